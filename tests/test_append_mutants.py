"""Planted mistakes in the append oracle must be caught by its pins.

Each mutant is a copy of oracle/append.py with one plausible mistake, placed
in a temporary copy of the oracle package; tests/test_append_oracle.py then
runs against that copy in a child process and must fail.  An unmodified copy
must pass.  CPU only; the oracle itself is never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

MUTANTS = {
    "position_off_by_one":  ("pos = kv[s] - q_len + i", "pos = kv[s] - q_len + i + 1"),
    "oldest_positions":     ("pos = kv[s] - q_len + i", "pos = i"),
    "page_slot_swapped":    ("blk, slot = bt[s, pos // bs], pos % bs", "blk, slot = bt[s, pos % bs], pos // bs"),
    "ties_away_from_zero":  ("((d_hi == d_lo) & (hi % 2 == 0))", "(d_hi == d_lo)"),
    "ties_toward_zero":     ("((d_hi == d_lo) & (hi % 2 == 0))", "False"),
    "no_subnormal_codes":   ("_POS = _E4M3[:127].copy()", "_POS = np.concatenate([[0.0], _E4M3[8:127]])"),
    "sign_dropped":         ("np.where(np.signbit(x), code | 0x80, code)", "code"),
    "scale_multiplied":     ("row.float().numpy() / np.float32(scale)", "row.float().numpy() * np.float32(scale)"),
    "k_into_v":             ("vc[blk, slot] = _stored(v_new[t]", "vc[blk, slot] = _stored(k_new[t]"),
}


def _run_pins(tmp_path, text):
    pkg = tmp_path / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), pkg,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__", "*.tmp"))
    (pkg / "append.py").write_text(text)
    tests = tmp_path / "tests"
    shutil.copytree(os.path.join(HERE, "golden"), tests / "golden")
    shutil.copy(os.path.join(HERE, "test_append_oracle.py"), tests)
    env = dict(os.environ, PYTHONPATH=str(tmp_path), OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           str(tests / "test_append_oracle.py")],
                          capture_output=True, text=True, env=env, cwd=str(tmp_path), timeout=300)


@pytest.fixture(scope="module")
def src_text():
    with open(os.path.join(ROOT, "oracle", "append.py")) as f:
        return f.read()


def test_unmutated_copy_passes(src_text, tmp_path):
    r = _run_pins(tmp_path, src_text)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, src_text, tmp_path):
    old, new = MUTANTS[name]
    assert src_text.count(old) == 1, f"mutation site for {name} not found exactly once"
    r = _run_pins(tmp_path, src_text.replace(old, new))
    assert r.returncode != 0, f"mutant {name} passed every pin"
