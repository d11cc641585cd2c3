"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of oracle/ua_oracle.c with one plausible mistake (a
dropped term, a wrong sign or index, a transposed operand, a wrong alignment),
compiled with gcc into a temporary directory and run through the quick pin
battery of tests/oracle_pins.py in a child process (a mutant may also read out
of bounds and crash, which counts as caught).  A mutant that passes every pin
means the pins have a blind spot.  CPU only; the oracle source itself is never
modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

MUTANTS = {
    "causal_top_left":        ("hi = ctx + i + 1;", "hi = i + 1;"),
    "causal_off_by_one":      ("hi = ctx + i + 1;", "hi = ctx + i;"),
    "ctx_off_by_one":         ("const int32_t ctx = kv_len - q_len;", "const int32_t ctx = kv_len - q_len + 1;"),
    "gqa_modulo_mapping":     ("h / (p->num_q_heads / p->num_kv_heads)", "h % p->num_kv_heads"),
    "page_index_swapped":     ("+ pos / p->block_size];", "+ pos % p->block_size];"),
    "slot_head_strides":      ("(int64_t)slot * p->kv_st_slot", "(int64_t)slot * p->kv_st_head"),
    "block_stride_dropped":   ("(int64_t)blk * p->kv_st_blk", "(int64_t)blk * p->kv_st_slot"),
    "scale_dropped":          ("z[j - lo] = p->scale * dot;", "z[j - lo] = dot;"),
    "k_scale_dropped":        ("* p->k_scale);", ");"),
    "v_scale_dropped":        ("* p->v_scale);", ");"),
    "lse_without_max":        ("*lse = m + log(denom);", "*lse = log(denom);"),
    "no_normalisation":       ("out[d] /= denom;", "out[d] /= 1.0;"),
    "q_head_stride":          ("(int64_t)h * p->q_st_head + d", "(int64_t)h * p->q_st_tok + d"),
    "seq_lookup_boundary":    ("t < p->cu_seqlens_q[s + 1]", "t <= p->cu_seqlens_q[s + 1]"),
    "fp8_bias":               ("ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 11)"),
    "fp8_subnormal":          ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "fp16_subnormal":         ("ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    "bf16_shift":             ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "combine_unweighted":     ("+= w * o_part", "+= o_part"),
    "combine_lse_without_max": ("lse[r] = L + log(wsum);", "lse[r] = log(wsum);"),
    "combine_no_normalise":   ("out[r * head_size + d] /= wsum;", "out[r * head_size + d] /= 1.0;"),
    "kv_range_ignored":       ("if (p->kv_hi >= 0 && p->kv_hi < hi)", "if (0)"),
    "window_left_off_by_one": ("lo = pos - p->win_left;", "lo = pos - p->win_left + 1;"),
    "window_left_ignored":    ("if (p->win_left >= 0 && pos - p->win_left > lo)", "if (0)"),
    "window_right_off_by_one": ("hi = pos + p->win_right + 1;", "hi = pos + p->win_right;"),
    "window_right_ignored":   ("if (p->win_right >= 0 && pos + p->win_right + 1 < hi)", "if (0)"),
    "alibi_sign":             ("z[j - lo] -= p->alibi[h]", "z[j - lo] += p->alibi[h]"),
    "alibi_from_context_start": ("fabs((double)(pos - j))", "fabs((double)(ctx - j))"),
    "alibi_without_abs":      ("fabs((double)(pos - j))", "((double)(pos - j))"),
    "alibi_kv_head_slope":    ("p->alibi[h] *", "p->alibi[g] *"),
    "alibi_before_scale":     ("z[j - lo] = p->scale * dot;\n        if (p->alibi)\n            z[j - lo] -= p->alibi[h] * fabs((double)(pos - j));",
                               "z[j - lo] = dot;\n        if (p->alibi)\n            z[j - lo] -= p->alibi[h] * fabs((double)(pos - j));\n        z[j - lo] *= p->scale;"),
}


@pytest.fixture(scope="module")
def src_text():
    with open(oracle.SRC) as f:
        return f.read()


def _battery_in_child(src_text, tmp_path):
    src = tmp_path / "mutant.c"
    src.write_text(src_text)
    so = oracle.build(force=True, src=str(src), out=str(tmp_path / "libmutant.so"))
    here = os.path.dirname(os.path.abspath(__file__))
    code = ("import sys; sys.path[:0] = [%r, %r]; import oracle, oracle_pins; "
            "oracle_pins.run_battery(oracle.load(%r))" % (here, os.path.dirname(here), so))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=300, env=env)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_unmutated_copy_passes(src_text, tmp_path):
    """Control: the same harness on an unmodified copy passes, so a failing
    mutant fails because of its mutation."""
    res = _battery_in_child(src_text, tmp_path)
    assert res.returncode == 0, res.stderr[-2000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, src_text, tmp_path):
    old, new = MUTANTS[name]
    assert src_text.count(old) == 1, f"mutation site for {name} not unique in the oracle"
    res = _battery_in_child(src_text.replace(old, new), tmp_path)
    assert res.returncode != 0, f"mutant {name} passed every pin"
