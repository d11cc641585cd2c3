"""The backward oracle against its pins, and planted mistakes against the pins.

A mutant is a copy of oracle/backward.py with one plausible mistake (a dropped
term, a wrong sign, a missing scale, the wrong operand or head mapping, an
overwrite instead of a sum), executed from a string; every mutant must fail
some pin of tests/backward_pins.py.  CPU only; the oracle source is never
modified.
"""
import os
import types

import numpy as np
import pytest

import backward_pins as pins
from oracle import backward


@pytest.mark.parametrize("check", pins.BATTERY, ids=lambda c: c.__name__)
def test_backward_oracle_pin(check):
    check(backward.attention_backward)


def test_backward_outputs_match_forward_oracle():
    # the backward's own O and LSE agree with the brute-force forward
    q, k, v, do, cq, ck, scale = pins._batch(41, [3, 8], [7, 8], 4, 2, 8)
    for causal in (True, False):
        got = backward.attention_backward(q, k, v, do, cq, ck, scale, causal)
        out = pins._forward_bruteforce(q, k, v, cq, ck, scale, causal)
        assert np.abs(got["out"] - out).max() < 1e-12


MUTANTS = {
    "delta_dropped":     ("dS = P * (dP - delta[:, None])", "dS = P * dP"),
    "ds_sign":           ("dS = P * (dP - delta[:, None])", "dS = P * (delta[:, None] - dP)"),
    "dk_scale_dropped":  ('res["dk"][k0:k1, g] += scale * (dS.T @ Qh)', 'res["dk"][k0:k1, g] += dS.T @ Qh'),
    "dq_with_values":    ('res["dq"][q0:q1, h] = scale * (dS @ Kg)', 'res["dq"][q0:q1, h] = scale * (dS @ Vg)'),
    "dk_overwritten":    ('res["dk"][k0:k1, g] += scale', 'res["dk"][k0:k1, g] = scale'),
    "dv_overwritten":    ('res["dv"][k0:k1, g] += P.T @ dOh', 'res["dv"][k0:k1, g] = P.T @ dOh'),
    "gqa_modulo":        ("g = h // G", "g = h % Hkv"),
    "causal_top_left":   ("pos = (kl - ql) + np.arange(ql)[:, None]", "pos = np.arange(ql)[:, None]"),
    "dp_with_keys":      ("dP = dOh @ Vg.T", "dP = dOh @ Kg.T"),
    "delta_from_dout":   ("delta = (O * dOh).sum(axis=1)", "delta = dOh.sum(axis=1)"),
}


@pytest.fixture(scope="module")
def src_text():
    with open(os.path.join(os.path.dirname(backward.__file__), "backward.py")) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_is_caught(src_text, name):
    old, new = MUTANTS[name]
    assert src_text.count(old) == 1, f"mutation site of {name} not unique"
    text = src_text.replace(old, new).replace("from .bruteforce import", "from oracle.bruteforce import")
    mod = types.ModuleType(f"backward_mutant_{name}")
    exec(compile(text, f"<mutant {name}>", "exec"), mod.__dict__)
    caught = []
    for check in pins.BATTERY:
        try:
            check(mod.attention_backward)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"mutant {name} passes every backward pin"
