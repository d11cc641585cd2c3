"""Pins of the fp8-compute oracle's second rounding: the softmax weights
rounded to e4m3fn before the weight-value product (page "flashatten takeaways
EP2 工程", section "源代码接口": the fp8 (e4m3) attention variants; page "Fused
Attention", the FA3 fp8 section).  CPU only.

What fixes the values here, independently of the oracle's code:
  * hand-checked roundings of chosen weights (ties to even, the subnormal
    range, the half-way point of the smallest subnormal);
  * torch's float8_e4m3fn cast (a library routine) on float32 inputs, which are
    exact in float64;
  * a designed batch (workloads.fp8_weight_pin_case) whose output element
    (row, d = j) is e4m3(w_j) / sum_k w_k for a single key j, with the weights
    in closed form 2^(-n/8) (rows of +1 queries) and 2^((n - 71)/8) (rows of
    -1 queries);
  * planted mistakes in copies of the rounding (flush of subnormals to zero,
    truncation toward zero), each of which must move that batch's expected
    output past the bound the GPU test applies.
"""
import numpy as np
import pytest
import torch

import oracle.fp8_compute as f8
import workloads as wk

# the GPU test's per-element bound on the designed batch: bf16 output rounding
# (unit roundoff 2^-8: 8 significant bits) plus the kernel's fp32 evaluation
# (relative 2^-16)
PIN_REL = 2.0 ** -8 + 2.0 ** -16


def pin_bound(ref):
    return PIN_REL * np.abs(ref)


@pytest.mark.parametrize("w,expect", [
    (0.0, 0.0),
    (1.0, 1.0),
    (1.0625, 1.0),              # half-way between 1 and 1.125: even mantissa (1.0)
    (1.1875, 1.25),             # half-way between 1.125 and 1.25: even mantissa (1.25)
    (0.3, 0.3125),              # 0.28125 < 0.3 < 0.3125, nearer the upper
    (2.0 ** -7, 2.0 ** -7),     # a subnormal, exact (4 * 2^-9)
    (3.4 * 2.0 ** -9, 3 * 2.0 ** -9),
    (3.6 * 2.0 ** -9, 4 * 2.0 ** -9),
    (1.5 * 2.0 ** -9, 2 * 2.0 ** -9),   # tie: code 2 is even
    (2.5 * 2.0 ** -9, 2 * 2.0 ** -9),   # tie: code 2 is even
    (2.0 ** -10, 0.0),          # half the smallest subnormal: ties to zero (even)
    (0.51 * 2.0 ** -9, 2.0 ** -9),
    (0.49 * 2.0 ** -9, 0.0),
    (7.6 * 2.0 ** -9, 2.0 ** -6),       # rounds up into the first normal binade
    (255.0, 256.0),             # 240 < 255 < 256: spacing 16 in [128, 256)
    (440.0, 448.0),
])
def test_round_weight_hand_checked(w, expect):
    assert f8.round_weight_e4m3(np.array([w]))[0] == expect


def test_round_weight_matches_torch_cast():
    # every float32 on a fine grid of [0, 448]: torch's float8_e4m3fn cast
    # rounds to nearest even; float32 inputs are exact in float64
    grid = np.concatenate([np.linspace(0, 2.0 ** -5, 20001), np.linspace(0, 2, 40001),
                           np.linspace(2, 448, 20001)]).astype(np.float32)
    ours = f8.round_weight_e4m3(grid.astype(np.float64))
    theirs = torch.from_numpy(grid).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, theirs)


@pytest.fixture(scope="module")
def pin():
    wl = wk.fp8_weight_pin_case()
    ref, ref_lse = f8.attention_rounded_weights(wl)
    return wl, ref, ref_lse


def closed_form(wl, row_sign):
    n = np.array([0] + wl.meta["n"], dtype=np.float64)
    w = 2.0 ** (-n / 8) if row_sign > 0 else 2.0 ** ((n - n.max()) / 8)
    return w


def test_pin_batch_against_closed_forms(pin):
    wl, ref, ref_lse = pin
    for t in range(wl.num_tokens):
        w = closed_form(wl, +1 if t % 2 == 0 else -1)
        want = f8.round_weight_e4m3(w) / w.sum()
        got = ref[t, 0]
        # d = j holds key j's rounded weight; key 0's value row is zero, and
        # d >= 64 is zero in every value row
        assert np.allclose(got[1:64], want[1:], rtol=1e-6, atol=0)
        assert np.all(got[0] == 0) and np.all(got[64:] == 0)
        zmax = 0.0 if t % 2 == 0 else max(wl.meta["n"]) * np.log(2.0) / 8
        assert abs(ref_lse[t, 0] - (zmax + np.log(w.sum()))) < 1e-6


def test_pin_batch_weights_far_from_rounding_boundaries(pin):
    # the kernel evaluates each weight in float32 (relative error well below
    # 1e-5 here); every weight sits at least 1e-3 (relative) away from an
    # e4m3 rounding boundary, so its rounded value is the same as the exact
    # weight's
    wl, _, _ = pin
    mids = (f8._POS[1:] + f8._POS[:-1]) / 2
    for sign in (+1, -1):
        w = closed_form(wl, sign)
        margin = np.min(np.abs(w[:, None] - mids[None, :]) / w[:, None], axis=1)
        assert margin.min() > 1e-3
        r = f8.round_weight_e4m3(w)
        assert ((w < 2.0 ** -6) & (r > 0)).sum() >= 15, "many subnormal weights are kept"
        assert (r > w).sum() >= 15 and (r < w).sum() >= 15, "rounding goes both ways"


def flush_subnormals(w):
    r = f8.round_weight_e4m3(w)
    return np.where(w < 2.0 ** -6, 0.0, r)


def toward_zero(w):
    pos = f8._POS
    i = np.clip(np.searchsorted(pos, w, side="right") - 1, 0, 126)
    return pos[i]


def toward_zero_subnormals_only(w):
    return np.where(w < 2.0 ** -6, toward_zero(w), f8.round_weight_e4m3(w))


@pytest.mark.parametrize("mutant", [flush_subnormals, toward_zero, toward_zero_subnormals_only])
def test_planted_rounding_mistakes_fail_the_bound(pin, mutant):
    wl, ref, _ = pin
    bad, _ = f8.attention_rounded_weights(wl, round_weights=mutant)
    assert np.any(np.abs(bad - ref) > pin_bound(ref)), mutant.__name__


def test_unmodified_copy_passes(pin):
    wl, ref, _ = pin
    again, _ = f8.attention_rounded_weights(wl, round_weights=lambda w: f8.round_weight_e4m3(w.copy()))
    assert np.all(np.abs(again - ref) <= pin_bound(ref))


def test_error_terms_closed_form_on_pin_batch(pin):
    # A = sum w |v| / sum w and B = sum_{w < 2^-6} min(w, 2^-10) |v| / sum w:
    # with one-hot values, element d = j is w_j / sum w and
    # [w_j < 2^-6] min(w_j, 2^-10) / sum w
    wl, _, _ = pin
    A, B, pre = f8.rounding_error_terms(wl)
    assert pre.all()
    for t in range(wl.num_tokens):
        w = closed_form(wl, +1 if t % 2 == 0 else -1)
        assert np.allclose(A[t, 0, 1:64], (w / w.sum())[1:], rtol=1e-6, atol=0)
        assert np.allclose(B[t, 0, 1:64], (np.where(w < 2.0 ** -6, np.minimum(w, 2.0 ** -10), 0) / w.sum())[1:], rtol=1e-6, atol=0)


def test_error_term_A_matches_c_oracle():
    # A by the dense numpy path equals the C oracle run on |V| (a second
    # implementation of sum w |v| / sum w)
    wl = wk.make_paged("f8terms", 4700, [1, 40, 70], [300, 40, 200], 8, 2, block_size=16,
                       kv_dtype="fp8_e4m3fn", causal=True)
    A, _, _ = f8.rounding_error_terms(wl)
    vabs = (wl.v_cache.view(torch.uint8) & 0x7F).view(torch.float8_e4m3fn)
    wv, _ = f8.attention_workload_fp8(wl, values=vabs)
    assert np.allclose(A, wv, rtol=1e-9, atol=1e-12)
