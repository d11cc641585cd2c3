"""CPU oracle for the fp8-compute mode of the attention call (TEST
INFRASTRUCTURE ONLY: only ``tests/``, the smoke check and the CPU-baseline leg
of ``bench.py`` may import it; it shares no code with the GPU library).

The mode (the fp8 attention variants of page "flashatten takeaways EP2 工程",
section "源代码接口"; the FA3 fp8 path of page "Fused Attention") runs the
query-key and weight-value products of sequences with q_len * (Hq / Hkv) > 32
rows on e4m3 operands, with two roundings:

1. each query row (token, head) is replaced by e4m3 codes of q / s with its
   own scale s = max|q_row| / 448 (float32 division; s = 1 for an all-zero
   row), values clamped to +-448 and rounded to the nearest code, ties to even
   (``quantize_rows``);
2. the softmax weights w_j = exp(z_j - z_ref), taken relative to a per-row
   reference z_ref, are rounded to the nearest e4m3fn value (ties to even,
   subnormals 2^-9 .. 7 * 2^-9 kept) before the weight-value product, while the
   normalising sum adds the unrounded weights:
       o = sum_j e4m3(w_j) v_j / sum_j w_j.
   The reference is the maximum of the first 64-key tile that holds a visible
   key, raised to a later tile's maximum only when that exceeds it by more
   than 8 in log2 units (our reading; the pages fix no quantisation of P).
   When a row's visible keys fit in one 64-key tile, or its first tile holds
   its maximum, the reference is the row's maximum score, and
   ``attention_rounded_weights`` computes the mode exactly (up to the
   rounding of the final output).

``attention_workload_fp8`` applies rounding 1 only, before the plain fp64
attention of ``oracle.attention``; parity tests on general batches bound the
effect of rounding 2 per element from the oracle's own weights.

Parity status: ``quantize_rows`` is pinned by tests/test_oracle.py (codes equal
torch's float8_e4m3fn cast of the same float32 quotients; the largest element
of a row maps to +-448; an all-zero row stays zero).  ``round_weight_e4m3`` and
``attention_rounded_weights`` are pinned by tests/test_fp8_weight_pin.py:
hand-checked roundings (ties to even, the subnormal range, the smallest
subnormal's half-way point), torch's float8_e4m3fn cast of exactly
representable float32 inputs, and a designed batch whose outputs isolate one
rounded weight per element against closed forms 2^(-n/8) / sum; planted
flush-to-zero and round-toward-zero copies of the rounding fail that batch's
bound.
"""
from __future__ import annotations

import numpy as np
import torch

from . import attention_workload
from .append import encode_e4m3fn
from .bruteforce import decode_e4m3fn_table, to_f64

_E4M3 = decode_e4m3fn_table()


def quantize_rows(q: torch.Tensor):
    """q [T, Hq, D] bf16/fp16 -> (codes uint8 [T, Hq, D], scales float32 [T, Hq],
    dequantised values float64 [T, Hq, D] = code value * scale)."""
    x = to_f64(q).astype(np.float32)                         # exact: 16-bit -> float32
    amax = np.abs(x).max(axis=-1)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    quot = (x / s[..., None]).astype(np.float32)              # float32 division
    quot = np.clip(quot, np.float32(-448.0), np.float32(448.0))
    codes = encode_e4m3fn(quot)
    deq = _E4M3[codes.astype(np.int64)] * s[..., None].astype(np.float64)
    return codes, s, deq


def prefill_rows_mask(wl) -> np.ndarray:
    """[T] bool: tokens of sequences with q_len * (Hq / Hkv) > 32 rows (the rows
    the mode applies to)."""
    cu = wl.cu_seqlens_q.numpy().astype(np.int64)
    G = wl.num_q_heads // wl.num_kv_heads
    mask = np.zeros(wl.num_tokens, dtype=bool)
    for s in range(wl.num_seqs):
        if (cu[s + 1] - cu[s]) * G > 32:
            mask[cu[s]:cu[s + 1]] = True
    return mask


def attention_workload_fp8(wl, rows=None, kv_range=None, threads=None, lib=None, values=None):
    """fp64 attention of the mode: queries of the prefill rows replaced by their
    e4m3 rounding (other rows unchanged).  values: optional replacement for
    the value cache (same dtype and shape), e.g. |V| for error bounds."""
    from workloads import Workload
    _, _, deq = quantize_rows(wl.q)
    q64 = torch.from_numpy(np.where(prefill_rows_mask(wl)[:, None, None], deq, to_f64(wl.q)))
    w = Workload(**{**wl.__dict__, "q": q64})
    if values is not None:
        w = Workload(**{**w.__dict__, "v_cache": values})
    return attention_workload(w, rows=rows, kv_range=kv_range, threads=threads, lib=lib)


def _dense_kv(wl, s: int, kl: int):
    """Keys and values 0 .. kl-1 of sequence s, gathered through its block table
    (position j: block table[s][j // bs], slot j % bs), decoded and scaled."""
    bs = wl.block_size
    bt = wl.block_table.numpy().astype(np.int64)
    ks = 1.0 if wl.k_scale is None else float(wl.k_scale)
    vs = 1.0 if wl.v_scale is None else float(wl.v_scale)
    K = np.stack([to_f64(wl.k_cache[bt[s, j // bs], j % bs]) for j in range(kl)]) * ks
    V = np.stack([to_f64(wl.v_cache[bt[s, j // bs], j % bs]) for j in range(kl)]) * vs
    return K, V


# codes 0 .. 126: zero and the positive finite e4m3fn values, increasing
_POS = _E4M3[:127]


def round_weight_e4m3(w: np.ndarray) -> np.ndarray:
    """Nearest e4m3fn value to each non-negative float64 weight w (w <= 448),
    ties to the code with an even mantissa; subnormals (multiples of 2^-9 below
    2^-6) are kept, weights below 2^-10 round to 0 and exactly 2^-10 ties to 0."""
    w = np.asarray(w, dtype=np.float64)
    hi = np.clip(np.searchsorted(_POS, w, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = w - _POS[lo]
    d_hi = _POS[hi] - w
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(pick_hi, _POS[hi], _POS[lo])


def attention_rounded_weights(wl, round_weights=round_weight_e4m3):
    """fp64 output [T, Hq, D] and natural-log LSE [T, Hq] of the mode with both
    roundings: prefill rows (q_len * G > 32) use their e4m3-rounded query and
    o = sum_j round_weights(w_j) v_j / sum_j w_j with w_j = exp(z_j - max z);
    other rows are plain attention.  Exact when each prefill row's reference
    is its maximum; this function requires every sequence's keys to fit one
    64-key tile (kv_len <= 64), which guarantees it.  Dense per-sequence
    numpy (small batches only)."""
    kv_lens = wl.kv_lens
    if kv_lens.max(initial=0) > 64:
        raise ValueError("rounded-weight oracle needs every kv_len <= 64 (one tile)")
    _, _, deq = quantize_rows(wl.q)
    pre = prefill_rows_mask(wl)
    q64 = np.where(pre[:, None, None], deq, to_f64(wl.q))
    cu = wl.cu_seqlens_q.numpy().astype(np.int64)
    T, Hq, D = q64.shape
    G = Hq // wl.num_kv_heads
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    for s in range(wl.num_seqs):
        ql, kl = int(cu[s + 1] - cu[s]), int(kv_lens[s])
        if ql == 0:
            continue
        K, V = _dense_kv(wl, s, kl)                 # [kl, Hkv, D] float64, scales applied
        for i in range(ql):
            t = int(cu[s]) + i
            vis = np.arange(kl) <= (kl - ql + i) if wl.causal else np.ones(kl, dtype=bool)
            for h in range(Hq):
                g = h // G
                z = wl.softmax_scale * (K[:, g, :] @ q64[t, h])
                z = np.where(vis, z, -np.inf)
                zmax = z.max()
                w = np.exp(z - zmax)
                wr = round_weights(w) if pre[t] else w
                out[t, h] = (wr[:, None] * V[:, g, :]).sum(axis=0) / w.sum()
                lse[t, h] = zmax + np.log(w.sum())
    return out, lse


def rounding_error_terms(wl):
    """Per output element, the two sums that bound the effect of the weight
    rounding for any running reference (dense per-sequence numpy, small and
    moderate batches):

        A = sum_j w_j |v_j| / sum_j w_j,
        B = sum_{j : w_j < 2^-6} min(w_j, 2^-10) |v_j| / sum_j w_j,

    with w_j = exp(z_j - max z) over the row's visible keys (prefill rows with
    their e4m3-rounded query).  The kernel rounds w'_j = 2^(x_j - m) against
    a reference m <= max z, so w'_j >= w_j, and later rescales it by a = 2^(m
    - M) <= 1 to the final reference M, where u_j = a w'_j and the final sum
    is L = sum u_j >= sum w_j with u_j / L = w_j / sum w.  Rounding to
    nearest e4m3 moves a normal weight by at most 2^-4 w'_j (contributing
    2^-4 u_j / L) and a subnormal one (w'_j < 2^-6, hence w_j < 2^-6) by at
    most min(w'_j, 2^-10) (contributing at most min(u_j, 2^-10) / L <=
    min(w_j, 2^-10) / sum w).  So the output moves by at most 2^-4 A + B.
    Returns (A, B, prefill mask [T]) with A, B float64 [T, Hq, D]."""
    _, _, deq = quantize_rows(wl.q)
    pre = prefill_rows_mask(wl)
    q64 = np.where(pre[:, None, None], deq, to_f64(wl.q))
    cu = wl.cu_seqlens_q.numpy().astype(np.int64)
    T, Hq, D = q64.shape
    G = Hq // wl.num_kv_heads
    A = np.zeros((T, Hq, D))
    B = np.zeros((T, Hq, D))
    for s in range(wl.num_seqs):
        ql, kl = int(cu[s + 1] - cu[s]), int(wl.kv_lens[s])
        if ql == 0:
            continue
        K, V = _dense_kv(wl, s, kl)
        Kh = np.repeat(K, G, axis=1)                           # [kl, Hq, D]
        Vh = np.abs(np.repeat(V, G, axis=1))
        z = np.einsum("ihd,jhd->hij", q64[cu[s]:cu[s + 1]], Kh) * wl.softmax_scale
        vis = np.ones((ql, kl), dtype=bool)
        if wl.causal:
            vis = np.arange(kl)[None, :] <= (kl - ql + np.arange(ql))[:, None]
        z = np.where(vis[None], z, -np.inf)
        w = np.exp(z - z.max(axis=-1, keepdims=True))          # [Hq, ql, kl]
        den = w.sum(axis=-1, keepdims=True)
        A[cu[s]:cu[s + 1]] = np.einsum("hij,jhd->ihd", w / den, Vh)
        small = np.where(w < 2.0 ** -6, np.minimum(w, 2.0 ** -10), 0.0) / den
        B[cu[s]:cu[s + 1]] = np.einsum("hij,jhd->ihd", small, Vh)
    return A, B, pre
