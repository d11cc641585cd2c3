"""CPU oracle for the KV-cache append (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, the smoke check in ``__graft_entry__.py`` and the CPU-baseline
leg of ``bench.py`` may import this module.  It shares no code with the GPU
library and imports nothing from it.

What it computes (page "flashatten takeaways EP2 工程", section "kv cache": a
sequence's cache grows by the new tokens' rows, K_{1:t+1} = [K_{1:t}; k_{t+1}];
page "vLLM Triton unified attention notes", section
kernel_unified_attention_2d: key position j of sequence s is slot j % bs of
physical block block_table[s][j / bs]): new token i of sequence s (packed row
cu_seqlens_q[s] + i) is written at key position kv_len(s) - q_len(s) + i, the
newest positions, as the attention's causal convention places the queries.

Stored value: a 16-bit cache receives the new row's bits unchanged; an fp8
e4m3fn cache receives, per element, the code nearest to x / scale computed in
float32 (the e4m3fn value set of the OCP format: bias 7, largest finite 448,
no infinities), ties to the code with an even mantissa, values beyond +-448
saturated.

Parity status: pinned by ``tests/test_append_oracle.py`` (hand-derived slot
positions in ``tests/golden/append_positions.json``, torch's saturating
float8_e4m3fn cast, round trips over all finite codes, untouched rows, page
relabelling).  Not "parity unpinned".
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np
import torch

from .bruteforce import decode_e4m3fn_table

_E4M3 = decode_e4m3fn_table()
_POS = _E4M3[:127].copy()        # codes 0x00 .. 0x7e: the non-negative finite values, increasing


def encode_e4m3fn(x: np.ndarray) -> np.ndarray:
    """uint8 e4m3fn codes nearest to the float32 values x (finite), ties to the
    code with an even mantissa, saturating at +-448; the sign of x (also of a
    value that rounds to zero) goes to bit 7."""
    x = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x).astype(np.float64), 448.0)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def _stored(row: torch.Tensor, cache_dtype: torch.dtype, scale: Optional[float]) -> torch.Tensor:
    """The cache content for one new [Hkv, D] row."""
    if cache_dtype == row.dtype:
        return row.clone()
    if cache_dtype != torch.float8_e4m3fn:
        raise TypeError(cache_dtype)
    xs = row.float().numpy() / np.float32(scale)          # float32 division, as stored
    return torch.from_numpy(encode_e4m3fn(xs)).view(torch.float8_e4m3fn)


def kv_append(k_new: torch.Tensor, v_new: torch.Tensor, cu_seqlens_q: torch.Tensor,
              seqused_k: torch.Tensor, block_table: torch.Tensor, k_cache: torch.Tensor,
              v_cache: torch.Tensor, k_scale: Optional[float] = None,
              v_scale: Optional[float] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Copies of k_cache / v_cache [NB, bs, Hkv, D] with the new tokens' rows of
    k_new / v_new [T, Hkv, D] written in (CPU tensors)."""
    kc, vc = k_cache.clone(), v_cache.clone()
    cu = cu_seqlens_q.numpy().astype(np.int64)
    kv = seqused_k.numpy().astype(np.int64)
    bt = block_table.numpy().astype(np.int64)
    bs = k_cache.shape[1]
    for s in range(len(kv)):
        q_len = cu[s + 1] - cu[s]
        for i in range(q_len):
            pos = kv[s] - q_len + i
            blk, slot = bt[s, pos // bs], pos % bs
            t = cu[s] + i
            kc[blk, slot] = _stored(k_new[t], k_cache.dtype, k_scale)
            vc[blk, slot] = _stored(v_new[t], v_cache.dtype, v_scale)
    return kc, vc
