"""CPU oracle for the fp8-compute mode of the attention call (TEST
INFRASTRUCTURE ONLY: only ``tests/``, the smoke check and the CPU-baseline leg
of ``bench.py`` may import it; it shares no code with the GPU library).

The mode (the fp8 attention variants of page "flashatten takeaways EP2 工程",
section "源代码接口"; the FA3 fp8 path of page "Fused Attention") runs the
query-key and weight-value products of sequences with q_len * (Hq / Hkv) > 32
rows on e4m3 operands: each query row (token, head) is replaced by e4m3 codes
of q / s with its own scale s = max|q_row| / 448 (float32 division; s = 1 for
an all-zero row), values clamped to +-448 and rounded to the nearest code,
ties to even.  That replacement is deterministic and is what this oracle
applies before the plain fp64 attention of ``oracle.attention``.  The second
rounding of the mode, of the softmax weights before the weight-value product,
depends on the kernel's running reference maximum and is not modelled: the
parity test bounds its effect instead.

Parity status: ``quantize_rows`` is pinned by tests/test_oracle.py (codes equal
torch's float8_e4m3fn cast of the same float32 quotients; the largest element
of a row maps to +-448; an all-zero row stays zero); the attention it feeds is
the pinned oracle.
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
