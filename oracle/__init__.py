"""CPU fp64 oracle for paged, variable-length attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may import this
package.  It shares no code with the GPU library (``paged_varlen_flashattention_amd``)
and imports nothing from it: it consumes the same seeded inputs
(``workloads.py``) and computes the plain definition of attention over a paged
KV cache in double precision.

Two independent implementations live here:

* ``ua_oracle.c`` (loaded through ctypes): per-row loops over visible keys,
  gathering K/V through the block table (see its header for the passages of the
  pages each step follows);
* ``bruteforce.py`` (numpy): materialises each sequence's dense K/V, builds the
  full score matrix, masks it and applies softmax.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle.py`` against closed forms, invariants, torch's fp64
scaled-dot-product attention and float8/bfloat16 casts, brute force, and
planted mutants.  No function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "ua_oracle.c")
LIB = os.path.join(_HERE, "libua_oracle.so")

UAO_BF16, UAO_FP16, UAO_FP8_E4M3FN, UAO_F64 = 0, 1, 2, 3
_DTYPE_CODES = {torch.bfloat16: UAO_BF16, torch.float16: UAO_FP16,
                torch.float8_e4m3fn: UAO_FP8_E4M3FN, torch.float64: UAO_F64}
_NAME_CODES = {"bf16": UAO_BF16, "fp16": UAO_FP16, "fp8_e4m3fn": UAO_FP8_E4M3FN}

_lib = None


def build(force: bool = True, src: str = SRC, out: str = LIB) -> str:
    """Compile the C oracle with gcc (plain -O2, no fast-math: IEEE double semantics)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    p, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.uao_attention.argtypes = [p, ctypes.c_int, i64, i64, p, p, ctypes.c_int, i64, i64, i64,
                                  p, p, p, i64, i32, i32, i32, i32, i32, dbl, ctypes.c_int,
                                  dbl, dbl, i32, i32, p, i64, p, p, ctypes.c_int]
    lib.uao_attention.restype = ctypes.c_int
    lib.uao_attention_ex.argtypes = [p, ctypes.c_int, i64, i64, p, p, ctypes.c_int, i64, i64, i64,
                                     p, p, p, i64, i32, i32, i32, i32, i32, dbl, ctypes.c_int,
                                     dbl, dbl, i32, i32, i32, i32, p, p, i64, p, p, ctypes.c_int]
    lib.uao_attention_ex.restype = ctypes.c_int
    lib.uao_combine.argtypes = [p, p, i32, i64, i32, p, p]
    lib.uao_combine.restype = ctypes.c_int
    lib.uao_decode.argtypes = [ctypes.c_int, p, p, i64]
    lib.uao_decode.restype = ctypes.c_int
    return lib


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the compiled oracle (building it first if it is missing or stale)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        build(force=False)
        _lib = _bind(ctypes.CDLL(LIB))
    return _lib


def _ptr(a) -> int:
    return a.data_ptr() if isinstance(a, torch.Tensor) else a.ctypes.data


def decode(raw: torch.Tensor, lib: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """Decode stored bf16 / fp16 / fp8_e4m3fn values to float64 with the C decoder."""
    lib = lib or load()
    raw = raw.contiguous()
    out = np.empty(raw.numel(), dtype=np.float64)
    rc = lib.uao_decode(_DTYPE_CODES[raw.dtype], raw.data_ptr(), out.ctypes.data, raw.numel())
    assert rc == 0
    return out.reshape(tuple(raw.shape))


def attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
              cu_seqlens_q: torch.Tensor, seqused_k: torch.Tensor, block_table: torch.Tensor,
              softmax_scale: float, causal: bool, k_scale: Optional[float] = None,
              v_scale: Optional[float] = None, rows: Optional[np.ndarray] = None,
              kv_range: Optional[Tuple[int, int]] = None, threads: Optional[int] = None,
              lib: Optional[ctypes.CDLL] = None, window: Tuple[int, int] = (-1, -1),
              alibi_slopes=None) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 attention over a paged KV cache.

    q [T, Hq, D] (bf16/fp16, or float64 for queries given exactly; any
    token/head strides, unit d stride);
    k_cache, v_cache [NB, bs, Hkv, D] (bf16/fp16/fp8_e4m3fn, unit d stride);
    cu_seqlens_q [S+1] int32; seqused_k [S] int32; block_table [S, W] int32.
    rows: optional int array [n, 2] of (token, head); default all rows,
    token-major.  kv_range=(lo, hi) restricts keys to absolute positions
    [lo, hi) (hi < 0: unbounded), which gives one split's partial result.
    window=(left, right): local attention, keys pos - left .. pos + right of
    the query at absolute position pos (negative: unbounded); alibi_slopes:
    [Hq] slopes, logit of key j minus slope[h] * |pos - j| (after the scale).
    Returns out [n, D] (or [T, Hq, D] for all rows) and lse [n] (or [T, Hq]),
    natural log.
    """
    lib = lib or load()
    for t in (q, k_cache, v_cache):
        if t.numel() and t.stride(-1) != 1:          # an empty tensor has no layout to check
            raise ValueError("unit stride along head_size required")
    if k_cache.stride() != v_cache.stride() or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must share dtype and strides")
    cu = cu_seqlens_q.to(torch.int32).contiguous()
    kv = seqused_k.to(torch.int32).contiguous()
    bt = block_table.to(torch.int32).contiguous()
    T, Hq, D = q.shape
    S = kv.numel()
    Hkv, bs = k_cache.shape[2], k_cache.shape[1]
    if rows is None:
        rows_arr = None
        n = T * Hq
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
        n = rows_arr.shape[0]
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    lo, hi = kv_range if kv_range is not None else (0, -1)
    fp8 = k_cache.dtype == torch.float8_e4m3fn
    if fp8 and (k_scale is None or v_scale is None):
        raise ValueError("fp8 KV needs k_scale and v_scale")
    if alibi_slopes is not None:
        alibi = np.ascontiguousarray(np.asarray(
            alibi_slopes.numpy() if isinstance(alibi_slopes, torch.Tensor) else alibi_slopes,
            dtype=np.float64).reshape(-1))
        if alibi.shape[0] != Hq:
            raise ValueError("alibi_slopes needs one slope per query head")
    else:
        alibi = None
    rc = lib.uao_attention_ex(
        q.data_ptr(), _DTYPE_CODES[q.dtype], q.stride(0), q.stride(1),
        k_cache.data_ptr(), v_cache.data_ptr(), _DTYPE_CODES[k_cache.dtype],
        k_cache.stride(0), k_cache.stride(1), k_cache.stride(2),
        cu.data_ptr(), kv.data_ptr(), bt.data_ptr(), bt.stride(0) if bt.dim() == 2 else 0,
        S, Hq, Hkv, D, bs, float(softmax_scale), int(bool(causal)),
        float(k_scale) if fp8 else 1.0, float(v_scale) if fp8 else 1.0,
        int(lo), int(hi), int(window[0]), int(window[1]),
        alibi.ctypes.data if alibi is not None else None,
        rows_arr.ctypes.data if rows_arr is not None else None, n,
        out.ctypes.data, lse.ctypes.data, int(threads or os.cpu_count() or 1))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    if rows is None:
        return out.reshape(T, Hq, D), lse.reshape(T, Hq)
    return out, lse


def attention_workload(wl, rows=None, kv_range=None, threads=None, lib=None):
    """attention() on any object with the fields of workloads.Workload."""
    return attention(wl.q, wl.k_cache, wl.v_cache, wl.cu_seqlens_q, wl.seqused_k, wl.block_table,
                     wl.softmax_scale, wl.causal, wl.k_scale, wl.v_scale, rows=rows,
                     kv_range=kv_range, threads=threads, lib=lib,
                     window=(getattr(wl, "window_left", -1), getattr(wl, "window_right", -1)),
                     alibi_slopes=getattr(wl, "alibi_slopes", None))


def combine(o_part: np.ndarray, lse_part: np.ndarray,
            lib: Optional[ctypes.CDLL] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Log-sum-exp merge of split partials: o_part [P, n, D], lse_part [P, n] (float64)."""
    lib = lib or load()
    o_part = np.ascontiguousarray(o_part, dtype=np.float64)
    lse_part = np.ascontiguousarray(lse_part, dtype=np.float64)
    P, n, D = o_part.shape
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    rc = lib.uao_combine(o_part.ctypes.data, lse_part.ctypes.data, P, n, D,
                         out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out, lse
