"""ctypes binding of the C ABI in include/ua.h (argument marshalling only).

Every step of the attention runs in the HIP kernels of libua.so; this module
only turns torch tensors into device pointers, strides and the caller's current
HIP stream.  When libua.so is missing every entry point raises: there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libua.so")
ABI_VERSION = 5

UA_OK, UA_ERR_INVALID_ARG, UA_ERR_UNSUPPORTED, UA_ERR_WORKSPACE, UA_ERR_HIP = 0, -1, -2, -3, -4
UA_ERR_SCRATCH = -5
NOALLOC_SCRATCH_BYTES = 64 << 20      # UA_NOALLOC_SCRATCH_BYTES
UA_BF16, UA_FP16, UA_FP8_E4M3FN = 0, 1, 2
_DTYPES = {torch.bfloat16: UA_BF16, torch.float16: UA_FP16, torch.float8_e4m3fn: UA_FP8_E4M3FN}

# Every symbol include/ua.h declares.
EXPORTS = ("ua_unified_attention", "ua_split_kv_combine", "ua_workspace_size", "ua_plan",
           "ua_status_string", "ua_abi_version", "ua_params_size", "ua_plan_info_size",
           "ua_kv_append", "ua_append_params_size", "ua_attn_params_init",
           "ua_attention_backward", "ua_bwd_workspace_size", "ua_bwd_params_size",
           "ua_unified_attention_noalloc")


class UAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class AttnParams(ctypes.Structure):
    """Mirror of ua_attn_params (field order and types as in include/ua.h)."""
    _fields_ = [
        ("abi_version", ctypes.c_uint32), ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("cu_seqlens_q", ctypes.c_void_p),
        ("seqused_k", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p), ("lse_out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64),
        ("q_stride_token", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
        ("o_stride_token", ctypes.c_int64), ("o_stride_head", ctypes.c_int64),
        ("kv_stride_block", ctypes.c_int64), ("kv_stride_slot", ctypes.c_int64),
        ("kv_stride_head", ctypes.c_int64),
        ("num_seqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32), ("block_table_stride", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
        ("num_splits", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("window_left", ctypes.c_int32), ("window_right", ctypes.c_int32),
        ("alibi_slopes", ctypes.c_void_p),
        ("fp8_compute", ctypes.c_int32), ("test_barrier_timeout", ctypes.c_int32),
    ]


class BwdParams(ctypes.Structure):
    """Mirror of ua_bwd_params (field order and types as in include/ua.h)."""
    _fields_ = [
        ("abi_version", ctypes.c_uint32), ("dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("dout", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64),
        ("num_seqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
        ("num_tokens_k", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_size", ctypes.c_int32),
    ]


class AppendParams(ctypes.Structure):
    """Mirror of ua_append_params (field order and types as in include/ua.h)."""
    _fields_ = [
        ("abi_version", ctypes.c_uint32), ("new_dtype", ctypes.c_int32),
        ("cache_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p), ("seqused_k", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("new_stride_token", ctypes.c_int64), ("new_stride_head", ctypes.c_int64),
        ("kv_stride_block", ctypes.c_int64), ("kv_stride_slot", ctypes.c_int64),
        ("kv_stride_head", ctypes.c_int64),
        ("num_seqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_size", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
        ("block_table_stride", ctypes.c_int32), ("reserved2", ctypes.c_int32),
    ]


class PlanInfo(ctypes.Structure):
    """Mirror of ua_plan_info."""
    _fields_ = [("block_m", ctypes.c_int32), ("block_q", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("num_waves", ctypes.c_int32),
                ("num_splits", ctypes.c_int32), ("kernels", ctypes.c_int32),
                ("grid_x", ctypes.c_int64), ("grid_y", ctypes.c_int64),
                ("decode_grid_x", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}


_lib: Optional[ctypes.CDLL] = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libua.so (built by paged_varlen_flashattention_amd.build).  Raises if absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m paged_varlen_flashattention_amd.build`"
                           " (there is no fallback path)")
    lib = ctypes.CDLL(p)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.ua_unified_attention.argtypes = [ctypes.POINTER(AttnParams), vp]
    lib.ua_unified_attention.restype = ctypes.c_int
    lib.ua_unified_attention_noalloc.argtypes = [ctypes.POINTER(AttnParams), vp]
    lib.ua_unified_attention_noalloc.restype = ctypes.c_int
    lib.ua_split_kv_combine.argtypes = [vp, vp, i32, i32, i32, i32, vp, i32, i64, i64, vp, vp]
    lib.ua_split_kv_combine.restype = ctypes.c_int
    lib.ua_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.ua_workspace_size.restype = ctypes.c_size_t
    lib.ua_plan.argtypes = [ctypes.POINTER(AttnParams), ctypes.POINTER(PlanInfo)]
    lib.ua_plan.restype = ctypes.c_int
    lib.ua_status_string.argtypes = [i32]
    lib.ua_status_string.restype = ctypes.c_char_p
    lib.ua_abi_version.argtypes = []
    lib.ua_abi_version.restype = ctypes.c_uint32
    lib.ua_params_size.restype = ctypes.c_size_t
    lib.ua_plan_info_size.restype = ctypes.c_size_t
    lib.ua_kv_append.argtypes = [ctypes.POINTER(AppendParams), vp]
    lib.ua_kv_append.restype = ctypes.c_int
    lib.ua_append_params_size.restype = ctypes.c_size_t
    lib.ua_attn_params_init.argtypes = [ctypes.POINTER(AttnParams)]
    lib.ua_attn_params_init.restype = None
    lib.ua_attention_backward.argtypes = [ctypes.POINTER(BwdParams), vp]
    lib.ua_attention_backward.restype = ctypes.c_int
    lib.ua_bwd_workspace_size.argtypes = [i32, i32]
    lib.ua_bwd_workspace_size.restype = ctypes.c_size_t
    lib.ua_bwd_params_size.restype = ctypes.c_size_t
    if lib.ua_abi_version() != ABI_VERSION:
        raise RuntimeError("libua.so ABI version mismatch")
    if lib.ua_params_size() != ctypes.sizeof(AttnParams) or \
            lib.ua_plan_info_size() != ctypes.sizeof(PlanInfo) or \
            lib.ua_append_params_size() != ctypes.sizeof(AppendParams) or \
            lib.ua_bwd_params_size() != ctypes.sizeof(BwdParams):
        raise RuntimeError("libua.so struct layout differs from the binding")
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load_library().ua_status_string(status).decode()
    except RuntimeError:
        return "libua.so not loaded"


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def workspace_size(num_tokens: int, num_q_heads: int, head_size: int, num_splits: int) -> int:
    return int(load_library().ua_workspace_size(num_tokens, num_q_heads, head_size, num_splits))


def make_params(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table, max_seqlen_q,
                max_seqlen_k, softmax_scale, causal, k_scale=None, v_scale=None, num_splits=1,
                lse=None, workspace=None, window=(-1, -1), alibi_slopes=None,
                fp8_compute=False, test_barrier_timeout=False) -> AttnParams:
    """Fill ua_attn_params from tensors (no copies, no device work)."""
    p = AttnParams()
    p.abi_version = ABI_VERSION
    p.q_dtype = _DTYPES.get(q.dtype, 99)
    p.kv_dtype = _DTYPES.get(k_cache.dtype, 99)
    p.causal = int(bool(causal))
    p.q, p.k_cache, p.v_cache, p.out = q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr()
    p.cu_seqlens_q, p.seqused_k = cu_seqlens_q.data_ptr(), seqused_k.data_ptr()
    p.block_table = block_table.data_ptr()
    p.k_scale, p.v_scale, p.lse_out = _ptr(k_scale), _ptr(v_scale), _ptr(lse)
    p.workspace = _ptr(workspace)
    p.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    p.q_stride_token, p.q_stride_head = q.stride(0), q.stride(1)
    p.o_stride_token, p.o_stride_head = out.stride(0), out.stride(1)
    if k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must share strides")
    if q.stride(-1) != 1 or out.stride(-1) != 1 or k_cache.stride(-1) != 1:
        raise ValueError("head_size must be the unit-stride dimension")
    p.kv_stride_block, p.kv_stride_slot, p.kv_stride_head = k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)
    p.num_seqs = seqused_k.numel()
    p.num_tokens = q.shape[0]
    p.num_q_heads = q.shape[1]
    p.num_kv_heads = k_cache.shape[2]
    p.head_size = q.shape[2]
    p.block_size = k_cache.shape[1]
    p.num_blocks = k_cache.shape[0]
    p.block_table_stride = block_table.stride(0) if block_table.dim() == 2 else block_table.numel()
    p.max_seqlen_q = int(max_seqlen_q)
    p.max_seqlen_k = int(max_seqlen_k)
    p.num_splits = int(num_splits)
    p.softmax_scale = float(softmax_scale)
    p.window_left, p.window_right = int(window[0]), int(window[1])
    if alibi_slopes is not None and (alibi_slopes.dtype != torch.float32 or
                                     alibi_slopes.numel() != q.shape[1]):
        raise ValueError("alibi_slopes must be fp32 with one slope per query head")
    p.alibi_slopes = _ptr(alibi_slopes)
    p.fp8_compute = int(bool(fp8_compute))
    p.test_barrier_timeout = int(bool(test_barrier_timeout))
    return p


def plan(params: AttnParams) -> dict:
    """The launch ua_unified_attention would make (host only)."""
    info = PlanInfo()
    st = load_library().ua_plan(ctypes.byref(params), ctypes.byref(info))
    if st != UA_OK:
        raise UAError(st, "ua_plan")
    return info.as_dict()


def auto_splits(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table, max_seqlen_q,
                max_seqlen_k, softmax_scale, causal, k_scale=None, v_scale=None, window=(-1, -1),
                alibi_slopes=None) -> int:
    """The split the planner picks for num_splits = 0 given unlimited workspace
    (host only, no device work), as the num_splits value that asks for it
    explicitly: n for n splits of every row, -n when only the decode rows are
    split n ways."""
    probe = make_params(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table,
                        max_seqlen_q, max_seqlen_k, softmax_scale, causal, k_scale, v_scale, 0,
                        None, None, window, alibi_slopes)
    probe.workspace, probe.workspace_bytes = 256, 1 << 62
    info = plan(probe)
    return -info["num_splits"] if info["kernels"] & 4 else info["num_splits"]


def unified_attention(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table,
                      max_seqlen_q, max_seqlen_k, softmax_scale, causal, k_scale=None,
                      v_scale=None, num_splits=1, lse=None, workspace=None, stream=None,
                      window=(-1, -1), alibi_slopes=None, fp8_compute=False,
                      test_barrier_timeout=False):
    """ua_unified_attention on torch device tensors; writes `out` (and `lse`).

    q [T, Hq, 128] bf16/fp16; k_cache, v_cache [NB, bs, Hkv, 128] (q dtype or
    float8_e4m3fn); out like q; cu_seqlens_q [S+1] int32; seqused_k [S] int32;
    block_table [S, W] int32; k_scale / v_scale 1-element fp32 device tensors for
    fp8 caches; lse optional [T, Hq] fp32; window (left, right) local attention
    bounds (-1 = unbounded); alibi_slopes optional [Hq] fp32 device tensor;
    fp8_compute: with an fp8 cache, prefill rows on the fp8 matrix cores.
    num_splits: 0 = auto, 1 = none, n > 1 = every row split n ways, -n =
    only the decode sequences' rows split n ways.  With a split (or auto) a
    workspace of workspace_size(..., |num_splits|) bytes is allocated here when
    none is given.  Enqueued on `stream` (default: torch's current stream).
    """
    if workspace is None and num_splits not in (1, -1):
        splits = abs(num_splits)
        if splits == 0:
            splits = auto_splits(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table,
                                 max_seqlen_q, max_seqlen_k, softmax_scale, causal, k_scale,
                                 v_scale, window, alibi_slopes)
        nbytes = workspace_size(q.shape[0], q.shape[1], q.shape[2], splits)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    p = make_params(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table, max_seqlen_q,
                    max_seqlen_k, softmax_scale, causal, k_scale, v_scale, num_splits, lse, workspace,
                    window, alibi_slopes, fp8_compute, test_barrier_timeout)
    st = load_library().ua_unified_attention(ctypes.byref(p), _stream_handle(stream))
    if st != UA_OK:
        raise UAError(st, "ua_unified_attention")
    return out


def unified_attention_noalloc(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table,
                              max_seqlen_q, max_seqlen_k, softmax_scale, causal, k_scale=None,
                              v_scale=None, num_splits=1, lse=None, stream=None, window=(-1, -1),
                              alibi_slopes=None, fp8_compute=False):
    """ua_unified_attention_noalloc on torch device tensors: as
    unified_attention, with the split partials in the library's per-device
    scratch (nothing is allocated, here or in the library)."""
    p = make_params(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table, max_seqlen_q,
                    max_seqlen_k, softmax_scale, causal, k_scale, v_scale, num_splits, lse, None,
                    window, alibi_slopes, fp8_compute)
    st = load_library().ua_unified_attention_noalloc(ctypes.byref(p), _stream_handle(stream))
    if st != UA_OK:
        raise UAError(st, "ua_unified_attention_noalloc")
    return out


def make_append_params(k_new, v_new, k_cache, v_cache, cu_seqlens_q, seqused_k, block_table,
                       k_scale=None, v_scale=None) -> AppendParams:
    """Fill ua_append_params from tensors (no copies, no device work)."""
    p = AppendParams()
    p.abi_version = ABI_VERSION
    p.new_dtype = _DTYPES.get(k_new.dtype, 99)
    p.cache_dtype = _DTYPES.get(k_cache.dtype, 99)
    p.k_new, p.v_new = k_new.data_ptr(), v_new.data_ptr()
    p.k_cache, p.v_cache = k_cache.data_ptr(), v_cache.data_ptr()
    p.cu_seqlens_q, p.seqused_k = cu_seqlens_q.data_ptr(), seqused_k.data_ptr()
    p.block_table = block_table.data_ptr()
    p.k_scale, p.v_scale = _ptr(k_scale), _ptr(v_scale)
    if k_new.stride() != v_new.stride():
        raise ValueError("k_new and v_new must share strides")
    if k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must share strides")
    p.new_stride_token, p.new_stride_head = k_new.stride(0), k_new.stride(1)
    p.kv_stride_block, p.kv_stride_slot, p.kv_stride_head = k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)
    p.num_seqs = seqused_k.numel()
    p.num_tokens = k_new.shape[0]
    p.num_kv_heads = k_new.shape[1]
    p.head_size = k_new.shape[2]
    p.block_size = k_cache.shape[1]
    p.num_blocks = k_cache.shape[0]
    p.block_table_stride = block_table.stride(0) if block_table.dim() == 2 else block_table.numel()
    return p


def kv_append(k_new, v_new, k_cache, v_cache, cu_seqlens_q, seqused_k, block_table,
              k_scale=None, v_scale=None, stream=None):
    """ua_kv_append on torch device tensors: writes the new tokens' rows of
    k_new / v_new [T, Hkv, 128] (bf16/fp16) into k_cache / v_cache
    [NB, bs, Hkv, 128] (same dtype, or float8_e4m3fn with 1-element fp32
    k_scale / v_scale) at positions seqused_k - q_len + i."""
    p = make_append_params(k_new, v_new, k_cache, v_cache, cu_seqlens_q, seqused_k, block_table,
                           k_scale, v_scale)
    st = load_library().ua_kv_append(ctypes.byref(p), _stream_handle(stream))
    if st != UA_OK:
        raise UAError(st, "ua_kv_append")


def split_kv_combine(o_partial, lse_partial, out, lse=None, stream=None):
    """ua_split_kv_combine: o_partial [P, T, Hq, D] fp32, lse_partial [P, T, Hq] fp32
    (both contiguous) -> out [T, Hq, D] bf16/fp16 (and lse [T, Hq] fp32)."""
    if not (o_partial.is_contiguous() and lse_partial.is_contiguous()):
        raise ValueError("partials must be contiguous")
    P, T, Hq, D = o_partial.shape
    st = load_library().ua_split_kv_combine(
        o_partial.data_ptr(), lse_partial.data_ptr(), P, T, Hq, D, out.data_ptr(),
        _DTYPES.get(out.dtype, 99), out.stride(0), out.stride(1), _ptr(lse), _stream_handle(stream))
    if st != UA_OK:
        raise UAError(st, "ua_split_kv_combine")
    return out


def bwd_workspace_size(num_tokens: int, num_q_heads: int) -> int:
    return int(load_library().ua_bwd_workspace_size(num_tokens, num_q_heads))


def make_bwd_params(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, dq, dk, dv,
                    softmax_scale, causal, workspace=None) -> BwdParams:
    """ua_bwd_params for contiguous q, out, dout, dq [T, Hq, 128] and k, v, dk,
    dv [Tk, Hkv, 128] (bf16 or fp16), lse [T, Hq] fp32, cu_seqlens_q and
    cu_seqlens_k [S + 1] int32."""
    p = BwdParams()
    p.abi_version = ABI_VERSION
    p.dtype = _DTYPES.get(q.dtype, 99)
    p.causal = 1 if causal else 0
    p.softmax_scale = float(softmax_scale)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout), ("lse", lse),
                    ("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k),
                    ("dq", dq), ("dk", dk), ("dv", dv), ("workspace", workspace)):
        if t is not None and name not in ("cu_seqlens_q", "cu_seqlens_k", "workspace") \
                and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        setattr(p, name, _ptr(t))
    p.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    p.num_seqs = cu_seqlens_q.numel() - 1
    p.num_tokens = q.shape[0]
    p.num_tokens_k = k.shape[0]
    p.num_q_heads = q.shape[1]
    p.num_kv_heads = k.shape[1]
    p.head_size = q.shape[2]
    return p


def attention_backward(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, dq, dk, dv,
                       softmax_scale, causal, workspace=None, stream=None):
    """ua_attention_backward on torch device tensors (see make_bwd_params).
    Allocates the workspace when none is given."""
    if workspace is None:
        n = bwd_workspace_size(q.shape[0], q.shape[1])
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    p = make_bwd_params(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, dq, dk, dv,
                        softmax_scale, causal, workspace)
    st = load_library().ua_attention_backward(ctypes.byref(p), _stream_handle(stream))
    if st != UA_OK:
        raise UAError(st, "ua_attention_backward")
    return dq, dk, dv
