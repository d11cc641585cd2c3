"""Unified paged, variable-length attention forward for MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of
include/ua.h (libua.so, built in-tree by ``python -m
paged_varlen_flashattention_amd.build``).  This package is the thin Python
binding over that ABI: torch supplies device memory and the stream, nothing
else.  Calls raise when libua.so is missing; there is no CPU path.
"""
from ._binding import (ABI_VERSION, EXPORTS, LIB_PATH, UA_BF16, UA_ERR_HIP, UA_ERR_INVALID_ARG,
                       UA_ERR_UNSUPPORTED, UA_ERR_WORKSPACE, UA_FP16, UA_FP8_E4M3FN, UA_OK,
                       AppendParams, AttnParams, BwdParams, PlanInfo, UAError, attention_backward,
                       auto_splits, bwd_workspace_size, kv_append, make_bwd_params,
                       load_library, make_append_params, make_params, plan,
                       split_kv_combine, status_string, unified_attention, workspace_size,
                       UA_ERR_SCRATCH, NOALLOC_SCRATCH_BYTES, unified_attention_noalloc)

__all__ = ["ABI_VERSION", "EXPORTS", "LIB_PATH", "AppendParams", "AttnParams", "BwdParams", "PlanInfo",
           "attention_backward", "bwd_workspace_size", "make_bwd_params",
           "UAError", "auto_splits", "kv_append", "make_append_params", "load_library", "make_params", "plan", "split_kv_combine", "status_string",
           "unified_attention", "unified_attention_noalloc", "workspace_size", "UA_OK",
           "UA_ERR_SCRATCH", "NOALLOC_SCRATCH_BYTES", "UA_ERR_INVALID_ARG",
           "UA_ERR_UNSUPPORTED", "UA_ERR_WORKSPACE", "UA_ERR_HIP", "UA_BF16", "UA_FP16",
           "UA_FP8_E4M3FN"]
