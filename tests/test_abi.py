"""The C-ABI library on the host: it loads, exports every symbol include/ua.h
declares, its structs match the binding, and every host-checkable violation
returns its documented status before any HIP call (ua_plan and the error paths
of ua_unified_attention / ua_split_kv_combine never touch a device, so fake,
never-dereferenced addresses are safe here).  CPU only."""
import ctypes
import math
import os
import re

import pytest

import paged_varlen_flashattention_amd as ua
from paged_varlen_flashattention_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ua.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libua.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ua_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return ua.load_library()


def test_exports_every_declared_symbol(lib):
    decl = declared_functions()
    assert decl, "no declarations parsed"
    assert sorted(ua.EXPORTS) == decl
    for name in decl:
        assert hasattr(lib, name), name


def test_struct_layout(lib):
    assert lib.ua_params_size() == ctypes.sizeof(B.AttnParams) == 240
    assert lib.ua_plan_info_size() == ctypes.sizeof(B.PlanInfo)
    assert lib.ua_abi_version() == B.ABI_VERSION


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4):
        assert lib.ua_status_string(st)
    assert lib.ua_status_string(12345) == b"unknown status"


FAKE = 1 << 20   # 16-byte (and 256-byte) aligned fake device address


def base_params(**kw):
    """A valid parameter set for config-3-like shapes with fake addresses."""
    p = B.AttnParams()
    lib = B.load_library()
    lib.ua_attn_params_init(ctypes.byref(p))
    p.q_dtype = p.kv_dtype = B.UA_BF16
    p.causal = 1
    for name in ("q", "k_cache", "v_cache", "out", "cu_seqlens_q", "seqused_k", "block_table"):
        setattr(p, name, FAKE)
    S, Hq, Hkv, D, bs = 256, 32, 8, 128, 16
    p.num_seqs, p.num_tokens, p.num_q_heads, p.num_kv_heads = S, S, Hq, Hkv
    p.head_size, p.block_size, p.num_blocks, p.block_table_stride = D, bs, 65536, 512
    p.q_stride_token, p.q_stride_head = Hq * D, D
    p.o_stride_token, p.o_stride_head = Hq * D, D
    p.kv_stride_block, p.kv_stride_slot, p.kv_stride_head = bs * Hkv * D, Hkv * D, D
    p.max_seqlen_q, p.max_seqlen_k = 1, 8192
    p.num_splits = 1
    p.softmax_scale = 1 / math.sqrt(128)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def plan_status(lib, p):
    info = B.PlanInfo()
    return lib.ua_plan(ctypes.byref(p), ctypes.byref(info)), info


def test_valid_plan_decode(lib):
    st, info = plan_status(lib, base_params())
    assert st == 0
    # every sequence has q_len * G = 4 <= 32 rows: only the decode kernel, one
    # workgroup per (sequence, kv head)
    assert info.kernels == 2 and info.grid_x == 0
    assert info.decode_grid_x == 256 * 8 and info.grid_y == 1 and info.num_waves == 4


def test_valid_plan_prefill(lib):
    p = base_params(num_seqs=4, num_tokens=16384, num_q_heads=32, num_kv_heads=32,
                    max_seqlen_q=4096, max_seqlen_k=4096, block_table_stride=256,
                    q_stride_token=32 * 128, o_stride_token=32 * 128,
                    kv_stride_block=16 * 32 * 128, kv_stride_slot=32 * 128)
    st, info = plan_status(lib, p)
    assert st == 0
    assert (info.block_m, info.block_q, info.tile_n, info.num_waves) == (128, 128, 64, 4)
    # prefill only: T - (S - 1) * max_seqlen_q = 4096 tokens, no sequence can
    # have q_len * G <= 32, so no decode workgroups are launched
    assert info.kernels == 1
    assert info.grid_x == (16384 // 128 + 4) * 32
    assert info.decode_grid_x == 0


def test_plan_gqa_block_q(lib):
    # G = 8: 128 rows = 16 tokens per prefill workgroup; q_len 2048 > 32 / 8
    p = base_params(num_seqs=68, num_tokens=8256, num_q_heads=64, num_kv_heads=8,
                    max_seqlen_q=2048, max_seqlen_k=16384, block_table_stride=1024,
                    q_stride_token=64 * 128, o_stride_token=64 * 128)
    st, info = plan_status(lib, p)
    assert st == 0 and info.block_q == 16 and info.kernels == 3
    assert info.grid_x == (8256 // 16 + 68) * 8 and info.decode_grid_x == 68 * 8


def test_plan_split_prefill_is_wide(lib):
    # long-context shape (query lens [1, 16], 131072 keys, 64/8 heads, 32
    # splits): the split launch with prefill work runs 8-wave workgroups; the
    # same call unsplit, and a decode-only split launch, keep 4 waves
    shape = dict(num_seqs=2, num_tokens=17, num_q_heads=64, num_kv_heads=8, max_seqlen_q=16,
                 max_seqlen_k=131072, block_table_stride=8192, num_blocks=16384,
                 q_stride_token=64 * 128, o_stride_token=64 * 128)
    need = lib.ua_workspace_size(17, 64, 128, 32)
    st, info = plan_status(lib, base_params(num_splits=32, workspace=FAKE, workspace_bytes=need,
                                            **shape))
    assert st == 0 and info.num_waves == 8 and info.num_splits == 32 and info.kernels == 3
    st, info = plan_status(lib, base_params(num_splits=1, **shape))
    assert st == 0 and info.num_waves == 4
    st, info = plan_status(lib, base_params(num_splits=8, workspace=FAKE,
                                            workspace_bytes=lib.ua_workspace_size(256, 32, 128, 8)))
    assert st == 0 and info.num_waves == 4 and info.kernels == 2


@pytest.mark.parametrize("field,value,status", [
    ("abi_version", 7, B.UA_ERR_INVALID_ARG),
    ("num_seqs", -1, B.UA_ERR_INVALID_ARG),
    ("num_tokens", -5, B.UA_ERR_INVALID_ARG),
    ("num_splits", 129, B.UA_ERR_INVALID_ARG),
    ("num_splits", -129, B.UA_ERR_INVALID_ARG),
    ("q_dtype", B.UA_FP8_E4M3FN, B.UA_ERR_UNSUPPORTED),
    ("q_dtype", 9, B.UA_ERR_INVALID_ARG),
    ("kv_dtype", B.UA_FP16, B.UA_ERR_UNSUPPORTED),
    ("kv_dtype", 9, B.UA_ERR_INVALID_ARG),
    ("head_size", 64, B.UA_ERR_UNSUPPORTED),
    ("head_size", 0, B.UA_ERR_INVALID_ARG),
    ("num_q_heads", 30, B.UA_ERR_INVALID_ARG),        # 30 % 8 != 0
    ("num_kv_heads", 0, B.UA_ERR_INVALID_ARG),
    ("block_size", 24, B.UA_ERR_UNSUPPORTED),
    ("block_size", 8, B.UA_ERR_UNSUPPORTED),
    ("block_size", 8192, B.UA_ERR_UNSUPPORTED),
    ("block_table_stride", 100, B.UA_ERR_INVALID_ARG),  # 100 * 16 < 8192
    ("softmax_scale", 0.0, B.UA_ERR_INVALID_ARG),
    ("softmax_scale", -0.1, B.UA_ERR_INVALID_ARG),
    ("softmax_scale", float("nan"), B.UA_ERR_INVALID_ARG),
    ("softmax_scale", float("inf"), B.UA_ERR_INVALID_ARG),
    ("causal", 2, B.UA_ERR_INVALID_ARG),
    ("q", None, B.UA_ERR_INVALID_ARG),
    ("k_cache", None, B.UA_ERR_INVALID_ARG),
    ("v_cache", None, B.UA_ERR_INVALID_ARG),
    ("out", None, B.UA_ERR_INVALID_ARG),
    ("cu_seqlens_q", None, B.UA_ERR_INVALID_ARG),
    ("seqused_k", None, B.UA_ERR_INVALID_ARG),
    ("block_table", None, B.UA_ERR_INVALID_ARG),
    ("q", FAKE + 8, B.UA_ERR_INVALID_ARG),             # not 16-byte aligned
    ("out", FAKE + 2, B.UA_ERR_INVALID_ARG),
    ("k_cache", FAKE + 4, B.UA_ERR_INVALID_ARG),
    ("lse_out", FAKE + 2, B.UA_ERR_INVALID_ARG),
    ("q_stride_head", 100, B.UA_ERR_INVALID_ARG),      # not a multiple of 8
    ("o_stride_token", 0, B.UA_ERR_INVALID_ARG),
    ("kv_stride_slot", -1024, B.UA_ERR_INVALID_ARG),
    ("kv_stride_slot", 1 << 26, B.UA_ERR_UNSUPPORTED),
    ("max_seqlen_q", -1, B.UA_ERR_INVALID_ARG),
    ("window_left", -2, B.UA_ERR_INVALID_ARG),
    ("window_right", -5, B.UA_ERR_INVALID_ARG),
    ("alibi_slopes", FAKE + 2, B.UA_ERR_INVALID_ARG),   # not 4-byte aligned
    ("fp8_compute", 2, B.UA_ERR_INVALID_ARG),
    ("test_barrier_timeout", 2, B.UA_ERR_INVALID_ARG),
    ("test_barrier_timeout", -1, B.UA_ERR_INVALID_ARG),
    ("fp8_compute", 1, B.UA_ERR_UNSUPPORTED),           # bf16 cache
])
def test_invalid_arguments(lib, field, value, status):
    p = base_params(**{field: value})
    st, info = plan_status(lib, p)
    assert st == status
    assert info.grid_x == 0
    # the launch entry point rejects the same call before touching HIP
    assert lib.ua_unified_attention(ctypes.byref(p), None) == status


def test_params_init_defaults(lib):
    p = B.AttnParams()
    ctypes.memset(ctypes.byref(p), 0xAB, ctypes.sizeof(p))
    lib.ua_attn_params_init(ctypes.byref(p))
    assert p.abi_version == B.ABI_VERSION and p.num_splits == 1
    assert (p.window_left, p.window_right) == (-1, -1)
    assert not p.alibi_slopes and not p.q and p.fp8_compute == 0 and p.test_barrier_timeout == 0
    lib.ua_attn_params_init(None)                           # no-op


def test_window_and_alibi_accepted(lib):
    assert plan_status(lib, base_params(window_left=0, window_right=0))[0] == B.UA_OK
    assert plan_status(lib, base_params(window_left=4096, window_right=-1,
                                        alibi_slopes=FAKE))[0] == B.UA_OK
    # ALiBi distances are exact in fp32 only below 2^24 positions
    p = base_params(alibi_slopes=FAKE, max_seqlen_k=(1 << 24) + 16,
                    block_table_stride=((1 << 24) + 16) // 16)
    assert plan_status(lib, p)[0] == B.UA_ERR_UNSUPPORTED


def test_fp8_compute_needs_fp8_cache_and_no_mask(lib):
    fp8 = dict(kv_dtype=B.UA_FP8_E4M3FN, k_scale=FAKE, v_scale=FAKE, fp8_compute=1)
    assert plan_status(lib, base_params(**fp8))[0] == B.UA_OK
    assert plan_status(lib, base_params(window_left=10, **fp8))[0] == B.UA_ERR_UNSUPPORTED
    assert plan_status(lib, base_params(alibi_slopes=FAKE, **fp8))[0] == B.UA_ERR_UNSUPPORTED


def test_fp8_requires_scales(lib):
    p = base_params(kv_dtype=B.UA_FP8_E4M3FN)
    assert plan_status(lib, p)[0] == B.UA_ERR_INVALID_ARG
    p = base_params(kv_dtype=B.UA_FP8_E4M3FN, k_scale=FAKE, v_scale=FAKE)
    assert plan_status(lib, p)[0] == B.UA_OK


def test_split_needs_workspace(lib):
    need = lib.ua_workspace_size(256, 32, 128, 8)
    assert need == 8 * 256 * 32 * 128 * 4 + 8 * 256 * 32 * 4
    assert plan_status(lib, base_params(num_splits=8))[0] == B.UA_ERR_WORKSPACE
    p = base_params(num_splits=8, workspace=FAKE, workspace_bytes=need - 1)
    assert plan_status(lib, p)[0] == B.UA_ERR_WORKSPACE
    p = base_params(num_splits=8, workspace=FAKE + 16, workspace_bytes=need)
    assert plan_status(lib, p)[0] == B.UA_ERR_WORKSPACE          # not 256-byte aligned
    p = base_params(num_splits=8, workspace=FAKE, workspace_bytes=need)
    st, info = plan_status(lib, p)
    assert st == 0 and info.num_splits == 8 and info.grid_y == 8
    assert lib.ua_unified_attention(ctypes.byref(base_params(num_splits=8)), None) == B.UA_ERR_WORKSPACE


MIXED = dict(num_seqs=68, num_tokens=8256, num_q_heads=64, num_kv_heads=8, max_seqlen_q=2048,
             max_seqlen_k=16384, block_table_stride=1024, q_stride_token=64 * 128,
             o_stride_token=64 * 128)


def test_plan_mixed_splits_decode_rows_only(lib):
    # 64 decode sequences + 4 prefill chunks of 2048 tokens (G = 8): automatic
    # choice keeps the prefill rows unsplit and splits the decode rows, one
    # split per 4096 keys of max_seqlen_k (16384 -> 4), in 4-wave workgroups
    # on a one-dimensional grid
    need = lib.ua_workspace_size(8256, 64, 128, 4)
    st, info = plan_status(lib, base_params(num_splits=0, workspace=FAKE, workspace_bytes=need,
                                            **MIXED))
    assert st == 0 and info.kernels == 7 and info.num_splits == 4 and info.num_waves == 4
    assert info.grid_y == 1 and info.decode_grid_x == 68 * 8 * 4
    p = base_params(num_splits=0, workspace=FAKE, workspace_bytes=1 << 40, **MIXED)
    p.max_seqlen_k, p.block_table_stride = 65536, 4096
    st, info = plan_status(lib, p)
    assert st == 0 and info.kernels == 7 and info.num_splits == 8          # at most 8
    assert info.grid_x == (8256 // 16 + 68) * 8
    # a workspace for 3 splits only: 3 decode splits; none: unsplit
    st, info = plan_status(lib, base_params(num_splits=0, workspace=FAKE,
                                            workspace_bytes=lib.ua_workspace_size(8256, 64, 128, 3),
                                            **MIXED))
    assert st == 0 and info.kernels == 7 and info.num_splits == 3
    st, info = plan_status(lib, base_params(num_splits=0, **MIXED))
    assert st == 0 and info.kernels == 3 and info.num_splits == 1 and info.decode_grid_x == 68 * 8
    # explicit -4: decode rows split 4 ways; -1: unsplit; 4: every row split
    st, info = plan_status(lib, base_params(num_splits=-4, workspace=FAKE,
                                            workspace_bytes=lib.ua_workspace_size(8256, 64, 128, 4),
                                            **MIXED))
    assert st == 0 and info.kernels == 7 and info.num_splits == 4 and info.grid_y == 1
    assert plan_status(lib, base_params(num_splits=-4, **MIXED))[0] == B.UA_ERR_WORKSPACE
    st, info = plan_status(lib, base_params(num_splits=-1, **MIXED))
    assert st == 0 and info.kernels == 3 and info.num_splits == 1
    st, info = plan_status(lib, base_params(num_splits=4, workspace=FAKE,
                                            workspace_bytes=lib.ua_workspace_size(8256, 64, 128, 4),
                                            **MIXED))
    assert st == 0 and info.kernels == 3 and info.grid_y == 4 and info.num_waves == 8


@pytest.mark.parametrize("extra,decode", [(5, False), (4, True), (0, True)])
def test_plan_decode_kernel_rule_gqa8(lib, extra, decode):
    # G = 8 (64 q heads, 8 kv heads): a sequence is a decode sequence when
    # q_len * 8 <= 32, i.e. q_len <= 4.  Three sequences, max_seqlen_q 100,
    # T = 200 + extra: the shortest has at least `extra` tokens, so the
    # decode kernel runs (bit 1, S x Hkv decode workgroups) only when extra <= 4
    p = base_params(num_seqs=3, num_tokens=200 + extra, num_q_heads=64, num_kv_heads=8,
                    max_seqlen_q=100, max_seqlen_k=2048,
                    q_stride_token=64 * 128, o_stride_token=64 * 128)
    st, info = plan_status(lib, p)
    assert st == 0 and info.kernels & 1 and bool(info.kernels & 2) == decode
    assert info.decode_grid_x == (3 * 8 if decode else 0) and info.num_splits == 1


def test_plan_no_decode_split_without_decode_rows(lib):
    # dense 4 x 4096 (G = 1): every sequence has 4096 tokens, none can be a
    # decode sequence, so automatic choice leaves the launch unsplit
    p = base_params(num_splits=0, num_seqs=4, num_tokens=16384, num_q_heads=32, num_kv_heads=32,
                    max_seqlen_q=4096, max_seqlen_k=4096, block_table_stride=256,
                    q_stride_token=32 * 128, o_stride_token=32 * 128,
                    kv_stride_block=16 * 32 * 128, kv_stride_slot=32 * 128,
                    workspace=FAKE, workspace_bytes=1 << 40)
    st, info = plan_status(lib, p)
    assert st == 0 and info.kernels == 1 and info.num_splits == 1
    # the bound T - (S - 1) * max_q <= 32 / G: 33 tokens left for the
    # shortest sequence rule a decode sequence out, 32 do not
    p.num_tokens = 3 * 4096 + 33
    st, info = plan_status(lib, p)
    assert st == 0 and info.kernels == 1 and info.num_splits == 1 and info.decode_grid_x == 0
    # an explicit decode-row split of a launch without decode rows runs unsplit
    p.num_splits = -4
    st, info = plan_status(lib, p)
    assert st == 0 and info.kernels == 1 and info.num_splits == 1
    p.num_splits = 0
    p.num_tokens = 3 * 4096 + 32
    p.max_seqlen_k, p.block_table_stride = 8192, 512
    st, info = plan_status(lib, p)
    assert st == 0 and info.kernels == 7 and info.num_splits == 2
    # decode-only launches: -n is an ordinary split
    st, info = plan_status(lib, base_params(num_splits=-4, workspace=FAKE,
                                            workspace_bytes=lib.ua_workspace_size(256, 32, 128, 4)))
    assert st == 0 and info.kernels == 2 and info.num_splits == 4 and info.grid_y == 4


def test_auto_splits_respect_workspace(lib):
    few = dict(num_seqs=16, num_tokens=16)                           # 128 workgroups unsplit
    st, info = plan_status(lib, base_params(num_splits=0, **few))
    assert st == 0 and info.num_splits == 1                        # no workspace: no split
    p = base_params(num_splits=0, workspace=FAKE, workspace_bytes=1 << 40, **few)
    st, info = plan_status(lib, p)
    assert st == 0 and 1 < info.num_splits <= 128
    small = lib.ua_workspace_size(16, 32, 128, 2)
    p = base_params(num_splits=0, workspace=FAKE, workspace_bytes=small, **few)
    st, info = plan_status(lib, p)
    assert st == 0 and info.num_splits == 2
    # decode-only: about 8 rounds of 2 workgroups per CU over 256 CUs (4096);
    # 256 x 8 (sequence, kv head) workgroups -> 2 splits, 4096 or more -> none
    p = base_params(num_splits=0, workspace=FAKE, workspace_bytes=1 << 40)
    st, info = plan_status(lib, p)
    assert st == 0 and info.num_splits == 2
    many = dict(num_seqs=512, num_tokens=512)
    p = base_params(num_splits=0, workspace=FAKE, workspace_bytes=1 << 40, **many)
    st, info = plan_status(lib, p)
    assert st == 0 and info.num_splits == 1


def test_workspace_size_edges(lib):
    assert lib.ua_workspace_size(256, 32, 128, 1) == 0
    assert lib.ua_workspace_size(0, 32, 128, 4) == 0
    assert lib.ua_workspace_size(17, 64, 128, 32) % 256 == 0


def test_empty_batch_is_noop(lib):
    p = base_params(num_seqs=0, q=None)
    assert plan_status(lib, p)[0] == B.UA_OK
    assert lib.ua_unified_attention(ctypes.byref(p), None) == B.UA_OK
    p = base_params(num_tokens=0, q=None)
    assert lib.ua_unified_attention(ctypes.byref(p), None) == B.UA_OK


def test_null_params(lib):
    info = B.PlanInfo()
    assert lib.ua_plan(None, ctypes.byref(info)) == B.UA_ERR_INVALID_ARG
    assert lib.ua_plan(ctypes.byref(base_params()), None) == B.UA_ERR_INVALID_ARG
    assert lib.ua_unified_attention(None, None) == B.UA_ERR_INVALID_ARG


@pytest.mark.parametrize("args,status", [
    (dict(num_splits=0), B.UA_ERR_INVALID_ARG),
    (dict(num_splits=129), B.UA_ERR_INVALID_ARG),
    (dict(head_size=64), B.UA_ERR_UNSUPPORTED),
    (dict(out_dtype=B.UA_FP8_E4M3FN), B.UA_ERR_UNSUPPORTED),
    (dict(out_dtype=7), B.UA_ERR_INVALID_ARG),
    (dict(o_partial=None), B.UA_ERR_INVALID_ARG),
    (dict(out=FAKE + 4), B.UA_ERR_INVALID_ARG),
    (dict(o_stride_head=12), B.UA_ERR_INVALID_ARG),
    (dict(num_tokens=0, o_partial=None), B.UA_OK),
])
def test_combine_invalid_arguments(lib, args, status):
    a = dict(o_partial=FAKE, lse_partial=FAKE, num_splits=4, num_tokens=17, num_q_heads=64,
             head_size=128, out=FAKE, out_dtype=B.UA_BF16, o_stride_token=64 * 128,
             o_stride_head=128, lse_out=None)
    a.update(args)
    st = lib.ua_split_kv_combine(a["o_partial"], a["lse_partial"], a["num_splits"], a["num_tokens"],
                                 a["num_q_heads"], a["head_size"], a["out"], a["out_dtype"],
                                 a["o_stride_token"], a["o_stride_head"], a["lse_out"], None)
    assert st == status


def test_binding_raises_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        B.load_library(str(tmp_path / "nope.so"))


# ------------------------------------------------------------------ ua_kv_append (host checks only)

def append_params(**kw):
    """A valid ua_append_params set with fake addresses (never launched here)."""
    p = B.AppendParams()
    p.abi_version = B.ABI_VERSION
    p.new_dtype = p.cache_dtype = B.UA_BF16
    for name in ("k_new", "v_new", "k_cache", "v_cache", "cu_seqlens_q", "seqused_k", "block_table"):
        setattr(p, name, FAKE)
    S, Hkv, D, bs = 4, 8, 128, 16
    p.num_seqs, p.num_tokens, p.num_kv_heads, p.head_size = S, 64, Hkv, D
    p.block_size, p.num_blocks, p.block_table_stride = bs, 1024, 64
    p.new_stride_token, p.new_stride_head = Hkv * D, D
    p.kv_stride_block, p.kv_stride_slot, p.kv_stride_head = bs * Hkv * D, Hkv * D, D
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_append_struct_layout(lib):
    assert lib.ua_append_params_size() == ctypes.sizeof(B.AppendParams) == 160


@pytest.mark.parametrize("field,value,status", [
    ("abi_version", 99, B.UA_ERR_INVALID_ARG),
    ("num_seqs", -1, B.UA_ERR_INVALID_ARG),
    ("num_tokens", -2, B.UA_ERR_INVALID_ARG),
    ("num_kv_heads", 0, B.UA_ERR_INVALID_ARG),
    ("head_size", 64, B.UA_ERR_UNSUPPORTED),
    ("block_size", 24, B.UA_ERR_INVALID_ARG),
    ("block_size", 8, B.UA_ERR_INVALID_ARG),
    ("new_dtype", B.UA_FP8_E4M3FN, B.UA_ERR_UNSUPPORTED),
    ("new_dtype", 7, B.UA_ERR_INVALID_ARG),
    ("cache_dtype", B.UA_FP16, B.UA_ERR_UNSUPPORTED),          # bf16 rows into an fp16 cache
    ("cache_dtype", 9, B.UA_ERR_INVALID_ARG),
    ("k_new", None, B.UA_ERR_INVALID_ARG),
    ("v_cache", None, B.UA_ERR_INVALID_ARG),
    ("block_table", None, B.UA_ERR_INVALID_ARG),
    ("new_stride_head", 100, B.UA_ERR_INVALID_ARG),
    ("kv_stride_slot", 0, B.UA_ERR_INVALID_ARG),
    ("k_cache", FAKE + 8, B.UA_ERR_INVALID_ARG),               # not 16-byte aligned
])
def test_append_invalid_args(lib, field, value, status):
    p = append_params(**{field: value})
    assert lib.ua_kv_append(ctypes.byref(p), None) == status


def test_append_fp8_needs_scales(lib):
    p = append_params(cache_dtype=B.UA_FP8_E4M3FN)
    assert lib.ua_kv_append(ctypes.byref(p), None) == B.UA_ERR_INVALID_ARG
    p = append_params(cache_dtype=B.UA_FP8_E4M3FN, k_scale=FAKE)
    assert lib.ua_kv_append(ctypes.byref(p), None) == B.UA_ERR_INVALID_ARG
    # both present, one not 4-byte aligned
    p = append_params(cache_dtype=B.UA_FP8_E4M3FN, k_scale=FAKE + 2, v_scale=FAKE)
    assert lib.ua_kv_append(ctypes.byref(p), None) == B.UA_ERR_INVALID_ARG


def test_append_empty_batch_is_noop(lib):
    assert lib.ua_kv_append(ctypes.byref(append_params(num_tokens=0, k_new=None)), None) == B.UA_OK
    assert lib.ua_kv_append(ctypes.byref(append_params(num_seqs=0, block_table=None)), None) == B.UA_OK
    assert lib.ua_kv_append(None, None) == B.UA_ERR_INVALID_ARG


# ---------------------------------------------------------------- backward

def bwd_params(**kw):
    p = B.BwdParams()
    p.abi_version = B.ABI_VERSION
    p.dtype = B.UA_BF16
    p.causal = 1
    p.softmax_scale = 0.088
    fake = 0x10000
    for name in ("q", "k", "v", "out", "dout", "lse", "cu_seqlens_q", "cu_seqlens_k", "dq", "dk", "dv",
                 "workspace"):
        setattr(p, name, fake)
        fake += 0x100000
    p.num_seqs, p.num_tokens, p.num_tokens_k = 2, 100, 300
    p.num_q_heads, p.num_kv_heads, p.head_size = 8, 2, 128
    p.workspace_bytes = lib_bwd_ws(100, 8)
    for k_, v_ in kw.items():
        setattr(p, k_, v_)
    return p


def lib_bwd_ws(T, Hq):
    return int(ua.load_library().ua_bwd_workspace_size(T, Hq))


def test_bwd_struct_layout(lib):
    assert lib.ua_bwd_params_size() == ctypes.sizeof(B.BwdParams) == 144


def test_bwd_workspace_size(lib):
    assert lib.ua_bwd_workspace_size(0, 8) == 0
    n = lib.ua_bwd_workspace_size(100, 8)
    assert n % 256 == 0 and n >= 2 * (100 * 8 + 64) * 4


@pytest.mark.parametrize("field,value,status", [
    ("abi_version", 99, B.UA_ERR_INVALID_ARG),
    ("dtype", B.UA_FP8_E4M3FN, B.UA_ERR_UNSUPPORTED),
    ("dtype", 7, B.UA_ERR_INVALID_ARG),
    ("causal", 2, B.UA_ERR_INVALID_ARG),
    ("head_size", 64, B.UA_ERR_UNSUPPORTED),
    ("num_kv_heads", 3, B.UA_ERR_INVALID_ARG),
    ("num_q_heads", 0, B.UA_ERR_INVALID_ARG),
    ("num_tokens", -1, B.UA_ERR_INVALID_ARG),
    ("softmax_scale", math.inf, B.UA_ERR_INVALID_ARG),
    ("q", None, B.UA_ERR_INVALID_ARG),
    ("dk", None, B.UA_ERR_INVALID_ARG),
    ("lse", None, B.UA_ERR_INVALID_ARG),
    ("cu_seqlens_k", None, B.UA_ERR_INVALID_ARG),
    ("dq", 0x10008, B.UA_ERR_INVALID_ARG),
    ("workspace", None, B.UA_ERR_WORKSPACE),
    ("workspace", 0x10010, B.UA_ERR_WORKSPACE),
    ("workspace_bytes", 1024, B.UA_ERR_WORKSPACE),
    ("num_tokens", 1 << 21, B.UA_ERR_UNSUPPORTED),
])
def test_bwd_invalid_arguments(lib, field, value, status):
    p = bwd_params(**{field: value})
    assert lib.ua_attention_backward(ctypes.byref(p), None) == status


def test_bwd_empty_is_noop(lib):
    assert lib.ua_attention_backward(ctypes.byref(bwd_params(num_seqs=0)), None) == B.UA_OK
    assert lib.ua_attention_backward(ctypes.byref(bwd_params(num_tokens=0, num_tokens_k=0)), None) == B.UA_OK
    assert lib.ua_attention_backward(None, None) == B.UA_ERR_INVALID_ARG


# ------------------------------------------------------------------ no-allocation entry point

def test_noalloc_rejects_splits_beyond_its_scratch(lib):
    # 256 rows x 32 heads: 128 splits need 128 * 256 * 32 * 129 * 4 B > 64 MiB
    p = base_params(num_splits=128)
    need = lib.ua_workspace_size(p.num_tokens, p.num_q_heads, 128, 128)
    assert need > B.NOALLOC_SCRATCH_BYTES
    assert lib.ua_unified_attention_noalloc(ctypes.byref(p), None) == B.UA_ERR_SCRATCH
    assert "scratch" in ua.status_string(B.UA_ERR_SCRATCH)


@pytest.mark.parametrize("field,value,status", [
    ("abi_version", 3, B.UA_ERR_INVALID_ARG),
    ("head_size", 64, B.UA_ERR_UNSUPPORTED),
    ("q", 0, B.UA_ERR_INVALID_ARG),
    ("num_splits", 129, B.UA_ERR_INVALID_ARG),
])
def test_noalloc_validates_like_the_workspace_entry(lib, field, value, status):
    p = base_params(**{field: value})
    assert lib.ua_unified_attention_noalloc(ctypes.byref(p), None) == status
    assert lib.ua_unified_attention_noalloc(None, None) == B.UA_ERR_INVALID_ARG


def test_noalloc_no_op_batches(lib):
    for kw in ({"num_seqs": 0}, {"num_tokens": 0}):
        assert lib.ua_unified_attention_noalloc(ctypes.byref(base_params(**kw)), None) == B.UA_OK
