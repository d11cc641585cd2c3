"""The no-allocation entry point (ua_unified_attention_noalloc), called through
the C ABI, against the entry point it varies (ua_unified_attention with a
caller workspace): the same kernels, so the outputs must agree bit for bit,
and both with the oracle.  Two calls in a row, the second with a smaller
input, so the second reuses the scratch the first filled."""
import ctypes

import numpy as np
import pytest
import torch

import gpu_helpers as H
import paged_varlen_flashattention_amd as ua
from paged_varlen_flashattention_amd import _binding as B
import workloads as wk

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")]


def both(wl, splits):
    d = H.to_device(wl)
    T, Hq = wl.num_tokens, wl.num_q_heads
    outs = []
    for noalloc in (False, True):
        out = torch.full_like(d["q"], float("nan"))
        lse = torch.full((T, Hq), float("nan"), dtype=torch.float32, device="cuda")
        args = (d["q"], d["k_cache"], d["v_cache"], out, d["cu_seqlens_q"], d["seqused_k"], d["block_table"],
                wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale, wl.causal, d["k_scale"], d["v_scale"])
        if noalloc:
            ua.unified_attention_noalloc(*args, num_splits=splits, lse=lse)
        else:
            ws = torch.empty(max(1, B.workspace_size(T, Hq, 128, abs(splits))), dtype=torch.uint8,
                             device="cuda")
            ua.unified_attention(*args, num_splits=splits, lse=lse, workspace=ws)
        torch.cuda.synchronize()
        outs.append((out, lse))
    return outs


def test_noalloc_two_calls_second_smaller():
    cases = [
        # larger first: mixed decode and prefill rows, 32 splits (two key groups)
        (wk.make_paged("noalloc_a", 5000, [1, 70, 1, 200, 3], [2000, 900, 64, 1500, 40], 8, 2,
                       block_size=16, causal=True), 32),
        # then smaller: fewer rows, fewer splits, an fp8 cache
        (wk.make_paged("noalloc_b", 5001, [1, 40], [700, 300], 8, 2, block_size=32,
                       kv_dtype="fp8_e4m3fn", causal=True), 3),
    ]
    for wl, splits in cases:
        H.say(f"noalloc {wl.name} T={wl.num_tokens} splits={splits}")
        (o_ws, l_ws), (o_na, l_na) = both(wl, splits)
        assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16)), "outputs differ"
        assert torch.equal(l_ws, l_na), "lse differs"
        H.compare(wl, o_na, l_na, what=f"noalloc {wl.name}")


def test_noalloc_unsplit_and_auto():
    wl = wk.make_paged("noalloc_c", 5002, [1, 1, 1], [3000, 500, 64], 32, 8, block_size=16, causal=True)
    for splits in (1, 0):
        H.say(f"noalloc decode batch splits={splits}")
        out = torch.full_like(wl.q, float("nan"), device="cuda")
        lse = torch.full((wl.num_tokens, wl.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
        d = H.to_device(wl)
        ua.unified_attention_noalloc(d["q"], d["k_cache"], d["v_cache"], out, d["cu_seqlens_q"],
                                     d["seqused_k"], d["block_table"], wl.max_seqlen_q, wl.max_seqlen_k,
                                     wl.softmax_scale, wl.causal, num_splits=splits, lse=lse)
        torch.cuda.synchronize()
        H.compare(wl, out, lse, what=f"noalloc splits {splits}")


def test_noalloc_decode_rows_split():
    # a mixed batch whose decode rows alone are split (-4), then a smaller one
    # (-2): the scratch keeps only the decode rows' partials
    cases = [
        (wk.make_paged("noalloc_d", 5003, [1, 90, 1, 4], [3000, 700, 64, 2100], 64, 8, block_size=16,
                       causal=True), -4),
        (wk.make_paged("noalloc_e", 5004, [2, 50], [900, 60], 32, 8, block_size=32, causal=False), -2),
    ]
    for wl, splits in cases:
        info = H.plan(wl, splits)
        assert info.kernels & 4 and info.num_splits == -splits, info.as_dict()
        H.say(f"noalloc {wl.name} T={wl.num_tokens} decode-row splits={-splits}")
        (o_ws, l_ws), (o_na, l_na) = both(wl, splits)
        assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16)), "outputs differ"
        assert torch.equal(l_ws, l_na), "lse differs"
        H.compare(wl, o_na, l_na, what=f"noalloc {wl.name}")
