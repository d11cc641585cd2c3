"""Parity of the KV-cache append (ua_kv_append through the C ABI) with the
oracle in oracle/append.py: the whole caches after the append, bit for bit
(16-bit caches receive the rows unchanged; fp8 caches the saturating,
round-to-nearest-even e4m3fn codes of x / scale, an integer decision taken in
float32 on both sides).  Every other cache row must be left as it was.
"""
import numpy as np
import pytest
import torch

import gpu_helpers as H
import oracle
import oracle.append as oa
import paged_varlen_flashattention_amd as ua
import workloads as wk

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")]


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.contiguous().cpu()
    return (t.view(torch.uint8) if t.element_size() == 1 else t.view(torch.int16)).numpy()


def run_append(c, dev="cuda", k_new=None, v_new=None):
    kn = (c["k_new"] if k_new is None else k_new).to(dev)
    vn = (c["v_new"] if v_new is None else v_new).to(dev)
    kc, vc = c["k_cache"].to(dev), c["v_cache"].to(dev)
    ks = None if c["k_scale"] is None else torch.tensor([c["k_scale"]], dtype=torch.float32, device=dev)
    vs = None if c["v_scale"] is None else torch.tensor([c["v_scale"]], dtype=torch.float32, device=dev)
    ua.kv_append(kn, vn, kc, vc, c["cu_seqlens_q"].to(dev), c["seqused_k"].to(dev),
                 c["block_table"].to(dev), ks, vs)
    torch.cuda.synchronize()
    return kc.cpu(), vc.cpu()


def check(c, got_k, got_v, what):
    ref_k, ref_v = oa.kv_append(c["k_new"], c["v_new"], c["cu_seqlens_q"], c["seqused_k"],
                                c["block_table"], c["k_cache"], c["v_cache"], c["k_scale"], c["v_scale"])
    for name, got, ref in (("k", got_k, ref_k), ("v", got_v, ref_v)):
        g, r = bits(got), bits(ref)
        bad = np.argwhere(g != r)
        assert bad.size == 0, f"{what}: {name}_cache differs at {len(bad)} elements, first {bad[:3].tolist()}"


CASES = []
for i, (nd, cd) in enumerate([("bf16", "bf16"), ("fp16", "fp16"), ("bf16", "fp8_e4m3fn"),
                              ("fp16", "fp8_e4m3fn")]):
    for j, (bs, hkv) in enumerate([(16, 2), (32, 1), (64, 8), (256, 2)]):
        for sat in ((False, True) if cd == "fp8_e4m3fn" else (False,)):
            CASES.append((10 * i + j + (5 if sat else 0), nd, cd, bs, hkv, sat))


@pytest.mark.parametrize("seed,nd,cd,bs,hkv,sat", CASES)
def test_append_random(seed, nd, cd, bs, hkv, sat):
    c = wk.append_case(seed, num_seqs=5, kv_heads=hkv, block_size=bs, new_dtype=nd,
                       cache_dtype=cd, saturate=sat)
    H.say(f"append random seed={seed} {nd}->{cd} bs={bs} Hkv={hkv} saturate={sat}")
    check(c, *run_append(c), f"seed {seed}")


def test_append_strided_new_rows():
    c = wk.append_case(3, num_seqs=3, kv_heads=2)
    T = c["k_new"].shape[0]
    big = torch.zeros(T, 5, 128, dtype=c["k_new"].dtype)
    big[:, 1:3] = c["k_new"]
    bigv = torch.zeros(T, 5, 128, dtype=c["v_new"].dtype)
    bigv[:, 1:3] = c["v_new"]
    H.say("append strided new rows")
    dev = "cuda"
    kn, vn = big.to(dev)[:, 1:3], bigv.to(dev)[:, 1:3]          # token stride 5*128, head stride 128
    kc, vc = run_append(c, k_new=kn, v_new=vn)
    check(c, kc, vc, "strided")


def test_append_rows_outside_sequences_not_read():
    c = wk.append_case(4, num_seqs=3, kv_heads=2)
    T = c["k_new"].shape[0]
    pad = torch.full((7, 2, 128), float("nan"), dtype=c["k_new"].dtype)
    kn = torch.cat([c["k_new"], pad])                          # 7 trailing rows of no sequence
    vn = torch.cat([c["v_new"], pad])
    H.say("append with trailing rows of no sequence")
    kc, vc = run_append(c, k_new=kn, v_new=vn)
    check(c, kc, vc, "trailing rows")


def test_append_empty_is_noop():
    c = wk.append_case(5, num_seqs=2)
    dev = "cuda"
    kc = c["k_cache"].to(dev)
    before = bits(kc)
    H.say("append with no tokens")
    ua.kv_append(c["k_new"][:0].to(dev), c["v_new"][:0].to(dev), kc, kc.clone(),
                 torch.zeros(3, dtype=torch.int32, device=dev), c["seqused_k"].to(dev),
                 c["block_table"].to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc), before)


@pytest.mark.parametrize("cache", ["bf16", "fp8_e4m3fn"])
def test_append_mixed_batch_full_size(cache):
    # the mixed chunked-prefill batch's 8256 new tokens x 8 kv heads appended
    # into its own cache (new rows: the first / second 8 query heads)
    wl = wk.config4()
    c = {"k_new": wl.q[:, :8].contiguous(), "v_new": wl.q[:, 8:16].contiguous(),
         "cu_seqlens_q": wl.cu_seqlens_q, "seqused_k": wl.seqused_k, "block_table": wl.block_table}
    if cache == "fp8_e4m3fn":
        c["k_cache"] = (wl.k_cache.float().clamp(-448, 448)).to(torch.float8_e4m3fn)
        c["v_cache"] = (wl.v_cache.float().clamp(-448, 448)).to(torch.float8_e4m3fn)
        c["k_scale"] = float(c["k_new"].float().abs().max()) / 448.0
        c["v_scale"] = float(c["v_new"].float().abs().max()) / 448.0
    else:
        c["k_cache"], c["v_cache"] = wl.k_cache, wl.v_cache
        c["k_scale"] = c["v_scale"] = None
    H.say(f"append mixed batch full size, {cache} cache")
    check(c, *run_append(c), f"mixed batch {cache}")


def test_append_then_attention():
    # append the new rows, then attend with queries of the same tokens: the
    # result must match the attention oracle on the oracle-appended cache
    c = wk.append_case(6, num_seqs=4, kv_heads=2, block_size=16)
    # N(0,1) rows, the regime the attention tolerance is stated for (the case
    # generator draws 3 x N(0,1))
    c["k_new"] = (c["k_new"].float() / 3).to(torch.bfloat16)
    c["v_new"] = (c["v_new"].float() / 3).to(torch.bfloat16)
    kc, vc = run_append(c)
    ref_k, ref_v = oa.kv_append(c["k_new"], c["v_new"], c["cu_seqlens_q"], c["seqused_k"],
                                c["block_table"], c["k_cache"], c["v_cache"])
    T = c["k_new"].shape[0]
    q = torch.from_numpy(np.random.default_rng(9).standard_normal((T, 8, 128)).astype(np.float32)).to(torch.bfloat16)
    bt = c["block_table"].clamp(min=0)
    wl = wk.Workload(name="append_then_attend", q=q, k_cache=ref_k, v_cache=ref_v,
                     cu_seqlens_q=c["cu_seqlens_q"], seqused_k=c["seqused_k"], block_table=bt,
                     softmax_scale=128 ** -0.5, causal=True)
    dev = "cuda"
    out = torch.empty_like(q, device=dev)
    H.say("append then attention")
    ua.unified_attention(q.to(dev), kc.to(dev), vc.to(dev), out, c["cu_seqlens_q"].to(dev),
                         c["seqused_k"].to(dev), bt.to(dev), wl.max_seqlen_q, wl.max_seqlen_k,
                         wl.softmax_scale, True)
    torch.cuda.synchronize()
    ref, _ = oracle.attention_workload(wl)
    err = float(np.abs(out.cpu().float().numpy().astype(np.float64) - ref).max())
    assert err <= H.TOL["bf16"], err


def test_decode_step_graph_capture():
    """A serving decode step -- append the new tokens' k/v rows, then attend over
    the grown cache -- captured as one HIP graph.  After fresh rows and queries
    are written in place by eager work, each replay equals the same two calls
    made eagerly, bit for bit (both caches, output and LSE), and the last state
    equals the append oracle and the attention oracle."""
    c = wk.append_case(77, num_seqs=6, max_new=3, max_prefix=300, kv_heads=2, block_size=16)
    H.say("decode step (append + attention) graph capture")
    dev = "cuda"
    T, Hq = c["k_new"].shape[0], 8
    gen = torch.Generator().manual_seed(77)
    kn, vn = c["k_new"].to(dev), c["v_new"].to(dev)
    kc, vc = c["k_cache"].to(dev), c["v_cache"].to(dev)
    cu, used, bt = c["cu_seqlens_q"].to(dev), c["seqused_k"].to(dev), c["block_table"].to(dev)
    q = torch.randn((T, Hq, 128), generator=gen).to(torch.bfloat16).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(T, Hq, dtype=torch.float32, device=dev)
    q_lens = c["cu_seqlens_q"][1:] - c["cu_seqlens_q"][:-1]
    mq, mk = int(q_lens.max()), int(c["seqused_k"].max())
    scale = 128 ** -0.5

    def step():
        ua.kv_append(kn, vn, kc, vc, cu, used, bt, None, None)
        ua.unified_attention(q, kc, vc, out, cu, used, bt, mq, mk, scale, True, lse=lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        # N(0, 1) rows, as in the attention workloads the 2e-2 bound is set for
        k_rows = torch.randn(tuple(kn.shape), generator=gen).to(kn.dtype)
        v_rows = torch.randn(tuple(vn.shape), generator=gen).to(vn.dtype)
        q_rows = torch.randn(tuple(q.shape), generator=gen).to(q.dtype)
        kn.copy_(k_rows)
        vn.copy_(v_rows)
        q.copy_(q_rows)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        g = [out.clone(), lse.clone(), kc.clone(), vc.clone()]
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        for name, a, b in (("out", g[0], out), ("lse", g[1], lse), ("k_cache", g[2], kc), ("v_cache", g[3], vc)):
            assert np.array_equal(bits(a) if a.dtype != torch.float32 else a.cpu().numpy(),
                                  bits(b) if b.dtype != torch.float32 else b.cpu().numpy()), f"replay {rep}: {name}"
    # every replay wrote the same slots, so the final caches are one append of
    # the last rows onto the original contents
    check(dict(c, k_new=k_rows, v_new=v_rows), kc.cpu(), vc.cpu(), "decode step graph")
    ref_k, ref_v = oa.kv_append(k_rows, v_rows, c["cu_seqlens_q"], c["seqused_k"], c["block_table"],
                                c["k_cache"], c["v_cache"], None, None)
    wl = wk.Workload("decode_step_graph", q_rows, ref_k, ref_v, c["cu_seqlens_q"], c["seqused_k"],
                     c["block_table"], scale, True)
    H.compare(wl, out, lse, what="decode step graph")
