"""GPU parity of the attention backward (ua_attention_backward, through the C
ABI) against the float64 oracle (oracle/backward.py).

Bound per entry, from the arithmetic of the kernels: P and dS are rounded to
the input dtype (unit roundoff u: 2^-8 bf16, 2^-11 fp16) before their
products, Delta comes from the 16-bit O, products accumulate in fp32 and the
result is rounded to the dtype once.  With the oracle's magnitudes (sums of
the absolute terms of each gradient entry, see oracle/backward.py) that gives
|err| <= 2u * mag; the tests allow 4u * mag + 1e-5.  Outputs start as NaN so
an unwritten entry fails.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.backward as ob
import oracle.bruteforce as bf
import paged_varlen_flashattention_amd as ua
import workloads as wk
from gpu_helpers import say

pytestmark = pytest.mark.gpu

U = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}


def _dev(t):
    return t.to("cuda")


def oracle_case(case, causal):
    return ob.attention_backward(case["q"], case["k"], case["v"], case["dout"],
                                 case["cu_seqlens_q"].numpy(), case["cu_seqlens_k"].numpy(),
                                 case["softmax_scale"], causal)


def hip_backward(case, causal, out, lse):
    q, k, v, do = (_dev(case[n]) for n in ("q", "k", "v", "dout"))
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    ua.attention_backward(q, k, v, _dev(out), do, _dev(lse), _dev(case["cu_seqlens_q"]),
                          _dev(case["cu_seqlens_k"]), dq, dk, dv, case["softmax_scale"], causal)
    torch.cuda.synchronize()
    return {n: bf.to_f64(t.cpu()) for n, t in (("dq", dq), ("dk", dk), ("dv", dv))}


def check_close(got, ref, u, what, case_name):
    for n in ("dq", "dk", "dv"):
        err = np.abs(got[n] - ref[n])
        tol = 4 * u * ref["mag_" + n] + 1e-5
        bad = ~(err <= tol)                       # NaN counts as bad
        assert not bad.any(), (f"{case_name} {what} {n}: {int(bad.sum())} of {bad.size} entries beyond "
                               f"4u*mag, worst err {np.nanmax(err):.3e}")


CASES = [
    # name, seed, q_lens, k_lens, Hq, Hkv, dtype, causal, scale, std
    ("ragged_gqa4_causal_bf16", 1, [1, 37, 130, 64], [50, 37, 300, 64], 8, 2, "bf16", True, None, 1.0),
    ("ragged_gqa4_full_bf16", 2, [1, 37, 130, 64], [50, 37, 300, 64], 8, 2, "bf16", False, None, 1.0),
    ("mha_causal_fp16", 3, [200, 33], [260, 33], 4, 4, "fp16", True, None, 1.0),
    ("mha_full_fp16", 4, [5, 100], [300, 7], 4, 4, "fp16", False, None, 1.0),
    ("gqa8_causal_bf16", 5, [96, 17], [160, 17], 16, 2, "bf16", True, None, 1.0),
    ("gqa3_partial_rows_fp16", 6, [45, 70], [45, 129], 6, 2, "fp16", True, None, 1.0),
    ("empty_seqs_and_one_key", 7, [0, 9, 4, 0], [0, 1, 4, 12], 4, 2, "bf16", False, None, 1.0),
    ("one_key_causal", 8, [1, 3, 1], [1, 3, 257], 4, 1, "fp16", True, None, 1.0),
    ("tutorial_test_shape", 9, [128, 128], [128, 128], 2, 2, "fp16", True, 0.5, 0.5),
    ("many_key_blocks_full", 10, [33, 64], [700, 515], 4, 2, "bf16", False, 0.2, 1.0),
]


@pytest.mark.parametrize("case_def", CASES, ids=[c[0] for c in CASES])
def test_backward_parity(case_def):
    name, seed, ql, kl, hq, hkv, dt, causal, scale, std = case_def
    case = wk.backward_case(seed, ql, kl, hq, hkv, dt, softmax_scale=scale, std=std)
    ref = oracle_case(case, causal)
    # the forward's outputs as the backward receives them: O in the dtype, LSE in fp32
    out = torch.from_numpy(ref["out"]).to(case["q"].dtype)
    lse = torch.from_numpy(ref["lse"]).to(torch.float32)
    say(f"backward parity: {name} q_lens={ql} k_lens={kl} heads {hq}/{hkv} {dt} causal={causal}")
    got = hip_backward(case, causal, out, lse)
    check_close(got, ref, U[dt], "vs oracle", name)


@pytest.mark.parametrize("i", range(40))
def test_backward_random_sweep(i):
    # seeded random batches across the backward's features
    # (workloads.backward_feature_case), every entry against the oracle
    case, causal = wk.backward_feature_case(i)
    dt = "fp16" if case["q"].dtype == torch.float16 else "bf16"
    ref = oracle_case(case, causal)
    out = torch.from_numpy(ref["out"]).to(case["q"].dtype)
    lse = torch.from_numpy(ref["lse"]).to(torch.float32)
    say(f"backward sweep {i}: q_lens={np.diff(case['cu_seqlens_q'].numpy()).tolist()} "
        f"k_lens={np.diff(case['cu_seqlens_k'].numpy()).tolist()} causal={causal} {dt}")
    got = hip_backward(case, causal, out, lse)
    check_close(got, ref, U[dt], "vs oracle", f"sweep {i}")


def _paged_view(case):
    """The dense k, v as a paged cache with 16-key pages (every cu_seqlens_k[s]
    a multiple of 16) and the tables that map it back."""
    k, v = case["k"], case["v"]
    Tk, Hkv, D = k.shape
    cu = case["cu_seqlens_k"].numpy()
    S = len(cu) - 1
    W = max(1, int(np.diff(cu).max() + 15) // 16)
    table = np.zeros((S, W), dtype=np.int32)
    for s in range(S):
        n = (cu[s + 1] - cu[s] + 15) // 16
        table[s, :n] = cu[s] // 16 + np.arange(n)
    return k.view(Tk // 16, 16, Hkv, D), v.view(Tk // 16, 16, Hkv, D), torch.from_numpy(table)


def hip_forward(case, causal):
    kc, vc, table = _paged_view(case)
    q = _dev(case["q"])
    out = torch.full_like(q, float("nan"))
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device="cuda")
    kl = torch.tensor(case["k_lens"], dtype=torch.int32)
    ua.unified_attention(q, _dev(kc), _dev(vc), out, _dev(case["cu_seqlens_q"]), _dev(kl), _dev(table),
                         max(case["q_lens"]), max(case["k_lens"]), case["softmax_scale"], causal, lse=lse)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("causal", [True, False])
def test_forward_then_backward(causal):
    """The training step as it runs: the HIP forward's O and LSE feed the HIP backward."""
    case = wk.backward_case(11, [64, 128, 16], [128, 256, 16], 8, 2, "bf16")
    say(f"forward then backward: causal={causal}")
    out, lse = hip_forward(case, causal)
    got = hip_backward(case, causal, out, lse)
    check_close(got, oracle_case(case, causal), U["bf16"], "after the HIP forward", "fwd_bwd")


def test_backward_full_size_sampled():
    """The backward benchmark's shape (batch 4, 32 heads, N 4096, fp16, scale 1.3,
    causal), O and LSE from the HIP forward.  The oracle checks dQ of sampled
    rows (each as a one-row problem over the keys it sees) and dK, dV of the
    last 48 keys of every sequence (only the last 48 rows see them), every
    entry of two whole (sequence, head) planes, and the dV rows of every
    (sequence, head) must sum to its dO rows."""
    case = wk.backward_bench()
    causal = True
    N, H = 4096, 32
    say("backward full size: batch 4, heads 32, N 4096, fp16, causal (forward then backward)")
    out, lse = hip_forward(case, causal)
    got = hip_backward(case, causal, out, lse)
    u = U["fp16"]
    rng = np.random.default_rng(5)
    for s in range(4):
        base = s * N
        rows = np.unique(np.concatenate([[0, 1, N - 1], rng.integers(0, N, 5)]))
        for i in rows:
            sub = {"q": case["q"][base + i:base + i + 1], "k": case["k"][base:base + i + 1],
                   "v": case["v"][base:base + i + 1], "dout": case["dout"][base + i:base + i + 1],
                   "cu_seqlens_q": torch.tensor([0, 1], dtype=torch.int32),
                   "cu_seqlens_k": torch.tensor([0, i + 1], dtype=torch.int32),
                   "softmax_scale": case["softmax_scale"]}
            ref = oracle_case(sub, causal)
            err = np.abs(got["dq"][base + i] - ref["dq"][0])
            tol = 4 * u * ref["mag_dq"][0] + 1e-5
            assert (err <= tol).all(), f"seq {s} row {i}: dQ err {np.nanmax(err):.3e}"
        m = 48
        sub = {"q": case["q"][base + N - m:base + N], "k": case["k"][base:base + N],
               "v": case["v"][base:base + N], "dout": case["dout"][base + N - m:base + N],
               "cu_seqlens_q": torch.tensor([0, m], dtype=torch.int32),
               "cu_seqlens_k": torch.tensor([0, N], dtype=torch.int32),
               "softmax_scale": case["softmax_scale"]}
        ref = oracle_case(sub, causal)
        for n in ("dk", "dv"):
            err = np.abs(got[n][base + N - m:base + N] - ref[n][N - m:])
            tol = 4 * u * ref["mag_" + n][N - m:] + 1e-5
            assert (err <= tol).all(), f"seq {s}: {n} of the last {m} keys, err {np.nanmax(err):.3e}"
        dO = bf.to_f64(case["dout"][base:base + N])                     # [N, H, D]
        sum_dv = got["dv"][base:base + N].sum(axis=0)
        want = dO.sum(axis=0)
        tol = 2 * u * np.abs(dO).sum(axis=0) + 1e-3
        assert (np.abs(sum_dv - want) <= tol).all(), f"seq {s}: dV rows do not sum to the dO rows"
    # every dQ, dK and dV entry of two whole (sequence, head) planes
    for s, h in ((0, 0), (3, H - 1)):
        base = s * N
        sub = {"q": case["q"][base:base + N, h:h + 1], "k": case["k"][base:base + N, h:h + 1],
               "v": case["v"][base:base + N, h:h + 1], "dout": case["dout"][base:base + N, h:h + 1],
               "cu_seqlens_q": torch.tensor([0, N], dtype=torch.int32),
               "cu_seqlens_k": torch.tensor([0, N], dtype=torch.int32),
               "softmax_scale": case["softmax_scale"]}
        ref = oracle_case(sub, causal)
        plane = {n: got[n][base:base + N, h:h + 1] for n in ("dq", "dk", "dv")}
        check_close(plane, ref, u, f"whole plane (sequence {s}, head {h})", "backward full size")
    assert np.isfinite(got["dq"]).all() and np.isfinite(got["dk"]).all() and np.isfinite(got["dv"]).all()


def test_training_step_graph_capture():
    """The forward (O, LSE) and the backward of one training step captured as
    one HIP graph (neither call synchronises, copies to the host or clears
    memory): after q, k, v and dO are overwritten in place by eager work, each
    replay's O, LSE, dQ, dK and dV equal the same calls made eagerly, bit for
    bit, and the last gradients equal the oracle's."""
    causal = True
    case = wk.backward_case(12, [64, 128, 16], [128, 256, 16], 8, 2, "bf16")
    say("training step (forward + backward) graph capture")
    kc, vc, table = _paged_view(case)
    q, k, v, do = (_dev(case[n]) for n in ("q", "k", "v", "dout"))
    kcd, vcd = k.view(kc.shape), v.view(vc.shape)        # the paged view of the same buffers
    cu_q, cu_k = _dev(case["cu_seqlens_q"]), _dev(case["cu_seqlens_k"])
    kl = _dev(torch.tensor(case["k_lens"], dtype=torch.int32))
    tb = _dev(table)
    T, Hq = q.shape[0], q.shape[1]
    out = torch.empty_like(q)
    lse = torch.empty(T, Hq, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ua.bwd_workspace_size(T, Hq), dtype=torch.uint8, device="cuda")
    mq, mk, scale = max(case["q_lens"]), max(case["k_lens"]), case["softmax_scale"]

    def step():
        ua.unified_attention(q, kcd, vcd, out, cu_q, kl, tb, mq, mk, scale, causal, lse=lse)
        ua.attention_backward(q, k, v, out, do, lse, cu_q, cu_k, dq, dk, dv, scale, causal, workspace=ws)

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
    gen = torch.Generator().manual_seed(12)
    results = (out, lse, dq, dk, dv)
    for rep in range(3):
        new = {n: torch.randn(tuple(t.shape), generator=gen).to(t.dtype) for n, t in
               (("q", q), ("k", k), ("v", v), ("dout", do))}
        for n, t in (("q", q), ("k", k), ("v", v), ("dout", do)):
            t.copy_(new[n])
        for t in results:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        snap = [t.clone() for t in results]
        for t in results:
            t.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "dq", "dk", "dv"), snap, results):
            ai = a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16)
            bi = b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)
            assert torch.equal(ai, bi), f"replay {rep}: {name}"
    got = {n: bf.to_f64(t.cpu()) for n, t in (("dq", dq), ("dk", dk), ("dv", dv))}
    ref = oracle_case(dict(case, **new), causal)
    check_close(got, ref, U["bf16"], "graph replay", "graph")
