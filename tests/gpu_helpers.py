"""Helpers shared by the GPU tests: move a workload to the device, run the HIP
path through the C ABI, compare with the oracle."""
from __future__ import annotations

import ctypes
import os
import sys

import numpy as np
import torch

import oracle
import oracle.bruteforce as bf
import paged_varlen_flashattention_amd as ua
from paged_varlen_flashattention_amd import _binding as B

TOL = {"bf16": 2e-2, "fp16": 2e-2, "fp8_e4m3fn": 6e-2}
LSE_TOL = 1e-3


def say(msg: str) -> None:
    """Name the case on stdout before a GPU step (flushed, so it survives a crash)."""
    print(msg, flush=True)
    sys.stdout.flush()


def has_gpu() -> bool:
    return torch.cuda.is_available()


def to_device(wl, dev="cuda"):
    d = {
        "q": wl.q.to(dev), "k_cache": wl.k_cache.to(dev), "v_cache": wl.v_cache.to(dev),
        "cu_seqlens_q": wl.cu_seqlens_q.to(dev), "seqused_k": wl.seqused_k.to(dev),
        "block_table": wl.block_table.to(dev),
        "k_scale": None if wl.k_scale is None else torch.tensor([wl.k_scale], dtype=torch.float32, device=dev),
        "v_scale": None if wl.v_scale is None else torch.tensor([wl.v_scale], dtype=torch.float32, device=dev),
        "alibi": None if getattr(wl, "alibi_slopes", None) is None
        else wl.alibi_slopes.to(torch.float32).contiguous().to(dev),
    }
    return d


def check_shapes(wl) -> None:
    """Host-side check that the inputs match what the kernel assumes, before any launch."""
    T, Hq, D = wl.q.shape
    NB, bs, Hkv, D2 = wl.k_cache.shape
    assert D == D2 == 128 and Hq % Hkv == 0
    cu = wl.cu_seqlens_q.numpy()
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    kv = wl.seqused_k.numpy()
    assert np.all(kv >= np.diff(cu)), "q_len > kv_len"
    bt = wl.block_table.numpy()
    for s, kl in enumerate(kv.tolist()):
        used = (kl + bs - 1) // bs
        assert used <= bt.shape[1]
        assert np.all((bt[s, :used] >= 0) & (bt[s, :used] < NB)), "block id out of range"
    slopes = getattr(wl, "alibi_slopes", None)
    assert slopes is None or slopes.numel() == Hq, "one ALiBi slope per query head"


def run(wl, dev_inputs=None, num_splits=None, want_lse=True, out=None, workspace=None, sync=True,
        fp8_compute=False):
    """The HIP path on a workload; returns (out, lse) device tensors."""
    check_shapes(wl)
    d = dev_inputs or to_device(wl)
    if out is None:
        out = torch.full_like(d["q"], float("nan"))
    lse = torch.full((wl.num_tokens, wl.num_q_heads), float("nan"), dtype=torch.float32,
                     device=d["q"].device) if want_lse else None
    ua.unified_attention(d["q"], d["k_cache"], d["v_cache"], out, d["cu_seqlens_q"], d["seqused_k"],
                         d["block_table"], wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale,
                         wl.causal, d["k_scale"], d["v_scale"],
                         num_splits=wl.num_splits if num_splits is None else num_splits,
                         lse=lse, workspace=workspace,
                         window=(getattr(wl, "window_left", -1), getattr(wl, "window_right", -1)),
                         alibi_slopes=d.get("alibi"), fp8_compute=fp8_compute)
    if sync:
        torch.cuda.synchronize()
    return out, lse


def plan(wl, num_splits=None):
    """The launch the library plans for a workload (host only; the workload's
    CPU tensors stand in for the device buffers and the workspace is unbounded)."""
    scales = [None if x is None else torch.tensor([x], dtype=torch.float32)
              for x in (wl.k_scale, wl.v_scale)]
    p = B.make_params(wl.q, wl.k_cache, wl.v_cache, wl.q, wl.cu_seqlens_q, wl.seqused_k,
                      wl.block_table, wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale, wl.causal,
                      *scales, wl.num_splits if num_splits is None else num_splits, None, None)
    p.workspace, p.workspace_bytes = 256, 1 << 62
    info = B.PlanInfo()
    st = B.load_library().ua_plan(ctypes.byref(p), ctypes.byref(info))
    assert st == B.UA_OK, st
    return info


def out_f64(out: torch.Tensor) -> np.ndarray:
    return bf.to_f64(out.cpu())


def compare(wl, out, lse, rows=None, tol=None, what=""):
    """Max abs error of the GPU output (and lse) against the oracle, on all rows
    or on the given (token, head) rows.  Returns the error figures."""
    if tol is None:
        tol = TOL["fp8_e4m3fn"] if wl.k_cache.dtype == torch.float8_e4m3fn else TOL["bf16"]
    g = out_f64(out)
    gl = lse.cpu().numpy().astype(np.float64) if lse is not None else None
    if rows is None:
        ref, ref_lse = oracle.attention_workload(wl)
        got = g
        got_lse = gl
    else:
        rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
        ref, ref_lse = oracle.attention_workload(wl, rows=rows)
        got = g[rows[:, 0], rows[:, 1]]
        got_lse = gl[rows[:, 0], rows[:, 1]] if gl is not None else None
    assert np.all(np.isfinite(got)), f"{what}: non-finite or unwritten GPU output"
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    mean = float(np.abs(got - ref).mean()) if got.size else 0.0
    res = {"max_abs_err": err, "mean_abs_err": mean, "tol": tol}
    if got_lse is not None:
        assert np.all(np.isfinite(got_lse)), f"{what}: unwritten lse"
        res["lse_max_abs_err"] = float(np.abs(got_lse - ref_lse).max()) if got_lse.size else 0.0
        assert res["lse_max_abs_err"] <= LSE_TOL, f"{what}: lse err {res}"
    assert err <= tol, f"{what}: max abs err {err:.4g} > {tol} ({res})"
    return res


def sample_rows(wl, n: int, seed: int = 0) -> np.ndarray:
    """n (token, head) rows: the first and last token of each sequence and of each
    128-token block boundary, plus uniform random picks."""
    rng = np.random.default_rng(seed)
    cu = wl.cu_seqlens_q.numpy()
    Hq = wl.num_q_heads
    picks = []
    for s in range(wl.num_seqs):
        a, b = int(cu[s]), int(cu[s + 1])
        if b > a:
            for t in {a, b - 1, min(b - 1, a + 127), min(b - 1, a + 128)}:
                picks.append((t, int(rng.integers(0, Hq))))
    m = max(0, n - len(picks))
    toks = rng.integers(0, wl.num_tokens, size=m)
    heads = rng.integers(0, Hq, size=m)
    picks += list(zip(toks.tolist(), heads.tolist()))
    return np.array(picks[: max(n, len(picks))], dtype=np.int64)
