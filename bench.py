"""Benchmark of the unified paged varlen attention forward on one MI355X.

Default workload (the headline): dense FA2 forward, batch 4 x 32 heads x 4096
tokens, head_dim 128, fp16, expressed as a paged cache with one contiguous block
table per sequence (block_size 16).  One step = one causal call + one full
(non-causal) call of ua_unified_attention on the same inputs.  The value is
algorithmic attention TFLOP/s: 4 * D * (visible query-key pairs) * heads,
summed over both calls, divided by the step time.

Other workloads (``--config c3|c4|c5|c2mask``) are measured the same way for
the record; c3 and c5 report KV-read GB/s.  c2mask is the dense causal batch
with a 1024-key sliding window (window_left 1023) and, as a second call, with
ALiBi slopes; its FLOPs count only the pairs the window leaves visible.
c2fp8 is the dense batch with an e4m3 cache in the fp8-compute mode (queries
and weights rounded to e4m3, fp8 MFMA), against the fp8 MFMA peak.

Prints ONE JSON line.  Inputs are resident in HBM before the timed region;
K steps run back to back between two device synchronisations.  Per-launch
durations come from HIP events recorded on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2516.6      # MI355X dense bf16 / fp16 MFMA
PEAK_MFMA_FP8_TFLOPS = 5000.0  # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c2", choices=["c2", "c3", "c4", "c5", "c2mask", "c2fp8", "append", "bwd"])
    ap.add_argument("--splits", type=int, default=None, help="override num_splits (c3: default the planner's choice; c5: default 32)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the oracle CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="c2: skip the decode half (c3 and c5 KV-read GB/s timed after the headline)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the measurements made after the timed region (cold-cache call "
                         "times, c3 split sweep, c4 sub-batches)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of --copy-bytes bytes (counter calibration)")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    return ap.parse_args()


def copy_calibration(nbytes: int, reps: int = 3) -> None:
    """A plain device-to-device copy of a known size: under rocprofv3 --pmc its
    FETCH_SIZE / WRITE_SIZE per dispatch calibrate what those counters read per
    byte actually moved."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def kernel_source_hash(tag: str = "") -> str:
    """Hash of the device sources behind a profiled kernel: the kernel file of
    that workload (the append kernel, the backward kernels or the attention
    forward) and the shared argument header."""
    kind = tag.split("_")[0]
    files = {"append": ["ua_append.hip"], "bwd": ["ua_backward.hip"]}.get(kind, ["ua_attention.hip"])
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_varlen_flashattention_amd", "csrc")
    for name in sorted(files + ["ua_internal.h"]):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_tag: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE counters
    (profiles/traffic_<tag>.txt, counters scaled by a plain-copy calibration),
    or None when no such record exists or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_source_hash") != kernel_source_hash(kernel_tag):
        return None
    return int(float(rec["bytes_per_launch"]))


def mfma_util_from_profiles(tag: str):
    """Matrix-pipe utilisation of a prefill workload's kernel measured with
    rocprofv3 (profiles/mfma_util_prefill.txt: MfmaUtil, the share of SIMD
    cycles the MFMA unit was busy, and the clock the counters imply), or None
    when there is no record for it or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", "mfma_util_prefill.txt")
    if not os.path.exists(path):
        return None
    rec, header = {}, None
    with open(path) as f:
        for line in f:
            if line.startswith("kernel_source_hash:"):
                if line.split(":", 1)[1].strip() != kernel_source_hash(tag):
                    return None
            elif line.startswith("workload"):
                header = line.split()
            elif header and line.strip():
                parts = line.split()
                rec[parts[0]] = dict(zip(header[1:], (float(x) for x in parts[1:])))
    r = rec.get(tag)
    if r is None:
        return None
    return {"mfma_busy_pct": r["mfma_util"], "clock_ghz": r["clock_ghz"], "frac_at_clock": r["frac_clock"]}


def build_calls(cfg: str, splits_override):
    """Returns (workload description, list of (label, workload, num_splits))."""
    import workloads as wk
    if cfg == "c2":
        wl_c = wk.config2(causal=True)
        wl_f = wk.Workload(**{**wl_c.__dict__, "causal": False,
                              "name": wl_c.name.replace("causal", "full")})
        return ("dense_fa2_fwd_b4_h32_n4096_d128_fp16_causal_and_full",
                [("full", wl_f, 1), ("causal", wl_c, 1)])
    if cfg == "c2fp8":
        wl_c = wk.config2(causal=True, kv_dtype="fp8_e4m3fn")
        wl_f = wk.Workload(**{**wl_c.__dict__, "causal": False,
                              "name": wl_c.name.replace("causal", "full")})
        wl_c.meta["fp8_compute"] = wl_f.meta["fp8_compute"] = True
        return ("dense_fa2_fwd_b4_h32_n4096_d128_fp16q_fp8kv_fp8compute_causal_and_full",
                [("full", wl_f, 1), ("causal", wl_c, 1)])
    if cfg == "c2mask":
        wl_c = wk.config2(causal=True)
        return ("dense_fa2_fwd_b4_h32_n4096_d128_fp16_causal_window1024_and_alibi",
                [("window", wk.with_mask(wl_c, 1023, -1, name="c2_causal_window1024"), 1),
                 ("alibi", wk.with_mask(wl_c, alibi=wk.alibi_slopes(32), name="c2_causal_alibi"), 1)])
    if cfg == "c3":
        wl = wk.config3()
        if splits_override is None:
            # the split count the library's planner picks (host only)
            import paged_varlen_flashattention_amd as ua
            s = ua.auto_splits(wl.q, wl.k_cache, wl.v_cache, wl.q, wl.cu_seqlens_q, wl.seqused_k,
                               wl.block_table, wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale,
                               wl.causal)
        else:
            s = splits_override
        return (f"decode_paged_gqa_256seq_32q8kv_bs16_splits{s}", [("decode", wl, s)])
    if cfg == "c4":
        wl = wk.config4()
        if splits_override is None:
            # the planner's choice: the decode rows split (-n), prefill rows not
            import paged_varlen_flashattention_amd as ua
            s = ua.auto_splits(wl.q, wl.k_cache, wl.v_cache, wl.q, wl.cu_seqlens_q, wl.seqused_k,
                               wl.block_table, wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale,
                               wl.causal)
        else:
            s = splits_override
        return (f"mixed_chunked_prefill_64dec_4x2048_64q8kv_bs32_splits{s}", [("mixed", wl, s)])
    s = 32 if splits_override is None else splits_override
    return (f"long_ctx_fp8kv_2x131072_64q8kv_splits{s}", [("long", wk.config5(), s)])


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU only: run it with --gpus 1 "
                          "(the attention call has no cross-GPU step: across GPUs it would run "
                          "unchanged on each GPU's share of kv heads or sequences)",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_bytes)
        return
    if args.config == "bwd":
        main_bwd(args)
        return
    if args.config == "append":
        main_append(args)
        return

    import numpy as np
    import torch

    import paged_varlen_flashattention_amd as ua

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    ua.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    workload_name, calls = build_calls(args.config, args.splits)
    prepared = []
    for label, wl, splits in calls:
        d = {
            "q": wl.q.to(dev), "k": wl.k_cache.to(dev), "v": wl.v_cache.to(dev),
            "cu": wl.cu_seqlens_q.to(dev), "kv": wl.seqused_k.to(dev), "bt": wl.block_table.to(dev),
            "ks": None if wl.k_scale is None else torch.tensor([wl.k_scale], device=dev),
            "vs": None if wl.v_scale is None else torch.tensor([wl.v_scale], device=dev),
            "alibi": None if wl.alibi_slopes is None else wl.alibi_slopes.to(dev),
            "window": (wl.window_left, wl.window_right),
            "f8": bool(wl.meta.get("fp8_compute", False)),
        }
        d["out"] = torch.empty_like(d["q"])
        ws = None
        if abs(splits) > 1:
            ws = torch.empty(ua.workspace_size(wl.num_tokens, wl.num_q_heads, 128, abs(splits)),
                             dtype=torch.uint8, device=dev)
        prepared.append((label, wl, splits, d, ws))
    stream = torch.cuda.current_stream()

    def call(wl, splits, d, ws):
        ua.unified_attention(d["q"], d["k"], d["v"], d["out"], d["cu"], d["kv"], d["bt"],
                             wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale, wl.causal,
                             d["ks"], d["vs"], num_splits=splits, workspace=ws, stream=stream,
                             window=d["window"], alibi_slopes=d["alibi"], fp8_compute=d.get("f8", False))

    for _ in range(args.warmup):
        for _, wl, splits, d, ws in prepared:
            call(wl, splits, d, ws)
    torch.cuda.synchronize()

    K = args.steps
    ev = {label: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(K)] for label, *_ in prepared}
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(K):
        for label, wl, splits, d, ws in prepared:
            e0, e1 = ev[label][k]
            e0.record(stream)
            call(wl, splits, d, ws)
            e1.record(stream)
    t_stop.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_stop)
    ms_per_step = ms_total / K

    per = {}
    for label, wl, splits, d, ws in prepared:
        durs = np.array([a.elapsed_time(b) for a, b in ev[label]])
        per[label] = {"ms_mean": float(durs.mean()), "ms_min": float(durs.min()),
                      "ms_median": float(np.median(durs)), "flops": wl.flops(),
                      "kv_bytes": wl.kv_bytes(), "splits": splits}

    compute_bound = args.config in ("c2", "c4", "c2mask", "c2fp8")
    peak_mfma = PEAK_MFMA_FP8_TFLOPS if args.config == "c2fp8" else PEAK_MFMA_TFLOPS
    if compute_bound:
        total_flops = sum(p["flops"] for p in per.values())
        value = total_flops / (ms_per_step * 1e-3) / 1e12
        metric, unit = "attention TFLOP/s (prefill)", "TFLOP/s"
    else:
        total_bytes = sum(p["kv_bytes"] for p in per.values())
        value = total_bytes / (ms_per_step * 1e-3) / 1e9
        metric, unit = "KV-read GB/s (decode)", "GB/s"

    def roofline(label, tag):
        p = per[label]
        if compute_bound:
            ach = p["flops"] / (p["ms_mean"] * 1e-3) / 1e12
            r = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak_mfma, "unit": "TFLOP/s",
                 "frac": round(ach / peak_mfma, 4)}
        else:
            ach = p["kv_bytes"] / (p["ms_mean"] * 1e-3) / 1e9
            r = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": round(ach / PEAK_HBM_GBS, 4)}
        r["traffic"] = traffic_from_profiles(tag)
        r["launch_ms_mean"] = round(p["ms_mean"], 4)
        if compute_bound:
            r["mfma_counters"] = mfma_util_from_profiles(tag)
        return r

    dominant = max(per, key=lambda k: per[k]["ms_mean"])
    result = {
        "metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"c2": "fp16", "c2mask": "fp16", "c2fp8": "f8 (e4m3 operands, fp32 accumulate)"}.get(args.config, "bf16"),
        "data": "synthetic (seeded N(0,1) q/k/v, paged cache)",
        "config": {"workload": workload_name, "calls_per_step": [p[0] for p in prepared]},
        "roofline": roofline(dominant, f"{args.config}_{dominant}"),
        "per_call": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                     for k, v in per.items()},
    }
    for label in per:
        if label != dominant:
            result[f"roofline_{label}"] = roofline(label, f"{args.config}_{label}")

    if not args.no_extras:
        extras(args, prepared, per, result, call, stream)
    cpu_items = [(label, wl, splits, None, None) for label, wl, splits, _, _ in prepared]
    if args.config == "c2" and not args.no_decode:
        # the decode half of the metric, after the headline's timed region
        # (it never enters `value`): KV-read GB/s of the decode batch at the
        # planner's split count and of the long-context batch at 32 splits
        del prepared
        torch.cuda.empty_cache()
        result["decode"] = decode_half(args, call, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cpu_items, compute_bound, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def decode_half(args, call, stream) -> dict:
    """KV-read GB/s of the two HBM-bound workloads, each with its own HBM
    roofline object: the 256-sequence decode batch (32/8 heads, bs 16, the
    planner's split count) and the long-context fp8 batch (2 x 131072 keys,
    32 splits).  Per workload: `steps` warm calls back to back, bracketed by
    HIP events on the launch stream (mean, median, min), and 10 calls with the
    L2/MALL flushed by a 512 MB write before each (median, min)."""
    import numpy as np
    import torch

    import paged_varlen_flashattention_amd as ua
    dev = torch.device("cuda:0")
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush = lambda: scrub.fill_(1)
    res = {}
    for cfg, tag in (("c3", "c3_decode"), ("c5", "c5_long")):
        name, calls = build_calls(cfg, None)
        label, wl, splits = calls[0]
        d = {"q": wl.q.to(dev), "k": wl.k_cache.to(dev), "v": wl.v_cache.to(dev),
             "cu": wl.cu_seqlens_q.to(dev), "kv": wl.seqused_k.to(dev), "bt": wl.block_table.to(dev),
             "ks": None if wl.k_scale is None else torch.tensor([wl.k_scale], device=dev),
             "vs": None if wl.v_scale is None else torch.tensor([wl.v_scale], device=dev),
             "alibi": None, "window": (-1, -1), "f8": False}
        d["out"] = torch.empty_like(d["q"])
        ws = None
        if abs(splits) > 1:
            ws = torch.empty(ua.workspace_size(wl.num_tokens, wl.num_q_heads, 128, abs(splits)),
                             dtype=torch.uint8, device=dev)
        fn = lambda: call(wl, splits, d, ws)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        warm = np.array([a.elapsed_time(b) for a, b in evs])
        cold = time_calls(fn, 50, stream, flush)
        kvb = wl.kv_bytes()
        ach = kvb / (warm.mean() * 1e-3) / 1e9
        res[cfg] = {
            "workload": name, "metric": "KV-read GB/s (decode)", "splits": splits,
            "value": round(ach, 1), "unit": "GB/s", "kv_bytes": kvb,
            "ms_mean": round(float(warm.mean()), 4), "ms_median": round(float(np.median(warm)), 4),
            "ms_min": round(float(warm.min()), 4), "ms_cold_median": round(float(np.median(cold)), 4),
            "ms_cold_min": round(float(cold.min()), 4),
            "GB/s_cold_median": round(kvb / (np.median(cold) * 1e-3) / 1e9, 1),
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic_from_profiles(tag),
                         "launch_ms_mean": round(float(warm.mean()), 4),
                         "kernel": "one ua_unified_attention call (attention kernel + split combine)"},
        }
        del d, ws
        torch.cuda.empty_cache()
    return res


def append_bytes(k_new, k_cache) -> int:
    """Algorithmic bytes of an append: every new k and v element read once and
    written once in the cache dtype."""
    return int(k_new.numel() * 2 * (k_new.element_size() + k_cache.element_size()))


def main_append(args) -> None:
    """KV-cache append (ua_kv_append): the dense batch's 4 x 4096 new tokens x
    32 kv heads (fp16) written into its paged cache (every position of the
    cache is a new token there).  Value: algorithmic GB/s (read + write)."""
    import numpy as np
    import torch

    import paged_varlen_flashattention_amd as ua
    import workloads as wk
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    ua.load_library()
    dev = torch.device("cuda:0")
    wl = wk.config2(causal=True)
    # the new rows are the batch's k and v rows in token order (q has the same shape)
    k_new = wl.q.to(dev)
    v_new = torch.flip(wl.q, dims=[2]).contiguous().to(dev)
    k_cache = torch.empty_like(wl.k_cache, device=dev)
    v_cache = torch.empty_like(wl.v_cache, device=dev)
    cu, kv, bt = wl.cu_seqlens_q.to(dev), wl.seqused_k.to(dev), wl.block_table.to(dev)
    stream = torch.cuda.current_stream()
    fn = lambda: ua.kv_append(k_new, v_new, k_cache, v_cache, cu, kv, bt, stream=stream)
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / K
    durs = np.array([a.elapsed_time(b) for a, b in evs])
    nbytes = append_bytes(k_new, k_cache)
    value = nbytes / (ms_step * 1e-3) / 1e9
    ach = nbytes / (durs.mean() * 1e-3) / 1e9
    result = {
        "metric": "KV-append GB/s (read + write)", "value": round(value, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic (seeded N(0,1) rows, paged cache)",
        "config": {"workload": "kv_append_b4_n4096_kvh32_d128_fp16_bs16", "tokens": int(k_new.shape[0]),
                   "kv_heads": int(k_new.shape[1])},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic_from_profiles("append_bulk"),
                     "launch_ms_mean": round(float(durs.mean()), 4)},
        "per_call": {"append": {"ms_mean": round(float(durs.mean()), 4), "ms_min": round(float(durs.min()), 4),
                                "ms_median": round(float(np.median(durs)), 4), "bytes": nbytes}},
    }
    if not args.no_extras:
        # the mixed batch's 8256 new tokens x 8 kv heads, into a bf16 and an fp8 cache
        w4 = wk.config4()
        kn4 = w4.q[:, :8].contiguous().to(dev)
        vn4 = w4.q[:, 8:16].contiguous().to(dev)
        cu4, kv4, bt4 = w4.cu_seqlens_q.to(dev), w4.seqused_k.to(dev), w4.block_table.to(dev)
        mixed = {}
        for name, cdt in (("bf16", torch.bfloat16), ("fp8_e4m3fn", torch.float8_e4m3fn)):
            kc4 = torch.empty(w4.k_cache.shape, dtype=cdt, device=dev)
            vc4 = torch.empty_like(kc4)
            sc = torch.tensor([0.01], dtype=torch.float32, device=dev) if cdt == torch.float8_e4m3fn else None
            f4 = lambda: ua.kv_append(kn4, vn4, kc4, vc4, cu4, kv4, bt4, sc, sc, stream=stream)
            for _ in range(3):
                f4()
            torch.cuda.synchronize()
            t = time_calls(f4, 20, stream)
            b4 = append_bytes(kn4, kc4)
            mixed[name] = {"ms_median": round(float(np.median(t)), 4),
                           "GB/s": round(b4 / (np.median(t) * 1e-3) / 1e9, 1), "bytes": b4}
        result["mixed_batch_append"] = mixed
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_append(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def bwd_flops(q_lens, k_lens, heads: int, causal: bool, D: int = 128) -> float:
    """Algorithmic FLOPs of a backward: 2.5x the forward's 4 * D per visible
    (query, key) pair and head (five 2 * D products per pair: the recomputed
    scores, dV, dP, dQ, dK)."""
    import numpy as np
    pairs = 0
    for ql, kl in zip(q_lens, k_lens):
        if causal:
            pos = kl - ql + np.arange(ql)
            pairs += int(np.clip(pos + 1, 0, kl).sum())
        else:
            pairs += ql * kl
    return 10.0 * D * pairs * heads


def main_bwd(args) -> None:
    """Attention backward on the backward benchmark shape: O and LSE from one
    (untimed) HIP forward; a step is one ua_attention_backward call (the dQ
    kernel, which also forms Delta, then the dK/dV kernel).  Value: algorithmic
    TFLOP/s."""
    import numpy as np
    import torch

    import paged_varlen_flashattention_amd as ua
    import workloads as wk
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    ua.load_library()
    dev = torch.device("cuda:0")
    case = wk.backward_bench()
    B, N, H = 4, 4096, 32
    causal = True
    q, k, v, do = (case[n].to(dev) for n in ("q", "k", "v", "dout"))
    cu_q, cu_k = case["cu_seqlens_q"].to(dev), case["cu_seqlens_k"].to(dev)
    # forward (paged view of the dense k, v: contiguous 16-key pages)
    kc, vc = k.view(B * N // 16, 16, H, 128), v.view(B * N // 16, 16, H, 128)
    table = (torch.arange(B * N // 16, dtype=torch.int32, device=dev).view(B, N // 16)).contiguous()
    kl = torch.full((B,), N, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(B * N, H, dtype=torch.float32, device=dev)
    ua.unified_attention(q, kc, vc, out, cu_q, kl, table, N, N, case["softmax_scale"], causal, lse=lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ua.bwd_workspace_size(B * N, H), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    fn = lambda: ua.attention_backward(q, k, v, out, do, lse, cu_q, cu_k, dq, dk, dv,
                                       case["softmax_scale"], causal, workspace=ws, stream=stream)
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / K
    durs = np.array([a.elapsed_time(b) for a, b in evs])
    flops = bwd_flops([N] * B, [N] * B, H, causal)
    value = flops / (ms_step * 1e-3) / 1e12
    ach = flops / (durs.mean() * 1e-3) / 1e12
    result = {
        "metric": "attention backward TFLOP/s (2.5x forward FLOPs)", "value": round(value, 1),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic (seeded N(0,1) q, k, v, dO; O and LSE from the HIP forward)",
        "config": {"workload": "attn_bwd_dense_b4_h32_n4096_d128_causal_fp16", "batch": B, "heads": H,
                   "seq_len": N, "softmax_scale": case["softmax_scale"]},
        "roofline": {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_MFMA_TFLOPS, 4), "traffic": traffic_from_profiles("bwd_call"),
                     "launch_ms_mean": round(float(durs.mean()), 4),
                     "kernel": "one ua_attention_backward call (dQ + dK/dV kernels)"},
        "per_call": {"backward": {"ms_mean": round(float(durs.mean()), 4), "ms_min": round(float(durs.min()), 4),
                                  "ms_median": round(float(np.median(durs)), 4), "flops": flops}},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_bwd(case, causal, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline_bwd(case, causal: bool, target_s: float) -> dict:
    """The float64 backward oracle, as it stands, on a bounded sample of the
    same workload: whole (sequence, head) problems (4096 x 4096) cycled until
    about target_s seconds; TFLOP/s by the same FLOP count."""
    import numpy as np

    import oracle.backward as ob
    N = case["q_lens"][0]
    H = case["q"].shape[1]
    S = len(case["q_lens"])
    work, elapsed, calls = 0.0, 0.0, 0
    cu = np.array([0, N])
    while elapsed < target_s:
        s, h = calls % S, (calls // S) % H
        sl = slice(s * N, (s + 1) * N)
        t0 = time.perf_counter()
        ob.attention_backward(case["q"][sl, h:h + 1], case["k"][sl, h:h + 1], case["v"][sl, h:h + 1],
                              case["dout"][sl, h:h + 1], cu, cu, case["softmax_scale"], causal)
        elapsed += time.perf_counter() - t0
        work += bwd_flops([N], [N], 1, causal)
        calls += 1
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    return {"value": round(work / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{calls} whole (sequence, head) backward problems of {N} x {N} by the numpy float64 "
                      f"oracle (BLAS threads {cores}), {elapsed:.1f} s on {platform.processor() or 'host'}"}


def cpu_baseline_append(wl, target_s: float) -> dict:
    """The append oracle, as it stands, on a bounded sample of the same batch:
    whole sequences appended one call each, cycling over the batch until about
    target_s seconds; GB/s of algorithmic bytes."""
    import torch

    import oracle.append as oa
    work, elapsed, calls = 0, 0.0, 0
    cu = wl.cu_seqlens_q.numpy()
    S = len(cu) - 1
    while elapsed < target_s:
        s = calls % S
        n = int(cu[s + 1] - cu[s])
        t0 = time.perf_counter()
        oa.kv_append(wl.q[cu[s]:cu[s + 1]], wl.q[cu[s]:cu[s + 1]], torch.tensor([0, n], dtype=torch.int32),
                     wl.seqused_k[s:s + 1], wl.block_table[s:s + 1], wl.k_cache, wl.v_cache)
        elapsed += time.perf_counter() - t0
        work += n * wl.q.shape[1] * wl.q.shape[2] * 2 * (2 + 2)
        calls += 1
    return {"value": round(work / elapsed / 1e9, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} whole-sequence appends ({n} tokens x {wl.q.shape[1]} kv heads each) of the "
                      f"same batch by the numpy oracle (single thread; each call also copies the caches it "
                      f"returns), {elapsed:.1f} s on {platform.processor() or 'host'}"}


def time_calls(fn, n: int, stream, flush=None):
    """Per-call durations (ms) of n calls of fn, each bracketed by HIP events on
    `stream`; with `flush`, it runs before every call, outside the events."""
    import numpy as np
    import torch
    durs = []
    for _ in range(n):
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        durs.append(e0.elapsed_time(e1))
    return np.array(durs)


def extras(args, prepared, per, result, call, stream) -> None:
    """Measurements made after the timed region (they do not enter `value`):
    per-call times with L2/MALL flushed before each call (a 512 MB write; median
    and min of 50 calls, after the warm-up and timed calls), the
    decode batch at splits 1/2/4/8, and the mixed batch's prefill-only and
    decode-only sub-batches with its roofline time max(F/P_mfma, B_KV/P_hbm)."""
    import numpy as np
    import torch

    import workloads as wk
    dev = torch.device("cuda:0")
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush = lambda: scrub.fill_(1)
    for label, wl, splits, d, ws in prepared:
        t = time_calls(lambda: call(wl, splits, d, ws), 50, stream, flush)
        per_r = result["per_call"][label]
        per_r["ms_cold_median"] = round(float(np.median(t)), 4)
        per_r["ms_cold_min"] = round(float(t.min()), 4)

    def run_sub(wl, splits):
        d = {"q": wl.q.to(dev), "k": wl.k_cache.to(dev), "v": wl.v_cache.to(dev),
             "cu": wl.cu_seqlens_q.to(dev), "kv": wl.seqused_k.to(dev), "bt": wl.block_table.to(dev),
             "ks": None if wl.k_scale is None else torch.tensor([wl.k_scale], device=dev),
             "vs": None if wl.v_scale is None else torch.tensor([wl.v_scale], device=dev),
             "alibi": None if wl.alibi_slopes is None else wl.alibi_slopes.to(dev),
             "window": (wl.window_left, wl.window_right),
             "f8": bool(wl.meta.get("fp8_compute", False))}
        d["out"] = torch.empty_like(d["q"])
        import paged_varlen_flashattention_amd as ua
        ws = None
        if abs(splits) > 1:
            ws = torch.empty(ua.workspace_size(wl.num_tokens, wl.num_q_heads, 128, abs(splits)),
                             dtype=torch.uint8, device=dev)
        fn = lambda: call(wl, splits, d, ws)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t = time_calls(fn, 20, stream)
        return float(np.median(t)), float(t.min())

    if args.config == "c3":
        wl = prepared[0][1]
        sweep = []
        for sp in (1, 2, 4, 8):
            med, mn = run_sub(wl, sp)
            sweep.append({"splits": sp, "ms_median": round(med, 4), "ms_min": round(mn, 4),
                          "GB/s": round(wl.kv_bytes() / (med * 1e-3) / 1e9, 1),
                          "hbm_frac": round(wl.kv_bytes() / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)})
        result["splits_sweep"] = sweep
    if args.config in ("c2fp8", "c5"):
        # the same calls in the other compute mode (c2fp8: 16-bit compute on
        # the e4m3 cache; c5: fp8 compute), timed apart, not part of `value`
        other = {}
        for label, wl, splits, d, ws in prepared:
            w2 = wk.Workload(**{**wl.__dict__, "meta": {**wl.meta, "fp8_compute": args.config == "c5"}})
            med, mn = run_sub(w2, splits)
            unit = "TFLOP/s" if args.config == "c2fp8" else "GB/s"
            val = w2.flops() / (med * 1e-3) / 1e12 if args.config == "c2fp8" else w2.kv_bytes() / (med * 1e-3) / 1e9
            other[label] = {"ms_median": round(med, 4), "ms_min": round(mn, 4), unit: round(val, 1)}
        result["fp8_compute" if args.config == "c5" else "sixteen_bit_compute"] = other
    if args.config == "c2mask":
        # the same causal batch without window or bias, for the cost of the
        # mask-and-bias path
        plain = wk.with_mask(prepared[0][1], -1, -1, None, name="c2_causal_plain")
        med, mn = run_sub(plain, 1)
        result["plain_causal"] = {"ms_median": round(med, 4), "ms_min": round(mn, 4),
                                  "TFLOP/s": round(plain.flops() / (med * 1e-3) / 1e12, 1)}
    if args.config == "c4":
        wl = prepared[0][1]
        ql = wl.q_lens
        dec = wk.subset(wl, [s for s in range(len(ql)) if ql[s] == 1], "c4_decode_part")
        pre = wk.subset(wl, [s for s in range(len(ql)) if ql[s] > 1], "c4_prefill_part")
        # the decode part alone unsplit and with the launch's decode split,
        # the prefill part alone, and the whole batch with no split at all
        ds = abs(prepared[0][2])
        med_d, _ = run_sub(dec, 1)
        med_ds, _ = run_sub(dec, ds) if ds > 1 else (med_d, None)
        med_p, _ = run_sub(pre, 1)
        med_u, _ = run_sub(wl, 1)
        t_mfma = wl.flops() / (PEAK_MFMA_TFLOPS * 1e12) * 1e6
        t_hbm = wl.kv_bytes() / (PEAK_HBM_GBS * 1e9) * 1e6
        t_roof = max(t_mfma, t_hbm)
        meas = per[prepared[0][0]]["ms_median"] * 1e3
        gbs = lambda ms: dec.kv_bytes() / (ms * 1e-3) / 1e9
        result["sub_batches"] = {
            "decode_only": {"splits": 1, "ms_median": round(med_d, 4), "GB/s": round(gbs(med_d), 1),
                            "hbm_frac": round(gbs(med_d) / PEAK_HBM_GBS, 4)},
            "decode_only_split": {"splits": ds, "ms_median": round(med_ds, 4),
                                  "GB/s": round(gbs(med_ds), 1),
                                  "hbm_frac": round(gbs(med_ds) / PEAK_HBM_GBS, 4)},
            "prefill_only": {"ms_median": round(med_p, 4),
                             "TFLOP/s": round(pre.flops() / (med_p * 1e-3) / 1e12, 1),
                             "mfma_frac": round(pre.flops() / (med_p * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4)},
            "whole_unsplit": {"ms_median": round(med_u, 4),
                              "TFLOP/s": round(wl.flops() / (med_u * 1e-3) / 1e12, 1)},
            "t_roof_us": round(t_roof, 1), "t_roof_mfma_us": round(t_mfma, 1),
            "t_roof_hbm_us": round(t_hbm, 1), "measured_us": round(meas, 1),
            "frac_of_roof": round(t_roof / meas, 4)}


def cpu_baseline(prepared, compute_bound: bool, target_s: float) -> dict:
    """The fp64 C oracle, as it stands, on a bounded sample of the same rows,
    timed on the host cores; scaled to the metric's unit."""
    import numpy as np

    import oracle

    threads = os.cpu_count() or 1
    rng = np.random.default_rng(0)
    work = 0.0
    elapsed = 0.0
    nrows = 0
    n = max(16, threads * 4)
    while elapsed < target_s and n <= 1 << 22:
        for label, wl, splits, d, ws in prepared:
            toks = rng.integers(0, wl.num_tokens, size=n)
            heads = rng.integers(0, wl.num_q_heads, size=n)
            rows = np.stack([toks, heads], axis=1)
            t0 = time.perf_counter()
            oracle.attention_workload(wl, rows=rows, threads=threads)
            elapsed += time.perf_counter() - t0
            nrows += n
            work += row_work(wl, toks, compute_bound)
        n *= 2
    value = work / elapsed / (1e12 if compute_bound else 1e9)
    return {"value": round(value, 6), "unit": "TFLOP/s" if compute_bound else "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{nrows} random (token, head) rows of the same workload, fp64 C oracle "
                      f"(OpenMP, {threads} threads), {elapsed:.1f} s on {platform.processor() or 'host'}"}


def row_work(wl, toks, compute_bound: bool) -> float:
    """Algorithmic flops (or KV bytes) of the given rows."""
    import numpy as np
    cu = wl.cu_seqlens_q.numpy()
    kv = wl.kv_lens
    s = np.searchsorted(cu, toks, side="right") - 1
    ql = cu[s + 1] - cu[s]
    i = toks - cu[s]
    pos = kv[s] - ql + i
    hi = np.minimum(kv[s], pos + 1) if wl.causal else kv[s]
    if wl.window_right >= 0:
        hi = np.minimum(hi, pos + wl.window_right + 1)
    lo = np.maximum(pos - wl.window_left, 0) if wl.window_left >= 0 else 0
    vis = np.maximum(hi - lo, 0)
    if compute_bound:
        return float(4.0 * wl.head_size * vis.sum())
    G = wl.num_q_heads // wl.num_kv_heads
    return float((vis * wl.head_size * wl.k_cache.element_size() * 2 / G).sum())


if __name__ == "__main__":
    main()
