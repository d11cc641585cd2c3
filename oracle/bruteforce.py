"""Numpy brute force for paged, variable-length attention (TEST INFRASTRUCTURE ONLY).

A second, independent reading of the same definition as ``ua_oracle.c``, in a
different shape: for each sequence it materialises the dense K and V of the
sequence by walking its logical positions through the page table (page "vLLM
Triton unified attention notes", section kernel_unified_attention_2d), repeats
the kv heads for the query heads they serve, builds the full score matrix,
masks it with the causal band offset by the cached context (bottom-right
alignment: query i sits at position kv_len - q_len + i), and applies the
softmax of the definition on page "flashatten takeaways EP2 工程", section
"kv cache".  float64 throughout; meant for tiny inputs.
"""
from __future__ import annotations

import numpy as np
import torch


def decode_e4m3fn_table() -> np.ndarray:
    """float64 value of each of the 256 OCP E4M3FN codes (bias 7, NaN = S.1111.111)."""
    codes = np.arange(256)
    sign = np.where(codes >> 7, -1.0, 1.0)
    e = (codes >> 3) & 0xF
    m = (codes & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * np.exp2(-6.0)
    val = np.where(e == 0, sub, normal) * sign
    val[(e == 15) & ((codes & 7) == 7)] = np.nan
    return val


_E4M3 = decode_e4m3fn_table()


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a bf16 / fp16 / fp8_e4m3fn tensor, decoded with numpy."""
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).numpy().astype(np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if t.dtype == torch.float16:
        return t.view(torch.int16).numpy().view(np.float16).astype(np.float64)
    if t.dtype == torch.float8_e4m3fn:
        return _E4M3[t.view(torch.uint8).numpy().astype(np.int64)]
    if t.dtype in (torch.float32, torch.float64):
        return t.numpy().astype(np.float64)
    raise TypeError(t.dtype)


def attention(q, k_cache, v_cache, cu_seqlens_q, seqused_k, block_table, softmax_scale,
              causal, k_scale=None, v_scale=None, window=(-1, -1), alibi_slopes=None):
    """Returns out [T, Hq, D] and lse [T, Hq] (natural log), float64.

    window=(left, right) keeps the band pos - left <= j <= pos + right of the
    dense score matrix (negative: no bound); alibi_slopes [Hq] adds
    -slope[h] * |pos - j| to every scaled score."""
    Q = to_f64(q)
    Kc = to_f64(k_cache) * (1.0 if k_scale is None else float(k_scale))
    Vc = to_f64(v_cache) * (1.0 if v_scale is None else float(v_scale))
    cu = cu_seqlens_q.numpy().astype(np.int64)
    kvl = seqused_k.numpy().astype(np.int64)
    bt = block_table.numpy().astype(np.int64)
    T, Hq, D = Q.shape
    bs, Hkv = Kc.shape[1], Kc.shape[2]
    G = Hq // Hkv
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    for s in range(len(kvl)):
        q0, q1 = cu[s], cu[s + 1]
        ql, kl = q1 - q0, kvl[s]
        if ql == 0:
            continue
        # dense K_s, V_s [kl, Hkv, D] by walking logical positions
        Ks = np.stack([Kc[bt[s, j // bs], j % bs] for j in range(kl)])
        Vs = np.stack([Vc[bt[s, j // bs], j % bs] for j in range(kl)])
        Kh = np.repeat(Ks, G, axis=1)          # [kl, Hq, D]: query head h uses kv head h // G
        Vh = np.repeat(Vs, G, axis=1)
        Qs = Q[q0:q1]                          # [ql, Hq, D]
        S_ = np.einsum("ihd,jhd->hij", Qs, Kh) * softmax_scale    # [Hq, ql, kl]
        pos_q = (kl - ql) + np.arange(ql)[:, None]                # [ql, 1]
        pos_k = np.arange(kl)[None, :]                            # [1, kl]
        if alibi_slopes is not None:
            slopes = np.asarray(alibi_slopes, dtype=np.float64).reshape(-1)
            S_ = S_ - slopes[:, None, None] * np.abs(pos_q - pos_k)[None]
        visible = np.ones((ql, kl), dtype=bool)
        if causal:
            visible &= pos_k <= pos_q
        if window[0] >= 0:
            visible &= pos_k >= pos_q - window[0]
        if window[1] >= 0:
            visible &= pos_k <= pos_q + window[1]
        S_ = np.where(visible[None], S_, -np.inf)
        mx = S_.max(axis=-1, keepdims=True)
        mx_safe = np.where(np.isfinite(mx), mx, 0.0)              # rows with no visible key
        P = np.exp(S_ - mx_safe)
        den = P.sum(axis=-1, keepdims=True)
        W = np.divide(P, den, out=np.zeros_like(P), where=den > 0)
        out[q0:q1] = np.einsum("hij,jhd->ihd", W, Vh)
        lse[q0:q1] = np.where(den > 0, mx_safe + np.log(np.where(den > 0, den, 1.0)), -np.inf)[..., 0].T
    return out, lse


def attention_workload(wl):
    slopes = getattr(wl, "alibi_slopes", None)
    return attention(wl.q, wl.k_cache, wl.v_cache, wl.cu_seqlens_q, wl.seqused_k, wl.block_table,
                     wl.softmax_scale, wl.causal, wl.k_scale, wl.v_scale,
                     window=(getattr(wl, "window_left", -1), getattr(wl, "window_right", -1)),
                     alibi_slopes=None if slopes is None else to_f64(slopes))
