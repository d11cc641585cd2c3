"""Backward of packed variable-length attention (TEST INFRASTRUCTURE ONLY).

Only tests/, the smoke check and the bench's CPU baseline use this module; the
product path never does.

What it computes (page "Fused Attention", the tutorial's backward: the
preprocess that forms Delta, the dK/dV loop and the dQ loop, each recomputing
P from the forward's per-row log-sum-exp): for the loss L = sum(dO * O) with
O = softmax(scale * Q K^T) V under the mask of the forward, the gradients

    P   = softmax(scale * Q K^T)               (rows with no visible key: 0)
    dV  = P^T dO
    dP  = dO V^T
    Delta_i = sum_d O_id dO_id                 (the preprocess)
    dS  = P * (dP - Delta)                     (row-wise broadcast of Delta)
    dQ  = scale * dS K
    dK  = scale * dS^T Q

per sequence and per query head; a kv head's dK and dV add up the
contributions of the Hq / Hkv query heads that read it (head h reads kv head
h // (Hq / Hkv), page "vLLM Triton unified attention notes", section
kernel_unified_attention_2d).  Layout: dense packed rows, as the tutorial's
[Z, H, N, D] tensors with the batch replaced by cu_seqlens: q, out, dout
[T, Hq, D] with sequence s on rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]; k, v
[Tk, Hkv, D] with sequence s on rows cu_seqlens_k[s] .. cu_seqlens_k[s+1].
The causal mask is aligned bottom-right as in the forward: query i of a
sequence with q_len queries and kv_len keys sits at key position
kv_len - q_len + i and sees keys j <= that position.

Everything is float64, matrix by matrix, straight from the formulas above;
Delta uses the exact O of the definition.  Besides the gradients it returns,
for the error bounds of the tests, the magnitudes

    mag_dv[j, d] = sum_i P_ij |dO_id|
    mag_dk[j, d] = scale * sum_i A_ij |Q_id|
    mag_dq[i, d] = scale * sum_j A_ij |K_jd|,   A_ij = P_ij (|dP_ij| + |Delta_i| + sum_d |O_id dO_id|)

(sums of the absolute terms each gradient is made of).
"""
from __future__ import annotations

import numpy as np

from .bruteforce import to_f64


def attention_backward(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, softmax_scale, causal):
    """q, dout [T, Hq, D]; k, v [Tk, Hkv, D] (any float dtype, read exactly);
    cu_seqlens_q, cu_seqlens_k [S + 1] int.  Returns a dict of float64 arrays:
    dq [T, Hq, D], dk, dv [Tk, Hkv, D], out [T, Hq, D], lse [T, Hq] (natural
    log, -inf for rows with no visible key), delta [T, Hq] and the magnitudes
    mag_dq, mag_dk, mag_dv."""
    Q, K, V, dO = to_f64(q), to_f64(k), to_f64(v), to_f64(dout)
    cq = np.asarray(cu_seqlens_q, dtype=np.int64).reshape(-1)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64).reshape(-1)
    T, Hq, D = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    scale = float(softmax_scale)
    res = {name: np.zeros(shape) for name, shape in
           (("dq", Q.shape), ("dk", K.shape), ("dv", V.shape), ("out", Q.shape),
            ("delta", (T, Hq)), ("mag_dq", Q.shape), ("mag_dk", K.shape), ("mag_dv", V.shape))}
    res["lse"] = np.full((T, Hq), -np.inf)
    for s in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[s], cq[s + 1], ck[s], ck[s + 1]
        ql, kl = q1 - q0, k1 - k0
        if ql == 0:
            continue
        pos = (kl - ql) + np.arange(ql)[:, None]          # key position of each query
        visible = np.ones((ql, kl), dtype=bool)
        if causal:
            visible &= np.arange(kl)[None, :] <= pos
        any_visible = visible.any(axis=1)
        for h in range(Hq):
            g = h // G
            Qh, Kg, Vg, dOh = Q[q0:q1, h], K[k0:k1, g], V[k0:k1, g], dO[q0:q1, h]
            S = np.where(visible, scale * (Qh @ Kg.T), -np.inf)
            m = np.where(any_visible, S.max(axis=1, initial=-np.inf), 0.0)
            E = np.where(visible, np.exp(S - m[:, None]), 0.0)
            den = E.sum(axis=1)
            P = E / np.where(den > 0, den, 1.0)[:, None]
            O = P @ Vg
            delta = (O * dOh).sum(axis=1)
            dP = dOh @ Vg.T
            dS = P * (dP - delta[:, None])
            res["dq"][q0:q1, h] = scale * (dS @ Kg)
            res["dk"][k0:k1, g] += scale * (dS.T @ Qh)
            res["dv"][k0:k1, g] += P.T @ dOh
            res["out"][q0:q1, h] = O
            res["delta"][q0:q1, h] = delta
            res["lse"][q0:q1, h] = np.where(den > 0, m + np.log(np.where(den > 0, den, 1.0)), -np.inf)
            A = P * (np.abs(dP) + np.abs(delta)[:, None] + np.abs(O * dOh).sum(axis=1)[:, None])
            res["mag_dv"][k0:k1, g] += P.T @ np.abs(dOh)
            res["mag_dk"][k0:k1, g] += scale * (A.T @ np.abs(Qh))
            res["mag_dq"][q0:q1, h] = scale * (A @ np.abs(Kg))
    return res
