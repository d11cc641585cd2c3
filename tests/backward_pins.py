"""Pins for the backward oracle (oracle/backward.py).

Every ``check_*`` takes a backward function with the signature of
``oracle.backward.attention_backward`` and raises AssertionError when it
disagrees with the pin.  ``tests/test_oracle_backward.py`` runs them on the
oracle and on copies of it with a planted mistake (each must fail a pin).

What pins what:
  * central finite differences of the loss sum(dO * O), O from the numpy
    brute-force forward (oracle/bruteforce.py, itself pinned to torch's
    scaled_dot_product_attention and closed forms): every gradient entry of
    tiny batches, causal and full, with GQA and a query longer than its keys;
  * torch autograd in float64 on the dense per-sequence formula (a library
    differentiation that shares nothing with the oracle's hand-written
    gradient formulas);
  * closed forms of the definition: with all keys of a head equal, the scores
    of a row are equal, so dQ = 0; with one key, P = 1 and dV is the sum of the
    dO rows, dQ = dK = 0; the rows of dS sum to zero, so the dK rows of a
    sequence and kv head sum to zero; the rows of P sum to one, so the dV rows
    sum to the dO rows of the rows that see any key; under the causal mask
    with q_len = kv_len the first query sees only key 0 and its dQ is 0.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle.bruteforce as bf


def _batch(seed, q_lens, k_lens, Hq, Hkv, D, scale=0.4):
    g = torch.Generator().manual_seed(seed)
    T, Tk = sum(q_lens), sum(k_lens)
    q = torch.randn(T, Hq, D, generator=g, dtype=torch.float64)
    k = torch.randn(Tk, Hkv, D, generator=g, dtype=torch.float64)
    v = torch.randn(Tk, Hkv, D, generator=g, dtype=torch.float64)
    do = torch.randn(T, Hq, D, generator=g, dtype=torch.float64)
    cq = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    ck = np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int64)
    return q, k, v, do, cq, ck, scale


def _forward_bruteforce(q, k, v, cq, ck, scale, causal):
    """O of the numpy brute force on a page-size-1 view of the dense k, v."""
    S = len(cq) - 1
    kl = np.diff(ck)
    width = max(1, int(kl.max()))
    table = np.zeros((S, width), dtype=np.int32)
    for s in range(S):
        table[s, :kl[s]] = ck[s] + np.arange(kl[s])
    out, _ = bf.attention(q, k[:, None], v[:, None], torch.from_numpy(cq.astype(np.int32)),
                          torch.from_numpy(kl.astype(np.int32)), torch.from_numpy(table), scale,
                          causal)
    return out


def check_finite_differences(fn):
    for causal in (True, False):
        q, k, v, do, cq, ck, scale = _batch(11, [3, 4, 2], [5, 4, 1], 4, 2, 4)
        got = fn(q, k, v, do, cq, ck, scale, causal)
        dO = do.numpy()
        h = 1e-6
        for name, t in (("dq", q), ("dk", k), ("dv", v)):
            num = np.zeros(t.shape)
            flat = t.view(-1)
            for idx in range(flat.numel()):
                old = float(flat[idx])
                flat[idx] = old + h
                lp = float((_forward_bruteforce(q, k, v, cq, ck, scale, causal) * dO).sum())
                flat[idx] = old - h
                lm = float((_forward_bruteforce(q, k, v, cq, ck, scale, causal) * dO).sum())
                flat[idx] = old
                num.reshape(-1)[idx] = (lp - lm) / (2 * h)
            err = np.abs(got[name] - num).max()
            assert err < 1e-6, f"{name} vs finite differences (causal={causal}): {err:.3e}"


def _autograd(q, k, v, do, cq, ck, scale, causal):
    q, k, v = (t.clone().requires_grad_(True) for t in (q, k, v))
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    outs = []
    for s in range(len(cq) - 1):
        qs, ks, vs = q[cq[s]:cq[s + 1]], k[ck[s]:ck[s + 1]], v[ck[s]:ck[s + 1]]
        ql, kl = qs.shape[0], ks.shape[0]
        kh = ks.repeat_interleave(G, dim=1).transpose(0, 1)      # [Hq, kl, D]
        vh = vs.repeat_interleave(G, dim=1).transpose(0, 1)
        sc = torch.matmul(qs.transpose(0, 1), kh.transpose(1, 2)) * scale   # [Hq, ql, kl]
        vis = torch.ones(ql, kl, dtype=torch.bool)
        if causal:
            vis = torch.arange(kl)[None, :] <= (kl - ql) + torch.arange(ql)[:, None]
        sc = sc.masked_fill(~vis, float("-inf"))
        p = torch.softmax(sc, dim=-1).nan_to_num(0.0)
        outs.append(torch.matmul(p, vh).transpose(0, 1))
    out = torch.cat(outs)
    (out * do).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def check_autograd(fn):
    for causal in (True, False):
        for seed, ql, kl, Hq, Hkv in ((21, [1, 17, 30], [9, 17, 45], 6, 2), (22, [12, 5], [8, 5], 4, 4)):
            q, k, v, do, cq, ck, scale = _batch(seed, ql, kl, Hq, Hkv, 16)
            got = fn(q, k, v, do, cq, ck, scale, causal)
            ref = _autograd(q, k, v, do, cq, ck, scale, causal)
            for name, r in zip(("dq", "dk", "dv"), ref):
                err = np.abs(got[name] - r).max()
                assert err < 1e-10, f"{name} vs autograd (causal={causal}, seed={seed}): {err:.3e}"


def check_equal_keys(fn):
    q, k, v, do, cq, ck, scale = _batch(31, [6, 3], [6, 9], 4, 2, 8)
    k[:] = k[0]                                   # every key of every head the same row
    for causal in (True, False):
        got = fn(q, k, v, do, cq, ck, scale, causal)
        assert np.abs(got["dq"]).max() < 1e-12, "dQ must vanish when all keys are equal"


def check_single_key(fn):
    q, k, v, do, cq, ck, scale = _batch(32, [4], [1], 4, 2, 8)
    got = fn(q, k, v, do, cq, ck, scale, False)
    assert np.abs(got["dq"]).max() < 1e-12 and np.abs(got["dk"]).max() < 1e-12
    G = 2
    want = do.numpy().reshape(4, 2, G, 8).sum(axis=(0, 2))      # heads 2g, 2g+1 read kv head g
    assert np.abs(got["dv"][0] - want).max() < 1e-12, "one key: dV = sum of dO over rows and group"


def check_row_sums(fn):
    for causal in (True, False):
        q, k, v, do, cq, ck, scale = _batch(33, [5, 7, 2], [9, 7, 1], 6, 3, 8)
        got = fn(q, k, v, do, cq, ck, scale, causal)
        G = 2
        dO = do.numpy()
        for s in range(len(cq) - 1):
            q0, q1, k0, k1 = cq[s], cq[s + 1], ck[s], ck[s + 1]
            assert np.abs(got["dk"][k0:k1].sum(axis=0)).max() < 1e-10, "dK rows must sum to 0"
            ql, kl = q1 - q0, k1 - k0
            sees = np.ones(ql, dtype=bool) if not causal else (kl - ql) + np.arange(ql) >= 0
            want = dO[q0:q1][sees].reshape(-1, 3, G, 8).sum(axis=(0, 2))
            assert np.abs(got["dv"][k0:k1].sum(axis=0) - want).max() < 1e-10, \
                "dV rows must sum to the dO rows that see a key"


def check_causal_first_row(fn):
    q, k, v, do, cq, ck, scale = _batch(34, [6], [6], 2, 1, 8)
    got = fn(q, k, v, do, cq, ck, scale, True)
    assert np.abs(got["dq"][0]).max() < 1e-12, "the first causal row sees one key: dQ = 0"
    assert np.abs(got["dq"][1:]).max() > 1e-3


BATTERY = [check_equal_keys, check_single_key, check_row_sums, check_causal_first_row,
           check_autograd, check_finite_differences]


def run_battery(fn) -> None:
    for check in BATTERY:
        check(fn)
