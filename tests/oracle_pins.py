"""Pins for the CPU oracle: checks that tie it to something other than itself.

Every ``check_*`` takes the ctypes handle of a compiled oracle and raises
AssertionError when the oracle disagrees with the pin.  ``tests/test_oracle.py``
runs them on the real oracle; ``tests/test_oracle_mutants.py`` runs them on
copies of the oracle with a planted mistake and requires that some pin fails.

What pins what:
  * closed forms written by hand (tests/golden/closed_forms.json): weights,
    bottom-right causal alignment, GQA grouping, a gather across a page boundary,
    the log-sum-exp merge;
  * torch's float64 scaled_dot_product_attention on dense, unpaged inputs (a
    library routine): paging, strides, masking and GQA against an implementation
    that knows nothing of pages;
  * torch's bfloat16 / float8_e4m3fn casts and numpy's float16: the decoders,
    over every code;
  * the numpy brute force (oracle/bruteforce.py) on many tiny seeded batches;
  * invariants of the definition: one key returns its value; equal keys return
    the mean of the visible values; relabelling physical pages changes nothing;
    replicating kv heads for every query head changes nothing; a one-hot value
    code returns the softmax weights; partial results over any split of the keys
    merge back into the whole;
  * local attention and ALiBi (the FA2 window / slope switches): a (0, 0)
    window returns the value at the query's own position exactly; with zero
    keys and one-hot values the ALiBi weights are r^|pos - j| normalised, whose
    sum is a closed-form geometric series (the sign, the absolute value, the
    bottom-right position and the per-head slope all show); zero slopes and a
    window wider than the sequence change no bit; and the numpy brute force on
    tiny batches with random windows and slopes.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import oracle.bruteforce as bf
import workloads as wk

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-12


# ----------------------------------------------------------------- helpers

def _dense_vec(sparse: dict, D: int) -> np.ndarray:
    v = np.zeros(D)
    for k, x in sparse.items():
        v[int(k)] = x
    return v


def golden_workload(case: dict, D: int) -> wk.Workload:
    """Build a paged bf16 batch from a sparse closed-form case.  Keys of each
    sequence are stored in reversed physical page order, so the page table is
    not the identity."""
    q_lens, kv_lens = case["q_lens"], case["kv_lens"]
    Hq, Hkv, bs = case["num_q_heads"], case["num_kv_heads"], case["block_size"]
    q = np.stack([[_dense_vec(h, D) for h in tok] for tok in case["q"]])
    pages = [(kl + bs - 1) // bs for kl in kv_lens]
    NB, W = sum(pages), max(pages)
    kc = np.zeros((NB, bs, Hkv, D))
    vc = np.zeros((NB, bs, Hkv, D))
    bt = np.zeros((len(kv_lens), W), dtype=np.int32)
    nxt = NB - 1
    tok = 0
    for s, kl in enumerate(kv_lens):
        for p in range(pages[s]):
            bt[s, p] = nxt
            nxt -= 1
        for j in range(kl):
            b, slot = bt[s, j // bs], j % bs
            kc[b, slot] = [_dense_vec(h, D) for h in case["k"][tok + j]]
            vc[b, slot] = [_dense_vec(h, D) for h in case["v"][tok + j]]
        tok += kl
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    to = lambda a: torch.from_numpy(a).to(torch.bfloat16)
    return wk.Workload(name=case["name"], q=to(q), k_cache=to(kc), v_cache=to(vc),
                       cu_seqlens_q=torch.from_numpy(cu),
                       seqused_k=torch.tensor(kv_lens, dtype=torch.int32),
                       block_table=torch.from_numpy(bt), softmax_scale=case["softmax_scale"],
                       causal=case["causal"])


def load_golden() -> dict:
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        return json.load(f)


def _close(a, b, tol=TOL, what=""):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    same_inf = np.array_equal(np.isneginf(a), np.isneginf(b))
    assert same_inf, f"{what}: -inf pattern differs"
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: finiteness differs"
    err = float(np.abs(a[fin] - b[fin]).max()) if fin.any() else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------- pins

def check_golden_attention(lib, impl="oracle"):
    g = load_golden()
    D = g["head_size"]
    for case in g["attention"]:
        wl = golden_workload(case, D)
        if impl == "oracle":
            out, lse = oracle.attention_workload(wl, lib=lib, threads=1)
        else:
            out, lse = bf.attention_workload(wl)
        exp_out = np.stack([[_dense_vec(h, D) for h in tok] for tok in case["expect_out"]])
        _close(out, exp_out, what=case["name"] + " out")
        _close(lse, np.array(case["expect_lse"]), what=case["name"] + " lse")


def check_golden_combine(lib):
    for case in load_golden()["combine"]:
        out, lse = oracle.combine(np.array(case["o_part"]), np.array(case["lse_part"]), lib=lib)
        _close(out, np.array(case["expect_out"]), what=case["name"])
        _close(lse, np.array(case["expect_lse"]), what=case["name"] + " lse")


def check_decoders(lib):
    """Every code of each storage format against an independent library cast."""
    codes8 = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    fp8 = codes8.view(torch.float8_e4m3fn)
    got = oracle.decode(fp8, lib=lib)
    ref = fp8.to(torch.float32).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "fp8 NaN codes"
    assert set(np.flatnonzero(np.isnan(got)).tolist()) == {0x7F, 0xFF}, "fp8 NaN = S.1111.111"
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]), "fp8 values vs torch float8_e4m3fn"
    assert np.array_equal(got[ok], bf.decode_e4m3fn_table()[ok]), "fp8 vs numpy table"
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    codes16 = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    b16 = codes16.view(torch.bfloat16)
    got = oracle.decode(b16, lib=lib)
    ref = b16.to(torch.float32).double().numpy()
    assert np.array_equal(got, ref, equal_nan=True), "bf16 decode"
    h16 = codes16.view(torch.float16)
    got = oracle.decode(h16, lib=lib)
    ref = h16.numpy().astype(np.float64)
    assert np.array_equal(got, ref, equal_nan=True), "fp16 decode"


def sdpa_reference(wl):
    """Dense attention by torch's float64 scaled_dot_product_attention, sequence by
    sequence, from the dense K/V the workload's tables describe (a contiguous or
    permuted page table is resolved with a plain index)."""
    Q = torch.from_numpy(bf.to_f64(wl.q))
    Kc = torch.from_numpy(bf.to_f64(wl.k_cache)) * (wl.k_scale or 1.0)
    Vc = torch.from_numpy(bf.to_f64(wl.v_cache)) * (wl.v_scale or 1.0)
    bs = wl.block_size
    G = wl.num_q_heads // wl.num_kv_heads
    out = torch.zeros(Q.shape, dtype=torch.float64)
    cu = wl.cu_seqlens_q.tolist()
    for s, kl in enumerate(wl.kv_lens.tolist()):
        ql = cu[s + 1] - cu[s]
        if ql == 0:
            continue
        pos = torch.arange(kl)
        blocks = wl.block_table[s].long()[pos // bs]
        K = Kc[blocks, pos % bs]                    # [kl, Hkv, D]
        V = Vc[blocks, pos % bs]
        K = K.repeat_interleave(G, dim=1).transpose(0, 1)   # [Hq, kl, D]
        V = V.repeat_interleave(G, dim=1).transpose(0, 1)
        q = Q[cu[s]:cu[s + 1]].transpose(0, 1)               # [Hq, ql, D]
        mask = None
        if wl.causal:
            mask = pos[None, :] <= (kl - ql + torch.arange(ql))[:, None]
        o = F.scaled_dot_product_attention(q, K, V, attn_mask=mask, scale=wl.softmax_scale)
        out[cu[s]:cu[s + 1]] = o.transpose(0, 1)
    return out.numpy()


def sdpa_cases():
    yield wk.make_paged("dense_causal", 2001, [40, 40], [40, 40], 4, 4, block_size=16,
                        dtype="fp16", table_mode="contiguous", causal=True)
    yield wk.make_paged("dense_full", 2002, [33, 17], [33, 17], 4, 2, block_size=16,
                        dtype="bf16", table_mode="contiguous", causal=False)
    yield wk.make_paged("prefix_causal_gqa", 2003, [1, 7, 20], [50, 19, 41], 8, 2, block_size=16,
                        dtype="bf16", table_mode="perm", causal=True)
    yield wk.make_paged("bs32_full_gqa8", 2004, [3, 1], [70, 33], 8, 1, block_size=32,
                        dtype="bf16", table_mode="perm", causal=False)
    yield wk.make_paged("fp8_kv", 2005, [1, 5], [45, 30], 8, 2, block_size=16, dtype="bf16",
                        kv_dtype="fp8_e4m3fn", table_mode="perm", causal=True)


def check_sdpa(lib, impl="oracle"):
    for wl in sdpa_cases():
        ref = sdpa_reference(wl)
        if impl == "oracle":
            out, _ = oracle.attention_workload(wl, lib=lib, threads=2)
        else:
            out, _ = bf.attention_workload(wl)
        _close(out, ref, tol=1e-12, what=f"sdpa {wl.name}")


def brute_cases(n: int):
    for s in range(n):
        kind = s % 5
        if kind == 0:
            yield wk.random_small(s)
        elif kind == 1:
            yield wk.random_small(s, heads=(8, 2))
        elif kind == 2:
            yield wk.random_small(s, heads=(8, 1), dtype="fp16")
        elif kind == 3:
            yield wk.random_small(s, heads=(4, 4), kv_dtype="fp8_e4m3fn")
        else:
            yield wk.random_small(s, heads=(2, 1), max_seqs=3, max_kv=40)


def check_bruteforce(lib, n: int = 200):
    for wl in brute_cases(n):
        o1, l1 = oracle.attention_workload(wl, lib=lib, threads=2)
        o2, l2 = bf.attention_workload(wl)
        _close(o1, o2, what=f"brute {wl.name} out")
        _close(l1, l2, what=f"brute {wl.name} lse")


def check_single_key(lib):
    """kv_len = 1 (so q_len <= 1): the output is v_0 exactly, lse = the one score."""
    wl = wk.make_paged("one_key", 2101, [1, 0, 1], [1, 1, 1], 4, 2, block_size=16, causal=True)
    out, lse = oracle.attention_workload(wl, lib=lib)
    v = bf.to_f64(wl.v_cache)
    bt = wl.block_table.numpy()
    for t, s in ((0, 0), (1, 2)):
        for h in range(4):
            assert np.array_equal(out[t, h], v[bt[s, 0], 0, h // 2]), "one key returns v_0"


def check_equal_keys(lib):
    """All keys equal: every visible key has the same score, so the output is the
    mean of the visible value rows and lse = z + ln(#visible).  Pins the mask
    extent of every row, causal (bottom-right) and full."""
    for causal in (True, False):
        wl = wk.make_paged("equal_keys", 2201, [3, 1, 6], [9, 20, 6], 2, 1, block_size=16,
                           causal=causal)
        wl.k_cache[:] = wl.k_cache[0, 0, 0]
        out, lse = oracle.attention_workload(wl, lib=lib)
        Q = bf.to_f64(wl.q)
        k0 = bf.to_f64(wl.k_cache[0, 0, 0])
        V = bf.to_f64(wl.v_cache)
        bt = wl.block_table.numpy()
        cu = wl.cu_seqlens_q.tolist()
        for s, kl in enumerate(wl.kv_lens.tolist()):
            ql = cu[s + 1] - cu[s]
            for i in range(ql):
                n_vis = (kl - ql + i + 1) if causal else kl
                rows = np.stack([V[bt[s, j // 16], j % 16, 0] for j in range(n_vis)])
                for h in range(2):
                    t = cu[s] + i
                    _close(out[t, h], rows.mean(axis=0), tol=1e-12, what="equal keys mean")
                    z = wl.softmax_scale * float(Q[t, h] @ k0)
                    _close(lse[t, h], z + math.log(n_vis), tol=1e-12, what="equal keys lse")


def check_page_relabel(lib):
    """Relabelling physical pages (cache'[pi(b)] = cache[b], table' = pi(table))
    leaves every output bit unchanged."""
    wl = wk.make_paged("relabel", 2301, [4, 1, 9], [30, 47, 9], 4, 2, block_size=16, causal=True)
    out, lse = oracle.attention_workload(wl, lib=lib)
    NB = wl.num_blocks
    pi = torch.from_numpy(np.random.default_rng(7).permutation(NB))
    k2 = torch.empty_like(wl.k_cache)
    v2 = torch.empty_like(wl.v_cache)
    k2[pi] = wl.k_cache
    v2[pi] = wl.v_cache
    bt2 = pi[wl.block_table.long()].to(torch.int32)
    out2, lse2 = oracle.attention(wl.q, k2, v2, wl.cu_seqlens_q, wl.seqused_k, bt2,
                                  wl.softmax_scale, wl.causal, lib=lib)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2), "page relabel changed bits"


def check_gqa_replication(lib):
    """Replicating each kv head for the G query heads it serves (Hkv' = Hq) and
    running with G = 1 gives the same result."""
    wl = wk.make_paged("gqa", 2401, [2, 5], [21, 5], 8, 2, block_size=16, causal=True)
    out, lse = oracle.attention_workload(wl, lib=lib)
    G = 4
    k2 = wl.k_cache.repeat_interleave(G, dim=2).contiguous()
    v2 = wl.v_cache.repeat_interleave(G, dim=2).contiguous()
    out2, lse2 = oracle.attention(wl.q, k2, v2, wl.cu_seqlens_q, wl.seqused_k, wl.block_table,
                                  wl.softmax_scale, wl.causal, lib=lib)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2), "GQA replication"


def check_value_codes(lib):
    """V = ones gives 1 everywhere; V = one-hot position code gives the softmax
    weights, which sum to 1 and whose ratios are exp(z_j - z_k) for scores z
    computed here with numpy from the decoded q and k."""
    wl = wk.make_paged("vcodes", 2501, [2, 3], [40, 3], 2, 2, block_size=16, causal=True)
    wl.v_cache[:] = 1.0
    out, _ = oracle.attention_workload(wl, lib=lib)
    _close(out, np.ones_like(out), tol=1e-13, what="V = ones")
    vc = torch.zeros_like(wl.v_cache)
    bt = wl.block_table.numpy()
    for s, kl in enumerate(wl.kv_lens.tolist()):
        for j in range(kl):
            vc[bt[s, j // 16], j % 16, :, j] = 1.0          # value of key j = e_j
    out, _ = oracle.attention(wl.q, wl.k_cache, vc, wl.cu_seqlens_q, wl.seqused_k,
                              wl.block_table, wl.softmax_scale, wl.causal, lib=lib)
    Q, K = bf.to_f64(wl.q), bf.to_f64(wl.k_cache)
    cu = wl.cu_seqlens_q.tolist()
    for s, kl in enumerate(wl.kv_lens.tolist()):
        ql = cu[s + 1] - cu[s]
        for i in range(ql):
            t = cu[s] + i
            vis = kl - ql + i + 1
            for h in range(2):
                p = out[t, h]
                assert abs(p.sum() - 1.0) < 1e-13, "weights sum to 1"
                assert np.all(p[vis:] == 0.0), "masked keys weigh 0"
                z = np.array([wl.softmax_scale * (Q[t, h] @ K[bt[s, j // 16], j % 16, h])
                              for j in range(vis)])
                ref = np.exp(z - z.max())
                _close(p[:vis], ref / ref.sum(), tol=1e-13, what="one-hot weights")


def check_split_algebra(lib):
    """Partials over any partition of the key range, merged with the log-sum-exp
    combine, reproduce the unsplit result; empty splits weigh nothing."""
    rng = np.random.default_rng(11)
    for wl in (wk.make_paged("split_a", 2601, [1, 16, 3], [300, 200, 3], 8, 2, block_size=16,
                             causal=True),
               wk.make_paged("split_b", 2602, [5], [77], 4, 4, block_size=32, causal=False,
                             kv_dtype="fp8_e4m3fn")):
        full, lse_full = oracle.attention_workload(wl, lib=lib)
        T, Hq, D = full.shape
        for P in (1, 2, 3, 8, 32):
            kmax = int(wl.kv_lens.max())
            cuts = np.sort(rng.integers(0, kmax + 1, size=P - 1))
            edges = [0] + cuts.tolist() + [kmax]
            parts = [oracle.attention_workload(wl, kv_range=(edges[p], edges[p + 1]), lib=lib)
                     for p in range(P)]
            o_part = np.stack([p[0].reshape(T * Hq, D) for p in parts])
            l_part = np.stack([p[1].reshape(T * Hq) for p in parts])
            out, lse = oracle.combine(o_part, l_part, lib=lib)
            _close(out.reshape(T, Hq, D), full, tol=1e-12, what=f"split P={P}")
            _close(lse.reshape(T, Hq), lse_full, tol=1e-12, what=f"split lse P={P}")
    # every split empty -> 0 and -inf, not NaN
    out, lse = oracle.combine(np.ones((3, 2, 4)), np.full((3, 2), -np.inf), lib=lib)
    assert np.all(out == 0.0) and np.all(np.isneginf(lse)), "all-empty combine"


def check_page_structure():
    """Structural facts the pages print for the tiny batch (page 1, test section)."""
    with open(os.path.join(GOLDEN, "page_structure.json")) as f:
        g = json.load(f)
    wl = wk.config1()
    assert wl.num_seqs == g["config1_num_seqs"]
    assert wl.num_q_heads == g["config1_num_q_heads"]
    assert wl.num_kv_heads == g["config1_num_kv_heads"]
    assert list(wl.block_table.shape) == g["config1_block_table_shape"]
    assert math.ceil(g["config1_longest_kv"] / g["config1_block_size"]) == g["config1_block_table_shape"][1]


# ----------------------------------------------------------------- local attention and ALiBi

def _value_lookup(wl, s, j, g):
    """Decoded (and scaled) value row of key j, kv head g, sequence s."""
    V = bf.to_f64(wl.v_cache) * (1.0 if wl.v_scale is None else wl.v_scale)
    bt = wl.block_table.numpy()
    bs = wl.block_size
    return V[bt[s, j // bs], j % bs, g]


def check_window_own_key(lib):
    """Window (0, 0), not causal: each query sees only the key at its own
    absolute position kv_len - q_len + i, so the output is that value row
    exactly; with q = 0 the one score is 0 and lse = 0."""
    for kv_dtype in (None, "fp8_e4m3fn"):
        wl = wk.make_paged("win_own", 2501, [2, 1, 5], [9, 30, 17], 4, 2, block_size=16,
                           causal=False, kv_dtype=kv_dtype)
        wl = wk.with_mask(wl, 0, 0)
        out, lse = oracle.attention_workload(wl, lib=lib)
        cu = wl.cu_seqlens_q.tolist()
        for s, kl in enumerate(wl.kv_lens.tolist()):
            ql = cu[s + 1] - cu[s]
            for i in range(ql):
                for h in range(4):
                    want = _value_lookup(wl, s, kl - ql + i, h // 2)
                    assert np.array_equal(out[cu[s] + i, h], want), "(0, 0) window returns v_pos"
        wl.q.zero_()
        _, lse0 = oracle.attention_workload(wl, lib=lib)
        assert np.array_equal(lse0, np.zeros_like(lse0)), "one zero score: lse = 0"


def _geometric(r, n):
    """sum_{d=0}^{n-1} r^d in closed form."""
    return n if r == 1.0 else (1.0 - r ** n) / (1.0 - r)


def check_alibi_geometric(lib):
    """Zero keys, one-hot values (key j -> e_j): the scores are the ALiBi bias
    alone, so out[j] = r^|pos - j| / Z with r = exp(-slope) and Z a geometric
    sum in closed form; lse = ln Z.  Causal (with and without a left window)
    and full, per-head slopes through GQA."""
    slopes = np.array([0.5, 0.25, 0.125, 0.0625, 1.5, 0.03125], dtype=np.float64)
    for causal, window in ((True, (-1, -1)), (True, (6, -1)), (False, (-1, -1)), (False, (4, 3))):
        wl = wk.make_paged("alibi_geo", 2601, [3, 1, 4], [20, 37, 9], 6, 2, block_size=16,
                           causal=causal)
        wl.k_cache.zero_()
        wl.v_cache.zero_()
        bt = wl.block_table.numpy()
        for s, kl in enumerate(wl.kv_lens.tolist()):
            for j in range(kl):
                wl.v_cache[bt[s, j // 16], j % 16, :, j] = 1.0
        wl = wk.with_mask(wl, window[0], window[1], torch.tensor(slopes, dtype=torch.float32))
        out, lse = oracle.attention_workload(wl, lib=lib)
        cu = wl.cu_seqlens_q.tolist()
        for s, kl in enumerate(wl.kv_lens.tolist()):
            ql = cu[s + 1] - cu[s]
            for i in range(ql):
                pos = kl - ql + i
                lo = max(0, pos - window[0]) if window[0] >= 0 else 0
                hi = min(kl - 1, pos + window[1]) if window[1] >= 0 else kl - 1
                if causal:
                    hi = min(hi, pos)
                for h in range(6):
                    r = math.exp(-float(np.float32(slopes[h])))
                    Z = _geometric(r, pos - lo + 1) + r * _geometric(r, hi - pos)
                    t = cu[s] + i
                    _close(lse[t, h], math.log(Z), tol=1e-12, what="alibi lse geometric")
                    want = np.zeros(wl.head_size)
                    for j in range(lo, hi + 1):
                        want[j] = r ** abs(pos - j) / Z
                    _close(out[t, h], want, tol=1e-12, what="alibi weights")


def check_mask_neutral_settings(lib):
    """Zero slopes and a window wider than every sequence change no bit."""
    wl = wk.make_paged("neutral", 2701, [1, 6, 3], [40, 6, 25], 4, 1, block_size=16, causal=True)
    base, lbase = oracle.attention_workload(wl, lib=lib)
    for w in (wk.with_mask(wl, alibi=torch.zeros(4)), wk.with_mask(wl, 10_000, 10_000)):
        out, lse = oracle.attention_workload(w, lib=lib)
        assert np.array_equal(out, base) and np.array_equal(lse, lbase), "neutral mask settings"


def check_mask_bruteforce(lib, n: int = 30):
    """Random windows, slopes, causal flags and GQA on tiny batches against the
    numpy brute force (dense band masks, an independent formulation)."""
    rng = np.random.default_rng(2801)
    for c in range(n):
        S = int(rng.integers(1, 4))
        kv = [int(rng.integers(1, 70)) for _ in range(S)]
        ql = [int(rng.integers(0, k + 1)) for k in kv]
        Hkv = int(rng.choice([1, 2]))
        Hq = Hkv * int(rng.choice([1, 2, 3]))
        wl = wk.make_paged("mask_bf", 2810 + c, ql, kv, Hq, Hkv, block_size=16,
                           causal=bool(rng.integers(0, 2)),
                           kv_dtype="fp8_e4m3fn" if c % 5 == 4 else None)
        left = int(rng.choice([-1, 0, 1, 5, 17]))
        right = int(rng.choice([-1, 0, 2, 9]))
        slopes = torch.tensor(rng.uniform(0.0, 1.0, Hq), dtype=torch.float32) if c % 2 else None
        wl = wk.with_mask(wl, left, right, slopes)
        a, la = oracle.attention_workload(wl, lib=lib)
        b, lb = bf.attention_workload(wl)
        _close(a, b, tol=1e-12, what=f"mask brute force case {c}")
        assert np.array_equal(np.isneginf(la), np.isneginf(lb)), "empty rows agree"
        fin = np.isfinite(lb)
        _close(la[fin], lb[fin], tol=1e-12, what=f"mask brute force lse case {c}")


QUICK_BATTERY = [
    check_golden_attention, check_golden_combine, check_decoders, check_single_key,
    check_equal_keys, check_page_relabel, check_gqa_replication, check_value_codes,
    check_split_algebra, check_sdpa,
    lambda lib: check_bruteforce(lib, n=25),
    check_window_own_key, check_alibi_geometric, check_mask_neutral_settings,
    lambda lib: check_mask_bruteforce(lib, n=12),
]


def run_battery(lib) -> None:
    for check in QUICK_BATTERY:
        check(lib)
