"""Seeded synthetic inputs for paged, variable-length attention.

This module only *draws* inputs: sequence lengths, query/key/value values and
block tables.  It holds none of the attention arithmetic, so both the CPU oracle
(``oracle/``) and the GPU library (``paged_varlen_flashattention_amd``) can be
fed from it without sharing any of the method's code.

Workloads follow the shapes of the pages:

* page "vLLM Triton unified attention notes", section ``test_triton_unified_attn``:
  packed queries ``[sum(q_len), Hq, D]``, a paged cache
  ``[num_blocks, block_size, Hkv, D]``, ``cu_seqlens_q`` as an inclusive prefix
  sum with a leading 0, and one block table row per sequence whose ids are drawn
  at random from the block pool;
* page "Fused Attention" (FA2 tutorial listing, benchmark section): dense
  batch 4 x 32 heads, N(0,1) values, which we express as one contiguous block
  table per sequence.

Every random draw comes from ``numpy.random.default_rng`` seeded by
``SeedSequence([config_id, stream_id, chunk])``; streams are 0 lengths, 1 q,
2 k, 3 v, 4 block ids.  Large tensors are drawn in fixed chunks of
``CHUNK`` elements (each chunk its own seed), so the values do not depend on how
many threads draw them.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np
import torch

CHUNK = 1 << 22          # elements per independently seeded chunk
FP8_MAX = 448.0          # largest finite OCP E4M3FN magnitude

STREAM_LENGTHS, STREAM_Q, STREAM_K, STREAM_V, STREAM_BLOCKS = 0, 1, 2, 3, 4

TORCH_DTYPES = {
    "bf16": torch.bfloat16,
    "fp16": torch.float16,
    "fp8_e4m3fn": torch.float8_e4m3fn,
}


@dataclass
class Workload:
    """One batch of inputs for a paged varlen attention call (CPU tensors)."""
    name: str
    q: torch.Tensor                 # [T, Hq, D] bf16 / fp16
    k_cache: torch.Tensor           # [NB, bs, Hkv, D] bf16 / fp16 / fp8_e4m3fn
    v_cache: torch.Tensor           # [NB, bs, Hkv, D]
    cu_seqlens_q: torch.Tensor      # [S+1] int32, cu[0] = 0
    seqused_k: torch.Tensor         # [S] int32, kv length including the new queries
    block_table: torch.Tensor       # [S, W] int32
    softmax_scale: float
    causal: bool
    k_scale: Optional[float] = None  # fp32 per-tensor dequant scales (fp8 KV only)
    v_scale: Optional[float] = None
    num_splits: int = 1
    meta: dict = field(default_factory=dict)
    window_left: int = -1            # local attention: keys pos - left .. pos + right (-1: unbounded)
    window_right: int = -1
    alibi_slopes: Optional[torch.Tensor] = None   # [Hq] fp32 ALiBi slopes, or None

    @property
    def q_lens(self) -> np.ndarray:
        cu = self.cu_seqlens_q.numpy().astype(np.int64)
        return cu[1:] - cu[:-1]

    @property
    def kv_lens(self) -> np.ndarray:
        return self.seqused_k.numpy().astype(np.int64)

    @property
    def num_seqs(self) -> int:
        return int(self.seqused_k.numel())

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_cache.shape[2])

    @property
    def head_size(self) -> int:
        return int(self.q.shape[2])

    @property
    def block_size(self) -> int:
        return int(self.k_cache.shape[1])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_seqlen_q(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(self.kv_lens.max()) if self.num_seqs else 0

    def visible_pairs(self) -> int:
        """Number of visible (query, key) pairs per query head (causal: bottom-right
        aligned; with a window, only keys pos - left .. pos + right)."""
        total = 0
        local = self.window_left >= 0 or self.window_right >= 0
        for ql, kl in zip(self.q_lens.tolist(), self.kv_lens.tolist()):
            if local:
                pos = np.arange(kl - ql, kl, dtype=np.int64)
                lo = np.maximum(pos - self.window_left, 0) if self.window_left >= 0 else np.zeros_like(pos)
                hi = np.full_like(pos, kl)
                if self.causal:
                    hi = np.minimum(hi, pos + 1)
                if self.window_right >= 0:
                    hi = np.minimum(hi, pos + self.window_right + 1)
                total += int(np.maximum(hi - lo, 0).sum())
            elif self.causal:
                ctx = kl - ql
                # query i sees keys 0 .. ctx + i
                total += ql * ctx + ql * (ql + 1) // 2
            else:
                total += ql * kl
        return total

    def flops(self) -> float:
        """Algorithmic FLOPs: two matmuls of 2*D flops per visible pair and head."""
        return 4.0 * self.head_size * self.num_q_heads * self.visible_pairs()

    def kv_bytes(self) -> int:
        """K and V bytes read once per (sequence, kv head)."""
        elt = self.k_cache.element_size()
        return int(self.kv_lens.sum()) * self.num_kv_heads * self.head_size * elt * 2


# --------------------------------------------------------------------------- draws

def _seed(config_id: int, stream: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(config_id), int(stream), int(chunk)]))


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_tensor(config_id: int, stream: int, shape: Sequence[int], dtype: str) -> torch.Tensor:
    """N(0,1) values rounded (round-to-nearest-even, by torch's cast) to bf16 or fp16."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=TORCH_DTYPES[dtype])
    step = 64 * CHUNK
    for lo in range(0, n, step):
        hi = min(n, lo + step)
        # lo is a multiple of CHUNK, so chunk seeds do not depend on the step
        vals = _normal_range(config_id, stream, lo, hi)
        out[lo:hi] = torch.from_numpy(vals).to(out.dtype)
    return out.view(*shape)


def _normal_range(config_id: int, stream: int, lo: int, hi: int) -> np.ndarray:
    """Elements [lo, hi) of the chunked stream (lo, hi multiples of CHUNK except at the end)."""
    assert lo % CHUNK == 0
    out = np.empty(hi - lo, dtype=np.float32)
    c0 = lo // CHUNK
    nchunks = (hi - lo + CHUNK - 1) // CHUNK

    def fill(k: int) -> None:
        a = k * CHUNK
        b = min(hi - lo, a + CHUNK)
        _seed(config_id, stream, c0 + k).standard_normal(b - a, dtype=np.float32, out=out[a:b])

    if nchunks <= 1:
        for k in range(nchunks):
            fill(k)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def fp8_quantised_tensor(config_id: int, stream: int, shape: Sequence[int]):
    """N(0,1) values quantised to OCP E4M3FN with one per-tensor scale.

    scale = amax(|x|) / 448 over the whole tensor; codes = RNE(x / scale), clamped
    to +-448, by torch's float8_e4m3fn cast.  Returns (codes, scale) where the
    dequantised value is codes * scale.
    """
    n = int(np.prod(shape))
    vals = _normal_range(config_id, stream, 0, n)
    amax = float(np.abs(vals).max()) if n else 1.0
    scale = np.float32(amax / FP8_MAX)
    codes = torch.empty(n, dtype=torch.float8_e4m3fn)
    step = 64 * CHUNK
    for lo in range(0, n, step):
        hi = min(n, lo + step)
        x = torch.from_numpy(vals[lo:hi]) / float(scale)
        codes[lo:hi] = x.clamp_(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes.view(*shape), float(scale)


def block_tables(config_id: int, num_seqs: int, width: int, num_blocks: int, mode: str,
                 kv_lens: Optional[Sequence[int]] = None, block_size: int = 16,
                 poison_unused: bool = False) -> torch.Tensor:
    """Per-sequence page tables.

    mode 'perm': a seeded random permutation of physical ids, perm(NB)[:S*W];
    mode 'replace': ids drawn uniformly with replacement from [0, NB);
    mode 'contiguous': sequence s owns blocks s*W .. s*W + W - 1.
    With poison_unused, entries past ceil(kv_len / block_size) are set to -1.
    """
    rng = _seed(config_id, STREAM_BLOCKS)
    if mode == "perm":
        if num_seqs * width > num_blocks:
            raise ValueError("pool too small for a permutation table")
        ids = rng.permutation(num_blocks)[: num_seqs * width].reshape(num_seqs, width)
    elif mode == "replace":
        ids = rng.integers(0, num_blocks, size=(num_seqs, width))
    elif mode == "contiguous":
        ids = np.arange(num_seqs * width).reshape(num_seqs, width)
        if num_seqs * width > num_blocks:
            raise ValueError("pool too small for contiguous tables")
    else:
        raise ValueError(mode)
    ids = ids.astype(np.int32)
    if poison_unused:
        assert kv_lens is not None
        for s, kl in enumerate(kv_lens):
            used = (int(kl) + block_size - 1) // block_size
            ids[s, used:] = -1
    return torch.from_numpy(np.ascontiguousarray(ids))


def uniform_ints(config_id: int, lo: int, hi: int, n: int, stream: int = STREAM_LENGTHS,
                 chunk: int = 0) -> np.ndarray:
    """n integers uniform on [lo, hi] inclusive."""
    return _seed(config_id, stream, chunk).integers(lo, hi + 1, size=n)


# --------------------------------------------------------------------------- builders

def make_paged(name: str, seed_id: int, q_lens: Sequence[int], kv_lens: Sequence[int],
               num_q_heads: int, num_kv_heads: int, head_size: int = 128,
               block_size: int = 16, num_blocks: Optional[int] = None,
               width: Optional[int] = None, dtype: str = "bf16", kv_dtype: Optional[str] = None,
               table_mode: str = "perm", causal: bool = True,
               softmax_scale: Optional[float] = None, num_splits: int = 1,
               poison_unused: bool = False) -> Workload:
    """A paged varlen batch with N(0,1) q/k/v, seeded by ``seed_id``."""
    q_lens = [int(x) for x in q_lens]
    kv_lens = [int(x) for x in kv_lens]
    if len(q_lens) != len(kv_lens):
        raise ValueError("q_lens and kv_lens differ in length")
    for ql, kl in zip(q_lens, kv_lens):
        if ql > kl:
            raise ValueError("q_len > kv_len is not a valid input")
    kv_dtype = kv_dtype or dtype
    S = len(q_lens)
    T = sum(q_lens)
    need = max([(kl + block_size - 1) // block_size for kl in kv_lens] + [1])
    W = width or need
    if W < need:
        raise ValueError("block table too narrow")
    if num_blocks is None:
        num_blocks = S * W if table_mode in ("perm", "contiguous") else max(S * W, 1)
    cu = np.zeros(S + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    q = normal_tensor(seed_id, STREAM_Q, (T, num_q_heads, head_size), dtype)
    cache_shape = (num_blocks, block_size, num_kv_heads, head_size)
    k_scale = v_scale = None
    if kv_dtype == "fp8_e4m3fn":
        k_cache, k_scale = fp8_quantised_tensor(seed_id, STREAM_K, cache_shape)
        v_cache, v_scale = fp8_quantised_tensor(seed_id, STREAM_V, cache_shape)
    else:
        k_cache = normal_tensor(seed_id, STREAM_K, cache_shape, kv_dtype)
        v_cache = normal_tensor(seed_id, STREAM_V, cache_shape, kv_dtype)
    bt = block_tables(seed_id, S, W, num_blocks, table_mode, kv_lens, block_size, poison_unused)
    return Workload(
        name=name, q=q, k_cache=k_cache, v_cache=v_cache,
        cu_seqlens_q=torch.from_numpy(cu), seqused_k=torch.tensor(kv_lens, dtype=torch.int32),
        block_table=bt,
        softmax_scale=softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(head_size),
        causal=causal, k_scale=k_scale, v_scale=v_scale, num_splits=num_splits,
        meta={"seed_id": seed_id, "table_mode": table_mode, "dtype": dtype, "kv_dtype": kv_dtype},
    )


def alibi_slopes(num_heads: int) -> torch.Tensor:
    """The customary ALiBi slopes for num_heads heads: the geometric sequence
    2^(-8 (h + 1) / n) for the next power of two n >= num_heads, interleaved as
    usual when num_heads is not a power of two.  fp32 [num_heads]."""
    def pow2(n):
        return [2.0 ** (-8.0 * (h + 1) / n) for h in range(n)]
    n = 1 << (max(num_heads, 1) - 1).bit_length()
    if n == num_heads:
        vals = pow2(n)
    else:
        half = n // 2
        vals = pow2(half) + pow2(n)[0::2][: num_heads - half]
    return torch.tensor(vals, dtype=torch.float32)


def with_mask(wl: Workload, window_left: int = -1, window_right: int = -1,
              alibi: Optional[torch.Tensor] = None, name: Optional[str] = None) -> Workload:
    """The same batch with local attention and / or ALiBi slopes."""
    return Workload(**{**wl.__dict__, "name": name or wl.name, "window_left": int(window_left),
                       "window_right": int(window_right), "alibi_slopes": alibi})


def config1() -> Workload:
    """Tiny paged varlen batch (page 1, test_triton_unified_attn shapes): 3 sequences,
    q_lens [1,5,129], kv_lens [1328,18,463], 4/4 heads, D 128, bs 16, 512 blocks,
    permutation block tables, bf16, causal, scale 1/sqrt(128)."""
    return make_paged("c1_tiny_paged", 1, [1, 5, 129], [1328, 18, 463], 4, 4, 128,
                      block_size=16, num_blocks=512, width=83, dtype="bf16",
                      table_mode="perm", causal=True)


def config2(causal: bool = True, batch: int = 4, heads: int = 32, seq: int = 4096,
            kv_dtype: Optional[str] = None) -> Workload:
    """Dense FA2 forward (page 3 tutorial benchmark family) as a paged layout with
    contiguous tables: batch 4, 32 heads, N 4096, D 128, fp16, causal or not.
    kv_dtype="fp8_e4m3fn": the same draws quantised into an e4m3 cache."""
    bs = 16
    W = seq // bs
    tag = "" if kv_dtype is None else "_fp8kv"
    return make_paged(f"c2_dense_b{batch}_h{heads}_n{seq}_{'causal' if causal else 'full'}{tag}", 2,
                      [seq] * batch, [seq] * batch, heads, heads, 128, block_size=bs,
                      num_blocks=batch * W, width=W, dtype="fp16", kv_dtype=kv_dtype,
                      table_mode="contiguous", causal=causal)


def config3_lengths(n: int = 256) -> np.ndarray:
    return uniform_ints(3, 512, 8192, n)


def config3(num_splits: int = 1, num_seqs: int = 256, num_blocks: int = 65536) -> Workload:
    """Decode-heavy paged GQA batch: 256 x (q 1, kv U{512..8192}), 32/8 heads, bs 16,
    tables with replacement over a 65536-block pool, bf16."""
    kv = config3_lengths(num_seqs)
    return make_paged(f"c3_decode_s{num_seqs}_splits{num_splits}", 3, [1] * num_seqs, kv, 32, 8, 128,
                      block_size=16, num_blocks=num_blocks, width=512, dtype="bf16",
                      table_mode="replace", causal=True, num_splits=num_splits)


def config4_lengths():
    dec_kv = uniform_ints(4, 1024, 16384, 64)
    prefix = uniform_ints(4, 0, 8192, 4, chunk=1)
    q_lens = [1] * 64 + [2048] * 4
    kv_lens = list(dec_kv) + [int(p) + 2048 for p in prefix]
    return q_lens, kv_lens


def config4() -> Workload:
    """Mixed chunked prefill: 64 decode sequences (q 1, kv U{1024..16384}) + 4 prefill
    chunks of 2048 tokens with cached prefix U{0..8192}; 64/8 heads, bs 32, bf16, causal."""
    q_lens, kv_lens = config4_lengths()
    return make_paged("c4_mixed_chunked_prefill", 4, q_lens, kv_lens, 64, 8, 128, block_size=32,
                      num_blocks=34816, width=512, dtype="bf16", table_mode="perm", causal=True)


def config5(num_splits: int = 32, kv_len: int = 131072) -> Workload:
    """Long-context split-KV: q_lens [1,16], kv 131072, 64/8 heads, bs 16, fp8 e4m3fn KV
    with per-tensor scales, bf16 q, 32 splits."""
    W = kv_len // 16
    return make_paged(f"c5_long_fp8_splits{num_splits}", 5, [1, 16], [kv_len, kv_len], 64, 8, 128,
                      block_size=16, num_blocks=2 * W, width=W, dtype="bf16",
                      kv_dtype="fp8_e4m3fn", table_mode="perm", causal=True,
                      num_splits=num_splits)


def subset(wl: Workload, seqs: Sequence[int], name: Optional[str] = None) -> Workload:
    """The sub-batch made of the given sequences (same caches and table rows;
    their query rows repacked in order)."""
    cu = wl.cu_seqlens_q.numpy().astype(np.int64)
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs]).astype(np.int64)
    lens = [int(cu[s + 1] - cu[s]) for s in seqs]
    new_cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    idx = torch.as_tensor(np.asarray(seqs, dtype=np.int64))
    return Workload(**{**wl.__dict__, "name": name or f"{wl.name}_subset",
                       "q": wl.q[torch.as_tensor(rows)].contiguous(), "cu_seqlens_q": new_cu,
                       "seqused_k": wl.seqused_k[idx].contiguous(),
                       "block_table": wl.block_table[idx].contiguous(), "meta": dict(wl.meta)})


def append_case(seed: int, *, num_seqs: int = 4, max_new: int = 40, max_prefix: int = 100,
                kv_heads: int = 2, block_size: int = 16, new_dtype: str = "bf16",
                cache_dtype: Optional[str] = None, saturate: bool = False) -> dict:
    """Seeded inputs of a KV-cache append (CPU tensors): new rows k_new / v_new
    [T, Hkv, 128] (N(0,1) x 3), lengths (q_len U{0..max_new}, at least one > 0;
    kv_len = prefix U{0..max_prefix} + q_len), permuted page tables (entries past
    each sequence's last page poisoned with -1), caches filled with unrelated
    values (finite fp8 codes for an fp8 cache), and for an fp8 cache per-tensor
    scales amax / 448 (or amax / 600 with `saturate`, so that some values
    exceed the largest code)."""
    cache_dtype = cache_dtype or new_dtype
    rng = _seed(4000 + seed, STREAM_LENGTHS)
    q_lens = rng.integers(0, max_new + 1, size=num_seqs)
    if q_lens.max() == 0:
        q_lens[0] = 1
    kv_lens = rng.integers(0, max_prefix + 1, size=num_seqs) + q_lens
    pages = np.maximum(1, (kv_lens + block_size - 1) // block_size)
    W = int(pages.max())
    NB = int(pages.sum()) + 7
    ids = rng.permutation(NB)
    bt = np.full((num_seqs, W), -1, dtype=np.int32)
    at = 0
    for s in range(num_seqs):
        bt[s, :pages[s]] = ids[at:at + pages[s]]
        at += pages[s]
    T = int(q_lens.sum())
    D = 128
    g = _seed(4000 + seed, STREAM_K)
    tdt = TORCH_DTYPES[new_dtype]
    k_new = torch.from_numpy((g.standard_normal((T, kv_heads, D)) * 3).astype(np.float32)).to(tdt)
    v_new = torch.from_numpy((g.standard_normal((T, kv_heads, D)) * 3).astype(np.float32)).to(tdt)
    shape = (NB, block_size, kv_heads, D)
    if cache_dtype == "fp8_e4m3fn":
        codes = g.integers(0, 0x7F, size=shape, dtype=np.uint8) | (g.integers(0, 2, size=shape, dtype=np.uint8) << 7)
        k_cache = torch.from_numpy(codes).view(torch.float8_e4m3fn)
        codes = g.integers(0, 0x7F, size=shape, dtype=np.uint8) | (g.integers(0, 2, size=shape, dtype=np.uint8) << 7)
        v_cache = torch.from_numpy(codes).view(torch.float8_e4m3fn)
        div = 600.0 if saturate else FP8_MAX
        k_scale = float(k_new.float().abs().max()) / div if T else 1.0
        v_scale = float(v_new.float().abs().max()) / div if T else 1.0
    else:
        k_cache = torch.from_numpy(g.standard_normal(shape).astype(np.float32)).to(TORCH_DTYPES[cache_dtype])
        v_cache = torch.from_numpy(g.standard_normal(shape).astype(np.float32)).to(TORCH_DTYPES[cache_dtype])
        k_scale = v_scale = None
    return {"k_new": k_new, "v_new": v_new,
            "cu_seqlens_q": torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]), dtype=torch.int32),
            "seqused_k": torch.tensor(kv_lens, dtype=torch.int32), "block_table": torch.from_numpy(bt),
            "k_cache": k_cache, "v_cache": v_cache, "k_scale": k_scale, "v_scale": v_scale}


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def random_small(seed: int, *, max_seqs: int = 4, max_kv: int = 70, heads=(4, 2),
                 block_size: Optional[int] = None, head_size: int = 128, dtype: str = "bf16",
                 kv_dtype: Optional[str] = None, causal: Optional[bool] = None,
                 allow_empty_q: bool = True) -> Workload:
    """A tiny random paged batch for brute-force comparisons (seed ids 1000 + seed)."""
    rng = _seed(1000 + seed, STREAM_LENGTHS)
    S = int(rng.integers(1, max_seqs + 1))
    kv = rng.integers(1, max_kv + 1, size=S)
    lo = 0 if allow_empty_q else 1
    ql = [int(rng.integers(lo, k + 1)) for k in kv]
    bs = block_size or int(rng.choice([16, 32]))
    c = bool(rng.integers(0, 2)) if causal is None else causal
    hq, hkv = heads
    return make_paged(f"rand{seed}", 1000 + seed, ql, kv.tolist(), hq, hkv, head_size,
                      block_size=bs, num_blocks=None, dtype=dtype, kv_dtype=kv_dtype,
                      table_mode="perm", causal=c,
                      softmax_scale=float(rng.uniform(0.02, 0.2)))


def random_feature_case(i: int) -> tuple:
    """Case i of a seeded sweep across the forward's features: G 1..16, 1-6
    sequences mixing decode-like (q 0..4), short and long prefill rows, kv up
    to q + 1000, bf16/fp16 queries, 16-bit or e4m3 caches, pages of 16-128,
    causal or full, default or random scales, split counts 1/auto/2..8 and
    decode-row splits, and now and then a local window and / or ALiBi.
    Returns (workload, num_splits)."""
    import random
    rng = random.Random(31000 + int(i))
    G = rng.choice([1, 2, 3, 4, 8, 16]); hkv = rng.choice([1, 2, 4]); hq = G * hkv
    ql, kl = [], []
    for _ in range(rng.randint(1, 6)):
        r = rng.random()
        q = rng.randint(0, 4) if r < 0.3 else (rng.randint(5, 70) if r < 0.65 else rng.randint(70, 200))
        ql.append(q)
        kl.append(max(1, q + rng.randint(0, 1000)))
    dtype = rng.choice(["bf16", "fp16"])
    kvd = rng.choice([None, None, "fp8_e4m3fn"])
    bs = rng.choice([16, 32, 64, 128])
    causal = rng.random() < 0.7
    scale = None if rng.random() < 0.5 else rng.uniform(0.02, 0.3)
    splits = rng.choice([1, 1, 0, 2, 3, 4, 8, -2, -4])
    wl = make_paged(f"sweep{i}", 31000 + int(i), ql, kl, hq, hkv, block_size=bs, dtype=dtype, kv_dtype=kvd,
                    causal=causal, softmax_scale=scale)
    if rng.random() < 0.25:
        left = rng.choice([-1, rng.randint(0, 300)])
        right = rng.choice([-1, rng.randint(0, 50)]) if not causal else -1
        slopes = alibi_slopes(hq) if rng.random() < 0.5 else None
        if left >= 0 or right >= 0 or slopes is not None:
            wl = with_mask(wl, left, right, slopes)
    return wl, splits


# --------------------------------------------------------------------------- backward

def backward_case(seed: int, q_lens: Sequence[int], k_lens: Sequence[int], num_q_heads: int,
                  num_kv_heads: int, dtype: str = "bf16", softmax_scale: Optional[float] = None,
                  std: float = 1.0) -> dict:
    """Seeded inputs of an attention backward on dense packed rows (CPU tensors):
    q, dout [T, Hq, 128] and k, v [Tk, Hkv, 128], N(0, std^2) rounded to the
    dtype (dout N(0, 1)); cu_seqlens_q / cu_seqlens_k [S + 1] int32 from the
    lengths; softmax_scale (default 1 / sqrt(128)).  The page's tutorial test
    draws N(0, 0.5^2) inputs with scale 0.5 and its benchmark N(0, 1) with
    scale 1.3."""
    T, Tk = int(sum(q_lens)), int(sum(k_lens))
    sid = 7000 + int(seed)
    q = normal_tensor(sid, 1, (T, num_q_heads, 128), dtype)
    k = normal_tensor(sid, 2, (Tk, num_kv_heads, 128), dtype)
    v = normal_tensor(sid, 3, (Tk, num_kv_heads, 128), dtype)
    if std != 1.0:
        q, k, v = ((t.float() * std).to(t.dtype) for t in (q, k, v))
    dout = normal_tensor(sid, 4, (T, num_q_heads, 128), dtype)
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]), dtype=torch.int32)
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(k_lens)]), dtype=torch.int32)
    return {"q": q, "k": k, "v": v, "dout": dout, "cu_seqlens_q": cu_q, "cu_seqlens_k": cu_k,
            "q_lens": list(map(int, q_lens)), "k_lens": list(map(int, k_lens)),
            "softmax_scale": 1.0 / math.sqrt(128) if softmax_scale is None else float(softmax_scale),
            "dtype": dtype}


def backward_bench(batch: int = 4, heads: int = 32, seq: int = 4096) -> dict:
    """The page's backward benchmark (fused-attention, bwd, causal): batch 4,
    32 heads, N 4096, fp16, N(0,1) inputs, scale 1.3; head size 128."""
    return backward_case(8, [seq] * batch, [seq] * batch, heads, heads, "fp16", softmax_scale=1.3)


def backward_feature_case(i: int) -> tuple:
    """Case i of a seeded sweep across the backward's features: G 1..8,
    1-4 sequences with empty, single-row, short and long query runs, keys
    at least the queries (causal) or anything from none to 450 (full),
    bf16/fp16, default or random scales.  Returns (case, causal)."""
    import random
    rng = random.Random(41000 + int(i))
    G = rng.choice([1, 2, 3, 4, 8]); hkv = rng.choice([1, 2])
    causal = rng.random() < 0.6
    ql, kl = [], []
    for _ in range(rng.randint(1, 4)):
        q = rng.choice([0, 1, rng.randint(2, 40), rng.randint(40, 150)])
        k = q + rng.randint(0, 300) if causal else rng.choice([0, rng.randint(1, 40), rng.randint(40, 450)])
        ql.append(q)
        kl.append(k)
    dt = rng.choice(["bf16", "fp16"])
    scale = None if rng.random() < 0.5 else rng.uniform(0.05, 0.6)
    return backward_case(41000 + int(i), ql, kl, G * hkv, hkv, dt, softmax_scale=scale), causal


def fp8_weight_pin_case(q_len: int = 40) -> Workload:
    """A designed batch for the e4m3 rounding of the softmax weights in the
    fp8-compute mode: one sequence of q_len queries (one head, so every row is
    a prefill row once q_len > 32) against 64 keys in an e4m3 cache (one tile).

    Inputs only: every query row is all +1 (even tokens) or all -1 (odd
    tokens); key 0 is all zeros and key j (1..63) holds -A_j at d 0 and -B_j at
    d 1, with A_j + B_j = n_j, n_j running over 1..71 without multiples of 8
    (A_j, B_j exact e4m3 values); value j (1..63) is one-hot at d = j, value 0
    is zero.  k_scale = v_scale = 1 and softmax_scale = float32(ln 2 / 8) /
    (448 * float32(1 / 448)): with the row's e4m3 query codes (all +-448 under
    the row scale 1/448), a +1 row's score of key j is -n_j * ln2 / 8, so its
    weights relative to the maximum (key 0) are 2^(-n_j / 8); a -1 row's are
    2^((n_j - 71) / 8)."""
    n = [x for x in range(1, 72) if x % 8 != 0]
    assert len(n) == 63
    D = 128
    q = torch.ones(q_len, 1, D, dtype=torch.float32)
    q[1::2] = -1.0
    k = torch.zeros(4, 16, 1, D, dtype=torch.float32)
    v = torch.zeros(4, 16, 1, D, dtype=torch.float32)
    e4m3_ints = [float(x) for x in range(0, 17)] + [float(x) for x in range(18, 33, 2)] + \
        [float(x) for x in range(36, 65, 4)] + [float(x) for x in range(72, 129, 8)]
    bt = [2, 0, 3, 1]                      # logical page p lives in physical block bt[p]
    for j, nj in enumerate(n, start=1):
        a = max(x for x in e4m3_ints if x <= nj and nj - x in e4m3_ints)
        k[bt[j // 16], j % 16, 0, 0] = -a
        k[bt[j // 16], j % 16, 0, 1] = -(nj - a)
        v[bt[j // 16], j % 16, 0, j] = 1.0
    kc = k.to(torch.float8_e4m3fn)
    vc = v.to(torch.float8_e4m3fn)
    assert torch.equal(kc.float(), k) and torch.equal(vc.float(), v), "values exact in e4m3"
    sq = float(np.float32(1.0) / np.float32(448.0))
    scale = float(np.float32(math.log(2.0) / 8.0 / (448.0 * sq)))
    return Workload(
        name="fp8_weight_pin", q=q.to(torch.bfloat16), k_cache=kc, v_cache=vc,
        cu_seqlens_q=torch.tensor([0, q_len], dtype=torch.int32),
        seqused_k=torch.tensor([64], dtype=torch.int32),
        block_table=torch.tensor([bt], dtype=torch.int32),
        softmax_scale=scale, causal=False, k_scale=1.0, v_scale=1.0,
        meta={"n": n, "fp8_compute": True})
