"""Pins of the KV-cache append oracle (oracle/append.py), CPU only.

- slot positions against a hand-derived fixture (tests/golden/append_positions.json);
- the fp8 e4m3fn encoder against torch's float8_e4m3fn cast (a library
  routine) after the saturation the definition states, on random values, every
  code value, every midpoint between neighbouring codes and values just off
  them, and the saturation edge;
- encode(decode(c)) == c for every finite code;
- rows other than the appended ones are untouched; relabelling physical block
  ids relabels the result.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import append as oa
from oracle.bruteforce import decode_e4m3fn_table

HERE = os.path.dirname(os.path.abspath(__file__))


def _fixture():
    with open(os.path.join(HERE, "golden", "append_positions.json")) as f:
        return json.load(f)


def _distinct_rows(T, Hkv, D=128, dtype=torch.bfloat16):
    # row (t, h) holds values that identify t and h exactly in bf16
    t = torch.arange(T, dtype=torch.float32).view(T, 1, 1)
    h = torch.arange(Hkv, dtype=torch.float32).view(1, Hkv, 1)
    d = torch.arange(D, dtype=torch.float32).view(1, 1, D)
    return (t * 4 + h + 1 + d * 0).to(dtype) * torch.where(d % 2 == 0, 1.0, -1.0).to(dtype)


def test_append_positions_golden():
    g = _fixture()
    bs, NB, Hkv = g["block_size"], g["num_blocks"], g["num_kv_heads"]
    cu = torch.tensor(g["cu_seqlens_q"], dtype=torch.int32)
    kv = torch.tensor(g["seqused_k"], dtype=torch.int32)
    bt = torch.tensor(g["block_table"], dtype=torch.int32)
    T = int(cu[-1])
    k_new = _distinct_rows(T, Hkv)
    v_new = -k_new
    sentinel = torch.full((NB, bs, Hkv, 128), 7.0, dtype=torch.bfloat16)
    kc, vc = oa.kv_append(k_new, v_new, cu, kv, bt, sentinel, sentinel.clone())
    written = set()
    for t, blk, slot in g["expected_token_block_slot"]:
        assert torch.equal(kc[blk, slot], k_new[t]) and torch.equal(vc[blk, slot], v_new[t])
        written.add((blk, slot))
    for blk in range(NB):
        for slot in range(bs):
            if (blk, slot) not in written:
                assert torch.all(kc[blk, slot] == 7.0) and torch.all(vc[blk, slot] == 7.0)


def _torch_saturating_fp8(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, np.float32)).clamp(-448.0, 448.0).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_cast():
    rng = np.random.default_rng(11)
    vals = decode_e4m3fn_table()
    finite = np.sort(np.unique(np.abs(vals[np.isfinite(vals)])))
    mids = (finite[1:] + finite[:-1]) / 2
    probes = [rng.standard_normal(100_000).astype(np.float32) * s for s in (1e-3, 0.05, 1, 30, 600)]
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
                           np.nextafter(mids.astype(np.float32), np.float32(-np.inf))])
    edge = np.float32([0.0, -0.0, 448.0, -448.0, 449.0, 464.0, 464.0001, 1e6, -1e6, 2.0**-10, -2.0**-10,
                       2.0**-9, 2.0**-9 * 0.5, 2.0**-9 * 1.5, 2.0**-9 * 2.5])
    x = np.concatenate(probes + [finite.astype(np.float32), -finite.astype(np.float32),
                                 mids.astype(np.float32), -mids.astype(np.float32), near, -near, edge])
    np.testing.assert_array_equal(oa.encode_e4m3fn(x), _torch_saturating_fp8(x))


def test_encode_ties_go_to_even_codes():
    vals = decode_e4m3fn_table()[:127]
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    exact = mids.astype(np.float64) == (vals[1:] + vals[:-1]) / 2      # representable midpoints
    codes = oa.encode_e4m3fn(mids[exact])
    assert np.all(codes % 2 == 0)


def test_encode_decode_round_trip_every_finite_code():
    vals = decode_e4m3fn_table()
    codes = np.arange(256)
    ok = np.isfinite(vals)
    np.testing.assert_array_equal(oa.encode_e4m3fn(vals[ok].astype(np.float32)), codes[ok].astype(np.uint8))


@pytest.mark.parametrize("cache_dtype", [torch.bfloat16, torch.float8_e4m3fn])
def test_append_untouched_rows_and_page_relabel(cache_dtype):
    rng = np.random.default_rng(5)
    bs, NB, Hkv, D = 16, 40, 2, 128
    q_lens = [3, 0, 20, 1]
    kv_lens = [3, 9, 33, 50]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]), dtype=torch.int32)
    kv = torch.tensor(kv_lens, dtype=torch.int32)
    bt = torch.tensor(rng.permutation(NB)[:16].reshape(4, 4), dtype=torch.int32)
    T = int(cu[-1])
    k_new = torch.from_numpy(rng.standard_normal((T, Hkv, D)).astype(np.float32)).to(torch.bfloat16)
    v_new = torch.from_numpy(rng.standard_normal((T, Hkv, D)).astype(np.float32)).to(torch.bfloat16)
    if cache_dtype == torch.float8_e4m3fn:
        base = torch.from_numpy(rng.integers(0, 126, size=(NB, bs, Hkv, D), dtype=np.uint8)).view(cache_dtype)
        ks, vs = 0.0123, 0.0456
    else:
        base = torch.from_numpy(rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32)).to(cache_dtype)
        ks = vs = None
    kc, vc = oa.kv_append(k_new, v_new, cu, kv, bt, base, base.clone(), ks, vs)
    touched = set()
    for s in range(4):
        for i in range(q_lens[s]):
            pos = kv_lens[s] - q_lens[s] + i
            touched.add((int(bt[s, pos // bs]), pos % bs))
    as_bits = lambda t: t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t.view(torch.int16)
    for blk in range(NB):
        for slot in range(bs):
            if (blk, slot) not in touched:
                assert torch.equal(as_bits(kc[blk, slot]), as_bits(base[blk, slot]))
    if cache_dtype == torch.float8_e4m3fn:
        # what was stored is torch's saturating cast of x / scale (float32 division)
        s, i = 2, 5
        pos = kv_lens[s] - q_lens[s] + i
        row = kc[int(bt[s, pos // bs]), pos % bs].view(torch.uint8).numpy()
        ref = _torch_saturating_fp8(k_new[int(cu[s]) + i].float().numpy() / np.float32(ks))
        np.testing.assert_array_equal(row, ref)
    # relabel physical ids: cache'[pi(b)] = cache[b], table' = pi(table)
    pi = torch.tensor(rng.permutation(NB), dtype=torch.int64)
    base2 = torch.empty_like(base)
    base2[pi] = base
    kc2, _ = oa.kv_append(k_new, v_new, cu, kv, pi[bt.long()].to(torch.int32), base2, base2.clone(), ks, vs)
    assert torch.equal(as_bits(kc2[pi]), as_bits(kc))
