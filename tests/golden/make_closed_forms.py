"""Writes closed_forms.json: tiny attention problems whose answer is exact by hand.

Inputs are small integers (exact in bf16); head_size is 128 with only a few
non-zero coordinates.  Expected outputs are exact expressions of the
definition (page "flashatten takeaways EP2 工程", section "kv cache":
O = softmax(q K^T * scale) V), evaluated with the standard library only.
"""
import json
import math
import os

D = 128


def vec(**nz):
    """A sparse head_size-128 vector: {coordinate: value}, every other coordinate 0."""
    return {k[1:]: x for k, x in nz.items()}


cases = []

# 1. Two keys, scale = ln 3: scores [0, ln 3] -> weights [1/4, 3/4].
#    V rows 4*e1 and 8*e1 -> o[1] = 1 + 6 = 7; lse = ln(1 + 3) = ln 4.
cases.append({
    "name": "two_keys_weights_quarter_three_quarters",
    "cite": "page 'flashatten takeaways EP2 工程', section 'kv cache', boxed O_{t+1} formula",
    "q_lens": [1], "kv_lens": [2], "num_q_heads": 1, "num_kv_heads": 1, "block_size": 16,
    "causal": False, "softmax_scale": math.log(3.0),
    "q": [[vec(d0=1.0)]],
    "k": [[vec()], [vec(d0=1.0)]],
    "v": [[vec(d1=4.0)], [vec(d1=8.0)]],
    "expect_out": [[vec(d1=7.0)]],
    "expect_lse": [[math.log(4.0)]],
})

# 2. Bottom-right causal alignment: q_len 2, kv_len 3, values v_j = (j+1) e2,
#    all scores 0 (q = 0).  Query 0 sits at position 1 and sees keys {0, 1}:
#    o = mean(1, 2) = 1.5, lse = ln 2.  Query 1 sees {0, 1, 2}: o = 2, lse = ln 3.
cases.append({
    "name": "causal_bottom_right_alignment",
    "cite": "page 'vLLM Triton unified attention notes', section kernel_unified_attention_2d "
            "(context_len = tokens before the current queries); reading: query i at position kv_len - q_len + i",
    "q_lens": [2], "kv_lens": [3], "num_q_heads": 1, "num_kv_heads": 1, "block_size": 16,
    "causal": True, "softmax_scale": 0.125,
    "q": [[vec()], [vec()]],
    "k": [[vec(d3=1.0)], [vec(d3=2.0)], [vec(d3=3.0)]],
    "v": [[vec(d2=1.0)], [vec(d2=2.0)], [vec(d2=3.0)]],
    "expect_out": [[vec(d2=1.5)], [vec(d2=2.0)]],
    "expect_lse": [[math.log(2.0)], [math.log(3.0)]],
})

# 3. GQA: 4 query heads share 2 kv heads (G = 2).  kv head 0 holds values 1*e0,
#    kv head 1 holds 10*e0; one key, so o = v exactly.  Query heads 0,1 -> kv 0;
#    heads 2,3 -> kv 1 (h // G, page 1 section kernel_unified_attention_2d).
cases.append({
    "name": "gqa_consecutive_grouping",
    "cite": "page 'vLLM Triton unified attention notes', section kernel_unified_attention_2d "
            "(num_queries_per_kv = Hq / Hkv; largest query head index Hq - 1)",
    "q_lens": [1], "kv_lens": [1], "num_q_heads": 4, "num_kv_heads": 2, "block_size": 16,
    "causal": True, "softmax_scale": 0.5,
    "q": [[vec(d0=1.0), vec(d0=2.0), vec(d0=3.0), vec(d0=4.0)]],
    "k": [[vec(d0=1.0), vec(d0=1.0)]],
    "v": [[vec(d0=1.0), vec(d0=10.0)]],
    "expect_out": [[vec(d0=1.0), vec(d0=1.0), vec(d0=10.0), vec(d0=10.0)]],
    "expect_lse": [[0.5, 1.0, 1.5, 2.0]],
})

# 4. Paged gather across two physical blocks (block_size 16, kv_len 17): key 16
#    lives in the second page.  q = e0, k_16 = 2 e0, every other key 0, scale ln 2:
#    scores 0 (x16) and 2 ln 2 -> weights 1 each for 16 keys and 4 for key 16.
#    v_j = e5 for j < 16, v_16 = 21 e5 -> o[5] = (16 + 4*21) / 20 = 5; lse = ln 20.
cases.append({
    "name": "page_boundary_gather",
    "cite": "page 'vLLM Triton unified attention notes', section kernel_unified_attention_2d "
            "(physical block from the page table, slot = position mod block_size)",
    "q_lens": [1], "kv_lens": [17], "num_q_heads": 1, "num_kv_heads": 1, "block_size": 16,
    "causal": True, "softmax_scale": math.log(2.0),
    "q": [[vec(d0=1.0)]],
    "k": [[vec()]] * 16 + [[vec(d0=2.0)]],
    "v": [[vec(d5=1.0)]] * 16 + [[vec(d5=21.0)]],
    "expect_out": [[vec(d5=5.0)]],
    "expect_lse": [[math.log(20.0)]],
})

# Split combine: two partials with lse ln 1 and ln 3, outputs a and b -> (a + 3b)/4, ln 4.
combine = {
    "name": "combine_two_partials",
    "cite": "page 'flashatten takeaways EP2 工程', section '源代码接口' (split partials corrected by a "
            "combine step); page 'Fused Attention', section FlashDecoding (global reduce)",
    "lse_part": [[0.0], [math.log(3.0)]],
    "o_part": [[[2.0, -4.0]], [[6.0, 8.0]]],
    "expect_out": [[5.0, 5.0]],
    "expect_lse": [math.log(4.0)],
}

here = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(here, "closed_forms.json"), "w") as f:
    json.dump({"head_size": D, "attention": cases, "combine": [combine]}, f, indent=1)
