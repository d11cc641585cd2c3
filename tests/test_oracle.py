"""The CPU oracle against its pins (closed forms, library routines, invariants,
brute force).  CPU only."""
import pytest

import oracle
import oracle_pins as pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


def test_golden_closed_forms(lib):
    pins.check_golden_attention(lib)


def test_golden_closed_forms_bruteforce(lib):
    pins.check_golden_attention(lib, impl="bruteforce")


def test_golden_combine(lib):
    pins.check_golden_combine(lib)


def test_decoders_every_code(lib):
    pins.check_decoders(lib)


def test_sdpa_library_pin(lib):
    pins.check_sdpa(lib)


def test_sdpa_library_pin_bruteforce(lib):
    pins.check_sdpa(lib, impl="bruteforce")


def test_bruteforce_200_cases(lib):
    pins.check_bruteforce(lib, n=200)


def test_single_key_returns_value(lib):
    pins.check_single_key(lib)


def test_equal_keys_mean_of_visible_values(lib):
    pins.check_equal_keys(lib)


def test_page_relabel_bitwise(lib):
    pins.check_page_relabel(lib)


def test_gqa_replication(lib):
    pins.check_gqa_replication(lib)


def test_value_codes_give_softmax_weights(lib):
    pins.check_value_codes(lib)


def test_split_algebra(lib):
    pins.check_split_algebra(lib)


def test_page_structure():
    pins.check_page_structure()


def test_window_own_key(lib):
    pins.check_window_own_key(lib)


def test_alibi_geometric(lib):
    pins.check_alibi_geometric(lib)


def test_mask_neutral_settings(lib):
    pins.check_mask_neutral_settings(lib)


def test_mask_bruteforce(lib):
    pins.check_mask_bruteforce(lib, n=40)


# ------------------------------------------------------------------ fp8-compute mode

def test_fp8_quantize_rows_matches_torch_cast():
    """The e4m3 codes of q / s equal torch's float8_e4m3fn cast of the same
    float32 quotients (a library routine), for bf16 and fp16 queries."""
    import numpy as np
    import torch
    import oracle.fp8_compute as f8
    import workloads as wk
    for dtype in ("bf16", "fp16"):
        wl = wk.make_paged("q8", 2901, [3, 40, 9], [300, 200, 50], 16, 2, block_size=16,
                           dtype=dtype, kv_dtype="fp8_e4m3fn")
        codes, s, deq = f8.quantize_rows(wl.q)
        x = (wl.q.float().numpy() / s[..., None]).astype(np.float32)
        ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes, ref)


def test_fp8_quantize_rows_scale_closed_forms():
    """The largest element of each row maps to +-448 exactly; an all-zero row
    keeps scale 1 and zero codes; deq = code value * scale."""
    import numpy as np
    import torch
    import oracle.fp8_compute as f8
    q = torch.randn(7, 4, 128, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    q[2, 1] = 0
    codes, s, deq = f8.quantize_rows(q)
    assert s[2, 1] == 1.0 and not codes[2, 1].any()
    vals = deq / s[..., None]
    amax_pos = np.abs(q.float().numpy()).argmax(axis=-1)
    for t in range(7):
        for h in range(4):
            if (t, h) == (2, 1):
                continue
            assert abs(vals[t, h, amax_pos[t, h]]) == 448.0


def test_fp8_compute_rows_mask():
    """The mode applies to sequences with q_len * G > 32 rows only."""
    import oracle.fp8_compute as f8
    import workloads as wk
    wl = wk.make_paged("q8m", 2902, [1, 4, 5, 0, 33], [10, 10, 10, 5, 40], 8, 1, block_size=16,
                       kv_dtype="fp8_e4m3fn")
    m = f8.prefill_rows_mask(wl)          # G = 8: q_len 5 -> 40 rows > 32, q_len 4 -> 32 rows
    assert m.tolist() == [False] * 5 + [True] * 5 + [True] * 33
