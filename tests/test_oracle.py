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
