"""Pins of the oracle's attention over the compressed cache (attn_decode).

Each pin fixes the result independently of the function's own arithmetic:
a single token returns its value, identical keys average the values, a
dominant key selects its value, and permuting tokens changes nothing; a
textbook loop on a three-token case is kept as a cross-check.  With an fp16
window, the textbook formula over the prefix and the window tokens, the
window alone, and a dominant window key."""
import oracle
from tests import oracle_pins as P


def test_single_token_returns_its_value():
    P.check_attn_single_token_returns_its_value(oracle)


def test_identical_keys_average_values():
    P.check_attn_identical_keys_average_values(oracle)


def test_dominant_key_selects_its_value():
    P.check_attn_dominant_key_selects_its_value(oracle)


def test_token_permutation_invariance():
    P.check_attn_token_permutation_invariance(oracle)


def test_plain_softmax_attention_on_small_case():
    P.check_attn_plain_softmax_attention_on_small_case(oracle)


def test_cache_layout():
    P.check_attn_cache_layout(oracle)


def test_dequant_rows_match_rowwise_inverse():
    P.check_attn_dequant_rows_match_rowwise_inverse(oracle)


def test_row_list_matches_single_rows():
    P.check_row_list_matches_single_rows(oracle)


def test_window_schedule_closed_form():
    P.check_window_schedule_closed_form(oracle)


def test_window_joins_the_softmax():
    P.check_attn_window_joins_the_softmax(oracle)


def test_window_alone():
    P.check_attn_window_alone(oracle)


def test_dominant_window_key_selects_its_value():
    P.check_attn_dominant_window_key_selects_its_value(oracle)
