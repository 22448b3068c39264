"""Pins of the oracle's other code widths (3, 4, 6, 8 bits) and per-channel
lambda: the 4-bit special case, hand-packed bit streams, exhaustive
round trips, a brute-force quantizer, the absmax-to-extreme-code rule, exact
power-of-two lambda scaling, an energy identity for general lambda, and the
error falling with the code width."""
import oracle
from tests import oracle_pins as P


def test_bits4_without_lambda_is_the_int4_path():
    P.check_ext_bits4_without_lambda_is_the_int4_path(oracle)


def test_pack_bits_layout_fixtures():
    P.check_pack_bits_layout_fixtures(oracle)


def test_pack_bits_exhaustive_round_trip():
    P.check_pack_bits_exhaustive_round_trip(oracle)


def test_quantizer_brute_force():
    P.check_ext_quantizer_brute_force(oracle)


def test_absmax_maps_to_extreme_codes():
    P.check_ext_absmax_maps_to_extreme_codes(oracle)


def test_lambda_power_of_two_is_exact_input_scaling():
    P.check_lambda_power_of_two_is_exact_input_scaling(oracle)


def test_lambda_energy_identity():
    P.check_lambda_energy_identity(oracle)


def test_error_falls_with_code_width():
    P.check_error_falls_with_code_width(oracle)
