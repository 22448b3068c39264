"""The oracle against what the pages and mathematics fix (CPU only)."""
import ast
import os

import numpy as np
import pytest

import oracle
from tests import oracle_pins as P


def test_splitmix64_published_vectors():
    P.check_splitmix64_published(oracle.splitmix64_stream)


def test_sign_vector_from_published_outputs():
    P.check_sign_vector_from_published(oracle.sign_vector)


def test_row_seed_rule():
    P.check_row_seed(oracle.row_seed)


def test_sign_matrix_uses_row_seed():
    m = oracle.sign_matrix(6, 16, 500, rows_per_seed=2, seed_period=2)
    for r in range(6):
        assert np.array_equal(m[r], oracle.sign_vector(500 + (r // 2) % 2, 16))


def test_sign_balance():
    # ~half of the signs are negative over many seeds (generator sanity)
    s = np.concatenate([oracle.sign_vector(k, 256) for k in range(40)])
    assert abs(np.mean(s)) < 0.05


def test_srft_orthonormal_bruteforce():
    P.check_orthonormal(oracle.srft_matrix)
    P.check_orthonormal(oracle.srft_matrix, ds=(64, 128, 256))


def test_srft_matches_numpy_rfft_ortho():
    P.check_srft_vs_library(oracle.srft_matrix)


def test_srft_closed_forms():
    P.check_srft_closed_forms(oracle.srft_matrix)


def test_srht_is_scaled_sylvester_hadamard():
    P.check_srht(oracle.srht_matrix)
    P.check_orthonormal(oracle.srht_matrix, ds=(2, 4, 8, 16, 64, 256))


def test_ruler_example():
    P.check_ruler(oracle.fp16_scale_from_absmax, oracle.quantize_with_scale)


def test_outlier_example():
    P.check_outlier(oracle.fp16_scale_from_absmax, oracle.quantize_with_scale)


def test_half_step_error_bound():
    P.check_half_step_bound(oracle.fp16_scale_from_absmax, oracle.quantize_with_scale)


def test_bruteforce_argmin_rounding():
    P.check_bruteforce_argmin(oracle.quantize_with_scale)


def test_scale_rounding_and_saturation():
    P.check_scale_rounding(oracle.fp16_scale_from_absmax)


def test_zero_group():
    P.check_zero_group(oracle.quantize_groups, oracle.dequantize_groups)


def test_mse_ordering_tensor_channel_group():
    P.check_mse_ordering(oracle.int4_roundtrip_blocks)


def test_nibble_layout_and_involution():
    P.check_nibbles(oracle.pack_nibbles, oracle.unpack_nibbles)


def test_impulse_end_to_end():
    P.check_impulse_end_to_end(oracle)


def test_roundtrip_energy_identity():
    P.check_roundtrip_energy(oracle)


def test_rotation_lowers_error_and_srft_close_to_srht():
    P.check_rotation_helps(oracle)


def test_shapes_and_dtypes():
    x = np.zeros((3, 128), dtype=np.float16)
    codes, scales = oracle.quant_fwd(x, 32, 1)
    assert codes.shape == (3, 64) and codes.dtype == np.uint8
    assert scales.shape == (3, 4) and scales.dtype == np.float16
    y = oracle.dequant_inv(codes, scales, 128, 32, 1)
    assert y.shape == (3, 128) and y.dtype == np.float16 and np.all(y == 0)
    codes, scales = oracle.quant_fwd(np.zeros((0, 64), dtype=np.float16), 64, 1)
    assert codes.shape == (0, 32) and scales.shape == (0, 1)


def test_oracle_is_independent_of_the_library():
    """The oracle imports only numpy/math and nothing from the product package."""
    src_dir = os.path.dirname(oracle.__file__)
    for name in os.listdir(src_dir):
        if not name.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(src_dir, name)).read())
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                mods = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                mods = [node.module or ""]
            else:
                continue
            for m in mods:
                assert m.split(".")[0] in {"numpy", "math", "__future__", "rtq_oracle", ""}, (name, m)


def test_group_scales():
    P.check_group_scales(oracle.quantize_groups)


def test_dequantize_hand_evaluated():
    P.check_dequantize_hand_evaluated(oracle.dequantize_groups)


def test_dequant_inv_hand_evaluated():
    P.check_dequant_inv_hand_evaluated(oracle)


def test_quantize_dequantize_half_step():
    P.check_quantize_dequantize_half_step(oracle.quantize_groups, oracle.dequantize_groups)


def test_quantize_divides_by_stored_fp16_scale():
    P.check_quantize_divides_by_stored_scale(oracle.quantize_groups)


def test_ext_quantize_divides_by_stored_fp16_scale():
    P.check_ext_divides_by_stored_scale(oracle)
