"""Plant plausible mistakes in a copy of the oracle (CPU only) and check that
at least one pin catches each of them.  The real oracle is never modified."""
import os
import types

import pytest

from tests import oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "rtq_oracle.py")


def mutated(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def all_pins(m):
    """Run every pin against module ``m``; return the names that failed."""
    checks = {
        "splitmix": lambda: P.check_splitmix64_published(m.splitmix64_stream),
        "signs": lambda: P.check_sign_vector_from_published(m.sign_vector),
        "row_seed": lambda: P.check_row_seed(m.row_seed),
        "srft_orth": lambda: P.check_orthonormal(m.srft_matrix),
        "srft_lib": lambda: P.check_srft_vs_library(m.srft_matrix),
        "srft_closed": lambda: P.check_srft_closed_forms(m.srft_matrix),
        "srht": lambda: P.check_srht(m.srht_matrix),
        "ruler": lambda: P.check_ruler(m.fp16_scale_from_absmax, m.quantize_with_scale),
        "outlier": lambda: P.check_outlier(m.fp16_scale_from_absmax, m.quantize_with_scale),
        "half_step": lambda: P.check_half_step_bound(m.fp16_scale_from_absmax, m.quantize_with_scale),
        "argmin": lambda: P.check_bruteforce_argmin(m.quantize_with_scale),
        "scale_round": lambda: P.check_scale_rounding(m.fp16_scale_from_absmax),
        "zero_group": lambda: P.check_zero_group(m.quantize_groups, m.dequantize_groups),
        "group_scales": lambda: P.check_group_scales(m.quantize_groups),
        "dequant_hand": lambda: P.check_dequantize_hand_evaluated(m.dequantize_groups),
        "dequant_inv_hand": lambda: P.check_dequant_inv_hand_evaluated(m),
        "quant_dequant_half_step": lambda: P.check_quantize_dequantize_half_step(m.quantize_groups,
                                                                                 m.dequantize_groups),
        "stored_scale": lambda: P.check_quantize_divides_by_stored_scale(m.quantize_groups),
        "ext_stored_scale": lambda: P.check_ext_divides_by_stored_scale(m),
        "mse_order": lambda: P.check_mse_ordering(m.int4_roundtrip_blocks),
        "nibbles": lambda: P.check_nibbles(m.pack_nibbles, m.unpack_nibbles),
        "impulse": lambda: P.check_impulse_end_to_end(m),
        "roundtrip": lambda: P.check_roundtrip_energy(m),
        "attn_single": lambda: P.check_attn_single_token_returns_its_value(m),
        "attn_same_keys": lambda: P.check_attn_identical_keys_average_values(m),
        "attn_dominant": lambda: P.check_attn_dominant_key_selects_its_value(m),
        "attn_perm": lambda: P.check_attn_token_permutation_invariance(m),
        "attn_textbook": lambda: P.check_attn_plain_softmax_attention_on_small_case(m),
        "attn_layout": lambda: P.check_attn_cache_layout(m),
        "attn_rows": lambda: P.check_attn_dequant_rows_match_rowwise_inverse(m),
        "row_list": lambda: P.check_row_list_matches_single_rows(m),
        "window": lambda: P.check_window_schedule_closed_form(m),
        "attn_window": lambda: P.check_attn_window_joins_the_softmax(m),
        "attn_window_alone": lambda: P.check_attn_window_alone(m),
        "attn_window_dominant": lambda: P.check_attn_dominant_window_key_selects_its_value(m),
        "ext_bits4": lambda: P.check_ext_bits4_without_lambda_is_the_int4_path(m),
        "ext_layout": lambda: P.check_pack_bits_layout_fixtures(m),
        "ext_roundtrip": lambda: P.check_pack_bits_exhaustive_round_trip(m),
        "ext_brute": lambda: P.check_ext_quantizer_brute_force(m),
        "ext_absmax": lambda: P.check_ext_absmax_maps_to_extreme_codes(m),
        "ext_lam_pow2": lambda: P.check_lambda_power_of_two_is_exact_input_scaling(m),
        "ext_lam_energy": lambda: P.check_lambda_energy_identity(m),
        "ext_order": lambda: P.check_error_falls_with_code_width(m),
    }
    failed = []
    for name, fn in checks.items():
        try:
            with __import__("numpy").errstate(all="ignore"):
                fn()
        except Exception:
            failed.append(name)
    return failed


MUTATIONS = {
    "srft drops sqrt2 on interior bins": (
        "R[2 * k - 1, :] = math.sqrt(2.0 / d) * np.cos(ang)",
        "R[2 * k - 1, :] = math.sqrt(1.0 / d) * np.cos(ang)"),
    "srft uses exp(+i...)": (
        "R[2 * k, :] = -math.sqrt(2.0 / d) * np.sin(ang)",
        "R[2 * k, :] = math.sqrt(2.0 / d) * np.sin(ang)"),
    "srft swaps Re/Im slots": (
        "R[2 * k - 1, :] = math.sqrt(2.0 / d) * np.cos(ang)\n        R[2 * k, :] = -math.sqrt(2.0 / d) * np.sin(ang)",
        "R[2 * k, :] = math.sqrt(2.0 / d) * np.cos(ang)\n        R[2 * k - 1, :] = -math.sqrt(2.0 / d) * np.sin(ang)"),
    "srft nyquist sign": (
        "R[d - 1, :] = np.where(n % 2 == 0, 1.0, -1.0) / math.sqrt(d)",
        "R[d - 1, :] = np.where(n % 2 == 0, -1.0, 1.0) / math.sqrt(d)"),
    "hadamard uses OR": (
        'H[i, k] = -1.0 if bin(i & k).count("1") % 2 else 1.0',
        'H[i, k] = -1.0 if bin(i | k).count("1") % 2 else 1.0'),
    "scale divides by 7": ("s = (a / 8.0).astype(np.float16)", "s = (a / 7.0).astype(np.float16)"),
    "scale rounds through fp32": (
        "s = (a / 8.0).astype(np.float16)", "s = (a / 8.0).astype(np.float32).astype(np.float16)"),
    "scale not saturated": (
        "(a / 8.0).astype(np.float16)\n    return np.where(np.isinf(s), np.float16(FP16_MAX), s).astype(np.float16)",
        "(a / 8.0).astype(np.float16)\n    return s.astype(np.float16)"),
    "b-bit scale not saturated": (
        "(a / float(1 << (bits - 1))).astype(np.float16)\n    return np.where(np.isinf(s), np.float16(FP16_MAX), s)"
        ".astype(np.float16)",
        "(a / float(1 << (bits - 1))).astype(np.float16)\n    return s.astype(np.float16)"),
    "clamp to [-7, 7]": ("INT4_MIN = -8", "INT4_MIN = -7"),
    "round half away from zero": (
        "return np.clip(np.rint(r), INT4_MIN, INT4_MAX).astype(np.int8)",
        "return np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), INT4_MIN, INT4_MAX).astype(np.int8)"),
    "truncate instead of round": (
        "return np.clip(np.rint(r), INT4_MIN, INT4_MAX).astype(np.int8)",
        "return np.clip(np.trunc(r), INT4_MIN, INT4_MAX).astype(np.int8)"),
    "zero scale divides by zero": (
        "r = np.where(s64 > 0, z / safe, 0.0)", "r = z / s64"),
    "absmax over the whole row": (
        "a = np.max(np.abs(zg), axis=-1)\n    s = fp16_scale_from_absmax(a)",
        "a = np.repeat(np.max(np.abs(zg), axis=(-1, -2))[..., None], zg.shape[-2], axis=-1)\n"
        "    s = fp16_scale_from_absmax(a)"),
    "b-bit absmax over the whole row": (
        "a = np.max(np.abs(zg), axis=-1)\n    s = fp16_scale_bits(a, bits)",
        "a = np.repeat(np.max(np.abs(zg), axis=(-1, -2))[..., None], zg.shape[-2], axis=-1)\n"
        "    s = fp16_scale_bits(a, bits)"),
    "nibbles swapped": ("return (lo | (hi << 4)).astype(np.uint8)", "return (hi | (lo << 4)).astype(np.uint8)"),
    "unpack without sign extension": ("lo = np.where(lo >= 8, lo - 16, lo)", "lo = lo"),
    "splitmix wrong multiplier": ("0xBF58476D1CE4E5B9", "0xBF58476D1CE4E5B8"),
    "sign from bit 0": ("[-1.0 if (o >> 63) & 1 else 1.0", "[-1.0 if o & 1 else 1.0"),
    "row seed without modulo": ("block %= seed_period", "block = block"),
    "inverse uses R instead of R^T": (
        "return D * (z @ rotation_matrix(rot, d))", "return D * (z @ rotation_matrix(rot, d).T)"),
    "inverse forgets the signs": (
        "return D * (z @ rotation_matrix(rot, d))", "return z @ rotation_matrix(rot, d)"),
    "attention reads values from the key rows": (
        "        for kv in (0, 1):\n            rows = cache_rows(layer, kv, st,",
        "        for kv in (0, 0):\n            rows = cache_rows(layer, kv, st,"),
    "attention rows use one seed for every row": (
        "    row_seeds = [row_seed(seed, int(r), rows_per_seed, seed_period) for r in rows]",
        "    row_seeds = [row_seed(seed, int(rows[0]), rows_per_seed, seed_period) for r in rows]"),
    "attention rows skip the sign flip": ("        u[idx] *= sign_vector(s, d)", "        u[idx] *= 1.0"),
    "row list ignored by the sign matrix": (
        "row0 + i if rows is None else int(rows[i])", "row0 + i"),
    "window flushed one token late": ("        if held == window:", "        if held == window + 1:"),
    "b-bit stream packed most significant bit first": (
        "            bit = (flat[:, i] >> k) & 1", "            bit = (flat[:, i] >> (bits - 1 - k)) & 1"),
    "b-bit scale divides by 2^b": (
        "        s = (a / float(1 << (bits - 1))).astype(np.float16)", "        s = (a / float(1 << bits)).astype(np.float16)"),
    "lambda applied after the rotation": (
        "    z = (D * x) @ rotation_matrix(rot, d).T\n    q, s, a = quantize_groups_bits(z, group, bits)",
        "    z = (D * np.asarray(x_f16, dtype=np.float16).astype(np.float64)) @ rotation_matrix(rot, d).T\n"
        "    z = z * (1.0 if lam_f16 is None else np.asarray(lam_f16, dtype=np.float16).astype(np.float64))\n"
        "    q, s, a = quantize_groups_bits(z, group, bits)"),
    "inverse multiplies by lambda": (
        "        u = u / np.asarray(lam_f16, dtype=np.float16).astype(np.float64)[None, :]",
        "        u = u * np.asarray(lam_f16, dtype=np.float16).astype(np.float64)[None, :]"),
    "b-bit clamp one code short": (
        "    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1\n    q = np.clip",
        "    lo, hi = -(1 << (bits - 1)) + 1, (1 << (bits - 1)) - 1\n    q = np.clip"),
    "attention window reads keys as values": (
        "                win = np.asarray(window[layer, kv, st, :window_tokens]",
        "                win = np.asarray(window[layer, 0, st, :window_tokens]"),
    "attention window drops its last token": (
        "                win = np.asarray(window[layer, kv, st, :window_tokens]",
        "                win = np.asarray(window[layer, kv, st, :window_tokens - 1]"),
    "attention window rounds through fp16 after the prefix": (
        "                part = np.concatenate([part, win])",
        "                part = np.concatenate([part.astype(np.float16).astype(np.float64), win])"),
    "attention drops the softmax scale": (
        "            sc = keys @ q[layer, st, g] * softmax_scale",
        "            sc = keys @ q[layer, st, g]"),
    "cache rows swap the kv and stream strides": (
        "    return layer * sl + kv * skv + stream * ss + st * np.arange(tokens, dtype=np.int64)",
        "    return layer * sl + kv * ss + stream * skv + st * np.arange(tokens, dtype=np.int64)"),
    "dequantize adds half a step": (
        "return (qg * s64[..., None]).reshape(q.shape)", "return ((qg + 0.5) * s64[..., None]).reshape(q.shape)"),
    "dequantize halves the scale": (
        "return (qg * s64[..., None]).reshape(q.shape)", "return (qg * (s64 / 2)[..., None]).reshape(q.shape)"),
    "dequantize uses the first group's scale for every group": (
        "return (qg * s64[..., None]).reshape(q.shape)", "return (qg * s64[..., :1, None]).reshape(q.shape)"),
    "quantizer divides by absmax/8 before its fp16 rounding": (
        "    q = quantize_with_scale(zg, s[..., None])",
        "    q = np.clip(np.rint(np.where(a[..., None] > 0, zg / np.where(a[..., None] > 0, a[..., None] / 8.0, 1.0),"
        " 0.0)), INT4_MIN, INT4_MAX).astype(np.int8)"),
    "b-bit quantizer divides by absmax/2^(b-1) before its fp16 rounding": (
        "    s64 = s.astype(np.float64)[..., None]", "    s64 = (a / float(1 << (bits - 1)))[..., None]"),
    "forward rotates before the sign flip": (
        "u = D * x\n    return u @ rotation_matrix(rot, d).T",
        "return D * (x @ rotation_matrix(rot, d).T)"),
}


# Mistakes in the dequantize step and in the choice of the divided scale must
# be caught by a pin written for that step, not only incidentally by a pin of
# some other part (such as the error ordering of the code widths).
DEDICATED = {
    "dequantize adds half a step": {"dequant_hand", "dequant_inv_hand", "quant_dequant_half_step"},
    "dequantize halves the scale": {"dequant_hand", "dequant_inv_hand", "quant_dequant_half_step"},
    "dequantize uses the first group's scale for every group": {"dequant_hand", "quant_dequant_half_step"},
    "quantizer divides by absmax/8 before its fp16 rounding": {"stored_scale"},
    "b-bit quantizer divides by absmax/2^(b-1) before its fp16 rounding": {"ext_stored_scale"},
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    failed = all_pins(mutated(old, new))
    assert failed, f"no pin catches the planted mistake: {name}"
    if name in DEDICATED:
        assert DEDICATED[name] <= set(failed), (name, sorted(failed))


def test_unmutated_copy_passes_every_pin():
    assert all_pins(mutated("INT4_MAX = 7", "INT4_MAX = 7")) == []
