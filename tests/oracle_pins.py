"""Pin checks for the oracle, written against what the pages and mathematics fix.

Each ``check_*`` takes the implementation under test as an argument, so the
same check serves the real oracle (tests/test_oracle_pins.py) and deliberately
broken copies of it (tests/test_oracle_mutations.py).  A check raises
AssertionError when the implementation disagrees with the pin.
"""

from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_fixture(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line)
    return rows


def _kv_fixture(name):
    out = {}
    for line in _read_fixture(name):
        key, val = line.split(":", 1)
        out[key.strip()] = [float(v) for v in val.split()]
    return out


# --- sign generator -------------------------------------------------------


def check_splitmix64_published(splitmix64_stream):
    """Published SplitMix64 outputs (golden file)."""
    for line in _read_fixture("splitmix64_vectors.txt"):
        vals = [int(v) for v in line.split()]
        seed, expect = vals[0], vals[1:]
        got = splitmix64_stream(seed, len(expect))
        assert list(got) == expect, f"splitmix64({seed}) = {got} != {expect}"


def check_sign_vector_from_published(sign_vector):
    """Signs of seed 1234567 follow from the top bits of the published outputs.

    6457827717110365317 < 2^63 -> +1, 3203168211198807973 -> +1,
    9817491932198370423 >= 2^63 -> -1, 4593380528125082431 -> +1,
    16408922859458223821 -> -1.
    """
    got = sign_vector(1234567, 5)
    assert np.array_equal(got, [1.0, 1.0, -1.0, 1.0, -1.0]), got
    # seed 0: first output 16294208416658607535 >= 2^63 -> -1
    assert sign_vector(0, 1)[0] == -1.0


def check_row_seed(row_seed):
    """Hand-evaluated cases of seed + ((r // rows_per_seed) % seed_period)."""
    cases = [
        # seed, row, rps, period, expected
        (100, 0, 0, 0, 100),
        (100, 12345, 0, 0, 100),
        (100, 9, 10, 0, 100),
        (100, 10, 10, 0, 101),
        (100, 25, 10, 0, 102),
        (100, 25, 10, 2, 100),
        (100, 35, 10, 2, 101),
        (100, 40960 * 33 + 7, 40960, 32, 101),
        ((1 << 64) - 1, 10, 10, 0, 0),  # wraps modulo 2^64
    ]
    for seed, row, rps, per, exp in cases:
        got = row_seed(seed, row, rps, per)
        assert got == exp, (seed, row, rps, per, got, exp)


# --- rotations ------------------------------------------------------------


def check_orthonormal(matrix_fn, ds=(2, 4, 8, 16)):
    """R^T R = I and R R^T = I, element by element, and ||R x|| = ||x||."""
    rng = np.random.default_rng(7)
    for d in ds:
        R = matrix_fn(d)
        assert R.shape == (d, d)
        G = np.zeros((d, d))
        for i in range(d):  # brute force dot products
            for j in range(d):
                G[i, j] = sum(R[k, i] * R[k, j] for k in range(d))
        assert np.max(np.abs(G - np.eye(d))) < 1e-12, f"R^T R != I at d={d}"
        assert np.max(np.abs(R @ R.T - np.eye(d))) < 1e-12
        for _ in range(5):
            x = rng.standard_normal(d)
            assert abs(np.linalg.norm(R @ x) - np.linalg.norm(x)) < 1e-12 * max(1, np.linalg.norm(x))


def pack_rfft_reference(x):
    """numpy.fft.rfft(norm='ortho') packed as [X0, s*ReX1, s*ImX1, ..., X_{d/2}], s = sqrt 2.

    Written from view_as_real(rfft) with the two always-zero imaginary parts
    (of X0 and X_{d/2}) dropped; independent of the explicit DFT matrix.
    """
    d = x.shape[-1]
    X = np.fft.rfft(x, norm="ortho")
    z = np.empty(x.shape[:-1] + (d,))
    z[..., 0] = X[..., 0].real
    z[..., 1:d - 1:2] = math.sqrt(2) * X[..., 1:d // 2].real
    z[..., 2:d - 1:2] = math.sqrt(2) * X[..., 1:d // 2].imag
    z[..., d - 1] = X[..., d // 2].real
    return z


def check_srft_vs_library(srft_matrix, ds=(4, 8, 16, 64, 128, 256)):
    rng = np.random.default_rng(11)
    for d in ds:
        R = srft_matrix(d)
        x = rng.standard_normal((7, d))
        assert np.max(np.abs(x @ R.T - pack_rfft_reference(x))) < 1e-12, f"d={d}"


def check_srft_closed_forms(srft_matrix, ds=(8, 64, 256)):
    """Inputs whose packed orthonormal DFT is known in closed form."""
    for d in ds:
        R = srft_matrix(d)
        n = np.arange(d)
        # unit impulse at 0: every X_k = 1/sqrt d
        z = R @ np.eye(d)[0]
        exp = np.zeros(d)
        exp[0] = exp[d - 1] = 1 / math.sqrt(d)
        exp[1:d - 1:2] = math.sqrt(2 / d)
        assert np.allclose(z, exp, atol=1e-13), "impulse"
        # constant 1: X0 = sqrt d, everything else 0
        z = R @ np.ones(d)
        exp = np.zeros(d)
        exp[0] = math.sqrt(d)
        assert np.allclose(z, exp, atol=1e-12), "constant"
        # (-1)^n: only the Nyquist bin, X_{d/2} = sqrt d
        z = R @ np.where(n % 2 == 0, 1.0, -1.0)
        exp = np.zeros(d)
        exp[d - 1] = math.sqrt(d)
        assert np.allclose(z, exp, atol=1e-12), "nyquist"
        for m in (1, d // 4, d // 2 - 1):
            # cos(2 pi m n / d): X_m = sqrt(d)/2 -> z_{2m-1} = sqrt(d/2)
            z = R @ np.cos(2 * math.pi * m * n / d)
            exp = np.zeros(d)
            exp[2 * m - 1] = math.sqrt(d / 2)
            assert np.allclose(z, exp, atol=1e-12), f"cos m={m}"
            # sin(2 pi m n / d): X_m = -i sqrt(d)/2 -> z_{2m} = -sqrt(d/2)
            z = R @ np.sin(2 * math.pi * m * n / d)
            exp = np.zeros(d)
            exp[2 * m] = -math.sqrt(d / 2)
            assert np.allclose(z, exp, atol=1e-12), f"sin m={m}"


def check_srht(srht_matrix, ds=(1, 2, 4, 8, 16, 64, 128, 256)):
    import scipy.linalg
    for d in ds:
        H = srht_matrix(d) * math.sqrt(d)
        assert np.array_equal(np.rint(H), H)
        assert np.array_equal(H, scipy.linalg.hadamard(d).astype(np.float64)), f"d={d}"
        assert np.array_equal(H @ H.T, d * np.eye(d))


# --- quantizer ------------------------------------------------------------


def check_ruler(fp16_scale_from_absmax, quantize_with_scale):
    fx = _kv_fixture("ruler_example.txt")
    vals = np.array(fx["values"])
    s = fp16_scale_from_absmax(np.max(np.abs(vals)))
    assert float(s) == fx["scale"][0], s
    q = quantize_with_scale(vals, s)
    # interior values land exactly on cells; -8 is a code, +8 is clipped to 7
    assert np.array_equal(q, np.clip(vals, -8, 7)), q


def check_outlier(fp16_scale_from_absmax, quantize_with_scale):
    fx = _kv_fixture("outlier_example.txt")
    vals = np.array(fx["values"])
    s = fp16_scale_from_absmax(np.max(np.abs(vals)))
    assert float(s) == fx["scale"][0], s
    q_small = quantize_with_scale(np.array(fx["small"]), s)
    assert len(set(q_small.tolist())) == 1, q_small  # one shared cell
    assert q_small[0] == 0


def check_half_step_bound(fp16_scale_from_absmax, quantize_with_scale):
    """|z - s q| <= s/2 before clipping ([P4]); <= s when the absmax element clips."""
    rng = np.random.default_rng(3)
    for trial in range(200):
        z = rng.standard_normal(32) * rng.choice([1e-3, 1.0, 30.0])
        if trial % 3 == 0:
            z[rng.integers(32)] *= 20.0
        s = fp16_scale_from_absmax(np.max(np.abs(z)))
        q = quantize_with_scale(z, s)
        s64 = float(s)
        r = z / s64
        err = np.abs(z - s64 * q)
        inside = (r <= 7.5) & (r >= -8.5)
        assert np.all(err[inside] <= s64 / 2 * (1 + 1e-12))
        # fp16 rounding of s moves absmax/s at most 2^-11 relative away from 8
        assert np.all(err <= s64 * (1 + 8 * 2.0 ** -11) + 1e-300)


def check_bruteforce_argmin(quantize_with_scale):
    """q = argmin_{c in [-8,7]} |z - s c|, ties to the even code."""
    rng = np.random.default_rng(5)
    s = np.float16(0.375)
    s64 = float(s)
    zs = list(rng.uniform(-10, 10, size=2000) * s64)
    zs += [(k + 0.5) * s64 for k in range(-10, 10)]  # exact ties
    zs += [-8.5 * s64, 7.5 * s64, 0.0, -0.0]
    for z in zs:
        cands = np.arange(-8, 8)
        err = np.abs(z - s64 * cands)
        best = cands[err == err.min()]
        want = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
        got = int(quantize_with_scale(np.array([z]), s)[0])
        assert got == want, (z / s64, got, want)


def check_scale_rounding(fp16_scale_from_absmax):
    """fp16 round-to-nearest-even of absmax/8, saturating at 65504."""
    cases = [
        (8.0, 1.0),
        (8 * (1 + 2.0 ** -11), 1.0),  # tie -> even mantissa
        (8 * (1 + 3 * 2.0 ** -11), 1 + 2.0 ** -9),  # tie -> even mantissa
        (8 * (1 + 2.0 ** -11 + 2.0 ** -30), 1 + 2.0 ** -10),  # just above tie
        (20.0, 2.5),
        (0.0, 0.0),
        (8 * 2.0 ** -24, 2.0 ** -24),  # smallest subnormal
        (8 * 2.0 ** -25, 0.0),  # tie between 0 and 2^-24 -> 0
        (8 * 70000.0, 65504.0),  # saturate
        (8 * 65504.0, 65504.0),
    ]
    for a, want in cases:
        got = float(fp16_scale_from_absmax(np.array(a)))
        assert got == want, (a, got, want)


def check_zero_group(quantize_groups, dequantize_groups):
    z = np.zeros((3, 64))
    z[1, 32:] = 1.0
    # nonzero values whose absmax/8 is below half the smallest fp16 subnormal:
    # the scale rounds to 0 and every code of the group must be 0
    z[2, :32] = np.linspace(-1e-9, 1e-9, 32)
    q, s, _ = quantize_groups(z, 32)
    assert float(s[0, 0]) == 0 and float(s[0, 1]) == 0 and float(s[1, 0]) == 0
    assert float(s[2, 0]) == 0
    assert np.all(q[0] == 0) and np.all(q[1, :32] == 0) and np.all(q[2, :32] == 0)
    assert np.all(dequantize_groups(q, s, 32)[0] == 0)


def check_mse_ordering(int4_roundtrip_blocks):
    """Per-tensor >= per-channel >= per-group 4-bit MSE on a matrix with small
    and large regions ([P4]: the tests it describes)."""
    rng = np.random.default_rng(9)
    w = rng.standard_normal((64, 256))
    w[5:9, :] *= 20.0       # large rows
    w[:, 100:104] *= 20.0   # large columns (hurt per-row, not per-group)
    def mse(br, bc):
        return float(np.mean((int4_roundtrip_blocks(w, br, bc) - w) ** 2))
    t, c, g = mse(64, 256), mse(1, 256), mse(1, 32)
    assert t > c > g, (t, c, g)


# --- packing --------------------------------------------------------------


def check_nibbles(pack_nibbles, unpack_nibbles):
    allb = np.arange(256, dtype=np.uint8)[None, :]
    assert np.array_equal(pack_nibbles(unpack_nibbles(allb)), allb)
    for line in _read_fixture("nibble_layout.txt"):
        w0, w1, b = line.split()
        got = int(pack_nibbles(np.array([[int(w0), int(w1)]]))[0, 0])
        assert got == int(b, 16), (w0, w1, hex(got), b)
        un = unpack_nibbles(np.array([[int(b, 16)]], dtype=np.uint8))[0]
        assert un.tolist() == [int(w0), int(w1)]


# --- whole pipeline -------------------------------------------------------


def check_impulse_end_to_end(oracle):
    """x = c * e_0 gives z = c * D_0 * R[:, 0], known in closed form."""
    for d, g in ((64, 32), (128, 32), (256, 32), (64, 64)):
        c = 3.0
        x = np.zeros((1, d), dtype=np.float16)
        x[0, 0] = c
        seed = 4242
        d0 = oracle.sign_vector(seed, d)[0]
        codes, scales = oracle.quant_fwd(x, g, seed)
        # every group holds a sqrt(2/d) * c entry, the largest magnitude
        big = math.sqrt(2.0 / d) * c
        s_exp = np.float16(big / 8)
        assert np.all(scales == s_exp), (scales, s_exp)
        q = oracle.unpack_nibbles(codes)[0]
        s64 = float(s_exp)
        z = np.zeros(d)
        z[0] = z[d - 1] = d0 * c / math.sqrt(d)
        z[1:d - 1:2] = d0 * big
        q_exp = np.clip(np.rint(z / s64), -8, 7)
        assert np.array_equal(q, q_exp), (q[:8], q_exp[:8])


def check_roundtrip_energy(oracle):
    """||y_fp64 - x|| = ||z_hat - z|| (R and D are orthogonal)."""
    rng = np.random.default_rng(13)
    for rot in ("srft", "srht"):
        for d, g in ((64, 32), (128, 32), (256, 32)):
            x = (rng.standard_normal((9, d)) * 2).astype(np.float16)
            det = oracle.forward_detail(x, g, 77, rot=rot)
            codes, scales = det["codes"], det["s"]
            _, u = oracle.dequant_inv(codes, scales, d, g, 77, rot=rot, return_fp64=True)
            zhat = oracle.dequantize_groups(det["q"], det["s"], g)
            lhs = np.linalg.norm(u - x.astype(np.float64), axis=1)
            rhs = np.linalg.norm(zhat - det["z"], axis=1)
            assert np.allclose(lhs, rhs, rtol=1e-9, atol=1e-12), (rot, d)


def check_rotation_helps(oracle):
    """Rotating before quantizing lowers int4 error on outlier data ([P1,
    "Before you celebrate, check the quality bill"]); SRFT and SRHT land
    close to each other ([P1, "First, the 17%"])."""
    rng = np.random.default_rng(21)
    d, g = 64, 32
    x = rng.standard_normal((2000, d))
    x[:, [3, 17]] *= 20.0
    x = x.astype(np.float16)
    x64 = x.astype(np.float64)
    err = {}
    for rot in ("none", "srft", "srht"):
        det = oracle.forward_detail(x, g, 5, rot=rot)
        _, u = oracle.dequant_inv(det["codes"], det["s"], d, g, 5, rot=rot, return_fp64=True)
        err[rot] = float(np.mean((u - x64) ** 2))
    assert err["srft"] < 0.5 * err["none"], err
    assert err["srht"] < 0.5 * err["none"], err
    # the pages compare the two on perplexity, not MSE; on this impulse-like
    # outlier data the flat Hadamard image of a spike is slightly better, so
    # the check only asks that neither is far from the other
    assert 1 / 1.5 < err["srft"] / err["srht"] < 1.5, err


def check_group_scales(quantize_groups):
    """Each group gets its own absmax/8 (hand-evaluated)."""
    z = np.zeros((1, 128))
    z[0, 5] = -8.0      # group 0 absmax 8   -> scale 1
    z[0, 40] = 16.0     # group 1 absmax 16  -> scale 2
    z[0, 70] = 0.5      # group 2 absmax 0.5 -> scale 1/16
    z[0, 127] = -20.0   # group 3 absmax 20  -> scale 2.5
    z[0, 100] = 2.5     # group 3: 2.5 / 2.5 = 1
    q, s, _ = quantize_groups(z, 32)
    assert s.astype(np.float64).tolist() == [[1.0, 2.0, 0.0625, 2.5]], s
    assert q[0, 5] == -8 and q[0, 40] == 7 and q[0, 70] == 7 and q[0, 127] == -8
    assert q[0, 100] == 1
    q, s, _ = quantize_groups(z, 64)
    assert s.astype(np.float64).tolist() == [[2.0, 2.5]], s
    assert q[0, 5] == -4 and q[0, 100] == 1


# fp16(0.1) and fp16(1/3), evaluated by hand: 0.1 = 1.6 * 2^-4 and the 10-bit
# mantissa 0.6 * 1024 = 614.4 rounds to 614, so fp16(0.1) = 1638/16384 =
# 819/8192; 1/3 = 1.333... * 2^-2 and 0.333... * 1024 = 341.33 rounds to 341,
# so fp16(1/3) = 1365/4096.  Neither equals the real number it stands for.
FP16_TENTH = 819 / 8192          # 0.0999755859375
FP16_THIRD = 1365 / 4096         # 0.333251953125


def check_dequantize_hand_evaluated(dequantize_groups):
    """x_hat = s * q with zero point 0, per group, with s the stored fp16 scale.

    The decode rule: [P4] "Quantization & Serving" (opening: the dequantized
    value of symmetric absmax quantization is s times the code) and [P3] "What
    Quantization Is, Mathematically" (decode multiplies the cell index by the
    scale; zero_point = 0 in the symmetric case).  Scales are fp16 values
    ([P3] "How Many Numbers Should One Scale Cover").  Every product below is
    evaluated by hand; two of the scales are not the real numbers 0.1 and 1/3
    but their fp16 roundings, and 65504 is the largest fp16 value.
    """
    cases = [
        # (codes, fp16 scales, group, expected x_hat)
        ([[-8, 7, 3, -1]], [[2.5, 0.375]], 2, [[-20.0, 17.5, 1.125, -0.375]]),
        # 3 * 819/8192 = 2457/8192; -8 * 819/8192 = -819/1024; scale 0 decodes to 0
        ([[3, -8, 0, 5]], [[FP16_TENTH, 0.0]], 2, [[2457 / 8192, -819 / 1024, 0.0, 0.0]]),
        # 7 * 1365/4096 = 9555/4096; -8 * 1365/4096 = -10920/4096; 65504 * (-8, 7, 0, 1)
        ([[7, -8, 1, -1, -8, 7, 0, 1]], [[FP16_THIRD, 65504.0]], 4,
         [[9555 / 4096, -10920 / 4096, 1365 / 4096, -1365 / 4096, -524032.0, 458528.0, 0.0, 65504.0]]),
        # two rows, one group per row
        ([[1, 2], [-3, 4]], [[0.5], [0.25]], 2, [[0.5, 1.0], [-0.75, 1.0]]),
    ]
    for q, s, g, want in cases:
        s16 = np.array(s, dtype=np.float16)
        assert np.array_equal(s16.astype(np.float64), np.array(s)), "fixture scales must be fp16 values"
        got = dequantize_groups(np.array(q, dtype=np.int8), s16, g)
        assert np.array_equal(np.asarray(got, dtype=np.float64), np.array(want)), (q, s, got, want)


def check_dequant_inv_hand_evaluated(oracle):
    """The whole inverse step on a hand-evaluated row with no rotation (R = I):
    unpack [P5] nibbles, dequantize (s * q), flip signs, round to fp16.

    Bytes 0x78 = (7 << 4) | 8 and 0xF3 = (15 << 4) | 3 hold the codes
    -8, 7, 3, -1 (low nibble first, two's complement).  The signs of seed
    1234567 are +1, +1, -1, +1 (from the top bits of its first published
    SplitMix64 outputs, checked in check_sign_vector_from_published).  With
    scales 2.5 and 0.375 over groups of 2: y = (-20, 17.5, -1.125, -0.375).
    """
    codes = np.array([[0x78, 0xF3]], dtype=np.uint8)
    scales = np.array([[2.5, 0.375]], dtype=np.float16)
    y = oracle.dequant_inv(codes, scales, 4, 2, 1234567, rot="none")
    assert y.dtype == np.float16
    assert y.astype(np.float64).tolist() == [[-20.0, 17.5, -1.125, -0.375]], y


def check_quantize_dequantize_half_step(quantize_groups, dequantize_groups):
    """Through both steps of the oracle: z_hat = dequantize(quantize(z)) lies on
    the grid s * {-8 .. 7} of its group's stored scale, and |z_hat - z| <= s/2
    for every value that is not clipped ([P4] "Quantization & Serving": the
    rounding error of absmax quantization is at most s/2 before clipping);
    a clipped value (only +absmax can clip, at 7.5 < a/s <= 8) errs by at most
    s (1 + 8 * 2^-11) (fp16 rounding of s moves a/s by at most 2^-11 relative)."""
    rng = np.random.default_rng(31)
    for trial in range(60):
        g = (32, 64, 128)[trial % 3]
        z = rng.standard_normal((5, 256)) * rng.choice([1e-3, 1.0, 40.0])
        z[:, rng.integers(256, size=3)] *= 25.0
        q, s, _ = quantize_groups(z, g)
        zhat = np.asarray(dequantize_groups(q, s, g), dtype=np.float64)
        s_el = np.repeat(s.astype(np.float64), g, axis=-1)
        k = zhat / s_el
        assert np.array_equal(k, np.rint(k)) and k.min() >= -8 and k.max() <= 7, "off the code grid"
        err = np.abs(zhat - z)
        r = z / s_el
        inside = (r <= 7.5) & (r >= -8.5)
        assert np.all(err[inside] <= s_el[inside] / 2 * (1 + 1e-12)), "more than half a step"
        assert np.all(err <= s_el * (1 + 8 * 2.0 ** -11)), "clipped error above one step"


def check_quantize_divides_by_stored_scale(quantize_groups):
    """Codes divide by the stored fp16 scale, not by absmax/8 before rounding.

    [P3] "How Many Numbers Should One Scale Cover": scales are fp16 values that
    are stored and moved, and the decode of [P3] "What Quantization Is,
    Mathematically" multiplies by that stored value; dividing by the same
    value keeps the round trip within half a step of it.

    Hand-evaluated group (absmax 0.8, so absmax/8 = 0.1, stored as
    fp16(0.1) = 819/8192):
      0.8     / (819/8192) = 8.00195...  -> 8, clamped to 7
      0.24995 / (819/8192) = 2.50011...  -> 3   (0.24995 / 0.1 = 2.4995 -> 2)
     -0.34995 / (819/8192) = -3.50035... -> -4  (-0.34995 / 0.1 = -3.4995 -> -3)
      0.0502  / (819/8192) = 0.5021...   -> 1
    """
    z = np.zeros((1, 32))
    z[0, :4] = [0.8, 0.24995, -0.34995, 0.0502]
    q, s, _ = quantize_groups(z, 32)
    assert float(s[0, 0]) == FP16_TENTH, s
    assert q[0, :4].tolist() == [7, 3, -4, 1], q[0, :4]
    assert np.all(q[0, 4:] == 0)


def check_ext_divides_by_stored_scale(m):
    """The same rule for b-bit codes: absmax 0.1 * 2^(b-1) gives the stored
    scale fp16(0.1) = 819/8192 for every width, and 0.24995 and -0.34995 take
    the codes 3 and -4 (dividing by 0.1 would give 2 and -3)."""
    for bits in m.CODE_BITS:
        z = np.zeros((1, 32))
        z[0, :3] = [0.1 * (1 << (bits - 1)), 0.24995, -0.34995]
        q, s, _ = m.quantize_groups_bits(z, 32, bits)
        assert float(s[0, 0]) == FP16_TENTH, (bits, s)
        assert q[0, 1] == 3 and q[0, 2] == -4, (bits, q[0, :3])


# ---------------------------------------------------------------------------
# Attention over the compressed cache
# ---------------------------------------------------------------------------


def _lm(streams, tcap):
    """Strides of the layer-major cache [layer][K, V][stream][token]."""
    return (2 * streams * tcap, streams * tcap, tcap, 1)


def _tm(layers, streams):
    """Strides of the time-major cache [token][layer][K, V][stream]."""
    return (2 * streams, streams, 1, 2 * layers * streams)


def _attn_cache(m, rng, layers, streams, tcap, d, group, seed, rps, per, rot, scale=1.0):
    n = layers * 2 * streams * tcap
    x = (rng.standard_normal((n, d)) * scale).astype(np.float16)
    codes, scales = m.quant_fwd(x, group, seed, rps, per, rot)
    return codes, scales


def _attn_values(m, codes, scales, rows, d, group, seed, rps, per, rot):
    """Rows dequantized one at a time through dequant_inv (row0 = the row)."""
    return np.stack([m.dequant_inv(codes[r:r + 1], scales[r:r + 1], d, group, seed, rps, per, rot, row0=int(r),
                                   return_fp64=True)[1][0] for r in rows])


def check_attn_dequant_rows_match_rowwise_inverse(m):
    """dequant_rows on scattered rows of different seeds equals dequant_inv
    applied to each row on its own (before the fp16 rounding)."""
    rng = np.random.default_rng(6)
    n, d, g = 40, 64, 32
    x = rng.standard_normal((n, d)).astype(np.float16)
    codes, scales = m.quant_fwd(x, g, 21, 4, 3, "srft")
    rows = np.array([37, 0, 5, 12, 13, 22, 9, 30])
    got = m.dequant_rows(codes, scales, rows, d, g, 21, 4, 3, "srft")
    want = _attn_values(m, codes, scales, rows, d, g, 21, 4, 3, "srft")
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def check_attn_single_token_returns_its_value(m):
    """With one cached token the softmax weight is 1: o is that token's value
    row, whatever the query (both layouts, per-layer seeds)."""
    rng = np.random.default_rng(1)
    L, S, Tc, d, g = 2, 3, 4, 64, 32
    for strides, rps in ((_lm(S, Tc), 2 * S * Tc), (_tm(L, S), 2 * S)):
        codes, scales = _attn_cache(m, rng, L, S, Tc, d, g, 77, rps, L, "srft")
        q = rng.standard_normal((L, S, 2, d)).astype(np.float16)
        o = m.attn_decode(q, codes, scales, strides, L, S, 1, 2, d, g, 77, rps, L, "srft")
        for l in range(L):
            for s in range(S):
                row = l * strides[0] + strides[1] + s * strides[2]
                v = _attn_values(m, codes, scales, [row], d, g, 77, rps, L, "srft")[0]
                assert np.allclose(o[l, s, 0], v, rtol=0, atol=1e-12)
                assert np.allclose(o[l, s, 1], v, rtol=0, atol=1e-12)


def check_attn_identical_keys_average_values(m):
    rng = np.random.default_rng(2)
    L, S, Tc, T, d, g = 1, 2, 8, 5, 128, 64
    st = _lm(S, Tc)
    codes, scales = _attn_cache(m, rng, L, S, Tc, d, g, 5, 0, 0, "srht")
    for s in range(S):
        rows = [s * Tc + t for t in range(T)]
        codes[rows] = codes[rows[0]]
        scales[rows] = scales[rows[0]]
    q = rng.standard_normal((L, S, 1, d)).astype(np.float16)
    o = m.attn_decode(q, codes, scales, st, L, S, T, 1, d, g, 5, 0, 0, "srht")
    for s in range(S):
        v = _attn_values(m, codes, scales, [S * Tc + s * Tc + t for t in range(T)], d, g, 5, 0, 0, "srht")
        assert np.allclose(o[0, s, 0], v.mean(axis=0), rtol=0, atol=1e-12)


def check_attn_dominant_key_selects_its_value(m):
    rng = np.random.default_rng(3)
    L, S, Tc, T, d, g = 1, 1, 6, 6, 64, 64
    codes, scales = _attn_cache(m, rng, L, S, Tc, d, g, 9, 0, 0, "srft", scale=0.01)
    keys = _attn_values(m, codes, scales, range(T), d, g, 9, 0, 0, "srft")
    # a query parallel to key 3, scaled so its score dominates by a wide margin
    q = (keys[3] / np.linalg.norm(keys[3]) * 4e4).astype(np.float16).reshape(1, 1, 1, d)
    o = m.attn_decode(q, codes, scales, _lm(S, Tc), L, S, T, 1, d, g, 9, 0, 0, "srft", softmax_scale=1.0)
    v = _attn_values(m, codes, scales, range(Tc, Tc + T), d, g, 9, 0, 0, "srft")
    assert np.allclose(o[0, 0, 0], v[3], rtol=0, atol=1e-9)


def check_attn_token_permutation_invariance(m):
    rng = np.random.default_rng(4)
    L, S, Tc, T, d, g = 1, 1, 7, 7, 64, 32
    codes, scales = _attn_cache(m, rng, L, S, Tc, d, g, 11, 0, 0, "srft")
    q = rng.standard_normal((1, 1, 3, d)).astype(np.float16)
    o1 = m.attn_decode(q, codes, scales, _lm(S, Tc), L, S, T, 3, d, g, 11, 0, 0, "srft")
    perm = rng.permutation(T)
    c2, s2 = codes.copy(), scales.copy()
    for base in (0, Tc):
        rows = np.arange(base, base + T)
        c2[rows] = codes[rows[perm]]
        s2[rows] = scales[rows[perm]]
    o2 = m.attn_decode(q, c2, s2, _lm(S, Tc), L, S, T, 3, d, g, 11, 0, 0, "srft")
    assert np.allclose(o1, o2, rtol=0, atol=1e-12)


def check_attn_plain_softmax_attention_on_small_case(m):
    """Against the textbook formula on explicit per-token values."""
    rng = np.random.default_rng(5)
    L, S, Tc, T, d, g = 1, 1, 3, 3, 64, 64
    codes, scales = _attn_cache(m, rng, L, S, Tc, d, g, 13, 0, 0, "srft")
    k = _attn_values(m, codes, scales, range(T), d, g, 13, 0, 0, "srft")
    v = _attn_values(m, codes, scales, range(Tc, Tc + T), d, g, 13, 0, 0, "srft")
    q16 = rng.standard_normal(d).astype(np.float16)
    qf = q16.astype(np.float64)
    e = [math.exp(float(np.dot(qf, k[t])) / 8.0) for t in range(T)]
    want = sum(e[t] * v[t] for t in range(T)) / sum(e)
    o = m.attn_decode(q16.reshape(1, 1, 1, d), codes, scales, _lm(S, Tc), L, S, T, 1, d, g, 13)
    assert np.allclose(o[0, 0, 0], want, rtol=1e-12, atol=1e-12)


def check_attn_cache_layout(m):
    """Enumerating (layer, kv, stream, token) through cache_rows visits every
    row once, in the order [layer][kv][stream][token] for the layer-major
    strides and [token][layer][kv][stream] for the time-major ones."""
    L, S, T = 2, 3, 4
    lm = [int(r) for l in range(L) for kv in (0, 1) for s in range(S) for r in m.cache_rows(l, kv, s, T, _lm(S, T))]
    assert lm == list(range(L * 2 * S * T))
    tm = {}
    for l in range(L):
        for kv in (0, 1):
            for s in range(S):
                for t, r in enumerate(m.cache_rows(l, kv, s, T, _tm(L, S))):
                    tm[(t, l, kv, s)] = int(r)
    assert [tm[k] for k in sorted(tm)] == list(range(L * 2 * S * T))



def _textbook_attention(q, keys, values, scale):
    """softmax(scale * keys q) values, written out term by term."""
    e = [math.exp(scale * float(np.dot(q, k))) for k in keys]
    return sum(w * v for w, v in zip(e, values)) / sum(e)


def check_attn_window_joins_the_softmax(m):
    """With an fp16 window, one softmax runs over the dequantized prefix and
    the window tokens: the textbook formula over both token lists (prefix
    rows through dequant_inv one at a time, window rows as given)."""
    rng = np.random.default_rng(8)
    L, S, Tc, T, W, Wc, G, d, g = 2, 2, 5, 4, 3, 4, 2, 64, 32
    codes, scales = _attn_cache(m, rng, L, S, Tc, d, g, 31, 2 * S * Tc, L, "srft")
    win = (rng.standard_normal((L, 2, S, Wc, d)) * 0.7).astype(np.float16)
    q = rng.standard_normal((L, S, G, d)).astype(np.float16)
    o = m.attn_decode(q, codes, scales, _lm(S, Tc), L, S, T, G, d, g, 31, 2 * S * Tc, L, "srft",
                      window=win, window_tokens=W)
    for l in range(L):
        for s in range(S):
            base = l * 2 * S * Tc + s * Tc
            k = _attn_values(m, codes, scales, range(base, base + T), d, g, 31, 2 * S * Tc, L, "srft")
            v = _attn_values(m, codes, scales, range(base + S * Tc, base + S * Tc + T), d, g, 31, 2 * S * Tc, L,
                             "srft")
            keys = list(k) + list(win[l, 0, s, :W].astype(np.float64))
            values = list(v) + list(win[l, 1, s, :W].astype(np.float64))
            for gi in range(G):
                want = _textbook_attention(q[l, s, gi].astype(np.float64), keys, values, 1.0 / 8.0)
                assert np.allclose(o[l, s, gi], want, rtol=1e-12, atol=1e-12)


def check_attn_window_alone(m):
    """With no quantized tokens the window is the whole context: the textbook
    formula on the window rows; rows past window_tokens are ignored."""
    rng = np.random.default_rng(9)
    L, S, Tc, W, Wc, d, g = 1, 2, 3, 5, 8, 128, 64
    codes, scales = _attn_cache(m, rng, L, S, Tc, d, g, 3, 0, 0, "srht")
    win = rng.standard_normal((L, 2, S, Wc, d)).astype(np.float16)
    win[:, :, :, W:] = np.float16(1e4)  # unused slots must not matter
    q = rng.standard_normal((L, S, 1, d)).astype(np.float16)
    o = m.attn_decode(q, codes, scales, _lm(S, Tc), L, S, 0, 1, d, g, 3, 0, 0, "srht", window=win, window_tokens=W)
    for s in range(S):
        want = _textbook_attention(q[0, s, 0].astype(np.float64), win[0, 0, s, :W].astype(np.float64),
                                   win[0, 1, s, :W].astype(np.float64), 1.0 / math.sqrt(d))
        assert np.allclose(o[0, s, 0], want, rtol=1e-12, atol=1e-12)


def check_attn_dominant_window_key_selects_its_value(m):
    """A query parallel to one window key, scaled far up, returns that window
    token's value."""
    rng = np.random.default_rng(10)
    L, S, Tc, T, Wc, d, g = 1, 1, 4, 4, 4, 64, 64
    codes, scales = _attn_cache(m, rng, L, S, Tc, d, g, 5, 0, 0, "srft", scale=0.01)
    win = (rng.standard_normal((L, 2, S, Wc, d)) * 0.01).astype(np.float16)
    key = win[0, 0, 0, 2].astype(np.float64)
    q = (key / np.linalg.norm(key) * 4e4).astype(np.float16).reshape(1, 1, 1, d)
    o = m.attn_decode(q, codes, scales, _lm(S, Tc), L, S, T, 1, d, g, 5, 0, 0, "srft", softmax_scale=1.0,
                      window=win, window_tokens=3)
    assert np.allclose(o[0, 0, 0], win[0, 1, 0, 2].astype(np.float64), rtol=0, atol=1e-9)


# ---------------------------------------------------------------------------
# Row lists and the decode-cache window
# ---------------------------------------------------------------------------


def check_row_list_matches_single_rows(m):
    """quant_fwd / dequant_inv with an explicit row list give, row by row,
    what a one-row call at that row index gives (the seed follows the row)."""
    rng = np.random.default_rng(7)
    d, g = 64, 32
    rows = np.array([5, 40, 41, 7, 130, 2])
    x = rng.standard_normal((len(rows), d)).astype(np.float16)
    codes, scales = m.quant_fwd(x, g, 99, 8, 5, "srft", rows=rows)
    y = m.dequant_inv(codes, scales, d, g, 99, 8, 5, "srft", rows=rows)
    for i, r in enumerate(rows):
        c1, s1 = m.quant_fwd(x[i:i + 1], g, 99, 8, 5, "srft", row0=int(r))
        assert np.array_equal(codes[i:i + 1], c1) and np.array_equal(scales[i:i + 1], s1)
        y1 = m.dequant_inv(c1, s1, d, g, 99, 8, 5, "srft", row0=int(r))
        assert np.array_equal(y[i:i + 1], y1)


def check_window_schedule_closed_form(m):
    """After a prefill of T0 tokens and k appends with a window of W tokens,
    T0 + W*floor(k/W) tokens are quantized and k mod W stay in fp16."""
    for t0, w in ((0, 16), (20, 16), (5, 4), (3, 1)):
        for k in range(0, 3 * w + 3):
            assert m.window_schedule(t0, k, w) == (t0 + w * (k // w), k % w), (t0, k, w)



# ---------------------------------------------------------------------------
# Other code widths and the per-channel lambda
# ---------------------------------------------------------------------------


def check_ext_bits4_without_lambda_is_the_int4_path(m):
    """b = 4 with no lambda gives exactly the int4 forward and inverse."""
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((12, 128)) * 3).astype(np.float16)
    for rot in ("srft", "srht"):
        c1, s1 = m.quant_fwd_ext(x, 32, 4, None, 5, 4, 3, rot)
        c2, s2 = m.quant_fwd(x, 32, 5, 4, 3, rot)
        assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
        assert np.array_equal(m.dequant_inv_ext(c1, s1, 128, 32, 4, None, 5, 4, 3, rot),
                              m.dequant_inv(c2, s2, 128, 32, 5, 4, 3, rot))


def check_pack_bits_layout_fixtures(m):
    """Hand-packed streams: code i in stream bits [i*b, (i+1)*b), least
    significant bit first, stream bit k = bit k%8 of byte k//8."""
    cases = [
        (3, [1, -1, 2, -4, 3, 0, -2, 1], [185, 56, 56]),
        (6, [5, -32, 31, -1], [5, 248, 253]),
        (8, [-128, 127, -1, 0], [128, 127, 255, 0]),
        (4, [3, -2], [0xE3]),
    ]
    for bits, codes, want in cases:
        got = m.pack_bits(np.array([codes]), bits)[0]
        assert got.tolist() == want, (bits, got.tolist(), want)
        assert m.unpack_bits(got[None], bits, len(codes))[0].tolist() == codes


def check_pack_bits_exhaustive_round_trip(m):
    for bits in m.CODE_BITS:
        vals = np.arange(-(1 << (bits - 1)), 1 << (bits - 1))
        d = ((len(vals) + 7) // 8) * 8 * 2
        row = np.resize(vals, d)[None, :]
        assert np.array_equal(m.unpack_bits(m.pack_bits(row, bits), bits, d), row), bits


def check_ext_quantizer_brute_force(m):
    """Each code is the argmin of |z - s q| over the b-bit range, ties to even."""
    rng = np.random.default_rng(22)
    for bits in m.CODE_BITS:
        z = rng.standard_normal((4, 64)) * 2.0
        z[0, 5] = 0.0
        q, s, _ = m.quantize_groups_bits(z, 32, bits)
        lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
        cand = np.arange(lo, hi + 1, dtype=np.float64)
        for r in range(z.shape[0]):
            for i in range(64):
                sc = float(s[r, i // 32])
                err = np.abs(z[r, i] - sc * cand)
                best = cand[err <= err.min() + 1e-12 * max(1.0, abs(z[r, i]))]
                want = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
                assert q[r, i] == want, (bits, r, i, q[r, i], want)


def check_ext_absmax_maps_to_extreme_codes(m):
    """s = absmax / 2^(b-1) per group: the group's -absmax lands on the lowest
    code, +absmax clips to the highest; a huge absmax saturates at 65504."""
    for bits in m.CODE_BITS:
        z = np.zeros((1, 64))
        z[0, 3], z[0, 9], z[0, 40] = 3.0, -3.0, 0.5
        q, s, _ = m.quantize_groups_bits(z, 32, bits)
        assert float(s[0, 0]) == float(np.float16(3.0 / (1 << (bits - 1))))
        assert float(s[0, 1]) == float(np.float16(0.5 / (1 << (bits - 1))))
        assert q[0, 9] == -(1 << (bits - 1)) and q[0, 3] == (1 << (bits - 1)) - 1
        assert float(m.fp16_scale_bits(np.array([1e9]), bits)[0]) == 65504.0


def check_lambda_power_of_two_is_exact_input_scaling(m):
    """With lambda a power of two per channel, the forward equals the plain
    forward of the scaled fp16 input and the inverse equals the plain inverse
    divided by lambda, exactly."""
    rng = np.random.default_rng(23)
    d = 64
    lam = (2.0 ** rng.integers(-2, 3, size=d)).astype(np.float16)
    x = rng.standard_normal((10, d)).astype(np.float16)
    for bits in (3, 4, 8):
        c1, s1 = m.quant_fwd_ext(x, 32, bits, lam, 9, 0, 0, "srft")
        c2, s2 = m.quant_fwd_ext((x.astype(np.float64) * lam).astype(np.float16), 32, bits, None, 9, 0, 0, "srft")
        assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
        _, u1 = m.dequant_inv_ext(c1, s1, d, 32, bits, lam, 9, return_fp64=True)
        _, u2 = m.dequant_inv_ext(c1, s1, d, 32, bits, None, 9, return_fp64=True)
        assert np.array_equal(u1, u2 / lam.astype(np.float64))


def check_lambda_energy_identity(m):
    """||lambda (.) (u - x)|| = ||z_hat - z|| per row: lambda multiplies before
    the orthogonal rotation and divides after the inverse."""
    rng = np.random.default_rng(24)
    d = 128
    lam = rng.uniform(0.25, 4.0, size=d).astype(np.float16)
    x = rng.standard_normal((6, d)).astype(np.float16)
    det = m.forward_detail_ext(x, 32, 3, lam, 3, 0, 0, "srft")
    zhat = m.dequantize_groups(det["q"], det["s"], 32)
    _, u = m.dequant_inv_ext(det["codes"], det["s"], d, 32, 3, lam, 3, return_fp64=True)
    lhs = np.linalg.norm(lam.astype(np.float64) * (u - x.astype(np.float64)), axis=1)
    rhs = np.linalg.norm(zhat - det["z"], axis=1)
    assert np.allclose(lhs, rhs, rtol=1e-9, atol=1e-12)


def check_error_falls_with_code_width(m):
    """Round-trip RMS error falls with the code width (3 > 4 > 6 > 8 bits),
    roughly by 2x per bit."""
    rng = np.random.default_rng(25)
    x = rng.standard_normal((64, 64)).astype(np.float16)
    err = {}
    for bits in m.CODE_BITS:
        c, s = m.quant_fwd_ext(x, 32, bits, None, 1)
        y = m.dequant_inv_ext(c, s, 64, 32, bits, None, 1).astype(np.float64)
        err[bits] = float(np.sqrt(np.mean((y - x.astype(np.float64)) ** 2)))
    assert err[3] > 1.5 * err[4] > 0 and err[4] > 3.0 * err[6] and err[6] > 3.0 * err[8], err
