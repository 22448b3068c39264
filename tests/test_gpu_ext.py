"""Forward and inverse with 3-, 4-, 6- and 8-bit codes and a per-channel
lambda, HIP path against the oracle (needs an MI355X).

Inputs are seeded fp16 rows (with outlier channels); the forward is compared
with oracle.forward_detail_ext and the inverse, run on the oracle's codes,
with oracle.dequant_inv_ext, under tests/parity.py's check_forward_ext and
check_inverse_ext.
"""
import numpy as np
import pytest

import oracle
from tests.conftest import gpu_available
from tests.parity import fp16_ulp, check_forward_ext, check_inverse_ext

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

torch = pytest.importorskip("torch")
import rotate_then_quantize_amd as rtq  # noqa: E402

DEV = "cuda"
SHAPES = sorted(rtq.EXT_SUPPORTED)


def rows(n, d, seed, outliers=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d))
    x[:, rng.choice(d, outliers, replace=False)] *= 15.0
    return x.astype(np.float16)


def lam_vector(d, seed):
    return np.random.default_rng(seed).uniform(0.25, 4.0, size=d).astype(np.float16)


def run_case(rot, d, g, bits, use_lam, n=200, seed=5, rps=0, per=0):
    x = rows(n, d, d + g + bits)
    lam = lam_vector(d, d + bits) if use_lam else None
    lam_t = torch.from_numpy(lam).to(DEV) if use_lam else None
    print(f"ext rot={rot} d={d} g={g} bits={bits} lambda={use_lam} n={n} rps={rps} per={per}", flush=True)
    codes, scales = rtq.quant_fwd_ext(rot, torch.from_numpy(x).to(DEV), g, bits, seed, lam_t, rps, per)
    torch.cuda.synchronize()
    check_forward_ext(x, codes.cpu().numpy(), scales.cpu().numpy(), g, bits, lam, seed, rps, per, rot)
    oc, os_ = oracle.quant_fwd_ext(x, g, bits, lam, seed, rps, per, rot)
    y = rtq.dequant_inv_ext(rot, torch.from_numpy(oc).to(DEV), torch.from_numpy(os_).to(DEV), d, g, bits, seed,
                            lam_t, rps, per)
    torch.cuda.synchronize()
    worst = check_inverse_ext(oc, os_, y.cpu().numpy(), d, g, bits, lam, seed, rps, per, rot)
    print(f"  inverse worst error / tolerance = {worst:.3f}", flush=True)


@pytest.mark.parametrize("rot", ["srft", "srht"])
@pytest.mark.parametrize("d,g", SHAPES)
@pytest.mark.parametrize("bits", [3, 4, 6, 8])
@pytest.mark.parametrize("use_lam", [False, True])
def test_widths_and_lambda(rot, d, g, bits, use_lam):
    run_case(rot, d, g, bits, use_lam)


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("bits", [3, 6])
@pytest.mark.parametrize("n", [1, 31, 32, 33, 63, 64, 65, 129])
def test_ragged_rows_and_seed_rules(bits, n, d):
    run_case("srft", d, 32, bits, True, n=n, rps=7, per=3)


@pytest.mark.parametrize("rot", ["srft", "srht"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 63, 65, 129])
def test_bits4_lambda_ragged_rows(rot, d, n):
    """4-bit codes with lambda below d = 256 run on the int4 tiles with the
    lambda multiply: partial tiles and a per-row seed rule."""
    run_case(rot, d, 32, 4, True, n=n, rps=5, per=3)


@pytest.mark.parametrize("rot", ["srft", "srht"])
@pytest.mark.parametrize("d", [128, 256])
def test_bits4_without_lambda_equals_the_int4_kernels(rot, d):
    """The general kernel with 4-bit codes and no lambda writes the same codes
    and scales as the fused int4 kernel, and the same fp16 outputs, except for
    SRHT at d <= 128, where the two inverse kernels round the dequantized
    values differently (each stays within the inverse tolerance of the
    oracle; here they agree within 2e-3 times the row's largest scale)."""
    x = torch.from_numpy(rows(500, d, 1)).to(DEV)
    c1, s1 = rtq.quant_fwd_ext(rot, x, 32, 4, 9, None, 11, 4)
    c2, s2 = rtq.quant_fwd(rot, x, 32, 9, 11, 4)
    y1 = rtq.dequant_inv_ext(rot, c1, s1, d, 32, 4, 9, None, 11, 4)
    y2 = rtq.dequant_inv(rot, c2, s2, d, 32, 9, 11, 4)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
    if rot == "srft" or d == 256:
        assert torch.equal(y1, y2)
    else:
        a, b = y1.double().cpu().numpy(), y2.double().cpu().numpy()
        s_row = s2.double().cpu().numpy().max(axis=1, keepdims=True)
        assert np.all(np.abs(a - b) <= 2e-3 * s_row + fp16_ulp(b)), np.max(np.abs(a - b) / (2e-3 * s_row))


def test_error_falls_with_code_width_on_the_gpu():
    x = torch.from_numpy(rows(4096, 64, 2)).to(DEV)
    err = {}
    for bits in rtq.CODE_BITS:
        c, s = rtq.srft_quant_fwd_ext(x, 32, bits, 3)
        y = rtq.srft_dequant_inv_ext(c, s, 64, 32, bits, 3)
        err[bits] = float(((y.float() - x.float()) ** 2).mean().sqrt())
    print("rms error by bits", err, flush=True)
    assert err[3] > 1.5 * err[4] > 0 and err[4] > 3 * err[6] and err[6] > 3 * err[8]
