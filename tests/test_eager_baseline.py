"""The eager four-operation baseline (eager_baseline.py, beside bench.py) is held
to the same parity bar as the fused kernels: it is measured beside them, so
it must compute the same thing.  CPU cases run here; the GPU case checks the
torch.fft / GPU elementwise path that bench.py times."""
import numpy as np
import pytest
import torch

import eager_baseline as eager
from rotate_then_quantize_amd import workloads as W
from tests import parity

CASES = [("srft", 64, 32), ("srft", 64, 64), ("srft", 128, 32), ("srft", 256, 32),
         ("srht", 64, 64), ("srht", 128, 64), ("srht", 256, 32)]


def _check(x, d, g, rot, seed, rps, per, device):
    xt = torch.from_numpy(x).to(device)
    codes, scales = eager.quant_fwd(xt, g, seed, rps, per, rot)
    st = parity.check_forward(x, codes.cpu().numpy(), scales.cpu().numpy(), g, seed, rps, per, rot,
                              allow_ties=True)
    assert st["code_ties"] <= 1e-5 * st["elements"] + 2
    oc, os_ = parity.oracle.quant_fwd(x, g, seed, rps, per, rot)
    y = eager.dequant_inv(torch.from_numpy(oc).to(device), torch.from_numpy(os_).to(device), d, g, seed, rps,
                          per, rot)
    parity.check_inverse(oc, os_, y.cpu().numpy(), d, g, seed, rps, per, rot)


@pytest.mark.parametrize("rot,d,g", CASES)
def test_eager_matches_oracle_cpu(rot, d, g):
    rng = np.random.default_rng(d + g)
    x = (rng.standard_normal((203, d)) * 2.0).astype(np.float16)
    x[5, 3] = 40.0
    _check(x, d, g, rot, seed=0x5EED + d, rps=9, per=4, device="cpu")


def test_eager_sign_rule_matches_oracle():
    s = eager.sign_matrix(50, 64, 77, rows_per_seed=7, seed_period=3, device="cpu").numpy()
    assert np.array_equal(s, parity.oracle.sign_matrix(50, 64, 77, 7, 3).astype(np.float32))


@pytest.mark.gpu
@pytest.mark.parametrize("wid", [2, 3, 4, 5])
def test_eager_matches_oracle_gpu(wid):
    w = W.WORKLOADS[wid].scaled(tokens=16 if wid != 3 else 3)
    x = W.generate(w, "cuda").cpu().numpy()
    rot = w.rots[-1]
    _check(x, w.d, w.group, rot, w.sign_seed, w.rows_per_seed, w.seed_period, device="cuda")
