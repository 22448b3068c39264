"""In-place append, row-mapped inverse and the decode cache with an fp16
window, HIP path against the oracle (needs an MI355X).

Inputs are seeded fp16 K/V; expected codes and scales come from the oracle's
forward on the same rows (with each cache row's own seed) and expected fp16
outputs from the oracle's inverse, under the tolerances of tests/parity.py.
Rows outside the block must keep a sentinel value.
"""
import numpy as np
import pytest

import oracle
from tests.conftest import gpu_available
from tests.parity import check_forward, check_inverse

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

torch = pytest.importorskip("torch")
import rotate_then_quantize_amd as rtq  # noqa: E402
from rotate_then_quantize_amd.decode_cache import DecodeCache  # noqa: E402

DEV = "cuda"
SHAPES = sorted(rtq.CACHE_SUPPORTED)
SENTINEL = 0xA5


def lm(streams, cap):
    return (2 * streams * cap, streams * cap, cap, 1)


def tm(layers, streams):
    return (2 * streams, streams, 1, 2 * layers * streams)


def block_rows(layers, streams, t0, n, strides):
    """Cache rows of a [layers][2][streams][n] block, in block order."""
    return np.array([l * strides[0] + kv * strides[1] + s * strides[2] + (t0 + j) * strides[3]
                     for l in range(layers) for kv in (0, 1) for s in range(streams) for j in range(n)],
                    dtype=np.int64)


def run_append(rot, d, g, layers, streams, cap, t0, n, strides, seed, rps, per, scale=1.0):
    rng = np.random.default_rng(d + g + t0)
    x = (rng.standard_normal((layers, 2, streams, n, d)) * scale).astype(np.float16)
    rows_total = layers * 2 * streams * cap
    codes = torch.full((rows_total, d // 2), SENTINEL, dtype=torch.uint8, device=DEV)
    scales = torch.full((rows_total, d // g), 7.0, dtype=torch.float16, device=DEV)
    print(f"append rot={rot} d={d} g={g} L={layers} S={streams} t0={t0} n={n} strides={strides}", flush=True)
    rtq.quant_append(rot, torch.from_numpy(x).to(DEV), codes, scales, strides, t0, g, seed, rps, per)
    torch.cuda.synchronize()
    ch, sh = codes.cpu().numpy(), scales.cpu().numpy()
    rows = block_rows(layers, streams, t0, n, strides)
    check_forward(x.reshape(-1, d), ch[rows], sh[rows], g, seed, rps, per, rot, rows=rows)
    others = np.setdiff1d(np.arange(rows_total), rows)
    assert np.all(ch[others] == SENTINEL) and np.all(sh[others] == np.float16(7.0)), "rows outside the block changed"
    return ch, sh, rows


@pytest.mark.parametrize("rot", ["srft", "srht"])
@pytest.mark.parametrize("d,g", SHAPES)
def test_append_layer_major(rot, d, g):
    L, S, C = 2, 3, 40
    run_append(rot, d, g, L, S, C, 7, 9, lm(S, C), 21, 2 * S * C, L)


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("t0,n", [(0, 1), (2, 3), (10, 16), (0, 70)])
def test_append_time_major(t0, n, d):
    L, S, C = 3, 4, 80
    run_append("srft", d, 32, L, S, C, t0, n, tm(L, S), 0x5EED * 3, 2 * S, L)


@pytest.mark.parametrize("rot,d", [("srft", 64), ("srft", 256), ("srht", 256)])
def test_append_seed_per_token_row(rot, d):
    """A seed rule that changes inside a tile takes the per-lane sign path."""
    L, S, C = 1, 2, 50
    run_append(rot, d, 32, L, S, C, 3, 40, lm(S, C), 5, 7, 0)


@pytest.mark.parametrize("rot", ["srft", "srht"])
def test_dequant_rows_seed_per_token_row(rot):
    """The row-mapped inverse with seeds that change inside a tile (d = 256)."""
    L, S, C, d, g = 1, 2, 50, 256, 32
    ch, sh, rows = run_append(rot, d, g, L, S, C, 3, 40, lm(S, C), 5, 7, 0)
    y = torch.zeros((L * 2 * S * C, d), dtype=torch.float16, device=DEV)
    rtq.dequant_rows(rot, torch.from_numpy(ch).to(DEV), torch.from_numpy(sh).to(DEV), y, L, S, 3, 40, lm(S, C), g, 5,
                     7, 0)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    check_inverse(ch[rows], sh[rows], yh[rows], d, g, 5, 7, 0, rot, rows=rows)
    others = np.setdiff1d(np.arange(L * 2 * S * C), rows)
    assert not yh[others].any(), "rows outside the block were written"


@pytest.mark.parametrize("rot", ["srft", "srht"])
@pytest.mark.parametrize("d,g", SHAPES)
def test_dequant_rows(rot, d, g):
    L, S, C, t0, n = 2, 3, 30, 4, 11
    strides = lm(S, C)
    rng = np.random.default_rng(3 + d + g)
    rows_total = L * 2 * S * C
    x = rng.standard_normal((rows_total, d)).astype(np.float16)
    codes, scales = oracle.quant_fwd(x, g, 8, 2 * S * C, L, rot)
    y = torch.full((rows_total, d), -3.0, dtype=torch.float16, device=DEV)
    print(f"dequant_rows rot={rot} d={d} g={g}", flush=True)
    rtq.dequant_rows(rot, torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV), y, L, S, t0, n,
                     strides, g, 8, 2 * S * C, L)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    rows = block_rows(L, S, t0, n, strides)
    check_inverse(codes[rows], scales[rows], yh[rows], d, g, 8, 2 * S * C, L, rot, rows=rows)
    others = np.setdiff1d(np.arange(rows_total), rows)
    assert np.all(yh[others] == np.float16(-3.0)), "rows outside the block changed"


def test_empty_block_is_a_no_op():
    x = torch.zeros((2, 2, 3, 0, 64), dtype=torch.float16, device=DEV)
    codes = torch.zeros((100, 32), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((100, 2), dtype=torch.float16, device=DEV)
    rtq.srft_quant_append(x, codes, scales, (0, 0, 0, 1), 0, 32, 1)
    assert int(codes.sum()) == 0


@pytest.mark.parametrize("rot,d,g", [("srft", 128, 32), ("srht", 64, 64), ("srft", 256, 32), ("srht", 256, 64)])
def test_decode_cache_window_cycle(rot, d, g):
    """Prefill 20 tokens, append 37 one at a time with a 16-token window:
    the quantized prefix, its dequantized copy and the window match the
    oracle and the window schedule after every append."""
    L, S, C, W, T0, K = 2, 3, 96, 16, 20, 37
    seed = 31
    rng = np.random.default_rng(11)
    toks = rng.standard_normal((L, 2, S, T0 + K, d)).astype(np.float16)
    cache = DecodeCache(L, S, C, d, g, seed, rot, W)
    cache.prefill(torch.from_numpy(np.ascontiguousarray(toks[:, :, :, :T0])).to(DEV))
    for k in range(1, K + 1):
        cache.append(torch.from_numpy(np.ascontiguousarray(toks[:, :, :, T0 + k - 1])).to(DEV))
        assert (cache.quantized, cache.held) == oracle.window_schedule(T0, k, W)
    torch.cuda.synchronize()
    print(f"decode cache rot={rot} d={d} g={g}: quantized {cache.quantized}, window {cache.held}", flush=True)
    nq, held = cache.quantized, cache.held
    rows = block_rows(L, S, 0, nq, cache.strides)
    x = toks[:, :, :, :nq].reshape(-1, d)
    ch, sh, ph = cache.codes.cpu().numpy(), cache.scales.cpu().numpy(), cache.prefix.cpu().numpy()
    check_forward(x, ch[rows], sh[rows], g, seed, cache.rows_per_seed, cache.seed_period, rot, rows=rows)
    check_inverse(ch[rows], sh[rows], ph[rows], d, g, seed, cache.rows_per_seed, cache.seed_period, rot, rows=rows)
    win = cache.window_kv.cpu().numpy()
    assert np.array_equal(win[:, :, :, :held], toks[:, :, :, nq:nq + held]), "window differs from the inputs"
    unused = np.setdiff1d(np.arange(L * 2 * S * C), rows)
    assert not ch[unused].any() and not ph[unused].any(), "rows past the quantized prefix were written"


def test_decode_cache_rejects_overflow():
    cache = DecodeCache(1, 1, 4, 64, 32, 1, "srft", window=2)
    tok = torch.zeros((1, 2, 1, 64), dtype=torch.float16, device=DEV)
    for _ in range(4):
        cache.append(tok)
    with pytest.raises(RuntimeError):
        cache.append(tok)
