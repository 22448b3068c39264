"""Decode attention over the int4 rotated cache, HIP path against the oracle
(needs an MI355X).

The cache is built on the CPU by the oracle's forward (or, at full size, drawn
as seeded random codes and scales on the device), the kernel runs through the
C ABI (ctypes binding), and every output element is compared with
oracle.attn_decode under the bound of tests/parity.py (check_attention).
"""
import math

import numpy as np
import pytest

import oracle
from tests.conftest import gpu_available
from tests.parity import check_attention, check_attention_window

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

torch = pytest.importorskip("torch")
import rotate_then_quantize_amd as rtq  # noqa: E402
from rotate_then_quantize_amd import workloads as W  # noqa: E402

DEV = "cuda"
ATTN = sorted(rtq.ATTN_SUPPORTED)


def lm(streams, tcap):
    return (2 * streams * tcap, streams * tcap, tcap, 1)


def tm(layers, streams):
    return (2 * streams, streams, 1, 2 * layers * streams)


def make_cache(rng, n, d, g, seed, rps, per, rot, scale=1.0, outliers=0):
    x = rng.standard_normal((n, d)) * scale
    if outliers:
        x[:, rng.choice(d, outliers, replace=False)] *= 15.0
    return oracle.quant_fwd(x.astype(np.float16), g, seed, rps, per, rot)


def gpu_attn(rot, q16, codes, scales, strides, tokens, g, seed, rps, per, softmax_scale=None, workspace=None):
    q = torch.from_numpy(np.ascontiguousarray(q16)).to(DEV)
    c = torch.from_numpy(np.ascontiguousarray(codes)).to(DEV)
    s = torch.from_numpy(np.ascontiguousarray(scales)).to(DEV)
    o = rtq.attn_decode(rot, q, c, s, strides, tokens, g, seed, rps, per, softmax_scale, workspace=workspace)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def run_case(rot, d, g, layers, streams, tokens, qpk, strides, n, seed=7, rps=0, per=0, softmax_scale=None,
             q_scale=1.0, v_scale=1.0, rng_seed=0, outliers=0, workspace=None):
    rng = np.random.default_rng(rng_seed)
    codes, scales = make_cache(rng, n, d, g, seed, rps, per, rot, v_scale, outliers)
    q16 = (rng.standard_normal((layers, streams, qpk, d)) * q_scale).astype(np.float16)
    ws = "auto" if workspace is None else f"{workspace.numel()} bytes"
    print(f"case rot={rot} d={d} g={g} L={layers} S={streams} T={tokens} G={qpk} strides={strides} workspace={ws}",
          flush=True)
    o_gpu = gpu_attn(rot, q16, codes, scales, strides, tokens, g, seed, rps, per, softmax_scale, workspace)
    o_orc = oracle.attn_decode(q16, codes, scales, strides, layers, streams, tokens, qpk, d, g, seed, rps, per,
                               rot, softmax_scale)
    worst = check_attention(o_gpu, o_orc, scales, strides, tokens, g)
    print(f"  worst error / (2e-3 s_v) = {worst:.3f}", flush=True)
    return worst


@pytest.mark.parametrize("rot", ["srft", "srht"])
@pytest.mark.parametrize("d,g", ATTN)
@pytest.mark.parametrize("qpk", [1, 3, 8])
def test_layer_major_per_layer_seeds(rot, d, g, qpk):
    L, S, T = 2, 3, 100  # four 32-token chunks, the last one ragged
    run_case(rot, d, g, L, S, T, qpk, lm(S, T), L * 2 * S * T, seed=11, rps=2 * S * T, per=L, outliers=2)


@pytest.mark.parametrize("rot", ["srft", "srht"])
@pytest.mark.parametrize("tokens", [1, 2, 31, 32, 33, 64, 65, 127, 128, 129, 200, 385])
def test_token_counts(rot, tokens):
    S = 2
    run_case(rot, 128, 32, 1, S, tokens, 6, lm(S, tokens), 2 * S * tokens, seed=5)


@pytest.mark.parametrize("d,g,qpk", [(128, 32, 6), (64, 32, 3), (64, 64, 1), (256, 32, 4), (256, 128, 8)])
def test_time_major_decode_layout(d, g, qpk):
    L, S, T = 3, 4, 70
    run_case("srft", d, g, L, S, T, qpk, tm(L, S), L * 2 * S * T, seed=0x5EED * 3, rps=2 * S, per=L)


@pytest.mark.parametrize("d,g", [(128, 32), (64, 64), (256, 32)])
def test_many_chunks_per_wave(d, g):
    S, T = 2, 1000  # 32 chunks: eight per wave, the ring wraps several times
    run_case("srft", d, g, 1, S, T, 4, lm(S, T), 2 * S * T, seed=3)


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("q_scale", [1e-3, 30.0, 600.0])
def test_query_magnitudes(q_scale, d):
    S, T = 2, 90
    run_case("srft", d, 32, 1, S, T, 5, lm(S, T), 2 * S * T, seed=9, q_scale=q_scale)


@pytest.mark.parametrize("v_scale", [1e-2, 300.0])
def test_cache_magnitudes(v_scale):
    S, T = 2, 90
    run_case("srft", 128, 64, 1, S, T, 2, lm(S, T), 2 * S * T, seed=9, v_scale=v_scale, q_scale=1.0 / v_scale)


@pytest.mark.parametrize("softmax_scale", [0.0, 1.0, -0.2])
def test_softmax_scales(softmax_scale):
    S, T = 2, 77
    run_case("srht", 64, 32, 1, S, T, 3, lm(S, T), 2 * S * T, seed=4, softmax_scale=softmax_scale)


def test_strided_cache_with_gaps():
    """Rows of a stream need not be adjacent: a token stride of 3 and unused rows between streams."""
    L, S, T = 2, 2, 50
    strides = (2 * S * 160, S * 160, 160, 3)
    run_case("srft", 128, 32, L, S, T, 2, strides, L * 2 * S * 160, seed=1)


# ---------------------------------------------------------------------------
# Token splits: few (layer, stream) pairs and long streams, so the call spreads
# each stream over several workgroups that merge through the workspace.
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("rot", ["srft", "srht"])
@pytest.mark.parametrize("d,g", ATTN)
def test_split_streams(rot, d, g):
    L, S, T, G = 1, 2, 1500, 3  # 47 chunks, the last one ragged
    assert rtq.attn_workspace_bytes(L, S, T, G, d) > 0, "this shape is meant to split"
    run_case(rot, d, g, L, S, T, G, lm(S, T), L * 2 * S * T, seed=21, outliers=2)


@pytest.mark.parametrize("T", [512, 513, 2047, 4100])
def test_split_token_counts(T):
    L, S, G = 2, 1, 8
    run_case("srft", 128, 32, L, S, T, G, lm(S, T), L * 2 * S * T, seed=23, rps=2 * S * T, per=L)


def test_split_workspace_sizes_and_reuse():
    """The same call with no workspace, a workspace for two splits, and the full
    workspace (twice, then again with fewer tokens: every call leaves the
    counters at zero) agrees with the oracle each time."""
    L, S, T, G, d, g = 1, 3, 1200, 4, 64, 32
    full = rtq.attn_workspace_bytes(L, S, T, G, d)
    assert full > 0
    pairs = L * S
    two = ((pairs * 4 + 255) // 256) * 256 + pairs * 2 * (((G * (d + 2)) + 3) // 4 * 4) * 4
    assert two < full
    ws_full = torch.zeros(full, dtype=torch.uint8, device=DEV)
    for ws in (torch.empty(0, dtype=torch.uint8, device=DEV), torch.zeros(two, dtype=torch.uint8, device=DEV),
               ws_full, ws_full):
        run_case("srft", d, g, L, S, T, G, lm(S, T), L * 2 * S * T, seed=31, workspace=ws)
    run_case("srft", d, g, L, S, 700, G, lm(S, T), L * 2 * S * T, seed=31, workspace=ws_full)
    assert int(ws_full[:256].sum()) == 0, "the counters are back at zero"


def test_split_matches_unsplit_closely():
    """Split and unsplit runs differ only by fp32 rounding of the merge."""
    rng = np.random.default_rng(5)
    L, S, T, G, d, g = 1, 2, 3000, 6, 128, 32
    codes, scales = make_cache(rng, L * 2 * S * T, d, g, 3, 0, 0, "srft")
    q16 = rng.standard_normal((L, S, G, d)).astype(np.float16)
    a = gpu_attn("srft", q16, codes, scales, lm(S, T), T, g, 3, 0, 0,
                 workspace=torch.empty(0, dtype=torch.uint8, device=DEV)).astype(np.float64)
    b = gpu_attn("srft", q16, codes, scales, lm(S, T), T, g, 3, 0, 0).astype(np.float64)
    scale = np.abs(a).max()
    assert np.abs(a - b).max() <= 2e-3 * scale, np.abs(a - b).max() / scale


def test_workspace_errors():
    q = torch.zeros((1, 1, 2, 128), dtype=torch.float16, device=DEV)
    c = torch.zeros((4096, 64), dtype=torch.uint8, device=DEV)
    s = torch.zeros((4096, 4), dtype=torch.float16, device=DEV)
    ws = torch.zeros(1 << 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(rtq.RTQError):
        rtq.srft_attn_decode(q, c, s, (0, 2048, 0, 1), 2048, 32, 1, workspace=ws[1:])   # misaligned
    with pytest.raises(rtq.RTQError):
        rtq.srft_attn_decode(q, c, s, (0, 2048, 0, 1), 2048, 32, 1, workspace=c.view(-1))  # overlaps the codes
    lib = rtq.library()
    st = lib.srft_attn_decode(q.data_ptr(), c.data_ptr(), s.data_ptr(), ws.data_ptr() + 4096, 1, 1, 2048, 2, 128, 32,
                              0, 2048, 0, 1, 1, 0, 0, 0.1, None, 64, None)  # size without a pointer
    assert st == rtq.RTQ_ERR_INVALID_ARG
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# The fp16 window of the newest tokens, in the same softmax as the int4 tokens.
# ---------------------------------------------------------------------------


def run_window_case(rot, d, g, L, S, T, W, Wc, G, seed=41, workspace=None):
    rng = np.random.default_rng(d + g + 7 * W + T)
    tcap = max(T, 1)
    rps = 2 * S * tcap if L > 1 else 0
    per = L if L > 1 else 0
    codes, scales = make_cache(rng, L * 2 * S * tcap, d, g, seed, rps, per, rot, outliers=2)
    win = (rng.standard_normal((L, 2, S, Wc, d)) * 1.5).astype(np.float16)
    q16 = rng.standard_normal((L, S, G, d)).astype(np.float16)
    print(f"window case rot={rot} d={d} g={g} L={L} S={S} T={T} W={W}/{Wc} G={G}", flush=True)
    q = torch.from_numpy(q16).to(DEV)
    c = torch.from_numpy(np.ascontiguousarray(codes)).to(DEV)
    sc = torch.from_numpy(np.ascontiguousarray(scales)).to(DEV)
    wt = torch.from_numpy(win).to(DEV)
    o = rtq.attn_decode(rot, q, c, sc, lm(S, tcap), T, g, seed, rps, per, window=wt, window_tokens=W,
                        workspace=workspace)
    torch.cuda.synchronize()
    o_orc = oracle.attn_decode(q16, codes, scales, lm(S, tcap), L, S, T, G, d, g, seed, rps, per, rot,
                               window=win, window_tokens=W)
    worst = check_attention_window(o.cpu().numpy(), o_orc, scales, lm(S, tcap), T, g, win, W)
    print(f"  worst error / bound = {worst:.3f}", flush=True)
    return o, (q, c, sc, wt, tcap, rps, per)


@pytest.mark.parametrize("rot", ["srft", "srht"])
@pytest.mark.parametrize("d,g", ATTN)
def test_window_joins_the_int4_tokens(rot, d, g):
    run_window_case(rot, d, g, 2, 3, 37, 5, 16, 3)


@pytest.mark.parametrize("rot", ["srft", "srht"])
@pytest.mark.parametrize("d,T,W,G", [(64, 100, 64, 8), (128, 1, 16, 6), (256, 70, 1, 4), (128, 33, 63, 1),
                                     (256, 40, 64, 8), (128, 300, 64, 8)])
def test_window_sizes(rot, d, T, W, G):
    """Window sizes up to the 64-token limit, with up to 8 queries per K/V head (the largest window
    work area)."""
    run_window_case(rot, d, 32, 1, 2, T, W, max(W, 16), G)


@pytest.mark.parametrize("rot", ["srft", "srht"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_window_without_int4_tokens(rot, d):
    """The first decode steps: nothing is quantized yet, the window is the whole context."""
    run_window_case(rot, d, 32, 2, 2, 0, 7, 16, 4)


@pytest.mark.parametrize("rot", ["srft", "srht"])
@pytest.mark.parametrize("d", [64, 128])
def test_window_with_token_splits(rot, d):
    """Only the workgroup that merges a stream's splits reads the window."""
    L, S, T = 1, 2, 1500
    assert rtq.attn_workspace_bytes(L, S, T, 4, d) > 0
    run_window_case(rot, d, 32, L, S, T, 16, 16, 4)


def test_empty_window_equals_plain_attention():
    o, (q, c, sc, wt, tcap, rps, per) = run_window_case("srft", 128, 32, 2, 2, 90, 0, 16, 5)
    o2 = rtq.attn_decode("srft", q, c, sc, lm(2, tcap), 90, 32, 41, rps, per)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)


@pytest.mark.parametrize("rot,d,g", [("srft", 128, 32), ("srht", 64, 64), ("srft", 256, 32)])
def test_decode_cache_attention(rot, d, g):
    """DecodeCache.attention after a prefill and single-token appends: one launch over the int4 prefix
    and the fp16 window, against the oracle on the tokens as they went in."""
    from rotate_then_quantize_amd.decode_cache import DecodeCache
    L, S, C, Wn, T0, K, G, seed = 2, 3, 96, 16, 20, 21, 3, 17
    rng = np.random.default_rng(3)
    toks = rng.standard_normal((L, 2, S, T0 + K, d)).astype(np.float16)
    cache = DecodeCache(L, S, C, d, g, seed, rot, Wn)
    cache.prefill(torch.from_numpy(np.ascontiguousarray(toks[:, :, :, :T0])).to(DEV))
    for k in range(K):
        cache.append(torch.from_numpy(np.ascontiguousarray(toks[:, :, :, T0 + k])).to(DEV))
    q16 = rng.standard_normal((L, S, G, d)).astype(np.float16)
    o = cache.attention(torch.from_numpy(q16).to(DEV))
    torch.cuda.synchronize()
    nq, held = cache.quantized, cache.held
    print(f"decode cache attention rot={rot} d={d}: {nq} int4 tokens, {held} in the window", flush=True)
    assert held > 0 and nq > T0
    codes, scales = cache.codes.cpu().numpy(), cache.scales.cpu().numpy()
    win = cache.window_kv.cpu().numpy()
    o_orc = oracle.attn_decode(q16, codes, scales, cache.strides, L, S, nq, G, d, g, seed, cache.rows_per_seed,
                               cache.seed_period, rot, window=win, window_tokens=held)
    check_attention_window(o.cpu().numpy(), o_orc, scales, cache.strides, nq, g, win, held)
    assert np.array_equal(win[:, :, :, :held], toks[:, :, :, nq:nq + held])
    # without the dequantized copy: the same int4 cache, window and attention output
    lean = DecodeCache(L, S, C, d, g, seed, rot, Wn, keep_prefix=False)
    lean.prefill(torch.from_numpy(np.ascontiguousarray(toks[:, :, :, :T0])).to(DEV))
    for k in range(K):
        lean.append(torch.from_numpy(np.ascontiguousarray(toks[:, :, :, T0 + k])).to(DEV))
    o2 = lean.attention(torch.from_numpy(q16).to(DEV))
    torch.cuda.synchronize()
    assert lean.prefix is None and (lean.quantized, lean.held) == (nq, held)
    assert torch.equal(lean.codes, cache.codes) and torch.equal(lean.scales, cache.scales)
    assert torch.equal(o2, o)


def test_empty_grid_is_a_no_op():
    q = torch.zeros((0, 3, 2, 128), dtype=torch.float16, device=DEV)
    c = torch.zeros((10, 64), dtype=torch.uint8, device=DEV)
    s = torch.zeros((10, 4), dtype=torch.float16, device=DEV)
    o = rtq.srft_attn_decode(q, c, s, (0, 0, 0, 1), 1, 32, 1)
    assert o.shape == q.shape


def test_argument_errors():
    q = torch.zeros((1, 1, 2, 128), dtype=torch.float16, device=DEV)
    c = torch.zeros((64, 64), dtype=torch.uint8, device=DEV)
    s = torch.zeros((64, 4), dtype=torch.float16, device=DEV)
    with pytest.raises(ValueError):
        rtq.srft_attn_decode(q, c, s, (0, 32, 0, 1), 0, 32, 1)          # no tokens
    with pytest.raises(ValueError):
        rtq.srft_attn_decode(q, c, s, (0, 32, 0, 1), 40, 32, 1)         # rows past the cache
    with pytest.raises(rtq.RTQError):
        rtq.srft_attn_decode(q, c, s, (0, 32, 0, 1), 8, 32, 1, 1, 0)    # a seed per row
    q9 = torch.zeros((1, 1, 9, 128), dtype=torch.float16, device=DEV)
    with pytest.raises(rtq.RTQError):
        rtq.srft_attn_decode(q9, c, s, (0, 32, 0, 1), 8, 32, 1)         # 9 query heads per K/V head
    q256 = torch.zeros((1, 1, 1, 256), dtype=torch.float16, device=DEV)
    c256 = torch.zeros((64, 128), dtype=torch.uint8, device=DEV)
    s256 = torch.zeros((64, 16), dtype=torch.float16, device=DEV)
    with pytest.raises(rtq.RTQError):
        rtq.srft_attn_decode(q256, c256, s256, (0, 32, 0, 1), 8, 16, 1)  # groups of 16 not built


# ---------------------------------------------------------------------------
# Full-size caches in the launch configuration the bench times, checked on
# sampled (layer, stream) pairs.  Codes are uniform over [-8, 7] and scales
# |N(0, 1)| * 0.3 in fp16 (the magnitude absmax/8 takes for unit-variance K/V).
# ---------------------------------------------------------------------------


def random_cache(n, d, g, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    codes = torch.randint(0, 256, (n, d // 2), generator=gen, device=DEV, dtype=torch.int32).to(torch.uint8)
    scales = (torch.randn((n, d // g), generator=gen, device=DEV).abs() * 0.3).to(torch.float16)
    return codes, scales


@pytest.mark.parametrize("wid", [3, 2, 5])
def test_workload_full_size_sampled(wid):
    w = W.WORKLOADS[wid]
    L, S, T, G, d, g = w.layers, w.streams, w.tokens, w.q_per_kv, w.d, w.group
    codes, scales = random_cache(w.n_rows, d, g, 100 + wid)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(200 + wid)
    q = torch.randn((L, S, G, d), generator=gen, device=DEV).to(torch.float16)
    print(f"full size {w.name}: L={L} S={S} T={T} G={G} rows={w.n_rows}", flush=True)
    o = rtq.srft_attn_decode(q, codes, scales, w.cache_strides, T, g, w.sign_seed, w.rows_per_seed, w.seed_period)
    torch.cuda.synchronize()
    rng = np.random.default_rng(wid)
    extra = 4 if T <= 4096 else 1  # the oracle takes a few seconds per 32768-token d = 256 stream
    pairs = [(0, 0), (L - 1, S - 1)] + [(int(rng.integers(L)), int(rng.integers(S))) for _ in range(extra)]
    qh, ch, sh, oh = q.cpu().numpy(), codes.cpu().numpy(), scales.cpu().numpy(), o.cpu().numpy()
    o_orc = oracle.attn_decode(qh, ch, sh, w.cache_strides, L, S, T, G, d, g, w.sign_seed, w.rows_per_seed,
                               w.seed_period, "srft", pairs=pairs)
    worst = check_attention(oh, o_orc, sh, w.cache_strides, T, g, pairs=pairs)
    print(f"  sampled pairs {pairs}: worst error / (2e-3 s_v) = {worst:.3f}", flush=True)
    del codes, scales, q, o
    torch.cuda.empty_cache()


@pytest.mark.parametrize("wid,win", [(3, 0), (3, 16), (2, 16), (5, 16)])
def test_bench_launch_full_size_sampled(wid, win):
    """The launch that the attention bench times, at full size: the per-head
    [layer][K, V][stream][token] layout with one sign seed per layer, the
    binding's token-split workspace, and (win > 0) that many fp16 window
    tokens per stream; sampled (layer, stream) pairs against the oracle."""
    w = W.WORKLOADS[wid]
    L, S, T, G, d, g = w.layers, w.streams, w.tokens, w.q_per_kv, w.d, w.group
    strides = (2 * S * T, S * T, T, 1)
    rps, per = (2 * S * T, L) if L > 1 else (0, 0)
    codes, scales = random_cache(L * 2 * S * T, d, g, 300 + wid)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(400 + wid)
    q = torch.randn((L, S, G, d), generator=gen, device=DEV).to(torch.float16)
    window = torch.randn((L, 2, S, max(win, 1), d), generator=gen, device=DEV).to(torch.float16)
    print(f"bench launch {w.name}: L={L} S={S} T={T} G={G} window={win} "
          f"splits workspace={rtq.attn_workspace_bytes(L, S, T, G, d)} B", flush=True)
    o = rtq.srft_attn_decode(q, codes, scales, strides, T, g, w.sign_seed, rps, per,
                             window=window if win else None, window_tokens=win)
    torch.cuda.synchronize()
    rng = np.random.default_rng(wid + win)
    extra = 3 if T <= 4096 else 0  # a 32768-token d = 256 stream takes the oracle a few seconds
    pairs = [(0, 0), (L - 1, S - 1)] + [(int(rng.integers(L)), int(rng.integers(S))) for _ in range(extra)]
    qh, ch, sh, oh = q.cpu().numpy(), codes.cpu().numpy(), scales.cpu().numpy(), o.cpu().numpy()
    wh = window.cpu().numpy()
    o_orc = oracle.attn_decode(qh, ch, sh, strides, L, S, T, G, d, g, w.sign_seed, rps, per, "srft", pairs=pairs,
                               window=wh if win else None, window_tokens=win)
    worst = check_attention_window(oh, o_orc, sh, strides, T, g, wh, win, pairs=pairs)
    print(f"  sampled pairs {pairs}: worst error / bound = {worst:.3f}", flush=True)
    del codes, scales, q, o, window
    torch.cuda.empty_cache()
