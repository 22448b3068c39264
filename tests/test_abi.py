"""The C ABI on the host: library loads, exports every declared symbol, and
rejects bad arguments before any HIP call (CPU only, no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import rotate_then_quantize_amd as rtq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rtq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(rtq.library_path()),
                                reason="librtq.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z_0-9]*\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(",
                                 src, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["rtq_attn_workspace_bytes", "rtq_status_string", "srft_attn_decode",
                                    "srft_attn_decode_noalloc", "srft_attn_decode_window", "srft_dequant_inv",
                                    "srft_dequant_inv_ext", "srft_dequant_rows", "srft_quant_append", "srft_quant_fwd",
                                    "srft_quant_fwd_ext", "srht_attn_decode", "srht_attn_decode_window",
                                    "srht_dequant_inv",
                                    "srht_dequant_inv_ext", "srht_dequant_rows", "srht_quant_append", "srht_quant_fwd",
                                    "srht_quant_fwd_ext"]


def test_library_exports_every_declared_symbol():
    lib = rtq.library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", rtq.library_path()], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(declared_functions()) <= exported
    # nothing else of ours leaks out of the shared object
    ours = {s for s in exported if "rtq" in s or "srft" in s or "srht" in s}
    assert ours == set(declared_functions()), ours


def test_status_strings():
    lib = rtq.library()
    for st, key in [(0, "RTQ_OK"), (1, "INVALID_ARG"), (2, "UNSUPPORTED"), (3, "RTQ_ERR_HIP")]:
        assert key in lib.rtq_status_string(st).decode()
    assert lib.rtq_status_string(99)


FWD = ["srft_quant_fwd", "srht_quant_fwd"]
INV = ["srft_dequant_inv", "srht_dequant_inv"]
A, B, C = 0x10000, 0x200000, 0x3000000  # distinct 16-byte aligned fake addresses (never dereferenced)


def call(name, p0, p1, p2, n, d, g, seed=1, rps=0, per=0):
    fn = getattr(rtq.library(), name)
    return fn(ctypes.c_void_p(p0), ctypes.c_void_p(p1), ctypes.c_void_p(p2), n, d, g, seed, rps, per, None)


@pytest.mark.parametrize("name", FWD + INV)
def test_rejects_bad_arguments_without_launching(name):
    assert call(name, A, B, C, -1, 64, 32) == rtq.RTQ_ERR_INVALID_ARG
    assert call(name, A, B, C, 10, 64, 32, rps=-1) == rtq.RTQ_ERR_INVALID_ARG
    assert call(name, A, B, C, 10, 64, 32, per=-1) == rtq.RTQ_ERR_INVALID_ARG
    for d, g in [(96, 32), (32, 32), (512, 32), (64, 16), (64, 128), (128, 256), (64, 48), (256, 512)]:
        assert call(name, A, B, C, 10, d, g) == rtq.RTQ_ERR_UNSUPPORTED, (d, g)
    # null and misaligned pointers
    assert call(name, 0, B, C, 10, 64, 32) == rtq.RTQ_ERR_INVALID_ARG
    assert call(name, A, 0, C, 10, 64, 32) == rtq.RTQ_ERR_INVALID_ARG
    assert call(name, A, B, 0, 10, 64, 32) == rtq.RTQ_ERR_INVALID_ARG
    assert call(name, A + 8, B, C, 10, 64, 32) == rtq.RTQ_ERR_INVALID_ARG
    assert call(name, A, B + 4, C, 10, 64, 32) == rtq.RTQ_ERR_INVALID_ARG
    assert call(name, A, B, C + 2, 10, 64, 32) == rtq.RTQ_ERR_INVALID_ARG
    # size overflow and the 32-bit row-index limit (0xFFFFFF00 rows per call)
    assert call(name, A, B, C, 1 << 62, 64, 32) == rtq.RTQ_ERR_INVALID_ARG
    assert call(name, A, B, C, 0xFFFFFF01, 64, 32) == rtq.RTQ_ERR_INVALID_ARG
    assert call(name, A, B, C, 1 << 32, 256, 32) == rtq.RTQ_ERR_INVALID_ARG


@pytest.mark.parametrize("name", FWD + INV)
def test_zero_rows_is_a_no_op(name):
    assert call(name, 0, 0, 0, 0, 64, 32) == rtq.RTQ_OK
    assert call(name, A, B, C, 0, 256, 32) == rtq.RTQ_OK


@pytest.mark.parametrize("name", FWD)
def test_forward_rejects_overlapping_buffers(name):
    n, d, g = 100, 64, 32  # x: 12800 B, codes: 3200 B, scales: 400 B
    assert call(name, A, A + 1024, C, n, d, g) == rtq.RTQ_ERR_INVALID_ARG   # codes inside x
    assert call(name, A, B, A + 4096, n, d, g) == rtq.RTQ_ERR_INVALID_ARG   # scales inside x
    assert call(name, A, B, B + 3184, n, d, g) == rtq.RTQ_ERR_INVALID_ARG   # scales overlap codes


@pytest.mark.parametrize("name", INV)
def test_inverse_rejects_overlapping_buffers(name):
    n, d, g = 100, 64, 32
    assert call(name, A + 1024, B, A, n, d, g) == rtq.RTQ_ERR_INVALID_ARG   # codes inside y
    assert call(name, A, B, A + 3000, n, d, g) == rtq.RTQ_ERR_INVALID_ARG        # y overlaps codes
    assert call(name, A, B, B - 16, n, d, g) == rtq.RTQ_ERR_INVALID_ARG         # y overlaps scales


ATTN = ["srft_attn_decode", "srht_attn_decode"]
Q, K, S_, O = 0x10000, 0x2000000, 0x6000000, 0x8000000  # q, codes, scales, out (never dereferenced)


WS = 0xA000000  # workspace (never dereferenced)


def attn_call(name, q=Q, codes=K, scales=S_, out=O, layers=2, streams=3, tokens=50, qpk=4, d=128, g=32,
              strides=(300, 150, 50, 1), seed=1, rps=0, per=0, softmax_scale=0.125, ws=0, ws_bytes=0):
    fn = getattr(rtq.library(), name)
    return fn(ctypes.c_void_p(q), ctypes.c_void_p(codes), ctypes.c_void_p(scales), ctypes.c_void_p(out),
              layers, streams, tokens, qpk, d, g, *strides, seed, rps, per, ctypes.c_float(softmax_scale),
              ctypes.c_void_p(ws), ws_bytes, None)


@pytest.mark.parametrize("name", ATTN)
def test_attention_rejects_bad_arguments_without_launching(name):
    bad = rtq.RTQ_ERR_INVALID_ARG
    assert attn_call(name, layers=-1) == bad
    assert attn_call(name, streams=-1) == bad
    assert attn_call(name, tokens=0) == bad
    assert attn_call(name, qpk=0) == bad
    assert attn_call(name, rps=-1) == bad
    assert attn_call(name, per=-1) == bad
    assert attn_call(name, strides=(300, 150, 50, -1)) == bad
    assert attn_call(name, softmax_scale=float("nan")) == bad
    assert attn_call(name, softmax_scale=float("inf")) == bad
    assert attn_call(name, layers=70000, streams=40000, strides=(0, 150, 50, 1)) == bad
    for kw in ({"q": 0}, {"codes": 0}, {"scales": 0}, {"out": 0}, {"q": Q + 8}, {"codes": K + 4},
               {"scales": S_ + 2}, {"out": O + 8}):
        assert attn_call(name, **kw) == bad, kw
    # rows past 2^56
    assert attn_call(name, strides=(1 << 60, 150, 50, 1)) == bad
    # unsupported shapes and head ratios
    for d, g in [(256, 512), (64, 128), (128, 16), (96, 32), (512, 32)]:
        assert attn_call(name, d=d, g=g) == rtq.RTQ_ERR_UNSUPPORTED, (d, g)
    assert attn_call(name, qpk=9) == rtq.RTQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ATTN)
def test_attention_requires_one_seed_per_key_and_value_sequence(name):
    bad = rtq.RTQ_ERR_INVALID_ARG
    L, S, T = 2, 3, 50
    lm = (2 * S * T, S * T, T, 1)
    tm = (2 * S, S, 1, 2 * L * S)
    assert attn_call(name, strides=lm, rps=1) == bad              # a seed per row
    assert attn_call(name, strides=lm, rps=T + 1) == bad          # blocks cut through the token sequences
    assert attn_call(name, strides=tm, rps=2 * S, per=2 * L) == bad   # time-major, period of two layers
    assert attn_call(name, strides=tm, rps=1, per=0) == bad


@pytest.mark.parametrize("name", ATTN)
def test_attention_empty_grid_is_a_no_op(name):
    assert attn_call(name, q=0, codes=0, scales=0, out=0, layers=0) == rtq.RTQ_OK
    assert attn_call(name, q=0, codes=0, scales=0, out=0, streams=0) == rtq.RTQ_OK


@pytest.mark.parametrize("name", ATTN)
def test_attention_rejects_overlapping_output(name):
    # q and out: 2*3*4*128*2 = 6144 B; codes reach row 299 (19200 B); scales 2400 B
    assert attn_call(name, out=Q + 4096) == rtq.RTQ_ERR_INVALID_ARG
    assert attn_call(name, out=K + 16384) == rtq.RTQ_ERR_INVALID_ARG
    assert attn_call(name, out=S_ - 4096) == rtq.RTQ_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ATTN)
def test_attention_rejects_bad_workspaces(name):
    bad = rtq.RTQ_ERR_INVALID_ARG
    assert attn_call(name, ws=WS, ws_bytes=0) == bad          # pointer without a size
    assert attn_call(name, ws=0, ws_bytes=4096) == bad        # size without a pointer
    assert attn_call(name, ws=WS + 8, ws_bytes=4096) == bad   # misaligned
    assert attn_call(name, ws=Q - 1024, ws_bytes=4096) == bad   # overlaps q
    assert attn_call(name, ws=O + 16, ws_bytes=4096) == bad     # overlaps out
    assert attn_call(name, ws=K + 4096, ws_bytes=4096) == bad   # overlaps the codes
    assert attn_call(name, ws=S_ - 16, ws_bytes=64) == bad      # overlaps the scales
    assert attn_call(name, q=0, codes=0, scales=0, out=0, layers=0, ws=WS, ws_bytes=4096) == rtq.RTQ_OK


def test_attention_workspace_size_query():
    f = rtq.attn_workspace_bytes
    # many (layer, stream) pairs or short streams: no split, no workspace
    assert f(28, 64, 2048, 6, 128) == 0
    assert f(1, 1, 255, 1, 64) == 0
    # invalid sizes
    for args in [(0, 1, 4096, 1, 64), (1, 0, 4096, 1, 64), (1, 1, 0, 1, 64), (1, 1, 4096, 0, 64),
                 (1, 1, 4096, 9, 64), (1, 1, 4096, 1, 0), (-1, 1, 4096, 1, 64)]:
        assert f(*args) == 0, args
    # few pairs, long streams: counters (256-byte block) + pairs * splits partials
    # of q_per_kv * (d + 2) floats rounded up to 4
    pairs, qpk, d = 160, 3, 64
    splits = 3  # 512 // 160 resident workgroups, below 4096 tokens / (32 * 8)
    assert f(32, 5, 4096, qpk, d) == 768 + pairs * splits * 200 * 4
    assert f(1, 1, 1 << 20, 8, 128) == 256 + 64 * (8 * 130) * 4  # capped at 64 splits
    assert f(1, 1, 2048, 8, 128) == 256 + 8 * (8 * 130) * 4       # 2048 tokens / (32 * 8)
    assert f(16, 16, 4096, 1, 64) == 1024 + 256 * 2 * 68 * 4     # 256 pairs: two per CU
    assert f(16, 17, 4096, 1, 64) == 0                            # 272 pairs: splitting needs a second round


WIN = 0xC000000  # window (never dereferenced)


def win_call(name, tokens=50, win=WIN, cap=16, wt=16, out=O, layers=2, streams=3, qpk=4, d=128, g=32):
    fn = getattr(rtq.library(), name + "_window")
    return fn(ctypes.c_void_p(Q), ctypes.c_void_p(K), ctypes.c_void_p(S_), ctypes.c_void_p(out), layers, streams,
              tokens, qpk, d, g, 300, 150, 50, 1, 1, 0, 0, ctypes.c_float(0.125), ctypes.c_void_p(win), cap, wt,
              ctypes.c_void_p(0), 0, None)


@pytest.mark.parametrize("name", ATTN)
def test_attention_window_rejects_bad_arguments(name):
    bad = rtq.RTQ_ERR_INVALID_ARG
    assert win_call(name, win=0, wt=4) == bad                 # window tokens without a window
    assert win_call(name, win=WIN + 8) == bad                 # misaligned window
    assert win_call(name, cap=8, wt=9) == bad                 # more tokens than slots
    assert win_call(name, wt=-1) == bad
    assert win_call(name, cap=-1, wt=0) == bad
    assert win_call(name, tokens=0, wt=0) == bad              # no token at all
    assert win_call(name, out=WIN + 4096) == bad              # out inside the window
    assert win_call(name, cap=65, wt=65) == rtq.RTQ_ERR_UNSUPPORTED
    assert win_call(name, d=96) == rtq.RTQ_ERR_UNSUPPORTED
    assert win_call(name, layers=0) == rtq.RTQ_OK


def test_decode_cache_rejects_windows_the_attention_cannot_read():
    """A DecodeCache whose window exceeds what *_attn_decode_window accepts
    fails at construction, not at its 65th append."""
    from rotate_then_quantize_amd.decode_cache import DecodeCache
    lim = rtq.ATTN_MAX_WINDOW
    assert win_call("srft_attn_decode", cap=lim + 1, wt=lim + 1) == rtq.RTQ_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        DecodeCache(1, 1, 256, 64, 32, 1, window=lim + 1, device="cpu")
    cache = DecodeCache(1, 1, 256, 64, 32, 1, window=lim, device="cpu")
    assert cache.window_kv.shape[3] == lim


MAPPED = ["srft_quant_append", "srht_quant_append", "srft_dequant_rows", "srht_dequant_rows"]


def mapped_call(name, a=A, b=B, c=C, layers=2, streams=3, t0=5, n=4, d=128, g=32, strides=(300, 150, 50, 1),
                seed=1, rps=0, per=0):
    fn = getattr(rtq.library(), name)
    return fn(ctypes.c_void_p(a), ctypes.c_void_p(b), ctypes.c_void_p(c), layers, streams, t0, n, d, g, *strides,
              seed, rps, per, None)


@pytest.mark.parametrize("name", MAPPED)
def test_mapped_rejects_bad_arguments_without_launching(name):
    bad = rtq.RTQ_ERR_INVALID_ARG
    for kw in ({"layers": -1}, {"streams": -1}, {"t0": -1}, {"n": -1}, {"rps": -1}, {"per": -1},
               {"strides": (300, 150, -50, 1)}, {"a": 0}, {"b": 0}, {"c": 0}, {"a": A + 8}, {"b": B + 4},
               {"c": C + 2}, {"strides": (1 << 60, 150, 50, 1)}, {"layers": 1 << 20, "streams": 1 << 10, "n": 1 << 10}):
        assert mapped_call(name, **kw) == bad, kw
    for d, g in [(256, 512), (96, 32), (64, 128), (128, 16)]:
        assert mapped_call(name, d=d, g=g) == rtq.RTQ_ERR_UNSUPPORTED, (d, g)


@pytest.mark.parametrize("name", MAPPED)
def test_mapped_empty_block_is_a_no_op(name):
    assert mapped_call(name, a=0, b=0, c=0, n=0) == rtq.RTQ_OK
    assert mapped_call(name, a=0, b=0, c=0, layers=0) == rtq.RTQ_OK


def test_mapped_rejects_overlapping_buffers():
    # block rows reach row 299 + 5 + 3 = ... ; codes 64 B/row, scales 8 B/row, x 256 B/row
    assert mapped_call("srft_quant_append", a=A, b=A + 1024) == rtq.RTQ_ERR_INVALID_ARG       # codes inside x
    assert mapped_call("srft_dequant_rows", a=A, b=B, c=A + 4096) == rtq.RTQ_ERR_INVALID_ARG  # y overlaps codes
    assert mapped_call("srft_dequant_rows", a=A, b=B, c=B - 64) == rtq.RTQ_ERR_INVALID_ARG    # y overlaps scales


EXT = ["srft_quant_fwd_ext", "srht_quant_fwd_ext", "srft_dequant_inv_ext", "srht_dequant_inv_ext"]
LAM = 0x9000000


def ext_call(name, a=A, b=B, c=C, n=10, d=64, g=32, bits=3, lam=0, seed=1, rps=0, per=0):
    fn = getattr(rtq.library(), name)
    return fn(ctypes.c_void_p(a), ctypes.c_void_p(b), ctypes.c_void_p(c), n, d, g, bits, ctypes.c_void_p(lam), seed,
              rps, per, None)


@pytest.mark.parametrize("name", EXT)
def test_ext_rejects_bad_arguments_without_launching(name):
    bad = rtq.RTQ_ERR_INVALID_ARG
    for kw in ({"n": -1}, {"rps": -1}, {"per": -1}, {"a": 0}, {"b": 0}, {"c": 0}, {"a": A + 8}, {"b": B + 4},
               {"c": C + 2}, {"lam": LAM + 2}, {"n": 0xFFFFFF01}):
        assert ext_call(name, **kw) == bad, kw
    for kw in ({"bits": 2}, {"bits": 5}, {"bits": 16}, {"d": 256, "g": 512}, {"d": 96}, {"g": 16}):
        assert ext_call(name, **kw) == rtq.RTQ_ERR_UNSUPPORTED, kw


@pytest.mark.parametrize("name", EXT)
def test_ext_zero_rows_is_a_no_op(name):
    assert ext_call(name, a=0, b=0, c=0, n=0) == rtq.RTQ_OK


def test_ext_rejects_overlapping_buffers():
    # n = 100, d = 64, 6 bits: x 12800 B, codes 4800 B, scales 400 B
    assert ext_call("srft_quant_fwd_ext", n=100, bits=6, b=A + 1024) == rtq.RTQ_ERR_INVALID_ARG    # codes in x
    assert ext_call("srft_quant_fwd_ext", n=100, bits=6, lam=B + 4784) == rtq.RTQ_ERR_INVALID_ARG   # lambda on codes
    assert ext_call("srft_dequant_inv_ext", n=100, bits=6, c=A + 4096) == rtq.RTQ_ERR_INVALID_ARG  # y on codes


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        rtq.srft_quant_fwd(x, 32, 1)
    with pytest.raises(TypeError):
        rtq.srft_quant_fwd(x.float(), 32, 1)


def test_binding_raises_when_library_missing(monkeypatch, tmp_path):
    """No fallback: with the shared library absent every entry point raises."""
    monkeypatch.setattr(rtq, "_LIB_PATH", str(tmp_path / "missing" / "librtq.so"))
    monkeypatch.setattr(rtq, "_lib", None)
    with pytest.raises(rtq.RTQError):
        rtq.library()
