"""rotate_then_quantize_amd -- fused rotate-then-quantize int4 K/V kernels for MI355X.

A thin binding over ``librtq.so`` (C ABI in ``include/rtq.h``).  It only checks
and marshals arguments: every step of the method runs in the HIP kernels.
PyTorch provides the device memory and the current stream.  There is no CPU
fallback: if the library is missing, every call raises.

    codes, scales = srft_quant_fwd(x, group, seed)        # x: [n, d] fp16 on the GPU
    y = srft_dequant_inv(codes, scales, d, group, seed)   # y: [n, d] fp16

The method ("Quantization Speed Is Often a Kernel Problem", sections "First,
the 17%" and "Fusing four steps into two kernels is not enough"): rotate each
K/V vector (SRFT, or the SRHT control), quantize it to int4 with one absmax
fp16 scale per group, and undo both when it is read back.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "srft_quant_fwd", "srft_dequant_inv", "srht_quant_fwd", "srht_dequant_inv",
    "srft_attn_decode", "srht_attn_decode", "srft_attn_decode_noalloc", "attn_workspace_bytes",
    "srft_quant_append", "srht_quant_append", "srft_dequant_rows", "srht_dequant_rows",
    "srft_quant_fwd_ext", "srht_quant_fwd_ext", "srft_dequant_inv_ext", "srht_dequant_inv_ext", "CODE_BITS",
    "RTQError", "library", "library_path", "ATTN_MAX_WINDOW", "SUPPORTED", "ATTN_SUPPORTED", "CACHE_SUPPORTED", "EXT_SUPPORTED",
]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG_DIR, "librtq.so")
_lib = None

RTQ_OK, RTQ_ERR_INVALID_ARG, RTQ_ERR_UNSUPPORTED, RTQ_ERR_HIP = 0, 1, 2, 3
# (d, group) pairs the library is built for
SUPPORTED = {(64, 32), (64, 64), (128, 32), (128, 64), (128, 128), (256, 32), (256, 64), (256, 128), (256, 256)}
# (d, group) pairs of the decode-attention kernels; at most 8 query heads per K/V head
ATTN_SUPPORTED = {(64, 32), (64, 64), (128, 32), (128, 64), (128, 128), (256, 32), (256, 64), (256, 128), (256, 256)}
# (d, group) pairs of the cache-layout entry points (*_quant_append, *_dequant_rows) and of the
# code-width / lambda entry points (*_ext)
CACHE_SUPPORTED = {(64, 32), (64, 64), (128, 32), (128, 64), (128, 128), (256, 32), (256, 64), (256, 128), (256, 256)}
EXT_SUPPORTED = {(64, 32), (64, 64), (128, 32), (128, 64), (128, 128), (256, 32), (256, 64), (256, 128), (256, 256)}
ATTN_MAX_Q_PER_KV = 8
# fp16 window tokens per stream that *_attn_decode_window accepts
ATTN_MAX_WINDOW = 64
# code widths of the *_ext entry points
CODE_BITS = (3, 4, 6, 8)


class RTQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def library():
    """The loaded ctypes handle of librtq.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RTQError(-1, f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                               "or python -m rotate_then_quantize_amd._build")
        lib = ctypes.CDLL(_LIB_PATH)
        fwd_args = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                    ctypes.c_int32, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
        for name in ("srft_quant_fwd", "srft_dequant_inv", "srht_quant_fwd", "srht_dequant_inv"):
            fn = getattr(lib, name)
            fn.argtypes = fwd_args
            fn.restype = ctypes.c_int
        attn_args = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                     ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                     ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                     ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p,
                     ctypes.c_size_t, ctypes.c_void_p]
        for name in ("srft_attn_decode", "srht_attn_decode"):
            fn = getattr(lib, name)
            fn.argtypes = attn_args
            fn.restype = ctypes.c_int
        win_args = attn_args[:18] + [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32] + attn_args[18:]
        for name in ("srft_attn_decode_window", "srht_attn_decode_window"):
            fn = getattr(lib, name)
            fn.argtypes = win_args
            fn.restype = ctypes.c_int
        lib.srft_attn_decode_noalloc.argtypes = attn_args[:18] + [ctypes.c_void_p]
        lib.srft_attn_decode_noalloc.restype = ctypes.c_int
        lib.rtq_attn_workspace_bytes.argtypes = [ctypes.c_int32] * 5
        lib.rtq_attn_workspace_bytes.restype = ctypes.c_size_t
        mapped_args = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                       ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
        for name in ("srft_quant_append", "srht_quant_append", "srft_dequant_rows", "srht_dequant_rows"):
            fn = getattr(lib, name)
            fn.argtypes = mapped_args
            fn.restype = ctypes.c_int
        ext_args = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                    ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                    ctypes.c_void_p]
        for name in ("srft_quant_fwd_ext", "srht_quant_fwd_ext", "srft_dequant_inv_ext", "srht_dequant_inv_ext"):
            fn = getattr(lib, name)
            fn.argtypes = ext_args
            fn.restype = ctypes.c_int
        lib.rtq_status_string.argtypes = [ctypes.c_int]
        lib.rtq_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _check(status: int) -> None:
    if status != RTQ_OK:
        msg = library().rtq_status_string(status).decode()
        raise RTQError(status, msg)


def _stream_handle(t, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, name, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _fwd(cname, x, group, seed, rows_per_seed, seed_period, codes, scales, stream):
    import torch
    _need(x, torch.float16, "x")
    if x.dim() != 2:
        raise ValueError("x must be [n, d]")
    n, d = x.shape
    if d % group or group <= 0:
        raise ValueError("group must divide d")
    if codes is None:
        codes = torch.empty((n, d // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((n, d // group), dtype=torch.float16, device=x.device)
    _need(codes, torch.uint8, "codes", (n, d // 2))
    _need(scales, torch.float16, "scales", (n, d // group))
    _check(getattr(library(), cname)(
        ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
        n, d, group, seed & ((1 << 64) - 1), rows_per_seed, seed_period, _stream_handle(x, stream)))
    return codes, scales


def _inv(cname, codes, scales, d, group, seed, rows_per_seed, seed_period, out, stream):
    import torch
    _need(codes, torch.uint8, "codes")
    if codes.dim() != 2 or codes.shape[1] * 2 != d:
        raise ValueError("codes must be [n, d/2]")
    n = codes.shape[0]
    if d % group or group <= 0:
        raise ValueError("group must divide d")
    _need(scales, torch.float16, "scales", (n, d // group))
    if out is None:
        out = torch.empty((n, d), dtype=torch.float16, device=codes.device)
    _need(out, torch.float16, "out", (n, d))
    _check(getattr(library(), cname)(
        ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(out.data_ptr()),
        n, d, group, seed & ((1 << 64) - 1), rows_per_seed, seed_period, _stream_handle(codes, stream)))
    return out


def srft_quant_fwd(x, group, seed, rows_per_seed=0, seed_period=0, codes=None, scales=None, stream=None):
    """Forward step with the SRFT rotation: returns (codes [n, d/2] uint8, scales [n, d/group] fp16)."""
    return _fwd("srft_quant_fwd", x, group, seed, rows_per_seed, seed_period, codes, scales, stream)


def srft_dequant_inv(codes, scales, d, group, seed, rows_per_seed=0, seed_period=0, out=None, stream=None):
    """Inverse step with the SRFT rotation: returns y [n, d] fp16."""
    return _inv("srft_dequant_inv", codes, scales, d, group, seed, rows_per_seed, seed_period, out, stream)


def srht_quant_fwd(x, group, seed, rows_per_seed=0, seed_period=0, codes=None, scales=None, stream=None):
    """Forward step with the SRHT (Walsh-Hadamard) control rotation."""
    return _fwd("srht_quant_fwd", x, group, seed, rows_per_seed, seed_period, codes, scales, stream)


def srht_dequant_inv(codes, scales, d, group, seed, rows_per_seed=0, seed_period=0, out=None, stream=None):
    """Inverse step with the SRHT (Walsh-Hadamard) control rotation."""
    return _inv("srht_dequant_inv", codes, scales, d, group, seed, rows_per_seed, seed_period, out, stream)


def attn_workspace_bytes(layers: int, streams: int, tokens: int, q_per_kv: int, d: int) -> int:
    """Bytes of workspace that let *_attn_decode split every stream's tokens as far as it would (0: no split)."""
    return int(library().rtq_attn_workspace_bytes(layers, streams, tokens, q_per_kv, d))


# Zero-filled attention workspaces kept per (device, stream): every completed
# call leaves its workspace zeroed again, and calls on one stream never overlap.
_workspaces = {}


def _attn_workspace(q, tokens, stream_handle):
    import torch
    layers, streams, q_per_kv, d = q.shape
    need = attn_workspace_bytes(layers, streams, tokens, q_per_kv, d)
    if need == 0:
        return None
    key = (q.device.index, stream_handle.value)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(need, dtype=torch.uint8, device=q.device)
        _workspaces[key] = ws
    return ws


def _attn(cname, q, codes, scales, strides, tokens, group, seed, rows_per_seed, seed_period, softmax_scale,
          out, stream, workspace=None, window=None, window_tokens=0, noalloc=False):
    import math
    import torch
    _need(q, torch.float16, "q")
    if q.dim() != 4:
        raise ValueError("q must be [layers, streams, q_per_kv, d]")
    layers, streams, q_per_kv, d = q.shape
    _need(codes, torch.uint8, "codes")
    if codes.dim() != 2 or codes.shape[1] * 2 != d:
        raise ValueError("codes must be [n, d/2]")
    if d % group or group <= 0:
        raise ValueError("group must divide d")
    _need(scales, torch.float16, "scales", (codes.shape[0], d // group))
    strides = tuple(int(v) for v in strides)
    if len(strides) != 4 or min(strides) < 0:
        raise ValueError("strides must be four non-negative row counts (layer, kv, stream, token)")
    if window is not None:
        _need(window, torch.float16, "window")
        if window.dim() != 5 or tuple(window.shape[:3]) != (layers, 2, streams) or window.shape[4] != d:
            raise ValueError(f"window must be [{layers}, 2, {streams}, capacity, {d}]")
        if not 0 <= window_tokens <= window.shape[3]:
            raise ValueError("window_tokens must lie in 0 .. window capacity")
    elif window_tokens:
        raise ValueError("window_tokens without a window")
    if tokens < (0 if window_tokens else 1):
        raise ValueError("tokens must be at least 1 (or 0 with a non-empty window)")
    if layers and streams and tokens:
        max_row = (layers - 1) * strides[0] + strides[1] + (streams - 1) * strides[2] + (tokens - 1) * strides[3]
        if max_row >= codes.shape[0]:
            raise ValueError(f"the cache has {codes.shape[0]} rows; the strides reach row {max_row}")
    if out is None:
        out = torch.empty_like(q)
    _need(out, torch.float16, "out", tuple(q.shape))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    sh = _stream_handle(q, stream)
    if noalloc:  # the library's static scratch holds the split partials
        args = [ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                ctypes.c_void_p(out.data_ptr()), layers, streams, tokens, q_per_kv, d, group, *strides,
                seed & ((1 << 64) - 1), rows_per_seed, seed_period, float(softmax_scale)]
        _check(library().srft_attn_decode_noalloc(*args, sh))
        return out
    if workspace is None:
        workspace = _attn_workspace(q, tokens, sh)
    if workspace is None or workspace.numel() == 0:
        ws_ptr, ws_bytes = None, 0
    else:
        _need(workspace, torch.uint8, "workspace")
        ws_ptr, ws_bytes = ctypes.c_void_p(workspace.data_ptr()), workspace.numel()
    args = [ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
            ctypes.c_void_p(out.data_ptr()), layers, streams, tokens, q_per_kv, d, group, *strides,
            seed & ((1 << 64) - 1), rows_per_seed, seed_period, float(softmax_scale)]
    if window is not None:
        args += [ctypes.c_void_p(window.data_ptr()), window.shape[3], window_tokens]
        cname += "_window"
    _check(getattr(library(), cname)(*args, ws_ptr, ws_bytes, sh))
    return out


def srft_attn_decode(q, codes, scales, strides, tokens, group, seed, rows_per_seed=0, seed_period=0,
                     softmax_scale=None, out=None, stream=None, workspace=None, window=None, window_tokens=0):
    """One decode step of attention over an SRFT int4 cache: q [layers, streams, q_per_kv, d] fp16
    attends over tokens 0..tokens-1 of its stream, whose key / value row is
    layer*strides[0] + kv*strides[1] + stream*strides[2] + token*strides[3] (kv 0 = K, 1 = V).
    Returns o like q (fp16); softmax_scale defaults to 1/sqrt(d).
    workspace: None = a zero-filled workspace kept per (device, stream), which lets the kernel split each
    stream's tokens over several workgroups when there are few streams; a uint8 tensor = that memory
    (zero-filled before its first use, see attn_workspace_bytes); an empty tensor = no split.
    window: an fp16 [layers, 2, streams, capacity, d] window of the newest tokens (unquantized, original
    domain) whose first window_tokens tokens join the softmax after the `tokens` int4 tokens; tokens may
    then be 0."""
    return _attn("srft_attn_decode", q, codes, scales, strides, tokens, group, seed, rows_per_seed, seed_period,
                 softmax_scale, out, stream, workspace, window, window_tokens)


def srft_attn_decode_noalloc(q, codes, scales, strides, tokens, group, seed, rows_per_seed=0, seed_period=0,
                             softmax_scale=None, out=None, stream=None):
    """srft_attn_decode whose token-split partials live in the library's static device scratch: the
    library allocates nothing (pass `out` to allocate nothing here either).  Calls that may overlap in
    time on one GPU share the scratch and race."""
    return _attn("srft_attn_decode_noalloc", q, codes, scales, strides, tokens, group, seed, rows_per_seed,
                 seed_period, softmax_scale, out, stream, noalloc=True)


def srht_attn_decode(q, codes, scales, strides, tokens, group, seed, rows_per_seed=0, seed_period=0,
                     softmax_scale=None, out=None, stream=None, workspace=None, window=None, window_tokens=0):
    """srft_attn_decode over an SRHT (Walsh-Hadamard) int4 cache."""
    return _attn("srht_attn_decode", q, codes, scales, strides, tokens, group, seed, rows_per_seed, seed_period,
                 softmax_scale, out, stream, workspace, window, window_tokens)


def attn_decode(rot, *args, **kw):
    return (srft_attn_decode if rot == "srft" else srht_attn_decode)(*args, **kw)


def _check_block(codes, scales, d, group, strides, layers, streams, t0, n_tokens):
    import torch
    _need(codes, torch.uint8, "codes")
    if codes.dim() != 2 or codes.shape[1] * 2 != d:
        raise ValueError("codes must be [rows, d/2]")
    if d % group or group <= 0:
        raise ValueError("group must divide d")
    _need(scales, torch.float16, "scales", (codes.shape[0], d // group))
    strides = tuple(int(v) for v in strides)
    if len(strides) != 4 or min(strides) < 0:
        raise ValueError("strides must be four non-negative row counts (layer, kv, stream, token)")
    if t0 < 0 or n_tokens < 0:
        raise ValueError("t0 and n_tokens must be non-negative")
    if layers and streams and n_tokens:
        max_row = (layers - 1) * strides[0] + strides[1] + (streams - 1) * strides[2] + (t0 + n_tokens - 1) * strides[3]
        if max_row >= codes.shape[0]:
            raise ValueError(f"the cache has {codes.shape[0]} rows; the strides reach row {max_row}")
    return strides


def _append(cname, x, codes, scales, strides, t0, group, seed, rows_per_seed, seed_period, stream):
    import torch
    _need(x, torch.float16, "x")
    if x.dim() != 5 or x.shape[1] != 2:
        raise ValueError("x must be [layers, 2, streams, n_tokens, d]")
    layers, _, streams, n_tokens, d = x.shape
    strides = _check_block(codes, scales, d, group, strides, layers, streams, t0, n_tokens)
    _check(getattr(library(), cname)(
        ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
        layers, streams, t0, n_tokens, d, group, *strides, seed & ((1 << 64) - 1), rows_per_seed, seed_period,
        _stream_handle(x, stream)))


def _rows(cname, codes, scales, y, layers, streams, t0, n_tokens, strides, group, seed, rows_per_seed,
          seed_period, stream):
    import torch
    d = codes.shape[1] * 2 if codes.dim() == 2 else 0
    strides = _check_block(codes, scales, d, group, strides, layers, streams, t0, n_tokens)
    _need(y, torch.float16, "y", (codes.shape[0], d))
    _check(getattr(library(), cname)(
        ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(y.data_ptr()),
        layers, streams, t0, n_tokens, d, group, *strides, seed & ((1 << 64) - 1), rows_per_seed, seed_period,
        _stream_handle(codes, stream)))
    return y


def srft_quant_append(x, codes, scales, strides, t0, group, seed, rows_per_seed=0, seed_period=0, stream=None):
    """Quantize x [layers, 2, streams, n_tokens, d] (fp16; axis 1 = K, V) into the cache rows of tokens
    t0 .. t0+n_tokens-1 (row = layer*s0 + kv*s1 + stream*s2 + token*s3), in place."""
    _append("srft_quant_append", x, codes, scales, strides, t0, group, seed, rows_per_seed, seed_period, stream)


def srht_quant_append(x, codes, scales, strides, t0, group, seed, rows_per_seed=0, seed_period=0, stream=None):
    """srft_quant_append with the SRHT rotation."""
    _append("srht_quant_append", x, codes, scales, strides, t0, group, seed, rows_per_seed, seed_period, stream)


def srft_dequant_rows(codes, scales, y, layers, streams, t0, n_tokens, strides, group, seed, rows_per_seed=0,
                      seed_period=0, stream=None):
    """Dequantize the cache rows of tokens t0 .. t0+n_tokens-1 of every (layer, kv, stream) into the same
    rows of y (an fp16 [rows, d] copy of the cache); other rows of y are left as they are."""
    return _rows("srft_dequant_rows", codes, scales, y, layers, streams, t0, n_tokens, strides, group, seed,
                 rows_per_seed, seed_period, stream)


def srht_dequant_rows(codes, scales, y, layers, streams, t0, n_tokens, strides, group, seed, rows_per_seed=0,
                      seed_period=0, stream=None):
    """srft_dequant_rows with the SRHT rotation."""
    return _rows("srht_dequant_rows", codes, scales, y, layers, streams, t0, n_tokens, strides, group, seed,
                 rows_per_seed, seed_period, stream)


def _lambda_ptr(lam, d, device):
    import torch
    if lam is None:
        return ctypes.c_void_p(0)
    _need(lam, torch.float16, "lam", (d,))
    if lam.device != device:
        raise ValueError("lam must be on the same device as the data")
    return ctypes.c_void_p(lam.data_ptr())


def _fwd_ext(cname, x, group, bits, lam, seed, rows_per_seed, seed_period, codes, scales, stream):
    import torch
    _need(x, torch.float16, "x")
    if x.dim() != 2:
        raise ValueError("x must be [n, d]")
    n, d = x.shape
    if d % group or group <= 0:
        raise ValueError("group must divide d")
    if bits not in CODE_BITS:
        raise ValueError(f"bits must be one of {CODE_BITS}")
    if codes is None:
        codes = torch.empty((n, d * bits // 8), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((n, d // group), dtype=torch.float16, device=x.device)
    _need(codes, torch.uint8, "codes", (n, d * bits // 8))
    _need(scales, torch.float16, "scales", (n, d // group))
    _check(getattr(library(), cname)(
        ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
        n, d, group, bits, _lambda_ptr(lam, d, x.device), seed & ((1 << 64) - 1), rows_per_seed, seed_period,
        _stream_handle(x, stream)))
    return codes, scales


def _inv_ext(cname, codes, scales, d, group, bits, lam, seed, rows_per_seed, seed_period, out, stream):
    import torch
    if bits not in CODE_BITS:
        raise ValueError(f"bits must be one of {CODE_BITS}")
    _need(codes, torch.uint8, "codes")
    if codes.dim() != 2 or codes.shape[1] * 8 != d * bits:
        raise ValueError("codes must be [n, d*bits/8]")
    n = codes.shape[0]
    if d % group or group <= 0:
        raise ValueError("group must divide d")
    _need(scales, torch.float16, "scales", (n, d // group))
    if out is None:
        out = torch.empty((n, d), dtype=torch.float16, device=codes.device)
    _need(out, torch.float16, "out", (n, d))
    _check(getattr(library(), cname)(
        ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(out.data_ptr()),
        n, d, group, bits, _lambda_ptr(lam, d, codes.device), seed & ((1 << 64) - 1), rows_per_seed, seed_period,
        _stream_handle(codes, stream)))
    return out


def srft_quant_fwd_ext(x, group, bits, seed, lam=None, rows_per_seed=0, seed_period=0, codes=None, scales=None,
                       stream=None):
    """Forward step with `bits`-bit codes (3, 4, 6, 8) and an optional per-channel fp16 lambda [d]:
    returns (codes [n, d*bits/8] uint8, scales [n, d/group] fp16)."""
    return _fwd_ext("srft_quant_fwd_ext", x, group, bits, lam, seed, rows_per_seed, seed_period, codes, scales,
                    stream)


def srht_quant_fwd_ext(x, group, bits, seed, lam=None, rows_per_seed=0, seed_period=0, codes=None, scales=None,
                       stream=None):
    """srft_quant_fwd_ext with the SRHT rotation."""
    return _fwd_ext("srht_quant_fwd_ext", x, group, bits, lam, seed, rows_per_seed, seed_period, codes, scales,
                    stream)


def srft_dequant_inv_ext(codes, scales, d, group, bits, seed, lam=None, rows_per_seed=0, seed_period=0, out=None,
                         stream=None):
    """Inverse step for `bits`-bit codes and an optional lambda: returns y [n, d] fp16."""
    return _inv_ext("srft_dequant_inv_ext", codes, scales, d, group, bits, lam, seed, rows_per_seed, seed_period,
                    out, stream)


def srht_dequant_inv_ext(codes, scales, d, group, bits, seed, lam=None, rows_per_seed=0, seed_period=0, out=None,
                         stream=None):
    """srft_dequant_inv_ext with the SRHT rotation."""
    return _inv_ext("srht_dequant_inv_ext", codes, scales, d, group, bits, lam, seed, rows_per_seed, seed_period,
                    out, stream)


def quant_fwd_ext(rot, *args, **kw):
    return (srft_quant_fwd_ext if rot == "srft" else srht_quant_fwd_ext)(*args, **kw)


def dequant_inv_ext(rot, *args, **kw):
    return (srft_dequant_inv_ext if rot == "srft" else srht_dequant_inv_ext)(*args, **kw)


def quant_append(rot, *args, **kw):
    return (srft_quant_append if rot == "srft" else srht_quant_append)(*args, **kw)


def dequant_rows(rot, *args, **kw):
    return (srft_dequant_rows if rot == "srft" else srht_dequant_rows)(*args, **kw)


def quant_fwd(rot, *args, **kw):
    return (srft_quant_fwd if rot == "srft" else srht_quant_fwd)(*args, **kw)


def dequant_inv(rot, *args, **kw):
    return (srft_dequant_inv if rot == "srft" else srht_dequant_inv)(*args, **kw)
