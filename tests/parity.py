"""Element-by-element comparison of the HIP path with the oracle.

Tolerances (the reading of the stated bar):
  * scales: bit-exact, except a 1-ulp fp16 difference in a group whose exact
    absmax/8 lies within 1e-6 (relative) of an fp16 rounding midpoint; such a
    group's codes are then checked against the oracle re-run with the GPU's
    scale.
  * codes: bit-exact, except elements whose oracle z/s lies within 1e-4 of
    k + 1/2, which may differ by +-1; at most 1e-5 of all elements may differ.
    The rate is asserted over a dedicated sample of 4 M codes per rotation
    (test_code_tie_rate_on_its_own_sample) and over every element compared in
    the session (TALLY, checked when the session ends); a single call may
    exceed it by at most two
    elements, since exact ties (SRHT of fp16 inputs gives dyadic values, about
    3.5e-6 of elements) make small inputs too noisy to resolve a 1e-5 rate.
    ``allow_ties`` lifts the count for inputs built to sit on ties.
  * outputs: the inverse is run on the same codes and scales on both sides;
    |y_gpu - y_oracle| <= max(2e-3 * s_row, 1 ulp of fp16 at y_oracle), where
    s_row is the largest scale of the row (fp16 output rounding can move a
    large value by one ulp, which exceeds 2e-3 * s on outlier channels).
"""
from __future__ import annotations

import numpy as np

import oracle


# (mismatching codes, compared codes) over the session, for the 1e-5 rate
TALLY = {"mismatch": 0, "elements": 0}


def fp16_ulp(v):
    v = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def near_fp16_midpoint(v, rel=1e-6):
    """True where v is within ``rel`` of a point where fp16 rounding changes."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        lo = (v * (1 - rel)).astype(np.float16)
        hi = (v * (1 + rel)).astype(np.float16)
    return lo.view(np.uint16) != hi.view(np.uint16)


def check_forward(x16, codes_gpu, scales_gpu, group, seed, rps=0, period=0, rot="srft", row0=0,
                  allow_ties=False, detail=None, rows=None):
    """Assert the GPU forward output matches the oracle; return mismatch stats."""
    x16 = np.asarray(x16, dtype=np.float16)
    n, d = x16.shape
    det = detail or oracle.forward_detail(x16, group, seed, rps, period, rot, row0, rows)
    s_orc = det["s"]
    s_gpu = np.asarray(scales_gpu, dtype=np.float16).reshape(s_orc.shape)
    diff = s_gpu.view(np.uint16) != s_orc.view(np.uint16)
    ulp_apart = np.abs(s_gpu.astype(np.float64) - s_orc.astype(np.float64)) <= fp16_ulp(s_orc) * (1 + 1e-9)
    amb = near_fp16_midpoint(det["a"] / 8.0)
    bad = diff & ~(amb & ulp_apart)
    if bad.any():
        r, j = np.argwhere(bad)[0]
        raise AssertionError(f"scale mismatch row {r} group {j}: gpu {s_gpu[r, j]!r} oracle {s_orc[r, j]!r} "
                             f"(absmax/8 = {det['a'][r, j] / 8!r}); {int(bad.sum())} bad scales")
    # reference codes: the oracle's, re-quantized with the GPU scale where allowed to differ
    z = det["z"].reshape(n, d // group, group)
    q_ref = det["q"].reshape(n, d // group, group).copy()
    if diff.any():
        q_ref[diff] = oracle.quantize_with_scale(z[diff], s_gpu[diff][:, None])
    s_used = np.where(diff, s_gpu, s_orc).astype(np.float64)[..., None]
    q_gpu = oracle.unpack_nibbles(np.asarray(codes_gpu, dtype=np.uint8)).reshape(q_ref.shape)
    mism = q_gpu != q_ref
    nm = int(mism.sum())
    if nm:
        with np.errstate(divide="ignore", invalid="ignore"):
            t = np.where(s_used > 0, z / np.where(s_used > 0, s_used, 1.0), 0.0)
        tie = np.abs((t - np.floor(t)) - 0.5) < 1e-4
        step = np.abs(q_gpu.astype(int) - q_ref.astype(int)) == 1
        ok = tie & step
        if not ok[mism].all():
            idx = np.argwhere(mism & ~ok)[0]
            raise AssertionError(f"code mismatch at row {idx[0]} coord {idx[1] * group + idx[2]}: gpu "
                                 f"{q_gpu[tuple(idx)]} oracle {q_ref[tuple(idx)]} z/s={t[tuple(idx)]!r}")
        if not allow_ties and nm > 1e-5 * q_ref.size + 2:
            raise AssertionError(f"{nm} tie mismatches out of {q_ref.size} elements (> 1e-5 + 2)")
    if not allow_ties:
        TALLY["mismatch"] += nm
        TALLY["elements"] += int(q_ref.size)
    return {"scale_1ulp": int(diff.sum()), "code_ties": nm, "elements": int(q_ref.size)}


def check_inverse(codes, scales, y_gpu, d, group, seed, rps=0, period=0, rot="srft", row0=0, rows=None):
    """Assert the GPU inverse of (codes, scales) matches the oracle's inverse of the same input
    (row i is cache row row0 + i, or rows[i] when a row list is given)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float16)
    y_orc, u = oracle.dequant_inv(codes, scales, d, group, seed, rps, period, rot, row0, return_fp64=True,
                                  rows=rows)
    y_gpu = np.asarray(y_gpu, dtype=np.float16)
    s_row = np.max(scales.astype(np.float64), axis=1, keepdims=True)
    tol = np.maximum(2e-3 * s_row, fp16_ulp(u)) * (1 + 1e-9)
    yg = y_gpu.astype(np.float64)
    yo = y_orc.astype(np.float64)
    both_inf = np.isinf(yg) & np.isinf(yo) & (np.sign(yg) == np.sign(yo))
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(yg - yo))
    bad = ~(err <= tol)
    if bad.any():
        r, c = np.argwhere(bad)[0]
        raise AssertionError(f"output mismatch row {r} col {c}: gpu {y_gpu[r, c]!r} oracle {y_orc[r, c]!r} "
                             f"(fp64 {u[r, c]!r}, tol {tol[r, c] if tol.shape[1] > 1 else tol[r, 0]!r}); "
                             f"{int(bad.sum())} bad")
    exact = float(np.mean(y_gpu.view(np.uint16) == y_orc.view(np.uint16))) if y_orc.size else 1.0
    rel = np.where(s_row > 0, err / np.where(s_row > 0, s_row, 1.0), 0.0)
    return {"max_err_over_s": float(np.max(rel, initial=0.0)), "exact_frac": exact}


def check_attention(o_gpu, o_orc, scales, strides, tokens, group, pairs=None):
    """Assert decode-attention outputs agree: for every (layer, stream, query,
    dim), |o_gpu - o_oracle| <= 2e-3 * s_v + 1 ulp of fp16 at o_oracle, where
    s_v is the largest value scale of that stream's cached tokens.  The output
    is a convex combination of the stream's dequantized value rows, so the
    per-row inverse bound (2e-3 times the row's scale) carries over with the
    stream's largest scale; the ulp term covers the final fp16 rounding.
    Returns the largest error in units of 2e-3 * s_v."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    layers, streams = o_orc.shape[:2]
    todo = [(l, s) for l in range(layers) for s in range(streams)] if pairs is None else pairs
    worst = 0.0
    for l, s in todo:
        rows = oracle.cache_rows(l, 1, s, tokens, strides)
        sv = float(np.max(np.asarray(scales[rows], dtype=np.float64)))
        err = np.abs(o_gpu[l, s] - o_orc[l, s])
        bound = 2e-3 * sv + fp16_ulp(o_orc[l, s])
        if not np.all(np.isfinite(o_gpu[l, s])) or np.any(err > bound):
            g, i = np.unravel_index(int(np.argmax(err - bound)), err.shape)
            raise AssertionError(f"attention mismatch at layer {l} stream {s} query {g} dim {i}: gpu "
                                 f"{o_gpu[l, s, g, i]!r} oracle {o_orc[l, s, g, i]!r} (bound {bound[g, i]:.3g}, "
                                 f"s_v {sv:.3g})")
        if sv > 0:
            worst = max(worst, float(np.max(err / (2e-3 * sv))))
    return worst


def check_attention_window(o_gpu, o_orc, scales, strides, tokens, group, window, window_tokens, pairs=None):
    """check_attention for attention over int4 tokens plus an fp16 window:
    |o_gpu - o_oracle| <= 2e-3 * s_v + 1 ulp of fp16 at o_oracle + 1e-5 *
    max |window value|.  s_v is the largest value scale of the stream's int4
    tokens (0 without any); the window values enter exactly, so the last term
    only covers fp32 arithmetic on them.  Returns the largest error in units
    of the bound."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    layers, streams = o_orc.shape[:2]
    todo = [(l, s) for l in range(layers) for s in range(streams)] if pairs is None else pairs
    worst = 0.0
    for l, s in todo:
        rows = oracle.cache_rows(l, 1, s, tokens, strides)
        sv = float(np.max(np.asarray(scales[rows], dtype=np.float64))) if tokens else 0.0
        wmax = float(np.max(np.abs(np.asarray(window[l, 1, s, :window_tokens], dtype=np.float64)))) \
            if window_tokens else 0.0
        err = np.abs(o_gpu[l, s] - o_orc[l, s])
        bound = 2e-3 * sv + fp16_ulp(o_orc[l, s]) + 1e-5 * wmax
        if not np.all(np.isfinite(o_gpu[l, s])) or np.any(err > bound):
            g, i = np.unravel_index(int(np.argmax(err - bound)), err.shape)
            raise AssertionError(f"attention mismatch at layer {l} stream {s} query {g} dim {i}: gpu "
                                 f"{o_gpu[l, s, g, i]!r} oracle {o_orc[l, s, g, i]!r} (bound {bound[g, i]:.3g})")
        worst = max(worst, float(np.max(err / bound)))
    return worst


def check_forward_ext(x16, codes_gpu, scales_gpu, group, bits, lam, seed, rps=0, period=0, rot="srft"):
    """check_forward for b-bit codes and an optional lambda: scales exact (or
    one fp16 ulp apart at an fp16 rounding midpoint of absmax/2^(b-1)); codes
    exact except +-1 at elements within 1e-4 of a rounding tie.  Returns the
    number of tie mismatches."""
    x16 = np.asarray(x16, dtype=np.float16)
    n, d = x16.shape
    det = oracle.forward_detail_ext(x16, group, bits, lam, seed, rps, period, rot)
    s_orc = det["s"]
    s_gpu = np.asarray(scales_gpu, dtype=np.float16).reshape(s_orc.shape)
    diff = s_gpu.view(np.uint16) != s_orc.view(np.uint16)
    ulp_apart = np.abs(s_gpu.astype(np.float64) - s_orc.astype(np.float64)) <= fp16_ulp(s_orc) * (1 + 1e-9)
    amb = near_fp16_midpoint(det["a"] / float(1 << (bits - 1)))
    bad = diff & ~(amb & ulp_apart)
    if bad.any():
        r, j = np.argwhere(bad)[0]
        raise AssertionError(f"scale mismatch row {r} group {j}: gpu {s_gpu[r, j]!r} oracle {s_orc[r, j]!r}")
    z = det["z"].reshape(n, d // group, group)
    s_used = np.where(diff, s_gpu, s_orc).astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(s_used > 0, z / np.where(s_used > 0, s_used, 1.0), 0.0)
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    q_ref = np.clip(np.rint(t), lo, hi)
    q_gpu = oracle.unpack_bits(np.asarray(codes_gpu, dtype=np.uint8), bits, d).reshape(q_ref.shape)
    mism = q_gpu != q_ref
    if mism.any():
        tie = np.abs((t - np.floor(t)) - 0.5) < 1e-4
        ok = tie & (np.abs(q_gpu.astype(int) - q_ref.astype(int)) == 1)
        if not ok[mism].all():
            idx = np.argwhere(mism & ~ok)[0]
            raise AssertionError(f"code mismatch row {idx[0]} coord {idx[1] * group + idx[2]}: gpu "
                                 f"{q_gpu[tuple(idx)]} oracle {q_ref[tuple(idx)]} z/s={t[tuple(idx)]!r}")
        assert int(mism.sum()) <= 1e-5 * q_ref.size + 2, f"{int(mism.sum())} tie mismatches"
    return int(mism.sum())


def check_inverse_ext(codes, scales, y_gpu, d, group, bits, lam, seed, rps=0, period=0, rot="srft"):
    """check_inverse for b-bit codes and an optional lambda: |y_gpu - y_oracle|
    <= max(2e-3 * s_row / |lambda_c|, 1 fp16 ulp of y_oracle) (lambda divides
    the output channel by channel)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float16)
    y_orc, u = oracle.dequant_inv_ext(codes, scales, d, group, bits, lam, seed, rps, period, rot, return_fp64=True)
    s_row = np.max(scales.astype(np.float64), axis=1, keepdims=True)
    lam64 = np.ones(d) if lam is None else np.abs(np.asarray(lam, dtype=np.float16).astype(np.float64))
    tol = np.maximum(2e-3 * s_row / lam64[None, :], fp16_ulp(u)) * (1 + 1e-9)
    err = np.abs(np.asarray(y_gpu, dtype=np.float16).astype(np.float64) - y_orc.astype(np.float64))
    bad = ~(err <= tol)
    if bad.any():
        r, c = np.argwhere(bad)[0]
        raise AssertionError(f"output mismatch row {r} col {c}: gpu {y_gpu[r, c]!r} oracle {y_orc[r, c]!r} "
                             f"(tol {tol[r, c]!r}); {int(bad.sum())} bad")
    return float(np.max(err / tol, initial=0.0))
