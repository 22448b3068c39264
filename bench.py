#!/usr/bin/env python3
"""Throughput of the fused SRFT int4 forward + inverse kernels on one MI355X.

One step = one pass of the whole path over one batch of synthetic K/V input:
the forward launch (sign flip, SRFT, per-group absmax, int4 rounding, nibble
packing) over every row, then the inverse launch (unpack, dequantize, inverse
SRFT, sign flip, fp16 store) over every row.  The default workload is the
largest configuration that fits one GPU, the Gemma-3-1B-shaped long-context
KV cache (26 layers x 2 x 16 sequences x 32768 tokens, d = 256, groups of
32, per-layer sign seeds): 27,262,976 vectors, 17.9 GB per direction.

Inputs are resident in HBM before timing starts.  Workloads smaller than
1 GiB cycle several replicas of the buffers so the 256 MB last-level cache
cannot hold a step's data.  Each kernel's duration is the median of 21
event-timed launches in a pass of its own after the timed steps.  Prints one
JSON line on stdout (human-readable notes go to stderr).

  python bench.py [--steps K] [--warmup W] [--workload 1..5] [--rot srft|srht]

With --attn it measures instead one decode step of attention that reads the
int4 cache directly (srft_attn_decode): every query head of every (layer,
stream) attends over all cached tokens (default: the Qwen2.5-1.5B decode
cache, 28 layers x 128 streams x 2049 tokens, 6 query heads per K/V head),
beside the unfused path (inverse kernel to an fp16 cache, then attention as
torch batched matmuls and softmax).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, public figure
KERNEL_REPS = 21  # event-timed samples per kernel (the median is reported)
METRIC = "K/V vectors/s and HBM GB/s (% of peak), fused SRFT-int4 quant+dequant, 1 GPU"
ATTN_METRIC = "decode-attention steps/s over the int4 rotated K/V cache (dequantized in registers), 1 GPU"
_CSRC = os.path.join(ROOT, "rotate_then_quantize_amd", "csrc")
# sources each kernel family is compiled from (a profile is current while their code is unchanged)
KERNEL_SOURCES = [os.path.join(_CSRC, f) for f in (
    "rtq.hip", "rtq_lane.hpp", "rtq_host.hpp", "rtq_device.hpp", "rtq_div.hpp", "rtq_mem.hpp")]
PAIR_SOURCES = KERNEL_SOURCES + [os.path.join(_CSRC, "rtq_pair.hpp")]  # d = 256 kernels
ATTN_SOURCES = [os.path.join(_CSRC, f) for f in ("rtq_attn.hip", "rtq_device.hpp", "rtq_mem.hpp")]


def kernel_sources(role: str, d: int):
    """The source files a kernel's code comes from (its profile summaries go stale when they change)."""
    if role == "attn_decode":
        return ATTN_SOURCES
    return PAIR_SOURCES if d == 256 else KERNEL_SOURCES


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_text(src: str) -> str:
    """Source with comments and blank runs removed: what the compiler sees."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash(sources=None) -> str:
    """Hash of the kernel sources' code (comments ignored)."""
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload_name: str, rot: str, kernel: str, d: int):
    """HBM bytes per launch from the committed PMC summary, if it was taken on
    the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{rot}_{workload_name}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha") != kernel_source_hash(kernel_sources(kernel, d)):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


KERNEL_ROLES = (("fwd_", "quant_fwd"), ("inv_", "dequant_inv"), ("attn::", "attn_decode"))


def attn_bytes(w, window: int = 0) -> int:
    """Algorithmic HBM bytes of one decode-attention launch over workload w:
    every K and V row's codes and scales once, the fp16 K and V rows of the
    `window` newest tokens once, plus the queries and outputs."""
    rows = w.layers * 2 * w.streams * w.tokens
    qo = 2 * w.layers * w.streams * w.q_per_kv * w.d * 2
    win = w.layers * 2 * w.streams * window * w.d * 2
    return rows * (w.d // 2 + 2 * (w.d // w.group)) + qo + win


def role_bytes(w, role: str) -> int:
    if role == "attn_decode":
        return attn_bytes(w)
    rows = w.new_rows if (w.new_tokens and role == "quant_fwd") else w.n_rows
    return rows * w.bytes_per_vector()


def role_sources(role: str, d: int):
    return kernel_sources(role, d)


def short_kernel_name(name: str) -> str:
    """'void rtq::fwd_lane_kernel<64, 32, 0>(...)' -> 'rtq::fwd_lane_kernel<64, 32, 0>'."""
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    name = name.replace("(anonymous namespace)", "{anon}")
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def kernel_role(name: str):
    short = short_kernel_name(name)
    if not short.startswith("rtq::"):
        return None
    for prefix, role in KERNEL_ROLES:
        if short[5:].startswith(prefix):
            return role
    return None


def find_csv(directory: str, suffix: str) -> str:
    hits = []
    for root, _, files in os.walk(directory):
        hits += [os.path.join(root, f) for f in files if f.endswith(suffix)]
    if len(hits) != 1:
        raise SystemExit(f"expected one *{suffix} under {directory}, found {hits}")
    return hits[0]


def find_profile(directory: str, csv_suffix: str):
    """('csv', path) when rocprofv3 wrote CSV files, else ('db', path) of its
    SQLite (rocpd) database, the default output format."""
    csvs, dbs = [], []
    for root, _, files in os.walk(directory):
        csvs += [os.path.join(root, f) for f in files if f.endswith(csv_suffix)]
        dbs += [os.path.join(root, f) for f in files if f.endswith(".db")]
    if len(csvs) == 1:
        return "csv", csvs[0]
    if len(dbs) == 1:
        return "db", dbs[0]
    raise SystemExit(f"expected one *{csv_suffix} or one *.db under {directory}, found {csvs + dbs}")


def trace_dispatches(trace_dir: str):
    """{kernel short name: [duration ns of each dispatch, in launch order]}
    from a rocprofv3 --kernel-trace run (CSV or rocpd database)."""
    kind, path = find_profile(trace_dir, "kernel_trace.csv")
    if kind == "db":
        import sqlite3
        con = sqlite3.connect(path)
        rows = [(n, int(b), int(e)) for n, b, e in con.execute("select name, start, end from kernels")]
        con.close()
    else:
        import csv
        raw = list(csv.DictReader(open(path)))
        if not raw:
            return {}
        keys = raw[0].keys()
        name_k = next(k for k in ("Kernel_Name", "KernelName", "Name") if k in keys)
        beg_k = next(k for k in ("Start_Timestamp", "BeginNs", "Start") if k in keys)
        end_k = next(k for k in ("End_Timestamp", "EndNs", "End") if k in keys)
        rows = [(r[name_k], int(r[beg_k]), int(r[end_k])) for r in raw]
    out = {}
    for name, b, e in sorted(rows, key=lambda r: r[1]):
        out.setdefault(short_kernel_name(name), []).append(e - b)
    return out


def summarize_trace(trace_dir: str, w, rot: str, command: str, attn: bool = False, window: int = 0,
                    skip: int = 0) -> None:
    """Write the rocprofv3 --kernel-trace --stats summary of a bench run
    (window: the fp16 window tokens of an --attn --window run).  The first
    `skip` dispatches of each library kernel (the bench's set-up and warm-up
    launches) are left out of its figures."""
    per = trace_dispatches(trace_dir)
    what = ("decode attention" + (f" with {window} fp16 window tokens" if window else "")) if attn \
        else "forward + inverse"
    lines = [f"# rocprofv3 kernel trace, {what}, workload {w.name} (d={w.d}, group={w.group}, {rot})",
             f"# command: {command}",
             f"# kernel_source_sha: {kernel_source_hash(kernel_sources('attn_decode' if attn else 'quant_fwd', w.d))}",
             f"# per library kernel, its first {skip} dispatch(es) (set-up and warm-up) are left out",
             "# kernel | dispatches used (skipped) | average us | median us | min us | max us",
             ]
    others = {k: v for k, v in per.items() if not k.startswith("rtq::")}
    total_ns = sum(sum(v) for v in per.values()) or 1
    used = {}
    for name, durs in per.items():
        if not name.startswith("rtq::"):
            continue
        kept = durs[skip:] if len(durs) > skip else durs
        used[name] = kept
        srt = sorted(kept)
        lines.append(f"{name} | {len(kept)} ({len(durs) - len(kept)}) | {sum(kept) / len(kept) / 1e3:.2f} | "
                     f"{srt[len(srt) // 2] / 1e3:.2f} | {srt[0] / 1e3:.2f} | {srt[-1] / 1e3:.2f}")
    if others:
        lines.append(f"other kernels (input generation, copies, baselines): {len(others)} kernels, "
                     f"{sum(len(v) for v in others.values())} calls, "
                     f"{100.0 * sum(sum(v) for v in others.values()) / total_ns:.1f}% of GPU time")
    for name, kept in used.items():
        role = kernel_role(name)
        if role and (role == "attn_decode") == attn:
            bytes_launch = attn_bytes(w, window) if role == "attn_decode" else role_bytes(w, role)
            avg = sum(kept) / len(kept)
            med = sorted(kept)[len(kept) // 2]
            lines.append(f"{role}_average_us: {avg / 1e3:.3f}")
            lines.append(f"{role}_median_us: {med / 1e3:.3f}")
            lines.append(f"{role}_algorithmic_GBps: {bytes_launch / avg:.1f}")
    suffix = f"_window{window}" if window else ""
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{'attn_' if attn else ''}{rot}_{w.name}{suffix}.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"wrote {path}")


def pmc_per_dispatch(directory: str, counter: str):
    """({kernel short name: mean counter value per dispatch}, {kernel: dispatches})
    from a rocprofv3 --pmc run (CSV or rocpd database); a counter's value of
    one dispatch is its sum over the rows recorded for that dispatch."""
    kind, path = find_profile(directory, "counter_collection.csv")
    per_dispatch = {}
    if kind == "db":
        import sqlite3
        con = sqlite3.connect(path)
        rows = con.execute("select kernel_name, dispatch_id, value from counters_collection where counter_name = ?",
                           (counter,)).fetchall()
        con.close()
    else:
        import csv
        rows = [(r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id", "")), r["Counter_Value"])
                for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    for name, did, val in rows:
        key = (short_kernel_name(name), did)
        per_dispatch[key] = per_dispatch.get(key, 0.0) + float(val)
    acc = {}
    for (name, _), v in per_dispatch.items():
        acc.setdefault(name, []).append(v)
    return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}


VALU_COUNTERS = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD",
                 "SQ_INSTS_VMEM_WR", "SQ_INSTS_SMEM")
SIMDS, CLOCK_HZ = 1024, 2.4e9  # MI355X: 256 CUs x 4 SIMDs, peak engine clock


EXTRA_COUNTERS = ("VALUBusy", "GRBM_GUI_ACTIVE", "LDSBankConflict", "TA_BUSY_avr", "TA_BUSY_max", "MemUnitBusy",
                  "MemUnitStalled")
XCDS = 8  # GRBM_GUI_ACTIVE is recorded once per XCD


def summarize_valu(pmc_dir: str, trace_dir: str, w, rot: str, commands, attn: bool = False, skip: int = 0,
                   extra_dirs=()) -> None:
    """Instruction mix per wave of each library kernel from one rocprofv3 --pmc
    pass of SQ counters (chip totals per dispatch), and the VALU issue time it
    implies: a wave64 VALU instruction occupies its SIMD for 4 cycles, so
    busy = SQ_INSTS_VALU * 4 / (SIMDs * clock * kernel time), with the kernel
    time from a rocprofv3 trace of the same command and the peak clock.
    extra_dirs: further --pmc runs of the same command; the counters of
    EXTRA_COUNTERS found there are listed, and with VALUBusy and
    GRBM_GUI_ACTIVE (busy cycles, summed over the XCDs) the measured cycles
    per VALU instruction (4 when every instruction issues at full rate) and the
    clock the kernel ran at (its busy cycles per XCD over its trace time)."""
    per = {c: pmc_per_dispatch(pmc_dir, c) for c in VALU_COUNTERS}
    extra = {}
    for d in extra_dirs:
        for c in EXTRA_COUNTERS:
            vals, _ = pmc_per_dispatch(d, c)
            if vals:
                extra[c] = vals
    durs = {}
    for name, ds in trace_dispatches(trace_dir).items():
        kept = ds[skip:] if len(ds) > skip else ds
        durs[name] = sum(kept) / len(kept)
    for kname, waves in per["SQ_WAVES"][0].items():
        role = kernel_role(kname)
        if not role or (role == "attn_decode") != attn or kname not in durs or waves <= 0:
            continue
        valu = per["SQ_INSTS_VALU"][0][kname]
        busy = valu * 4.0 / (SIMDS * CLOCK_HZ * durs[kname] * 1e-9)
        lines = [f"# instruction mix of {kname}, workload {w.name} (d={w.d}, group={w.group}, {rot})"]
        lines += [f"# command ({c}): {cmd}" for c, cmd in commands]
        lines += [f"kernel: {kname}", f"kernel_source_sha: {kernel_source_hash(role_sources(role, w.d))}",
                  f"dispatches: {per['SQ_WAVES'][1][kname]}", f"waves_per_dispatch: {waves:.0f}"]
        for c in VALU_COUNTERS[1:]:
            lines.append(f"{c.lower()}_per_wave: {per[c][0][kname] / waves:.1f}")
        lines += [f"kernel_average_us: {durs[kname] / 1e3:.2f}",
                  f"valu_busy_estimate: {busy:.3f}",
                  "# valu_busy_estimate = SQ_INSTS_VALU * 4 cycles / (1024 SIMDs * 2.4 GHz * kernel time)"
                  + ("; MFMA instructions count as VALU instructions here" if attn else "")]
        got = {c: v[kname] for c, v in extra.items() if kname in v}
        for c, v in got.items():
            lines.append(f"pmc_{c}: {v:.4g}")
        if "VALUBusy" in got and "GRBM_GUI_ACTIVE" in got:
            cycles = got["GRBM_GUI_ACTIVE"] / XCDS
            per_inst = got["VALUBusy"] / 100.0 * cycles * SIMDS / valu
            lines += [f"valu_cycles_per_instruction: {per_inst:.3f}",
                      f"clock_GHz_while_running: {cycles / (durs[kname] * 1e-9) / 1e9:.3f}",
                      "# valu_cycles_per_instruction = VALUBusy * (GRBM_GUI_ACTIVE / 8 XCDs) * 1024 SIMDs / "
                      "SQ_INSTS_VALU; clock = (GRBM_GUI_ACTIVE / 8) / kernel time"]
        path = os.path.join(ROOT, "profiles", f"valu_{role}_{rot}_{w.name}.txt")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        log(f"wrote {path}")


def read_valu(workload_name: str, rot: str, kernel: str, d: int):
    """VALU instructions per wave and the busy estimate from the committed
    summary, if it was taken on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"valu_{kernel}_{rot}_{workload_name}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha") != kernel_source_hash(kernel_sources(kernel, d)):
        return None
    try:
        return {"valu_insts_per_wave": float(vals["sq_insts_valu_per_wave"]),
                "busy_estimate": float(vals["valu_busy_estimate"]),
                "source": os.path.relpath(path, ROOT)}
    except (KeyError, ValueError):
        return None


def summarize_traffic(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, cal_mib, w, rot, commands) -> None:
    """HBM bytes per launch of each kernel: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) scaled by what the same counters read for a plain device copy of
    a known size."""
    known_kib = cal_mib * 1024.0
    cal = {}
    for counter, d in (("FETCH_SIZE", cal_fetch_dir), ("WRITE_SIZE", cal_write_dir)):
        vals, _ = pmc_per_dispatch(d, counter)
        copies = {k: v for k, v in vals.items() if "copy" in k.lower()}
        if not copies:
            raise SystemExit(f"no copy kernel in {d}: {sorted(vals)}")
        name, kib = max(copies.items(), key=lambda kv: kv[1])
        cal[counter] = (known_kib / kib, name, kib)
    fetch, nf = pmc_per_dispatch(fetch_dir, "FETCH_SIZE")
    write, nw = pmc_per_dispatch(write_dir, "WRITE_SIZE")
    for kname in sorted(set(fetch) & set(write)):
        role = kernel_role(kname)
        if not role:
            continue
        algo = role_bytes(w, role)
        fb = fetch[kname] * cal["FETCH_SIZE"][0] * 1024.0
        wb = write[kname] * cal["WRITE_SIZE"][0] * 1024.0
        lines = [f"# HBM traffic of {kname}, workload {w.name} (d={w.d}, group={w.group}, {rot})"]
        lines += [f"# command ({c}): {cmd}" for c, cmd in commands]
        lines += [
            f"kernel: {kname}",
            f"kernel_source_sha: {kernel_source_hash(role_sources(role, w.d))}",
            f"dispatches_fetch: {nf[kname]}",
            f"dispatches_write: {nw[kname]}",
            f"fetch_kib_per_dispatch_raw: {fetch[kname]:.1f}",
            f"write_kib_per_dispatch_raw: {write[kname]:.1f}",
            f"copy_calibration_kernel: {cal['FETCH_SIZE'][1]}",
            f"copy_calibration_bytes_each_way: {cal_mib} MiB",
            f"copy_fetch_kib_raw: {cal['FETCH_SIZE'][2]:.1f}",
            f"copy_write_kib_raw: {cal['WRITE_SIZE'][2]:.1f}",
            f"fetch_scale: {cal['FETCH_SIZE'][0]:.4f}",
            f"write_scale: {cal['WRITE_SIZE'][0]:.4f}",
            f"hbm_read_bytes_per_launch: {fb:.0f}",
            f"hbm_write_bytes_per_launch: {wb:.0f}",
            f"hbm_bytes_per_launch: {fb + wb:.0f}",
            f"algorithmic_bytes_per_launch: {algo}",
            f"traffic_over_algorithmic: {(fb + wb) / algo:.4f}",
        ]
        path = os.path.join(ROOT, "profiles", f"traffic_{role}_{rot}_{w.name}.txt")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        log(f"wrote {path}")


def graph_replay(w, sets, replicas, fwd_fn, inv_fn, steps, bpv, replays=5):
    """The same steps captured once into a HIP graph and replayed: launch
    overhead and event markers are gone, the kernels and their dispatch gaps
    remain.  The outputs of the last replay are compared with a direct call."""
    import torch
    n_inv = w.n_rows
    n_fwd = w.new_rows if w.new_tokens else w.n_rows

    def args_on(stream_handle, i):
        x, codes, scales, y = sets[i % replicas][2]
        xin = x[n_inv - n_fwd:] if w.new_tokens else x
        cin, sin = (codes[n_inv - n_fwd:], scales[n_inv - n_fwd:]) if w.new_tokens else (codes, scales)
        fa = (ctypes.c_void_p(xin.data_ptr()), ctypes.c_void_p(cin.data_ptr()), ctypes.c_void_p(sin.data_ptr()),
              n_fwd, w.d, w.group, w.sign_seed, w.rows_per_seed, w.seed_period, stream_handle)
        _, codes2, scales2, y2 = sets[(i + 1) % replicas][2]
        ia = (ctypes.c_void_p(codes2.data_ptr()), ctypes.c_void_p(scales2.data_ptr()), ctypes.c_void_p(y2.data_ptr()),
              n_inv, w.d, w.group, w.sign_seed, w.rows_per_seed, w.seed_period, stream_handle)
        return fa, ia

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            h = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for i in range(steps):
                fa, ia = args_on(h, i)
                if fwd_fn(*fa) or inv_fn(*ia):
                    raise RuntimeError("launch failed during capture")
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(replays):
        g.replay()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / (replays * steps)
    # replayed outputs equal a direct call on the same inputs
    last = steps - 1
    x, codes, scales, y = sets[last % replicas][2]
    ref_c, ref_s = codes.clone(), scales.clone()
    _, _, _, y_next = sets[(last + 1) % replicas][2]
    ref_y = y_next.clone()
    torch.cuda.synchronize()
    fa, ia = args_on(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), last)
    fwd_fn(*fa)
    inv_fn(*ia)
    torch.cuda.synchronize()
    same = bool(torch.equal(ref_c, codes) and torch.equal(ref_s, scales) and torch.equal(ref_y, y_next))
    fwd_bytes, inv_bytes = n_fwd * bpv, n_inv * bpv
    return {
        "ms_per_step": ms,
        "value": max(n_fwd, n_inv) / (ms * 1e-3),
        "unit": "vectors/s",
        "hbm_gbps_step": (fwd_bytes + inv_bytes) / (ms * 1e6),
        "steps_per_graph": steps,
        "replays": replays,
        "outputs_match_direct_call": same,
    }


def eager_baseline(w, sets, replicas, rot, fused_ms_step, stream, steps=3, warmup=1):
    """The same step as four separate torch operations (rotate with torch.fft,
    quantize, dequantize, inverse rotate) on the same buffers; signs are
    precomputed.  Workloads whose fp32 intermediates would not fit are run in
    row chunks of whole seed blocks (each chunk's signs are one broadcast
    row), every chunk still as the four operations.  Measurement only."""
    import torch
    import eager_baseline as eager
    n_inv = w.n_rows
    n_fwd = w.new_rows if w.new_tokens else w.n_rows
    budget = 1 << 30  # bytes of one fp32 [rows, d] intermediate per chunk
    rps, per = w.rows_per_seed, w.seed_period
    if n_inv * w.d * 4 <= 4 * budget:
        chunk_rows, repeat = n_inv, False
    elif rps and per and rps * per * w.d * 4 <= budget:
        # whole cycles of the seed rule: every chunk has the first chunk's signs
        chunk_rows, repeat = rps * per * max(1, budget // (rps * per * w.d * 4)), True
    elif rps and rps * w.d * 4 <= budget:
        chunk_rows, repeat = rps, False  # one seed block per chunk: its signs are one row
    else:
        raise SystemExit("eager baseline: no chunking rule for this workload")
    chunks, first = [], None
    for r0 in range(0, n_inv, chunk_rows):
        r1 = min(n_inv, r0 + chunk_rows)
        if chunk_rows == n_inv:
            sg = eager.sign_matrix(n_inv, w.d, w.sign_seed, rps, per)
        elif repeat:
            if first is None:
                first = eager.sign_matrix(chunk_rows, w.d, w.sign_seed, rps, per)
            sg = first[:r1 - r0]
        else:
            sg = eager.sign_matrix(1, w.d, w.sign_seed, rps, per, row0=r0)
        chunks.append((r0, r1, sg))
    if w.new_tokens:  # the decode step quantizes only the new token's rows
        fwd_chunks = [(n_inv - n_fwd, n_inv,
                       eager.sign_matrix(n_fwd, w.d, w.sign_seed, rps, per, row0=n_inv - n_fwd))]
    else:
        fwd_chunks = chunks

    def step(i):
        x, codes, scales, _ = sets[i % replicas][2]
        _, codes2, scales2, _ = sets[(i + 1) % replicas][2]
        out = []
        for r0, r1, sg in fwd_chunks:
            out.append(eager.quant_fwd(x[r0:r1], w.group, 0, rot=rot, signs=sg))
        for r0, r1, sg in chunks:
            out.append(eager.dequant_inv(codes2[r0:r1], scales2[r0:r1], w.d, w.group, 0, rot=rot, signs=sg))
            del out[-1]
        return out

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for i in range(steps):
        step(warmup + i)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    torch.cuda.empty_cache()
    return {
        "ms_per_step": ms,
        "value": max(n_fwd, n_inv) / (ms * 1e-3),
        "unit": "vectors/s",
        "fused_speedup": ms / fused_ms_step,
        "steps": steps,
        "row_chunks": len(chunks),
        "chunk_rows": chunk_rows,
        "ops": "rotate (torch.fft.rfft or Hadamard matmul), quantize, dequantize, inverse rotate (irfft): "
               "separate torch operations on the GPU, fp32 intermediates in HBM",
    }


def host_info() -> dict:
    """The host the oracle baseline ran on: CPU model and the cores this
    process may use (the oracle's BLAS threads are reported as "cores")."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count() or 1
    return {"cpu_model": model, "affinity_cores": affinity}


def cpu_baseline(w, x_gpu, rot, seconds):
    """The oracle, as it is, on consecutive 65536-row chunks of the same
    workload until ``seconds`` of CPU time are spent (input copy excluded)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    chunk = 65536
    done, spent, r0, passes = 0, 0.0, 0, 0
    while spent < seconds:
        r1 = min(w.n_rows, r0 + chunk)
        xs = x_gpu[r0:r1].cpu().numpy()
        t0 = time.perf_counter()
        codes, scales = oracle.quant_fwd(xs, w.group, w.sign_seed, w.rows_per_seed, w.seed_period, rot, row0=r0)
        oracle.dequant_inv(codes, scales, w.d, w.group, w.sign_seed, w.rows_per_seed, w.seed_period, rot, row0=r0)
        spent += time.perf_counter() - t0
        done += r1 - r0
        r0 = r1
        if r0 >= w.n_rows:
            r0, passes = 0, passes + 1
    where = (f"{passes} full pass(es) plus {r0} rows" if passes else f"the first {done}") + f" of the {w.n_rows}-row workload"
    return {
        "value": done / spent,
        "unit": "vectors/s",
        "cores": threads,
        "host": host_info(),
        "kind": "oracle",
        "sample": f"{done} rows ({where}), forward + inverse each, fp64 numpy oracle in {chunk}-row chunks, "
                  f"{spent:.1f} s of oracle time (device-to-host copies excluded)",
    }


def attn_unfused_baseline(w, rot, fused_ms, dev, steps=10, warmup=2):
    """The unfused consumer: the inverse kernel dequantizes the whole cache to
    fp16 (kv-major, so K and V are contiguous [layers*streams, tokens, d]
    blocks), then attention runs as torch.bmm, softmax in fp32, torch.bmm.
    Measurement only."""
    import torch
    import rotate_then_quantize_amd as rtq
    L, S, T, G, d, g = w.layers, w.streams, w.tokens, w.q_per_kv, w.d, w.group
    n = L * 2 * S * T
    gen = torch.Generator(device=dev)
    gen.manual_seed(4321)
    codes = torch.randint(0, 256, (n, d // 2), generator=gen, device=dev, dtype=torch.uint8)
    scales = (torch.randn((n, d // g), generator=gen, device=dev).abs_() * 0.3).to(torch.float16)
    y = torch.empty((n, d), dtype=torch.float16, device=dev)
    q = torch.randn((L * S, G, d), generator=gen, device=dev).to(torch.float16)
    qt = q.transpose(1, 2).contiguous()
    scale = 1.0 / math.sqrt(d)

    def step():
        rtq.dequant_inv(rot, codes, scales, d, g, w.sign_seed, S * T, L, out=y)
        k = y[: n // 2].view(L * S, T, d)
        v = y[n // 2:].view(L * S, T, d)
        sc = torch.bmm(k, qt)                                   # [L*S, T, G]
        p = torch.softmax(sc.float() * scale, dim=1).to(torch.float16)
        return torch.bmm(p.transpose(1, 2).contiguous(), v)     # [L*S, G, d]

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(steps):
        step()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    del codes, scales, y
    torch.cuda.empty_cache()
    return {
        "ms_per_step": ms,
        "value": 1e3 / ms,
        "unit": "steps/s",
        "fused_speedup": ms / fused_ms,
        "steps": steps,
        "ops": f"{rot}_dequant_inv of every K/V row to fp16 (this library), then torch.bmm (K q^T), "
               "fp32 softmax, torch.bmm (P V) on the GPU",
    }


def attn_cpu_baseline(w, codes_gpu, scales_gpu, q_gpu, rot, seconds, strides, rps, per):
    """oracle.attn_decode, as it is, on consecutive (layer, stream) pairs of
    the same cache until ``seconds`` of CPU time are spent."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    codes, scales, q = codes_gpu.cpu().numpy(), scales_gpu.cpu().numpy(), q_gpu.cpu().numpy()
    L, S = w.layers, w.streams
    done, spent = 0, 0.0
    while spent < seconds and done < L * S:
        pair = (done // S, done % S)
        t0 = time.perf_counter()
        oracle.attn_decode(q, codes, scales, strides, L, S, w.tokens, w.q_per_kv, w.d, w.group,
                           w.sign_seed, rps, per, rot, pairs=[pair])
        spent += time.perf_counter() - t0
        done += 1
    return {
        "value": done / spent / (L * S),
        "unit": "steps/s",
        "cores": threads,
        "host": host_info(),
        "kind": "oracle",
        "sample": f"{done} of the {L * S} (layer, stream) pairs ({w.tokens} tokens, {w.q_per_kv} queries each), "
                  f"fp64 numpy oracle, {spent:.1f} s of oracle time; steps/s = pairs/s / {L * S}",
    }


def attn_main(args, w, dev):
    import torch
    import rotate_then_quantize_amd as rtq
    rot, W = args.rot, args.window
    lib = rtq.library()
    if W:
        fn = lib.srft_attn_decode_window if rot == "srft" else lib.srht_attn_decode_window
    else:
        fn = lib.srft_attn_decode if rot == "srft" else lib.srht_attn_decode
    L, S, T, G, d, g = w.layers, w.streams, w.tokens, w.q_per_kv, w.d, w.group
    if w.kv != 2:
        raise SystemExit(f"workload {w.wid} ({w.name}) holds no K/V pair per stream; decode attention needs one "
                         f"(workloads 2, 3, 4 and 5 do)")
    n = w.n_rows
    if args.attn_layout == "heads":
        strides = (2 * S * T, S * T, T, 1)
        rps, per = (2 * S * T, L) if L > 1 else (0, 0)   # one sign seed per layer
    else:
        strides, rps, per = w.cache_strides, w.rows_per_seed, w.seed_period
    cache_bytes = n * (d // 2 + 2 * (d // g))
    replicas = args.replicas or max(1, math.ceil((1 << 30) / cache_bytes))
    log(f"decode attention, workload {w.name}: L={L} S={S} T={T} G={G} d={d} group={g} rot={rot}, "
        f"{replicas} cache replica(s) of {cache_bytes / 1e6:.1f} MB" + (f", fp16 window of {W} tokens" if W else ""))
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    scale = ctypes.c_float(1.0 / math.sqrt(d))
    # token-split workspace (zero-filled once; every call leaves it zeroed)
    ws_bytes = rtq.attn_workspace_bytes(L, S, T, G, d)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    ws_ptr = ctypes.c_void_p(ws.data_ptr() if ws_bytes else None)
    sets = []
    for _ in range(replicas):
        codes = torch.randint(0, 256, (n, d // 2), generator=gen, device=dev, dtype=torch.uint8)
        scales = (torch.randn((n, d // g), generator=gen, device=dev).abs_() * 0.3).to(torch.float16)
        q = torch.randn((L, S, G, d), generator=gen, device=dev).to(torch.float16)
        out = torch.empty_like(q)
        a = (ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
             ctypes.c_void_p(out.data_ptr()), L, S, T, G, d, g, *strides, w.sign_seed, rps, per, scale)
        keep = (codes, scales, q, out)
        if W:
            win = torch.randn((L, 2, S, W, d), generator=gen, device=dev).to(torch.float16)
            a += (ctypes.c_void_p(win.data_ptr()), W, W)
            keep += (win,)
        sets.append((a + (ws_ptr, ws_bytes, sh), keep))
    torch.cuda.synchronize()

    def step(i):
        st = fn(*sets[i % replicas][0])
        if st:
            raise RuntimeError(lib.rtq_status_string(st).decode())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    # the kernel's own time: median of KERNEL_REPS event-timed samples, in a pass after the timed steps
    k_ms, (k_min, k_max), k_reps = time_launches(fn, [sets[k % replicas][0] for k in range(KERNEL_REPS)], stream)
    nbytes = attn_bytes(w, W)
    achieved = nbytes / k_ms / 1e6
    log(f"step {ms_step * 1e3:.1f} us | kernel {k_ms * 1e3:.1f} us {achieved:.0f} GB/s "
        f"({100 * achieved / HBM_PEAK_GBPS:.1f}% of {HBM_PEAK_GBPS:.0f})")
    result = {
        "metric": ATTN_METRIC,
        "value": args.steps / (t1 - t0),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 mfma, f32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": w.name, "layers": L, "streams": S, "tokens": T, "q_per_kv": G, "d": d, "group": g,
            "rotation": rot, "layout": "[layer][K,V][stream][token]" if args.attn_layout == "heads" else w.layout,
            "cache_strides": list(strides),
            "cache_replicas": replicas, "cache": "uniform int4 codes, |N(0,1)|*0.3 fp16 scales",
            "token_split_workspace_bytes": ws_bytes,
            "window_tokens": W,
        },
        "kernel_us": {"attn_decode": k_ms * 1e3, "attn_decode_min_max": [k_min * 1e3, k_max * 1e3],
                      "launches_per_sample": k_reps,
                      "timing": f"median of {KERNEL_REPS} samples, each a run of back-to-back launches (one "
                                f"launch when a launch takes 1 ms or more) between two hipEvents on the launch "
                                f"stream, in a pass after the timed steps"},
        "roofline": {
            "kernel": f"{rot}_attn_decode d={d} g={g} q_per_kv={G}",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            # the counter summaries cover the launch without a window
            "traffic": None if W else read_traffic(w.name, rot, "attn_decode", w.d),
            "algorithmic_bytes_per_launch": nbytes,
        },
        "valu": None if W else read_valu(w.name, rot, "attn_decode", w.d),
    }
    result["hbm_copy"] = measured_copy(dev)
    if not args.no_eager and not W:
        result["unfused_baseline"] = attn_unfused_baseline(w, rot, ms_step, dev)
    if not args.no_cpu_baseline and not W:
        codes, scales, q, _ = sets[0][1]
        result["cpu_baseline"] = attn_cpu_baseline(w, codes, scales, q, rot, args.cpu_seconds, strides, rps, per)
    print(json.dumps(result), flush=True)


def decode_cache_main(args, w, dev):
    """Per-step cost of keeping a dequantized fp16 prefix with a 16-token fp16
    window (append each token to the window; every 16th step quantize the
    window in place and dequantize just those rows), against dequantizing
    the whole cache every step; and a whole decode step whose consumer is
    the int4 attention (append + one attention launch, no dequantized
    copy)."""
    import torch
    import rotate_then_quantize_amd as rtq
    from rotate_then_quantize_amd.decode_cache import DecodeCache
    rot, W = args.rot, 16
    L, S, T, d, g = w.layers, w.streams, w.tokens - 1, w.d, w.group  # prefix tokens; one more per step
    steps = max(W, (args.steps // W) * W)
    cap = T + steps
    log(f"decode cache, workload {w.name}: L={L} S={S} prefix {T} tokens, window {W}, {steps} steps, d={d} g={g}")
    cache = DecodeCache(L, S, cap, d, g, w.sign_seed, rot, W, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    cache.prefill(torch.randn((L, 2, S, T, d), generator=gen, device=dev).to(torch.float16))
    new = torch.randn((steps + args.warmup, L, 2, S, d), generator=gen, device=dev).to(torch.float16)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    # the window policy: `steps` appends (steps / 16 window flushes)
    ev[0].record(stream)
    for i in range(steps):
        cache.append(new[i])
    ev[1].record(stream)
    torch.cuda.synchronize()
    window_ms = ev[0].elapsed_time(ev[1]) / steps
    # one flush alone: quantize 16 tokens in place + refresh their dequantized rows
    t0 = cache.quantized - W
    blk = torch.randn((L, 2, S, W, d), generator=gen, device=dev).to(torch.float16)
    flush_ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for _ in range(2):
        rtq.quant_append(rot, blk, cache.codes, cache.scales, cache.strides, t0, g, cache.seed,
                         cache.rows_per_seed, cache.seed_period)
        rtq.dequant_rows(rot, cache.codes, cache.scales, cache.prefix, L, S, t0, W, cache.strides, g, cache.seed,
                         cache.rows_per_seed, cache.seed_period)
    flush_ev[0].record(stream)
    rtq.quant_append(rot, blk, cache.codes, cache.scales, cache.strides, t0, g, cache.seed, cache.rows_per_seed,
                     cache.seed_period)
    flush_ev[1].record(stream)
    rtq.dequant_rows(rot, cache.codes, cache.scales, cache.prefix, L, S, t0, W, cache.strides, g, cache.seed,
                     cache.rows_per_seed, cache.seed_period)
    flush_ev[2].record(stream)
    torch.cuda.synchronize()
    append_ms, rows_ms = flush_ev[0].elapsed_time(flush_ev[1]), flush_ev[1].elapsed_time(flush_ev[2])
    # without the dequantized prefix: quantize the new token, dequantize every cached row, each step
    n_all = cache.codes.shape[0]
    y = torch.empty((n_all, d), dtype=torch.float16, device=dev)
    for _ in range(args.warmup):
        rtq.dequant_inv(rot, cache.codes, cache.scales, d, g, cache.seed, cache.rows_per_seed, cache.seed_period,
                        out=y)
    tok = new[0].reshape(L, 2, S, 1, d).contiguous()
    full_steps = 20
    ev[0].record(stream)
    for i in range(full_steps):
        rtq.quant_append(rot, tok, cache.codes, cache.scales, cache.strides, cap - 1, g, cache.seed,
                         cache.rows_per_seed, cache.seed_period)
        rtq.dequant_inv(rot, cache.codes, cache.scales, d, g, cache.seed, cache.rows_per_seed, cache.seed_period,
                        out=y)
    ev[1].record(stream)
    torch.cuda.synchronize()
    full_ms = ev[0].elapsed_time(ev[1]) / full_steps
    # A whole decode step with the int4 attention as the consumer (no dequantized copy kept): append the
    # token (every 16th step quantizes the window in place), then one attention launch over the int4
    # prefix and the fp16 window.
    del y
    lean = DecodeCache(L, S, T + args.warmup + steps, d, g, w.sign_seed, rot, W, dev, keep_prefix=False)
    lean.prefill(torch.randn((L, 2, S, T, d), generator=gen, device=dev).to(torch.float16))
    q = torch.randn((L, S, w.q_per_kv, d), generator=gen, device=dev).to(torch.float16)
    o = torch.empty_like(q)
    for i in range(args.warmup):
        lean.append(new[i])
        lean.attention(q, out=o)
    torch.cuda.synchronize()
    dsteps = steps  # a multiple of 16: every phase of the window schedule equally often
    ev[0].record(stream)
    for i in range(dsteps):
        lean.append(new[i])
        lean.attention(q, out=o)
    ev[1].record(stream)
    torch.cuda.synchronize()
    decode_ms = ev[0].elapsed_time(ev[1]) / dsteps
    del lean
    rows_flush = L * 2 * S * W
    bpv = w.bytes_per_vector()
    log(f"window policy {window_ms * 1e3:.1f} us/step | flush: append {append_ms * 1e3:.1f} us + refresh "
        f"{rows_ms * 1e3:.1f} us ({rows_flush} rows) | full re-dequantize {full_ms * 1e3:.1f} us/step | "
        f"decode step with int4 attention {decode_ms * 1e3:.1f} us")
    result = {
        "metric": "decode-step cache maintenance time, dequantized prefix + 16-token fp16 window, 1 GPU",
        "value": window_ms * 1e3,
        "unit": "us/step",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": window_ms,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": L, "streams": S, "prefix_tokens": T, "window": W, "d": d,
                   "group": g, "rotation": rot, "layout": "[layer][K,V][stream][token]", "capacity": cap},
        "flush": {"append_us": append_ms * 1e3, "refresh_us": rows_ms * 1e3, "rows": rows_flush,
                  "append_GBps": rows_flush * bpv / append_ms / 1e6, "refresh_GBps": rows_flush * bpv / rows_ms / 1e6},
        "full_redequantize": {"us_per_step": full_ms * 1e3, "rows": n_all,
                              "ops": "append of the new token + dequant_inv of every cache row, each step"},
        "speedup_vs_full_redequantize": full_ms / window_ms,
        "decode_step_with_int4_attention": {
            "us_per_step": decode_ms * 1e3, "steps": dsteps, "q_per_kv": w.q_per_kv,
            "ops": "append of the new token (the window quantized in place every 16th step) + one "
                   "attention launch over the int4 prefix and the fp16 window; no dequantized copy kept"},
    }
    print(json.dumps(result), flush=True)


def ext_main(args, w, dev):
    """Forward + inverse with each code width (3, 4, 6, 8 bits) and a
    per-channel lambda, on the workload's rows: the same step as the default
    bench (forward over every row, then inverse over every row of another
    replica), one line with every width."""
    import torch
    import rotate_then_quantize_amd as rtq
    rot = args.rot
    lib = rtq.library()
    fwd_fn = lib.srft_quant_fwd_ext if rot == "srft" else lib.srht_quant_fwd_ext
    inv_fn = lib.srft_dequant_inv_ext if rot == "srft" else lib.srht_dequant_inv_ext
    n, d, g = w.n_rows, w.d, w.group
    x0 = W_generate(w, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    lam = (torch.rand((d,), generator=gen, device=dev) * 3.75 + 0.25).to(torch.float16)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    lp = ctypes.c_void_p(lam.data_ptr())
    out = {}
    for bits in rtq.CODE_BITS:
        footprint = n * (2 * d + d * bits // 8 + 2 * (d // g) + 2 * d)
        replicas = args.replicas or max(1, math.ceil((1 << 30) / footprint))
        sets = []
        for r in range(replicas):
            x = x0 if r == 0 else x0.clone()
            codes = torch.empty((n, d * bits // 8), dtype=torch.uint8, device=dev)
            scales = torch.empty((n, d // g), dtype=torch.float16, device=dev)
            y = torch.empty((n, d), dtype=torch.float16, device=dev)
            fa = (ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                  n, d, g, bits, lp, w.sign_seed, w.rows_per_seed, w.seed_period, sh)
            ia = (ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                  n, d, g, bits, lp, w.sign_seed, w.rows_per_seed, w.seed_period, sh)
            sets.append((fa, ia, (x, codes, scales, y)))
        for fa, _, _ in sets:
            assert fwd_fn(*fa) == 0
        torch.cuda.synchronize()
        steps = max(20, args.steps // 4)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for i in range(args.warmup):
            fwd_fn(*sets[i % replicas][0])
            inv_fn(*sets[(i + 1) % replicas][1])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            ev = evs[i] if i % 5 == 0 else None
            if ev:
                ev[0].record(stream)
            s1 = fwd_fn(*sets[i % replicas][0])
            if ev:
                ev[1].record(stream)
            s2 = inv_fn(*sets[(i + 1) % replicas][1])
            if ev:
                ev[2].record(stream)
            if s1 or s2:
                raise RuntimeError(lib.rtq_status_string(s1 or s2).decode())
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        sampled = [evs[i] for i in range(steps) if i % 5 == 0]
        f_ms = sum(e[0].elapsed_time(e[1]) for e in sampled) / len(sampled)
        i_ms = sum(e[1].elapsed_time(e[2]) for e in sampled) / len(sampled)
        bpv = 2 * d + d * bits // 8 + 2 * (d // g)
        out[bits] = {"step_us": (t1 - t0) * 1e6 / steps, "forward_us": f_ms * 1e3, "inverse_us": i_ms * 1e3,
                     "forward_GBps": n * bpv / f_ms / 1e6, "inverse_GBps": n * bpv / i_ms / 1e6,
                     "bytes_per_vector": bpv, "vectors_per_s": n * steps / (t1 - t0), "buffer_replicas": replicas}
        log(f"bits {bits}: step {out[bits]['step_us']:.1f} us | fwd {f_ms * 1e3:.1f} us "
            f"{out[bits]['forward_GBps']:.0f} GB/s | inv {i_ms * 1e3:.1f} us {out[bits]['inverse_GBps']:.0f} GB/s")
        del sets
        torch.cuda.empty_cache()
    head = out[4]
    dom = "inverse" if head["inverse_us"] >= head["forward_us"] else "forward"
    achieved = head[f"{dom}_GBps"]
    result = {
        "metric": "K/V vectors/s, fused forward + inverse with per-channel lambda, 4-bit codes (3/6/8-bit beside), 1 GPU",
        "value": head["vectors_per_s"],
        "unit": "vectors/s",
        "n_gpus": 1,
        "steps": max(20, args.steps // 4),
        "warmup": args.warmup,
        "ms_per_step": head["step_us"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "rows": n, "d": d, "group": g, "rotation": rot,
                   "lambda": "uniform(0.25, 4) fp16 per channel"},
        "by_bits": {str(b): v for b, v in out.items()},
        "roofline": {"kernel": f"{rot}_{'dequant_inv' if dom == 'inverse' else 'quant_fwd'}_ext bits=4 lambda",
                     "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None},
    }
    result["hbm_copy"] = measured_copy(dev)
    print(json.dumps(result), flush=True)


def W_generate(w, dev):
    from rotate_then_quantize_amd import workloads as W
    return W.generate(w, dev)


def measured_copy(dev, mib: int = 1024, reps: int = 10) -> dict:
    """Achievable HBM rate: a device-to-device copy of `mib` MiB (read plus
    written bytes over the median event-timed copy), reported beside the
    published peak."""
    import torch
    nbytes = mib << 20
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    stream = torch.cuda.current_stream(dev)
    b.copy_(a)
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        b.copy_(a)
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sorted(times)[len(times) // 2]
    del a, b
    return {"GBps": 2 * nbytes / ms / 1e6, "bytes_each_way": nbytes,
            "kind": f"torch device-to-device copy, (read + written bytes) / median of {reps} event-timed copies"}


def time_launches(fn, arg_sets, stream, min_ms: float = 1.0):
    """Median, min and max duration in ms of one launch of fn(*a), a cycling
    through arg_sets: each of len(arg_sets) samples is R back-to-back launches
    between two events recorded on `stream` (the launch stream), divided by R.
    R = 1 when one launch takes at least min_ms; shorter kernels take enough
    launches per sample to fill min_ms, so the few microseconds an event
    marker costs do not count as kernel time."""
    import torch

    def sample(r, k0):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for j in range(r):
            st = fn(*arg_sets[(k0 + j) % len(arg_sets)])
            if st:
                raise RuntimeError(f"launch failed with status {st}")
        e1.record(stream)
        return e0, e1

    torch.cuda.synchronize()
    e0, e1 = sample(1, 0)
    torch.cuda.synchronize()
    reps = max(1, math.ceil(min_ms / max(e0.elapsed_time(e1), 1e-3)))
    evs = [sample(reps, k) for k in range(len(arg_sets))]
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) / reps for e0, e1 in evs)
    return ms[len(ms) // 2], (ms[0], ms[-1]), reps


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=None, choices=[1, 2, 3, 4, 5],
                    help="workload id (default 5; 3 with --attn or --decode-cache)")
    ap.add_argument("--attn", action="store_true",
                    help="measure decode attention over the int4 cache instead of forward + inverse")
    ap.add_argument("--ext", action="store_true",
                    help="measure forward + inverse with 3/4/6/8-bit codes and a per-channel lambda")
    ap.add_argument("--decode-cache", action="store_true",
                    help="measure the dequantized-prefix cache with a 16-token fp16 window (workload 3 by default)")
    ap.add_argument("--attn-layout", choices=["heads", "workload"], default="heads",
                    help="attention cache layout: 'heads' = [layer][K,V][stream][token] (each head's tokens "
                         "contiguous, as a per-layer [batch, heads, tokens, d] cache), 'workload' = the "
                         "workload's own row order")
    ap.add_argument("--rot", choices=["srft", "srht"], default="srft")
    ap.add_argument("--window", type=int, default=0, metavar="W",
                    help="with --attn: also attend to W fp16 tokens per stream (0-64)")
    ap.add_argument("--replicas", type=int, default=0, help="buffer sets cycled per step (0 = enough to exceed 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-eager", action="store_true", help="skip the eager four-operation torch baseline")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the same steps replayed from one captured HIP graph")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (PMC counter calibration)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write profiles/kernel_trace_*.txt from a rocprofv3 --kernel-trace --stats CSV directory")
    ap.add_argument("--trace-skip", type=int, default=0, metavar="N",
                    help="with --summarize-trace: leave each library kernel's first N dispatches out")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write profiles/traffic_*.txt from four rocprofv3 --pmc CSV directories")
    ap.add_argument("--summarize-valu", nargs="+", metavar="DIR",
                    help="PMC TRACE [EXTRA ...]: write profiles/valu_*.txt from a rocprofv3 --pmc run of SQ "
                         "instruction counters, a kernel trace of the same command and optional further --pmc "
                         "runs (VALUBusy, GRBM_GUI_ACTIVE, LDSBankConflict, TA_BUSY, MemUnitBusy / MemUnitStalled)")
    ap.add_argument("--command", action="append", default=[],
                    help="command line(s) that produced the profile directories, recorded in the summary")
    args = ap.parse_args()
    if args.window and (not args.attn or not 0 < args.window <= 64):
        ap.error("--window takes 1 to 64 tokens and goes with --attn")
    if args.workload is None:
        args.workload = 3 if (args.attn or args.decode_cache) else 5

    if args.summarize_trace or args.summarize_traffic or args.summarize_valu:
        from rotate_then_quantize_amd import workloads as W
        w = W.WORKLOADS[args.workload]
        if args.summarize_valu:
            if len(args.summarize_valu) < 2:
                ap.error("--summarize-valu takes PMC TRACE [EXTRA ...]")
            pmc, trace, *extra_dirs = args.summarize_valu
            n_cmd = 1 + len(extra_dirs)
            cmds = [("SQ counters" if i == 0 else "extra counters", c)
                    for i, c in enumerate(args.command[-n_cmd:])]
            summarize_valu(pmc, trace, w, args.rot, cmds, args.attn, args.trace_skip, extra_dirs)
        if args.summarize_trace:
            summarize_trace(args.summarize_trace, w, args.rot, " ; ".join(args.command), args.attn, args.window,
                            args.trace_skip)
        if args.summarize_traffic:
            names = ("FETCH_SIZE", "WRITE_SIZE", "copy FETCH_SIZE", "copy WRITE_SIZE")
            cmds = list(zip(names, args.command[-4:])) if len(args.command) >= 4 else []
            summarize_traffic(*args.summarize_traffic, args.calibrate_copy or 256, w, args.rot, cmds)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log("bench.py measures one GPU and has no multi-GPU path: rows are independent, so the work "
            "shards by layer, K/V head or batch with no exchange, each GPU running the same kernels on "
            "its share. Run with --gpus 1.")
        sys.exit(2)

    import torch
    import rotate_then_quantize_amd as rtq
    from rotate_then_quantize_amd import workloads as W

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        nbytes = args.calibrate_copy << 20
        a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copied {nbytes} bytes 5 times")
        return

    w = W.WORKLOADS[args.workload]
    if args.attn:
        attn_main(args, w, dev)
        return
    if args.decode_cache:
        decode_cache_main(args, w, dev)
        return
    if args.ext:
        ext_main(args, w, dev)
        return
    rot = args.rot
    if rot not in w.rots:
        log(f"note: workload {w.name} is specified with {w.rots}; running {rot} anyway")
    lib = rtq.library()
    fwd_fn = lib.srft_quant_fwd if rot == "srft" else lib.srht_quant_fwd
    inv_fn = lib.srft_dequant_inv if rot == "srft" else lib.srht_dequant_inv

    # rows of one step: decode = new token's rows forward, whole cache inverse
    n_inv = w.n_rows
    n_fwd = w.new_rows if w.new_tokens else w.n_rows
    bpv = w.bytes_per_vector()
    footprint = n_fwd * 2 * w.d + n_inv * (w.d // 2 + 2 * (w.d // w.group)) + n_inv * 2 * w.d
    replicas = args.replicas or max(1, math.ceil((1 << 30) / footprint))
    log(f"workload {w.name}: fwd rows {n_fwd}, inv rows {n_inv}, d={w.d}, group={w.group}, rot={rot}, "
        f"{replicas} buffer replica(s) of {footprint / 1e6:.1f} MB")

    x0 = W.generate(w, dev)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    sets = []
    for r in range(replicas):
        x = x0 if r == 0 else x0.clone()
        codes = torch.empty((n_inv, w.d // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((n_inv, w.d // w.group), dtype=torch.float16, device=dev)
        y = torch.empty((n_inv, w.d), dtype=torch.float16, device=dev)
        xin = x[n_inv - n_fwd:] if w.new_tokens else x
        cin, sin = (codes[n_inv - n_fwd:], scales[n_inv - n_fwd:]) if w.new_tokens else (codes, scales)
        if w.new_tokens:  # the cached prefix is already quantized
            st = fwd_fn(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(codes.data_ptr()),
                        ctypes.c_void_p(scales.data_ptr()), n_inv, w.d, w.group, w.sign_seed,
                        w.rows_per_seed, w.seed_period, sh)
            assert st == 0, lib.rtq_status_string(st)
        fa = (ctypes.c_void_p(xin.data_ptr()), ctypes.c_void_p(cin.data_ptr()), ctypes.c_void_p(sin.data_ptr()),
              n_fwd, w.d, w.group, w.sign_seed, w.rows_per_seed, w.seed_period, sh)
        ia = (ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(y.data_ptr()),
              n_inv, w.d, w.group, w.sign_seed, w.rows_per_seed, w.seed_period, sh)
        sets.append((fa, ia, (x, codes, scales, y)))
    torch.cuda.synchronize()

    # Every replica's codes exist before the first inverse reads them.
    for fa, _, _ in sets:
        st = fwd_fn(*fa)
        assert st == 0, lib.rtq_status_string(st)
    torch.cuda.synchronize()

    def step(i, ev_start=None, ev_mid=None):
        # The inverse reads the replica the forward wrote two steps earlier, so
        # its codes come from HBM rather than from the 256 MB last-level cache.
        fa = sets[i % replicas][0]
        ia = sets[(i + 1) % replicas][1]
        if ev_start is not None:
            ev_start.record(stream)
        s1 = fwd_fn(*fa)
        if ev_mid is not None:
            ev_mid.record(stream)
        s2 = inv_fn(*ia)
        if s1 or s2:
            raise RuntimeError(lib.rtq_status_string(s1 or s2).decode())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    # Kernel durations: KERNEL_REPS event-timed samples of each kernel on its
    # own, after the timed steps (so --steps does not change how many samples
    # there are); the median of the per-launch durations (time_launches).
    # Launches cycle the replicas as the steps do.
    fwd_ms, fwd_spread, fwd_reps = time_launches(fwd_fn, [sets[i % replicas][0] for i in range(KERNEL_REPS)],
                                                 stream)
    inv_ms, inv_spread, inv_reps = time_launches(inv_fn, [sets[(i + 1) % replicas][1] for i in range(KERNEL_REPS)],
                                                 stream)
    fwd_bytes, inv_bytes = n_fwd * bpv, n_inv * bpv
    fwd_gbps, inv_gbps = fwd_bytes / fwd_ms / 1e6, inv_bytes / inv_ms / 1e6
    vectors = max(n_fwd, n_inv)
    value = vectors * args.steps / (t1 - t0)
    step_gbps = (fwd_bytes + inv_bytes) / (ms_step * 1e6)
    dominant = "inv" if inv_ms >= fwd_ms else "fwd"
    dom_ms, dom_bytes = (inv_ms, inv_bytes) if dominant == "inv" else (fwd_ms, fwd_bytes)
    achieved = dom_bytes / dom_ms / 1e6
    kname = {"fwd": "quant_fwd", "inv": "dequant_inv"}[dominant]
    traffic = read_traffic(w.name, rot, kname, w.d)
    log(f"step {ms_step * 1e3:.1f} us | fwd {fwd_ms * 1e3:.1f} us {fwd_gbps:.0f} GB/s "
        f"({100 * fwd_gbps / HBM_PEAK_GBPS:.1f}%) | inv {inv_ms * 1e3:.1f} us {inv_gbps:.0f} GB/s "
        f"({100 * inv_gbps / HBM_PEAK_GBPS:.1f}%) | step {step_gbps:.0f} GB/s")

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "rows_forward": n_fwd, "rows_inverse": n_inv, "d": w.d, "group": w.group,
            "rotation": rot, "rows_per_seed": w.rows_per_seed, "seed_period": w.seed_period,
            "io": "fp16 in/out, int4 codes, fp16 scales", "buffer_replicas": replicas,
        },
        "hbm_gbps": {"step": step_gbps, "forward": fwd_gbps, "inverse": inv_gbps,
                     "peak": HBM_PEAK_GBPS, "bytes_per_vector": bpv},
        "kernel_us": {"forward": fwd_ms * 1e3, "inverse": inv_ms * 1e3,
                      "forward_min_max": [fwd_spread[0] * 1e3, fwd_spread[1] * 1e3],
                      "inverse_min_max": [inv_spread[0] * 1e3, inv_spread[1] * 1e3],
                      "launches_per_sample": [fwd_reps, inv_reps],
                      "timing": f"median of {KERNEL_REPS} samples per kernel, each sample a run of back-to-back "
                                "launches (one launch when a launch takes 1 ms or more) between two hipEvents on "
                                "the launch stream, in a pass after the timed steps"},
        "roofline": {
            "kernel": f"{rot}_{kname} d={w.d} g={w.group}",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
        },
        "valu": read_valu(w.name, rot, kname, w.d),
    }
    result["hbm_copy"] = measured_copy(dev)
    if not args.no_graph:
        result["graph_replay"] = graph_replay(w, sets, replicas, fwd_fn, inv_fn, args.steps, bpv)
    if not args.no_eager:
        result["eager_baseline"] = eager_baseline(w, sets, replicas, rot, ms_step, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, x0, rot, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
