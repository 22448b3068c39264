"""Host logic of bench.py that needs no GPU: the algorithmic byte counts
behind the roofline, argument checks, and the kernel source lists that the
profile summaries are keyed on."""
import os
import subprocess
import sys

import bench
from rotate_then_quantize_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_attention_bytes_closed_form():
    w = W.WORKLOADS[3]  # 28 layers x 128 streams x 2049 tokens, d = 128, g = 32, 6 queries
    rows = 28 * 2 * 128 * 2049
    per_row = 128 // 2 + 2 * (128 // 32)          # codes + fp16 scales
    qo = 2 * 28 * 128 * 6 * 128 * 2               # queries in, outputs out
    assert bench.attn_bytes(w) == rows * per_row + qo == 1_068_490_752
    window = 28 * 2 * 128 * 16 * 128 * 2          # fp16 K and V rows of 16 window tokens
    assert bench.attn_bytes(w, 16) == 1_068_490_752 + window


def test_forward_inverse_bytes_per_vector():
    # fp16 in/out + int4 codes + fp16 scales: 2d + d/2 + 2d/g
    for wid, per in [(1, 162), (2, 164), (3, 328), (4, 162), (5, 656)]:
        w = W.WORKLOADS[wid]
        assert w.bytes_per_vector() == per
        assert bench.role_bytes(w, "dequant_inv") == w.n_rows * per


def test_profile_source_lists_exist():
    for role in ("quant_fwd", "dequant_inv", "attn_decode"):
        for d in (64, 128, 256):
            srcs = bench.kernel_sources(role, d)
            assert srcs and all(os.path.isfile(s) for s in srcs), (role, d, srcs)
    assert any(s.endswith("rtq_pair.hpp") for s in bench.kernel_sources("quant_fwd", 256))
    assert not any(s.endswith("rtq_pair.hpp") for s in bench.kernel_sources("quant_fwd", 64))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_window_needs_attention_and_a_size_in_range():
    for args in (["--window", "3"], ["--attn", "--window", "65"]):
        r = run_bench(*args)
        assert r.returncode == 2 and "--window takes 1 to 64 tokens" in r.stderr, (args, r.stderr[-300:])


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr), (r.stdout + r.stderr)[-300:]


def test_host_info_names_the_cpu():
    info = bench.host_info()
    assert info["affinity_cores"] >= 1 and isinstance(info["cpu_model"], str)
