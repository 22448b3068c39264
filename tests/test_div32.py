"""Host-side check of the multiply-high division the kernels use for the
per-row seed rule seed + ((r / rows_per_seed) % seed_period).

The header is compiled into a small host program that compares div32 and
seed_of_block(seed_block(r)) with plain integer division over edge cases and
random draws; no GPU is involved."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

PROGRAM = r"""
#include <stdio.h>
#include <stdlib.h>
#include "rtq_div.hpp"
using namespace rtq;
int main() {
  unsigned d, n; unsigned long long seed; unsigned rps, per, row;
  char op[8];
  long bad = 0, count = 0;
  while (scanf("%7s", op) == 1) {
    if (op[0] == 'D') {
      if (scanf("%u %u", &d, &n) != 2) return 2;
      const Div32 v = make_div32(d);
      if (div32(n, v) != n / d) { if (bad < 5) printf("div %u / %u -> %u\n", n, d, div32(n, v)); ++bad; }
    } else {
      if (scanf("%llu %u %u %u", &seed, &rps, &per, &row) != 4) return 2;
      SeedRule s{seed, rps, per, make_div32(rps ? rps : 1), make_div32(per ? per : 1)};
      unsigned long long blk = rps ? row / rps : 0;
      unsigned long long want = seed + (per ? blk % per : blk);
      unsigned long long got = seed_of_block(seed_block(row, s), s);
      if (got != want) { if (bad < 5) printf("seed %llu %u %u %u -> %llu want %llu\n", seed, rps, per, row, got, want); ++bad; }
    }
    ++count;
  }
  printf("checked %ld bad %ld\n", count, bad);
  return bad != 0;
}
"""


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("div32")
    src = d / "div32_check.cpp"
    src.write_text(PROGRAM)
    exe = d / "div32_check"
    cmd = [HIPCC, "-O2", "-std=c++20", "-I", os.path.join(ROOT, "rotate_then_quantize_amd", "csrc"),
           str(src), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    return str(exe)


def run_checker(exe, lines):
    out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert f"checked {len(lines)} bad 0" in out.stdout


def test_div32_matches_integer_division(checker):
    rng = np.random.default_rng(5)
    top = 0xFFFFFFFF
    divisors = [1, 2, 3, 5, 7, 10, 37, 63, 64, 65, 100, 641, 1 << 16, 65537, 6700417,
                (1 << 31) - 1, 1 << 31, (1 << 31) + 1, top - 1, top]
    divisors += [int(v) for v in rng.integers(1, top, 40, dtype=np.uint64)]
    lines = []
    for d in divisors:
        ns = {0, 1, d - 1, d, d + 1, 2 * d - 1, 2 * d, top, top - 1, top - d % (1 << 32)}
        q = top // d
        ns |= {q * d - 1, q * d, min(q * d + d - 1, top)}
        ns |= {int(v) for v in rng.integers(0, top, 200, dtype=np.uint64)}
        lines += [f"D {d} {n}" for n in sorted(ns) if 0 <= n <= top]
    run_checker(checker, lines)


def test_seed_rule_matches_definition(checker):
    rng = np.random.default_rng(6)
    lines = []
    for rps, per in [(0, 0), (0, 5), (1, 0), (1, 7), (10, 3), (37, 5), (64, 0), (100, 2), (4097, 16),
                     (1 << 20, 3), (0xFFFFFF00, 2)]:
        seed = int(rng.integers(0, 1 << 63, dtype=np.uint64)) * 2 + 1
        rows = {0, 1, 63, 64, 0xFFFFFEFF} | {int(v) for v in rng.integers(0, 0xFFFFFF00, 100, dtype=np.uint64)}
        if rps:
            rows |= {rps - 1, rps, rps * 3 - 1, rps * 3}
        lines += [f"S {seed} {rps} {per} {r}" for r in sorted(rows) if r < 1 << 32]
    # the 64-bit seed wraps modulo 2^64
    lines.append(f"S {(1 << 64) - 2} 1 0 5")
    run_checker(checker, lines)
