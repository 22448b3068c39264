"""Build librtq.so (the HIP kernels and the C ABI) in-tree for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "librtq.so")
SOURCES = [os.path.join(PKG_DIR, "csrc", "rtq.hip"), os.path.join(PKG_DIR, "csrc", "rtq_attn.hip")]
HEADERS = [os.path.join(PKG_DIR, "csrc", "rtq_device.hpp"), os.path.join(PKG_DIR, "csrc", "rtq_div.hpp"),
           os.path.join(PKG_DIR, "csrc", "rtq_mem.hpp"), os.path.join(ROOT, "include", "rtq.h")]


def hipcc_command(out: str = LIB_PATH, extra: list[str] | None = None) -> list[str]:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return [
        hipcc, "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-shared",
        "-fvisibility=hidden", "-I", os.path.join(ROOT, "include"),
        # no packed fp32 (v_pk_*_f32) anywhere in the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        *(extra or []), "-o", out, *SOURCES,
    ]


def build_library(verbose: bool = False) -> str:
    """Compile librtq.so every time it is called; return its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-4000:]}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
