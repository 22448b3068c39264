"""Build librtq.so (the HIP kernels and the C ABI) in-tree for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "librtq.so")
CSRC = os.path.join(PKG_DIR, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("rtq.hip", "rtq_attn.hip", "rtq_cache.hip", "rtq_ext.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("rtq_device.hpp", "rtq_div.hpp", "rtq_mem.hpp", "rtq_lane.hpp",
                                           "rtq_host.hpp", "rtq_pair.hpp")] + [os.path.join(ROOT, "include", "rtq.h")]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-fvisibility=hidden",
    "-I", os.path.join(ROOT, "include"),
    # no packed fp32 (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def hipcc_command(out: str = LIB_PATH, extra: list[str] | None = None) -> list[str]:
    """One command that compiles and links every source (used for one-off variant builds)."""
    return [_hipcc(), *FLAGS, "-shared", *(extra or []), "-o", out, *SOURCES]


def build_library(verbose: bool = False, extra: list[str] | None = None, out: str = LIB_PATH) -> str:
    """Compile every source in parallel and link librtq.so, every time it is called; return its path."""
    with tempfile.TemporaryDirectory(prefix="rtq_build_") as tmp:
        objs, cmds = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            objs.append(obj)
            cmds.append([_hipcc(), *FLAGS, *(extra or []), "-c", src, "-o", obj])
        workers = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))

        def run(cmd):
            if verbose:
                print(" ".join(cmd), flush=True)
            return subprocess.run(cmd, capture_output=True, text=True)

        with ThreadPoolExecutor(workers) as pool:
            results = list(pool.map(run, cmds))
        for cmd, res in zip(cmds, results):
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed ({res.returncode}) on {cmd[-3]}:\n{res.stderr[-4000:]}")
        tmp_lib = out + ".tmp"
        link = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib, *objs]
        res = run(link)
        if res.returncode != 0:
            raise RuntimeError(f"link failed ({res.returncode}):\n{res.stderr[-4000:]}")
        os.replace(tmp_lib, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
