"""Build libqg.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run ``python -m gemm_qgemv_amd.build``; ``__graft_entry__.build()`` calls
``build()``. The library is written next to this file and loaded from there.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "qg.hip")
OUT = os.path.join(HERE, "libqg.so")
PROBE_SRC = os.path.join(HERE, "csrc", "probe.hip")
PROBE_OUT = os.path.join(HERE, "libqgprobe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # IEEE float32: no fast-math, fp32 denormals kept
    "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero",
    # no packed-FP32 instructions (plain float code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(out: str = OUT, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Build libqg.so and the measurement-only libqgprobe.so."""
    _hipcc(PROBE_SRC, PROBE_OUT, extra, verbose)
    return _hipcc(SRC, out, extra, verbose)


def _hipcc(src: str, out: str, extra: list[str] | None, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed to build {os.path.basename(out)}")
    errs = [l for l in res.stderr.splitlines()
            if "warning" in l and "packed-fp32-ops" not in l]
    if errs and verbose:
        sys.stderr.write("\n".join(errs) + "\n")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
