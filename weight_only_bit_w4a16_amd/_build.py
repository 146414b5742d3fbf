"""Build the gfx950 HIP library ``libw4a16.so`` in-tree with hipcc.

Each source compiles to an object in ``_build/`` (in parallel), then one
shared link.  Packed-fp32 VALU forms are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libw4a16.so")
PROBE_LIB = os.path.join(PKG, "libw4a16_probe.so")  # measurement kernels (bench.py --bounds)
PROBE_SOURCES = ["probe.hip"]
SOURCES = ["api.cpp", "dequant.hip", "skinny.hip", "mid.hip", "tiled.hip", "ragged.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip():
        print(out)
    return obj


def _link(lib: str, objs) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.check_call(cmd)
    os.replace(tmp, lib)


def build(jobs: int = 4) -> str:
    """Build libw4a16.so (the GEMM library) and libw4a16_probe.so (the
    measurement kernels); returns the GEMM library's path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(LIB, objs[:len(SOURCES)])
    _link(PROBE_LIB, objs[len(SOURCES):])
    return LIB


if __name__ == "__main__":
    print(build())
