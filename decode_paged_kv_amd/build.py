"""Build libpkv.so in-tree with hipcc for gfx950.

``python -m decode_paged_kv_amd.build`` compiles every source under
``csrc/`` to an object (in parallel) and links ``decode_paged_kv_amd/libpkv.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
CALIB = os.path.join(HERE, "calib")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpkv.so")
# the benchmark's calibration kernels (matrix-core rate and shader clock); not part of libpkv
CALIB_LIB = os.path.join(HERE, "libpkv_calib.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instruction selection anywhere in this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the kernels never produce NaNs (masked scores are -inf next to a finite
    # running max), so max/min need no NaN canonicalisation
    "-fno-honor-nans",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libpkv")
    return path


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", *HIPCC_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{res.stderr}")
    return obj


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile all sources and link libpkv.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra_flags or [])
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    build_calib(extra)
    return LIB


def build_calib(extra: list[str] | None = None) -> str:
    """Compile the calibration kernels into libpkv_calib.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(os.path.join(CALIB, f) for f in os.listdir(CALIB) if f.endswith(".hip"))
    objs = [_compile(src, list(extra or [])) for src in srcs]
    tmp = CALIB_LIB + ".tmp"
    res = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, CALIB_LIB)
    return CALIB_LIB


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
