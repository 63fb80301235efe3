"""Build libssmscan.so (HIP kernels for gfx950 + the C ABI) in the package directory.

    python -m selective_state_space_49_amd.build

Every HIP translation unit is compiled with floating-point contraction off (the
kernels write their fused multiply-adds explicitly) and with packed fp32 math
disabled. The library is placed next to this file so that it travels with the
source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libssmscan.so")
OBJDIR = os.path.join(HERE, "_build")

ARCH = "gfx950"
HIP_SOURCES = ["scan_real.hip", "scan_complex.hip", "step.hip", "scan_bwd.hip", "scan_mimo.hip",
               "input_bwd.hip", "scratch.hip"]
CPP_SOURCES = ["api.cpp"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _compile(src: str, verbose: bool, objdir: str, defines) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *[f"-D{d}" for d in defines]]
    if src.endswith(".hip"):
        cmd += DEVICE
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source and link libssmscan.so; returns the library path.

    out and defines (NAME=VALUE strings, e.g. build-time tuning knobs) allow
    building variants elsewhere; the default is the package's own library.
    """
    objdir = OBJDIR if out == LIB else out + ".objs"
    os.makedirs(objdir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, objdir, defines), HIP_SOURCES + CPP_SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libssmscan.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
