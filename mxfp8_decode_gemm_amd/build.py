"""Build the HIP library libmxgemm.so for gfx950 with hipcc (in-tree).

Usage: python -m mxfp8_decode_gemm_amd.build   (or build() from Python).
Every .hip file under csrc/ is compiled to an object in parallel, then
linked into mxfp8_decode_gemm_amd/lib/libmxgemm.so.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(LIBDIR, "libmxgemm.so")
ARCH = "gfx950"

# -packed-fp32-ops: no packed FP32 VALU instructions in any kernel.
# atomic optimizer off: it rewrites a one-lane counter atomic into a wave
# scan whose result is waited for at once, which would hold the workgroup
# for a device-scope round trip where the count's result is needed only at
# the end of the kernel.
# FP32 denormals kept (the default, stated): the activation quantizer scales
# BF16 subnormals exactly by a power of two before converting them.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return exe


def _run(cmd: list[str]) -> None:
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False) -> str:
    """Compile and link the library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs]
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as pool:
        futs = [pool.submit(_run, [hipcc, *HIPCC_FLAGS, "-c", s, "-o", o])
                for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
