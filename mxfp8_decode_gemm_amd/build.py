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


# Host-side sanitizers for the C-ABI layer only (argument validation, size
# arithmetic, descriptor handling): api.hip's host code is compiled with
# AddressSanitizer and UndefinedBehaviorSanitizer (-Xarch_host: the device
# code is built as usual) and linked with the regular objects of the other
# sources. Loading it needs the ASan runtime preloaded (HOST_ASAN_RUNTIME).
HOST_SAN_LIB = os.path.join(LIBDIR, "libmxgemm_hostsan.so")
HOST_SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
]


def host_asan_runtime() -> str:
    """The clang ASan runtime of this ROCm toolchain (for LD_PRELOAD)."""
    import glob

    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("the clang ASan runtime was not found under /opt/rocm/llvm")
    return hits[-1]


def build_host_sanitized(verbose: bool = False) -> str:
    """Build libmxgemm_hostsan.so (after build(): it reuses its objects)."""
    hipcc = _hipcc()
    srcs = sources()
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    api = os.path.join(CSRC, "api.hip")
    san_obj = os.path.join(BUILD, "api.hostsan.o")
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"]
    _run([hipcc, *flags, *HOST_SAN_FLAGS, "-c", api, "-o", san_obj])
    others = [o for s, o in zip(srcs, objs) if os.path.basename(s) != "api.hip"]
    tmp = HOST_SAN_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *HOST_SAN_FLAGS, "-o", tmp, san_obj,
          *others])
    os.replace(tmp, HOST_SAN_LIB)
    if verbose:
        print(f"built {HOST_SAN_LIB}")
    return HOST_SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
