"""Build the HIP library in-tree: paged_kv_cache_36_amd/libpkv.so (gfx950 only).

    python -m paged_kv_cache_36_amd.build [--save-temps DIR]

hipcc cross-compiles for gfx950 without a GPU present.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpkv.so")
SOURCES = ["pkv_kernels.hip", "pkv_append.hip", "pkv_prefill.hip", "pkv_compress.hip",
           "pkv_noalloc.hip", "pkv_plan.cpp", "pkv_api.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    # no packed-fp32 instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: with AGPR accumulators the prefill
    # loop copied its whole accumulator out and back on every key tile
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpkv.so)")


def build(save_temps: str | None = None, verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC]
    if save_temps:
        # -save-temps=obj writes beside the output, so build into that folder
        save_temps = os.path.abspath(save_temps)
        os.makedirs(save_temps, exist_ok=True)
        tmp = os.path.join(save_temps, "libpkv.so.tmp")
        cmd += ["-save-temps=obj", "-o", tmp]
        cwd = save_temps
    else:
        cmd += ["-o", tmp]
        cwd = PKG
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


C_TEST_SRC = os.path.join(ROOT, "tests", "c_abi", "pkv_c_abi_test.cpp")
C_TEST_BIN = os.path.join(ROOT, "tests", "c_abi", "pkv_c_abi_test")


def build_c_test(verbose: bool = False) -> str:
    """The C++ test program of the C ABI (host code only: hipMalloc'd buffers
    and the library's entry points, no Python), linked against the in-tree
    libpkv.so. Build the library first."""
    cmd = [hipcc(), "--offload-arch=gfx950", "-O2", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", INCLUDE, C_TEST_SRC, "-o", C_TEST_BIN + ".tmp",
           "-L", PKG, "-lpkv", "-Wl,-rpath,$ORIGIN/../../paged_kv_cache_36_amd"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
        raise RuntimeError(f"hipcc failed on the C ABI test ({res.returncode}):\n{err}")
    os.replace(C_TEST_BIN + ".tmp", C_TEST_BIN)
    return C_TEST_BIN


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.save_temps, args.verbose))
    print(build_c_test(args.verbose))


if __name__ == "__main__":
    main()
