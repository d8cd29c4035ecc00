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
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpkv.so")
SOURCES = ["pkv_kernels.hip", "pkv_append.hip", "pkv_prefill.hip", "pkv_compress.hip",
           "pkv_noalloc.hip", "pkv_plan.cpp", "pkv_api.cpp"]

# flags of every compile
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
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


_NOISE = "is not a recognized feature for this target"


def _run(cmd: list[str], cwd: str, what: str, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if _NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {what} ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def compile_cmd(src: str, obj: str, save_temps: bool = False) -> list[str]:
    """The hipcc line that compiles one source of the library to an object."""
    cmd = [hipcc(), *HIPCC_FLAGS]
    if save_temps:
        cmd += ["-save-temps=obj"]
    return cmd + ["-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]


def build(save_temps: str | None = None, verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link them into
    libpkv.so in-tree."""
    out_dir = os.path.abspath(save_temps) if save_temps else os.path.join(PKG, "_objs")
    os.makedirs(out_dir, exist_ok=True)
    objs = [os.path.join(out_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1, 8)) as pool:
        futs = [pool.submit(_run, compile_cmd(s, o, bool(save_temps)), out_dir, s, verbose)
                for s, o in zip(SOURCES, objs)]
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], PKG,
         "the link", verbose)
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
