"""Build libmoe.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m mixture_experts_grouped_router_amd.build [-v]

Compiles every ``csrc/*.hip`` / ``csrc/*.cpp`` to an object in
``_build/`` (in parallel), then links ``libmoe.so`` next to this file.
Always recompiles: the call is the "does it build" check.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # GEMM epilogues walk all 256 accumulators of a lane with
                # fully unrolled loops; a partial unroll would index the
                # accumulator array dynamically and move it to scratch
                "-mllvm", "-pragma-unroll-threshold=1000000"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
          "-Wno-unused-result", "-Wno-unused-command-line-argument",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def sources():
    out = []
    for name in sorted(os.listdir(CSRC)):
        if name.endswith(".hip") or name.endswith(".cpp"):
            out.append(os.path.join(CSRC, name))
    return out


def _compile(src: str, verbose: bool, bdir: str = BUILD,
             extra: list | None = None) -> str:
    obj = os.path.join(bdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *(extra or []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        # host pass warns about the device-only feature flag: harmless
        lines = [l for l in r.stderr.splitlines()
                 if "packed-fp32-ops" not in l and l.strip()]
        if lines:
            print("\n".join(lines), flush=True)
    return obj


def build(verbose: bool = False, jobs: int | None = None,
          out: str | None = None, extra: list | None = None) -> str:
    """Compile and link; `out` and `extra` (additional hipcc flags, e.g.
    -D options) build another copy of the library elsewhere."""
    lib = out or LIB
    bdir = BUILD if out is None else out + ".objs"
    os.makedirs(bdir, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)), 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, bdir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
