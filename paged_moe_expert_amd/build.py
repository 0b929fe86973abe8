"""Build librimuru.so in-tree with hipcc for gfx950.

    python -m paged_moe_expert_amd.build

Compiles the host allocator and the HIP kernels into one shared library next
to this file. Always recompiles; the result replaces the old library only
once the compiler has succeeded.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "librimuru.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in
           ("allocator.cpp", "moe_routing.hip", "moe_gemm_stream.hip", "moe_gemm_tiled.hip", "moe_gemm_prefill.hip",
            "moe_layer.hip", "expert_upload.cpp", "adjuster.cpp", "attention.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (set HIPCC)")


def flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Wall", "-Wno-unused-function",
            # packed fp32 VALU forms stay off: plain fp32 code only
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile the library to `out`; defines are extra -D macros (tile tuning).

    Translation units compile in parallel to objects beside `out`, then link."""
    dflags = [f"-D{d}" for d in defines]
    noise = "is not a recognized feature for this target"

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msg}")
        if verbose and msg.strip():
            print(msg)

    objdir = out + ".objs"
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in SOURCES]
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        list(ex.map(lambda so: run([hipcc()] + flags() + dflags + ["-c", so[0], "-o", so[1]]),
                    zip(SOURCES, objs)))
    tmp = out + ".tmp"
    run([hipcc()] + flags() + ["-shared"] + objs + ["-o", tmp])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
