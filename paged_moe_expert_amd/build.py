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

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "librimuru.so")
SOURCES = [os.path.join(HERE, "csrc", "allocator.cpp"),
           os.path.join(HERE, "csrc", "moe_kernels.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (set HIPCC)")


def flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function",
            # packed fp32 VALU forms stay off: plain fp32 code only
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile the library to `out`; defines are extra -D macros (tile tuning)."""
    tmp = out + ".tmp"
    cmd = [hipcc()] + flags() + [f"-D{d}" for d in defines] + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
