"""Build libmxmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m combine_topk_ids_expert_amd.build

The library is written next to this file, where the binding loads it.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmxmoe.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # Only explicitly written fused multiply-adds; no contraction of a*b+c.
    "-ffp-contract=off",
    # Keep the compiler from forming packed fp32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(out_path: str = LIB, extra_flags: list[str] | None = None, verbose: bool = False) -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    tmp = out_path + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *(extra_flags or []), "-I", os.path.join(ROOT, "include"),
           *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
