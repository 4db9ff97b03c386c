"""Build libmxmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc,
and its bounds-checked twin libmxmoe_checked.so (the same sources with
MXMOE_CHECKED defined: every kernel access is checked against the call's
arrays; a debugging library, see mx_bounds_checked in include/mxmoe.h).

    python -m combine_topk_ids_expert_amd.build            # both
    python -m combine_topk_ids_expert_amd.build --product  # libmxmoe.so only

The libraries are written next to this file, where the binding loads them.
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
LIB_CHECKED = os.path.join(PKG, "libmxmoe_checked.so")
CHECKED_FLAGS = ["-DMXMOE_CHECKED=1"]
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


def build_checked(out_path: str = LIB_CHECKED, verbose: bool = False) -> str:
    return build(out_path, CHECKED_FLAGS, verbose)


def build_all(verbose: bool = False) -> list[str]:
    """Both libraries, compiled side by side."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(2) as pool:
        jobs = [pool.submit(build, LIB, None, verbose), pool.submit(build_checked, LIB_CHECKED, verbose)]
        return [j.result() for j in jobs]


if __name__ == "__main__":
    v = "-v" in sys.argv
    if "--product" in sys.argv:
        print(build(verbose=v))
    else:
        print("\n".join(build_all(verbose=v)))
