"""Build the plain-C end-to-end test program (end_to_end.c).

It is host C, compiled with gcc against the HIP runtime, include/mxmoe.h and
two libraries found next to it at run time: libmxmoe.so (the product) and
liboracle.so (the CPU oracle, test infrastructure).  Both must be built
first (combine_topk_ids_expert_amd.build, oracle.build).

    python -m tests.c_abi.build
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "end_to_end.c")
EXE = os.path.join(HERE, "end_to_end")
PKG = os.path.join(ROOT, "combine_topk_ids_expert_amd")
ORACLE = os.path.join(ROOT, "oracle")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    for lib in (os.path.join(PKG, "libmxmoe.so"), os.path.join(ORACLE, "liboracle.so")):
        if not os.path.exists(lib):
            raise FileNotFoundError(f"{lib} is missing: build the library and the oracle first")
    rpath = "$ORIGIN/../../combine_topk_ids_expert_amd:$ORIGIN/../../oracle:" + f"{ROCM}/lib"
    tmp = EXE + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", f"{ROCM}/include", "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp,
           "-L", PKG, "-lmxmoe", "-L", ORACLE, "-loracle", "-L", f"{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{rpath}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
