"""The combine kernel's row loads, read from its gfx950 assembly (CPU only).

Each wave of combine_vec_kernel issues the k row loads of a token before it
waits for any of them.  A compiler wait between two of those loads
serializes them and halves the kernel's bandwidth, with identical results,
so no parity test sees it; this test compiles combine.hip for gfx950 and
checks every instantiation's row loads (the non-temporal ones) for an
`s_waitcnt vmcnt` between them.
"""

import os
import re
import shutil
import subprocess

import pytest

from combine_topk_ids_expert_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "combine_topk_ids_expert_amd", "csrc", "combine.hip")


@pytest.fixture(scope="module")
def combine_asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    out = tmp_path_factory.mktemp("isa") / "combine.s"
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run([hipcc, *flags, "-I", os.path.join(ROOT, "include"), "--cuda-device-only",
                    "-S", SRC, "-o", str(out)], check=True, capture_output=True)
    return out.read_text()


def _kernels(asm: str, prefix: str):
    for m in re.finditer(r"^(_ZN\w*%s\w*):" % prefix, asm, re.M):
        start = m.start()
        yield m.group(1), asm[start:asm.index(".Lfunc_end", start)].splitlines()


def test_row_loads_are_issued_together(combine_asm):
    seen = 0
    for name, body in _kernels(combine_asm, "combine_vec_kernel"):
        loads = [i for i, ln in enumerate(body)
                 if re.search(r"^\s*global_load_dwordx[24]\b.*\bnt\b", ln)]
        assert len(loads) >= 8, name
        waits = [a for a, b in zip(loads, loads[1:])
                 if any("s_waitcnt vmcnt" in body[i] for i in range(a + 1, b))]
        assert not waits, f"{name}: a wait between row loads at lines {waits[:4]}"
        seen += 1
    # 3 y dtypes x 3 output dtypes x 4 weight forms x 2 store policies
    assert seen == 72
