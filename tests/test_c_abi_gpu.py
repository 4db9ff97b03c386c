"""The library from plain C on the GPU: tests/c_abi/end_to_end.c drives
prepare -> dispatch -> combine, prepare_dispatch and the no-alloc routing
through include/mxmoe.h with the HIP runtime alone (no Python, no PyTorch in
that process) and compares every output byte with the CPU oracle; it then
prints the host and GPU time per call at the decode shape."""

import os
import subprocess

import pytest

from tests.c_abi import build as c_build


@pytest.mark.gpu
def test_c_program_matches_oracle():
    if not os.path.exists(c_build.EXE):
        pytest.fail(f"{c_build.EXE} is missing: build it with `python -m tests.c_abi.build` "
                    "(the driver's build() does)")
    print("c_abi end_to_end: running", c_build.EXE, flush=True)
    proc = subprocess.run([c_build.EXE, "--host-cost"], capture_output=True, text=True,
                          timeout=240)
    print(proc.stdout, flush=True)
    assert proc.returncode == 0, proc.stderr[-3000:] + proc.stdout[-2000:]
    assert proc.stdout.count(": ok\n") == 5, proc.stdout
    assert "every case matches the oracle" in proc.stdout
    assert proc.stdout.count("host_cost: ") == 4, proc.stdout
