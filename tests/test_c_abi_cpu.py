"""The plain-C test program builds with gcc against include/mxmoe.h alone
and resolves libmxmoe.so and the oracle next to it (CPU only; the GPU run is
tests/test_c_abi_gpu.py)."""

import os
import subprocess

from tests.c_abi import build as c_build


def test_c_program_builds_and_links(tmp_path):
    if not os.path.exists(c_build.EXE):
        c_build.build()
    out = subprocess.run(["ldd", c_build.EXE], capture_output=True, text=True, check=True).stdout
    assert "not found" not in out, out
    libs = {ln.split()[0]: ln.split("=>")[1].split("(")[0].strip()
            for ln in out.splitlines() if "=>" in ln}
    root = os.path.dirname(os.path.dirname(c_build.HERE))
    assert os.path.realpath(libs["libmxmoe.so"]) == os.path.join(
        root, "combine_topk_ids_expert_amd", "libmxmoe.so")
    assert os.path.realpath(libs["liboracle.so"]) == os.path.join(root, "oracle", "liboracle.so")
