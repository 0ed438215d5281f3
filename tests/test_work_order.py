"""The work-order maps shared by the grouped GEMMs and the one-token kernels
(XCD-contiguous ranges, column groups of row tiles) are bijections: compiled
for the host from the library's own header and run on the CPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "sparse_mixture_experts_amd", "csrc")


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not found")
def test_work_order_maps_are_bijections(tmp_path):
    exe = str(tmp_path / "work_order")
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-O1", "-I", CSRC, os.path.join(HERE, "host", "work_order.cpp"),
                    "-o", exe], check=True, capture_output=True)
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0 and "bad=0" in out.stdout, out.stdout + out.stderr
