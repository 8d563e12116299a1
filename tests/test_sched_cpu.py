"""CPU checks of the work-item maps the kernels use (csrc/attn_sched.h), compiled with g++ as host code:
bijections onto (head, tile) items, heads kept on one XCD, persistent rounds that are permutations of
their items, and the persistent grid sized from the compute-unit and XCD counts."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "tiled_online_softmax_02_amd", "csrc")


def test_work_item_maps(tmp_path):
    exe = str(tmp_path / "sched_check")
    cmd = ["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + CSRC,
           os.path.join(HERE, "sched_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail("compile failed:\n" + r.stderr)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
