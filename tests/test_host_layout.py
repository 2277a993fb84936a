"""Host logic without a GPU: the workspace layout (moe_groupgemm_amd/csrc/mk_common.h) is
compiled with g++ into tests/host_layout_check.cpp, which checks that the layout grows with
the capacity and that a workspace sized for cap tokens holds every array, task index, queue
slot and trace record of every batch B <= cap under adversarial routing histograms."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "moe_groupgemm_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_workspace_layout_holds_every_batch(tmp_path):
    exe = str(tmp_path / "host_layout_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-I", CSRC, os.path.join(HERE, "host_layout_check.cpp"),
                    "-o", exe], check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout[-4000:]
    assert " 0 failures" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_capacity_lookups_from_two_threads_on_one_plan(tmp_path):
    exe = str(tmp_path / "host_capacity_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-pthread", "-I", CSRC,
                    os.path.join(HERE, "host_capacity_check.cpp"), "-o", exe], check=True, capture_output=True,
                   text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout[-4000:]
    assert " 0 failures" in r.stdout
