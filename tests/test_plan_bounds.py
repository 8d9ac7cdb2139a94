"""The work-decomposition formulas shared by the host sizing and the planner kernel, built for
the host and checked without a GPU: a call sized for a capacity (graph_max_seq_len) never
gets more work items on the device than the host sized its lists and grids for, whatever
the device lengths (padding rows of length 0 included).  See tests/host/plan_bounds.cpp."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def plan_bounds_exe(tmp_path_factory):
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    exe = str(tmp_path_factory.mktemp("plan_bounds") / "plan_bounds")
    src = os.path.join(ROOT, "tests", "host", "plan_bounds.cpp")
    inc = os.path.join(ROOT, "paged_kv_attention_05_amd", "csrc")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-x", "hip", "-I", inc, src, "-o", exe],
                   check=True, capture_output=True, text=True)
    return exe


def test_capacity_sized_plans_never_outgrow_the_host_sizing(plan_bounds_exe):
    res = subprocess.run([plan_bounds_exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "checked" in res.stdout
