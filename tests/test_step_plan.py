"""Host logic of the M = 1 step kernel's row plan (csrc/step_plan.h): built
with the host compiler and run on the CPU (tests/step_plan_check.cpp)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_INCLUDE = "/opt/rocm/include"


def test_step_row_plan(tmp_path):
    cxx = shutil.which("g++")
    if not cxx or not os.path.exists(os.path.join(HIP_INCLUDE, "hip", "hip_runtime.h")):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path / "step_plan_check")
    subprocess.run([cxx, "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE,
                    "-I", os.path.join(ROOT, "verify_gemm_amd", "csrc"),
                    os.path.join(ROOT, "tests", "step_plan_check.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.splitlines()
    layer = [ln for ln in lines if ln.startswith("layer job")]
    # q, k, v on disjoint runs of workgroups covering the grid; gate and up
    # on halves; o, down and the lm_head on every workgroup
    runs = [(int(ln.split("wg0=")[1].split()[0]), int(ln.split("wgn=")[1])) for ln in layer]
    assert runs[:3] == [(0, 86), (86, 85), (171, 85)]
    assert runs[3] == (0, 256) and runs[6] == (0, 256) and runs[7] == (0, 256)
    assert runs[4:6] == [(0, 128), (128, 128)]
    # the stage of tests/test_gpu_pass.py::test_step_stage_spread_over_grid:
    # every matrix on the whole grid, the 300-row one's extra rows from
    # workgroup 235 on, wrapping past the last workgroup
    spread = [ln for ln in lines if ln.startswith("spread job")]
    assert [ln.split("wg0=")[1] for ln in spread] == ["0 wgn=256 rr=235", "235 wgn=256 rr=0", "235 wgn=256 rr=44"]
    assert lines[-1] == "random cases ok: 3000"
