"""The kernels' work decomposition on the host: `xcd_remap` (whole (b, h) groups dealt round-robin
over the XCDs) is a permutation of the workgroup ids for every launch shape, and `block_work` then
gives each (split, b*H + h, Q tile) to exactly one workgroup.  The check program includes the
kernels' own header (`csrc/attn_common.h`), built with hipcc for the host; no GPU is used."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_work_decomposition_is_a_bijection(tmp_path):
    exe = tmp_path / "block_order_check"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I",
                    os.path.join(ROOT, "transformer_scaled_dot_amd", "csrc"), "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi", "block_order_check.hip"), "-o", str(exe)],
                   check=True, capture_output=True, timeout=300)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ")
