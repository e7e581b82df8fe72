"""The LDS ring's tile layout, checked on the CPU: a host program built from
the kernel header's own helpers walks every copy slot, every MFMA reader
offset and the bank spread (tests/lds_layout_check.hip)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_lds_ring_layout(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "lds_layout_check")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{ROOT}/include", f"-I{ROOT}/varlen_attention_serving_amd/csrc",
           os.path.join(ROOT, "tests", "lds_layout_check.hip"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout
