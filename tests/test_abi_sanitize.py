"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU, no GPU).

abi.cpp (argument checks, workspace plans, status strings, the device check) is rebuilt with
both sanitizers on its host code only, linked with the library's kernel objects and
tests/abi_sanitize_driver.cpp, which calls every entry point with bad arguments, the host-only
functions over their argument ranges, and valid arguments up to the device check (there is no
GPU here, so nothing is launched). A sanitizer finding aborts the driver.
"""
import glob
import os
import shutil
import subprocess

import pytest

from block_sparse_linear_pool_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# sanitizers on host code only: each flag right after -Xarch_host
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.mark.timeout(300)
def test_abi_host_code_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    kernels = sorted(glob.glob(os.path.join(build.BUILD_DIR, "*.hip.o")))
    if len(kernels) < 7:
        build.build()
        kernels = sorted(glob.glob(os.path.join(build.BUILD_DIR, "*.hip.o")))
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *SAN]
    abi_o, drv_o, exe = (str(tmp_path / n) for n in ("abi.o", "drv.o", "drv"))
    steps = [
        [HIPCC, *common, "-fPIC", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form", "-x", "hip", "-c",
         os.path.join(build.CSRC, "abi.cpp"), "-o", abi_o],
        [HIPCC, *common, "-x", "hip", "-c", os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp"),
         "-o", drv_o],
        [HIPCC, "--offload-arch=gfx950", *SAN[:4], drv_o, abi_o, *kernels, "-o", exe],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert r.stdout.startswith("ok: 0 unexpected")
