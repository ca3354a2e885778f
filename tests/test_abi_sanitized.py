"""The C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer: ep_abi.hip is built with both sanitizers on its
host code only and linked with tests/abi_validation_driver.c, which calls
every entry point down its argument checks; nothing reaches the GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_validation_paths_under_sanitizers(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "combine_ep_plan_02_amd", "csrc")]
    abi_o = str(tmp_path / "abi.o")
    drv_o = str(tmp_path / "drv.o")
    exe = str(tmp_path / "abi_validation")
    # the device code is built too (the object must carry its code object),
    # unoptimised enough to keep this test to a few seconds of compile time
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san, *inc, "-c",
                    os.path.join(ROOT, "combine_ep_plan_02_amd", "csrc", "ep_abi.hip"), "-o", abi_o],
                   check=True, capture_output=True)
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", *inc[:2], "-c",
                    os.path.join(ROOT, "tests", "abi_validation_driver.c"), "-o", drv_o],
                   check=True, capture_output=True)
    subprocess.run([HIPCC, *san, drv_o, abi_o, "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
