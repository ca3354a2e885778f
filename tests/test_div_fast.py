"""The quantising kernels' per-row division, emulated on the host with fmaf
(tests/div_fast_check.c), against IEEE binary32 division: the refined row
reciprocal over every mantissa from both floats around 1/s (the accuracy
v_rcp_f32 is specified to), and the quotients at and around every E4M3FN and
int8 rounding boundary, at powers of two, all-ones mantissas and log-uniform
scales over the fast path's range [2^-60, 2^60]."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _cpu_has_fma() -> bool:
    try:
        return " fma " in open("/proc/cpuinfo").read().replace("\n", " ")
    except OSError:
        return False


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_row_division_matches_ieee(tmp_path):
    exe = str(tmp_path / "div_fast_check")
    flags = ["-O2", "-std=c11", "-Wall", "-ffp-contract=off", "-fno-fast-math"]
    if _cpu_has_fma():
        flags.append("-mfma")       # fmaf inline; without it libm's fmaf is exact too
    subprocess.run(["gcc", *flags, "-o", exe, os.path.join(HERE, "div_fast_check.c"), "-lm"],
                   check=True)
    res = subprocess.run([exe, "20000", "300", "11"], capture_output=True, text=True, timeout=600)
    print(res.stdout)
    assert res.returncode == 0, res.stdout
    lines = dict(l.split(" ", 1) for l in res.stdout.strip().splitlines() if not l.startswith("mismatch"))
    assert lines["reciprocals"].startswith("50331648 mismatches 0")
    assert lines["quotients"].endswith("mismatches 0")
