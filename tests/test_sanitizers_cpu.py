"""The oracle and the library's host-only code built with AddressSanitizer and
UndefinedBehaviorSanitizer and run on the CPU (no GPU code is built this way): every
out-of-range access or undefined operation stops the run with a report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, exe, tmp_path):
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0", OMP_NUM_THREADS="4")
    p = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "AddressSanitizer" not in p.stderr and "runtime error" not in p.stderr, p.stderr
    return p.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    out = _run(["gcc", *SAN, "-fopenmp", "-std=c11", "-Wall", "-o", exe,
                os.path.join(HERE, "oracle_sanitize.c"), os.path.join(ROOT, "oracle", "kev_oracle.c"), "-lm"],
               exe, tmp_path)
    assert "all checks passed" in out


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_sanitize")
    out = _run(["g++", *SAN, "-std=c++17", "-Wall", "-o", exe, os.path.join(HERE, "host_sanitize.cpp"),
                os.path.join(ROOT, "segment_isolated_packed_amd", "csrc", "kev_host.cpp")], exe, tmp_path)
    assert "all checks passed" in out
