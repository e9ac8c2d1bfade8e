"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code: the
planner (hca_plan.cpp, with a driver that builds plans over random and edge
configurations and reads every export back) and the CPU oracle (with a driver
running every pass in every mode and input type).  Host compilers only (g++ /
gcc); no GPU code is built here.  Any sanitizer report fails the run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="no host compiler")


def test_planner_under_asan_ubsan(tmp_path):
    exe = tmp_path / "plan_driver"
    subprocess.check_call(["g++", "-std=c++17"] + SAN + [
        "-I" + os.path.join(ROOT, "include"),
        "-I" + os.path.join(ROOT, "block_sparse_compressed_amd", "csrc"),
        os.path.join(HERE, "plan_driver.cpp"),
        os.path.join(ROOT, "block_sparse_compressed_amd", "csrc", "hca_plan.cpp"),
        "-o", str(exe)])
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-5000:]
    assert "failures 0" in res.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_driver"
    subprocess.check_call(["gcc", "-std=c11", "-fopenmp"] + SAN + [
        os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "hca_oracle.c"),
        "-lm", "-o", str(exe)])
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-5000:]
    assert "oracle problems 24" in res.stdout
