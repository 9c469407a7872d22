"""The oracle and the host planner under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Both are built here with gcc / g++ (host code only: no HIP) into a temporary directory and run as
their own processes:
  * tests/sanitize/oracle_check.c -- every oracle function over all small shapes, with buffers of
    exactly the size each call may touch, plus the tiled-vs-plain self-consistency;
  * tests/sanitize/plan_check.cpp -- edge_masking_vector_amd/csrc/plan.cpp over a grid of shapes,
    strides, bases, tiles and paths, replaying the kernels' index mapping of every accepted plan
    and requiring exact coverage of the tensor (maps) or of its sub-tiles (transpose).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    rc, out = _run(["gcc", "-std=c99", *SAN, "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(ROOT, "tests", "sanitize", "oracle_check.c"),
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV, timeout=600)
    assert rc == 0 and "0 failures" in out, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_planner_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_check")
    rc, out = _run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "sanitize", "plan_check.cpp"),
                    os.path.join(ROOT, "edge_masking_vector_amd", "csrc", "plan.cpp"), "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV, timeout=900)
    assert rc == 0 and " 0 failures" in out, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
