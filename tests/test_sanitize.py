"""Host builds with AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
the C oracle (oracle/liboracle.c) on edge-case inputs, and the C ABI's
validation and batched-plan layer (w4_api.cpp, compiled for the host with
stub kernel launchers) on valid and invalid arguments.  Each program exits
non-zero on a failed check; a sanitizer report aborts it."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _run(cmd, tmp, exe, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp)
    assert r.returncode == 0, r.stderr[-3000:]
    e = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", **(env or {}))
    r = subprocess.run([exe], capture_output=True, text=True, env=e, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    cmd = ["gcc", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", *SAN,
           os.path.join(ROOT, "oracle", "liboracle.c"), os.path.join(HERE, "oracle_check.c"),
           "-o", exe, "-lm"]
    assert "oracle_check ok" in _run(cmd, str(tmp_path), exe, {"OMP_NUM_THREADS": "2"})


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_api_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_check")
    csrc = os.path.join(ROOT, "weight_only_bit_unpack_amd", "csrc")
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", csrc, os.path.join(csrc, "w4_api.cpp"),
           os.path.join(HERE, "api_check.cpp"), "-o", exe]
    assert "api_check ok" in _run(cmd, str(tmp_path), exe)
