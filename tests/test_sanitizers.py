"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code (CPU
only): the fp64 oracle (attnres_oracle.c) run over every function on small
inputs, and the C front end (attnres_api.cpp, with stub launchers) driven
through every entry point's validation paths.  Any invalid memory access,
leak or undefined behaviour aborts the driver (-fno-sanitize-recover=all)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]


def _run(cmd, cwd):
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", *SAN, "-Wall", "-Wno-unknown-pragmas", "-o", exe,
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "attnres_oracle.c"),
          "-lm"], tmp_path)
    out = _run([exe], tmp_path)
    assert "0 failures" in out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers not found")
def test_front_end_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "api_san")
    csrc = os.path.join(ROOT, "depth_wise_attention_attnres_amd", "csrc")
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I" + os.path.join(ROOT, "include"), "-I" + csrc, "-o", exe,
          os.path.join(csrc, "attnres_api.cpp"), os.path.join(HERE, "api_stubs.cpp"),
          os.path.join(HERE, "api_driver.cpp"), "-pthread"], tmp_path)
    out = _run([exe], tmp_path)
    assert "0 failures" in out
