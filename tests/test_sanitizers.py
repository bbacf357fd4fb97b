"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Two small drivers are built with the sanitizers and run: one takes the
oracle over ragged sizes, non-finite values and both 8-bit formats with
exactly sized buffers; the other takes the library's host side (list
validation, chunking, workspace tables, argument checks of every entry
point) through valid and invalid lists with stand-ins for the kernel
launchers that abort if reached.  No GPU code is built with a sanitizer."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")


def run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", *SAN, "-fsanitize=float-cast-overflow", "-std=c11", "-ffp-contract=off",
                    "-o", exe, os.path.join(HERE, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], check=True)
    assert "oracle driver ok" in run(exe)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_the_build_catches_a_planted_overrun(tmp_path):
    exe = str(tmp_path / "oracle_driver_short")
    subprocess.run(["gcc", *SAN, "-std=c11", "-ffp-contract=off", "-DPLANTED_OVERRUN", "-o", exe,
                    os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
                    "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="no g++ or ROCm headers")
def test_library_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_driver")
    subprocess.run(["g++", *SAN, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-o", exe, os.path.join(HERE, "host_driver.cpp"),
                    os.path.join(HERE, "no_launch.cpp"),
                    os.path.join(ROOT, "mixed_precision_sharded_amd", "csrc", "api.cpp"),
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    assert "host driver ok" in run(exe)
