"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Two small drivers are built with the sanitizers and run: one takes the
oracle over ragged sizes, non-finite values and both 8-bit formats with
exactly sized buffers; the other takes the library's host side (list
validation, chunking, workspace tables, argument checks of every entry
point) through valid and invalid lists with stand-ins for the kernel
launchers that abort if reached.  A third drives the library's table
uploads against a fake in-order device (tests/sanitize/fake_device.cpp):
list changes must never make the host wait, copies must come from pinned
buffers, and a staging buffer must not be reused before its copy ran.  A
fourth takes 400 seeded random lists through every entry point against the
same fake device, which checks the tables each launch finds (chunk map,
alignment heads, the one-tensor entry, the whole-model flag, grid bounds);
planted planning mistakes must make it fail.  No GPU code is built with a
sanitizer."""
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


UPLOAD_SOURCES = [os.path.join(HERE, "upload_driver.cpp"), os.path.join(HERE, "fake_device.cpp")]


def build_upload_driver(exe, api_cpp):
    subprocess.run(["g++", *SAN, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-o", exe, *UPLOAD_SOURCES, api_cpp], check=True)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="no g++ or ROCm headers")
def test_table_uploads_never_wait_for_the_device(tmp_path):
    exe = str(tmp_path / "upload_driver")
    build_upload_driver(exe, os.path.join(ROOT, "mixed_precision_sharded_amd", "csrc", "api.cpp"))
    assert "upload driver ok" in run(exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="no g++ or ROCm headers")
@pytest.mark.parametrize("plant,symptom", [
    # staging buffers treated as free before their copies ran
    ("const hipError_t e = hipEventQuery(u.in_flight.front().done);",
     "a launch found another list's tables"),
    # an upload that waits for the previous one
    ("int rc = reap_uploads(u);",
     "hipEventSynchronize: a call made the host wait"),
])
def test_the_upload_driver_catches_planted_mistakes(tmp_path, plant, symptom):
    src = os.path.join(ROOT, "mixed_precision_sharded_amd", "csrc", "api.cpp")
    text = open(src).read()
    assert plant in text
    if "hipEventQuery" in plant:
        bad = "const hipError_t e = hipSuccess; (void)hipEventQuery(u.in_flight.front().done);"
    else:
        bad = ("if (!u.in_flight.empty()) (void)hipEventSynchronize(u.in_flight.back().done); "
               "int rc = reap_uploads(u);")
    d = tmp_path / "csrc"
    d.mkdir()
    for name in os.listdir(os.path.dirname(src)):
        if name.endswith(".h"):
            shutil.copy(os.path.join(os.path.dirname(src), name), d / name)
    (tmp_path / "include").mkdir()
    shutil.copy(os.path.join(ROOT, "include", "mps_adamw.h"), tmp_path / "include" / "mps_adamw.h")
    planted = d / "api.cpp"
    planted.write_text(text.replace(plant, bad).replace('"../../include/mps_adamw.h"',
                                                        '"../include/mps_adamw.h"'))
    exe = str(tmp_path / "upload_driver_planted")
    build_upload_driver(exe, str(planted))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode != 0 and symptom in r.stderr, r.stdout + r.stderr


PLAN_SOURCES = [os.path.join(HERE, "plan_driver.cpp"), os.path.join(HERE, "fake_device.cpp")]


def planted_api(tmp_path, plant, bad):
    """A copy of api.cpp with `plant` replaced by `bad`, beside copies of the
    headers it includes."""
    src = os.path.join(ROOT, "mixed_precision_sharded_amd", "csrc", "api.cpp")
    text = open(src).read()
    assert plant in text
    d = tmp_path / "csrc"
    d.mkdir()
    for name in os.listdir(os.path.dirname(src)):
        if name.endswith(".h"):
            shutil.copy(os.path.join(os.path.dirname(src), name), d / name)
    (tmp_path / "include").mkdir()
    shutil.copy(os.path.join(ROOT, "include", "mps_adamw.h"), tmp_path / "include" / "mps_adamw.h")
    planted = d / "api.cpp"
    planted.write_text(text.replace(plant, bad).replace('"../../include/mps_adamw.h"',
                                                        '"../include/mps_adamw.h"'))
    return str(planted)


def build_plan_driver(exe, api_cpp):
    subprocess.run(["g++", *SAN, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-o", exe, *PLAN_SOURCES, api_cpp], check=True)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="no g++ or ROCm headers")
def test_planning_on_random_lists(tmp_path):
    exe = str(tmp_path / "plan_driver")
    build_plan_driver(exe, os.path.join(ROOT, "mixed_precision_sharded_amd", "csrc", "api.cpp"))
    assert "plan driver ok" in run(exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="no g++ or ROCm headers")
@pytest.mark.parametrize("plant,bad,symptom", [
    # the bf16 gradient's alignment taken with fp32 elements
    ("e.head = common_head(e, bf16);", "e.head = common_head(e, false);",
     "table check: head of a tensor"),
    # a tensor's last partial chunk dropped from the count
    ("n_chunks += (e.numel + plan.chunk_elems - 1) / plan.chunk_elems;",
     "n_chunks += e.numel / plan.chunk_elems;", "table check: chunk map"),
    # a list whose elements sit in one tensor not recognised as such
    ("plan.solo_tensor = i;", "plan.solo_tensor = -1;", "table check: the one-tensor index"),
])
def test_the_plan_checks_catch_planted_mistakes(tmp_path, plant, bad, symptom):
    exe = str(tmp_path / "plan_driver_planted")
    build_plan_driver(exe, planted_api(tmp_path, plant, bad))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode != 0 and symptom in r.stderr, r.stdout + r.stderr
