"""The C ABI: the library loads, exports every function the header declares,
and rejects bad arguments with error codes before touching the GPU.

Runs without a GPU: only host-side validation paths are called (no kernel is
launched and no HIP call is made on these paths).
"""
import ctypes
import os
import re
import subprocess

import pytest

from mixed_precision_sharded_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mps_adamw.h")

EINVAL, EWORKSPACE = -22, -28


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\([^;{]*\)\s*;", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from mixed_precision_sharded_amd import build
        build.build()
    return binding.lib()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "adamw_workspace_bytes", "adamw_workspace_release", "grad_norm_sq", "clip_coef",
        "adamw_multi_tensor_step", "adamw_clipped_step", "adamw_clipped_step_noalloc",
        "adamw_fused_step", "adamw_fused_status", "adamw_last_error",
        "adamw8_workspace_bytes", "adamw8_grad_norm_sq", "adamw8_multi_tensor_step",
        "adamw8_clipped_step",
        "adamw8_quantize", "adamw8_dequantize"])


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def fake_list(n=2, numel=1000, base=0x7f0000000000, misalign=0):
    arr = (binding.MpsTensor * n)()
    for i in range(n):
        off = base + i * (1 << 24) + misalign
        arr[i] = binding.MpsTensor(off, off + 4096 * 1024, off + 8192 * 1024, off + 12288 * 1024,
                                   None, numel)
    return arr


def test_workspace_bytes(lib):
    arr = fake_list(3, 5000)
    size = lib.adamw_workspace_bytes(arr, 3)
    assert size > 0 and size < 1 << 20
    # chunk tables grow with the parameter count, the fixed part does not
    big = lib.adamw_workspace_bytes(fake_list(3, 50_000_000), 3)
    assert big > size
    assert big < 50_000_000 * 3 // 900  # a 4-byte map slot per chunk of 4096: ~1 B per 1000


def test_workspace_bytes_rejects_bad_lists(lib):
    assert lib.adamw_workspace_bytes(None, 1) == 0
    assert "NULL" in binding.last_error()
    assert lib.adamw_workspace_bytes(fake_list(1), 0) == 0
    bad = fake_list(1)
    bad[0].numel = -1
    assert lib.adamw_workspace_bytes(bad, 1) == 0
    assert "numel" in binding.last_error()


def test_argument_errors(lib):
    arr = fake_list(1, 4096)
    ws = ctypes.c_void_p(0x7e0000000000)
    good = dict(coef=None, step=ctypes.c_void_p(0x7d0000000000), lr=3e-4, b1=0.9, b2=0.95,
                eps=1e-8, wd=0.1)

    def step(**kw):
        a = {**good, **kw}
        return lib.adamw_multi_tensor_step(arr, 1, 0, a["coef"], None, a["step"], a["lr"],
                                           a["b1"], a["b2"], a["eps"], a["wd"], ws, 1 << 30, None)

    assert step(step=None) == EINVAL
    assert step(b1=1.0) == EINVAL
    assert step(b2=-0.1) == EINVAL
    assert step(lr=float("nan")) == EINVAL
    assert step(lr=-1.0) == EINVAL
    assert step(eps=float("inf")) == EINVAL
    assert step(wd=-0.1) == EINVAL
    assert "weight_decay" in binding.last_error()
    # wrong dtype code, empty list, NULL state with numel > 0
    assert lib.adamw_multi_tensor_step(arr, 1, 7, None, None, good["step"], 3e-4, 0.9, 0.95,
                                       1e-8, 0.1, ws, 1 << 30, None) == EINVAL
    assert lib.adamw_multi_tensor_step(arr, 0, 0, None, None, good["step"], 3e-4, 0.9, 0.95,
                                       1e-8, 0.1, ws, 1 << 30, None) == EINVAL
    nostate = fake_list(1)
    nostate[0].master = None
    assert lib.adamw_multi_tensor_step(nostate, 1, 0, None, None, good["step"], 3e-4, 0.9,
                                       0.95, 1e-8, 0.1, ws, 1 << 30, None) == EINVAL
    # fp32 state not 4-byte aligned; bf16 gradient not 2-byte aligned
    odd = fake_list(1, misalign=2)
    assert lib.adamw_multi_tensor_step(odd, 1, 0, None, None, good["step"], 3e-4, 0.9, 0.95,
                                       1e-8, 0.1, ws, 1 << 30, None) == EINVAL
    odd1 = fake_list(1, misalign=1)
    assert lib.grad_norm_sq(odd1, 1, 1, ctypes.c_void_p(0x7d0000000000), 0.0, 1.0, None, ws,
                            1 << 30, None) == EINVAL
    # a clip output needs a finite positive max_norm and grad_scale
    out, coef = ctypes.c_void_p(0x7d0000000000), ctypes.c_void_p(0x7d0000000100)
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert lib.grad_norm_sq(arr, 1, 0, out, bad, 1.0, coef, ws, 1 << 30, None) == EINVAL
        assert lib.grad_norm_sq(arr, 1, 0, out, 1.0, bad, coef, ws, 1 << 30, None) == EINVAL
    assert "grad_scale" in binding.last_error()


def test_workspace_errors(lib):
    arr = fake_list(1, 4096)
    step = ctypes.c_void_p(0x7d0000000000)
    need = lib.adamw_workspace_bytes(arr, 1)
    args = (arr, 1, 0, None, None, step, 3e-4, 0.9, 0.95, 1e-8, 0.1)
    assert lib.adamw_multi_tensor_step(*args, None, need, None) == EWORKSPACE
    assert lib.adamw_multi_tensor_step(*args, ctypes.c_void_p(0x7e0000000040), need,
                                       None) == EWORKSPACE
    assert "aligned" in binding.last_error()
    assert lib.adamw_multi_tensor_step(*args, ctypes.c_void_p(0x7e0000000000), need - 1,
                                       None) == EWORKSPACE
    assert "too small" in binding.last_error()
    assert lib.grad_norm_sq(arr, 1, 0, ctypes.c_void_p(0x7d0000000000), 1.0, 1.0, None, None,
                            need, None) == EWORKSPACE
    assert lib.grad_norm_sq(arr, 1, 0, None, 1.0, 1.0, None, ctypes.c_void_p(0x7e0000000000),
                            need, None) == EINVAL


@pytest.mark.parametrize("entry", ["adamw_clipped_step", "adamw_fused_step"])
def test_whole_step_argument_errors(lib, entry):
    arr = fake_list(1, 4096)
    ws = ctypes.c_void_p(0x7e0000000000)
    step = ctypes.c_void_p(0x7d0000000000)

    def call(**kw):
        a = dict(mn=1.0, scale=1.0, step=step, lr=3e-4, b1=0.9, b2=0.95, eps=1e-8, wd=0.1,
                 ws=ws, size=1 << 30)
        a.update(kw)
        extra = (None,) if entry == "adamw_clipped_step" else ()
        return getattr(lib, entry)(arr, 1, 0, a["mn"], a["scale"], 0, None, None, a["step"],
                                   a["lr"], a["b1"], a["b2"], a["eps"], a["wd"], a["ws"],
                                   a["size"], None, *extra)

    assert call(step=None) == EINVAL
    assert call(mn=0.0) == EINVAL
    assert call(scale=float("nan")) == EINVAL
    assert call(b1=1.0) == EINVAL
    assert call(wd=-1.0) == EINVAL
    assert call(ws=None) == EWORKSPACE
    assert call(size=16) == EWORKSPACE


def test_clip_argument_errors(lib):
    p = ctypes.c_void_p(0x7d0000000000)
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert lib.clip_coef(p, bad, 1.0, p, None) == EINVAL
        assert lib.clip_coef(p, 1.0, bad, p, None) == EINVAL
    assert lib.clip_coef(None, 1.0, 1.0, p, None) == EINVAL
    assert lib.clip_coef(p, 1.0, 1.0, None, None) == EINVAL


def test_release_unknown_workspace_is_harmless(lib):
    assert lib.adamw_workspace_release(ctypes.c_void_p(0x1234500)) == 0


def fake_list8(n=2, numel=1000, base=0x7f0000000000, misalign=0):
    arr = (binding.MpsTensor8 * n)()
    for i in range(n):
        off = base + i * (1 << 26) + misalign
        arr[i] = binding.MpsTensor8(off, off + (8 << 20), off + (16 << 20), off + (24 << 20),
                                    off + (32 << 20), off + (40 << 20), None, numel)
    return arr


def test_8bit_workspace_bytes(lib):
    size8 = lib.adamw8_workspace_bytes(fake_list8(3, 5000), 3)
    size = lib.adamw_workspace_bytes(fake_list(3, 5000), 3)
    # one more 32-byte record per tensor for the 8-bit state (tables are padded to 256 bytes)
    assert size <= size8 <= size + 3 * 32 + 256
    many = lib.adamw8_workspace_bytes(fake_list8(40, 5000), 40)
    assert many >= lib.adamw_workspace_bytes(fake_list(40, 5000), 40) + 40 * 32 - 256
    assert lib.adamw8_workspace_bytes(None, 1) == 0
    bad = fake_list8(1)
    bad[0].numel = -5
    assert lib.adamw8_workspace_bytes(bad, 1) == 0 and "numel" in binding.last_error()


def test_8bit_argument_errors(lib):
    arr = fake_list8(1, 4096)
    ws = ctypes.c_void_p(0x7e0000000000)
    step = ctypes.c_void_p(0x7d0000000000)

    def call(a=arr, dtype=0, step=step, b1=0.9, wd=0.1, ws=ws, size=1 << 30):
        return lib.adamw8_multi_tensor_step(a, 1, dtype, None, None, step, 3e-4, b1, 0.95, 1e-8,
                                            wd, ws, size, None)

    assert call(step=None) == EINVAL
    assert call(b1=1.0) == EINVAL
    assert call(wd=float("nan")) == EINVAL
    assert call(dtype=5) == EINVAL
    for field in ("master", "exp_avg_codes", "exp_avg_scales", "exp_avg_sq_codes",
                  "exp_avg_sq_scales", "grad"):
        broken = fake_list8(1, 4096)
        setattr(broken[0], field, None)
        assert call(a=broken) == EINVAL, field
    assert call(a=fake_list8(1, 4096, misalign=2)) == EINVAL       # fp32 master
    assert call(ws=None) == EWORKSPACE
    assert call(size=64) == EWORKSPACE
    out = ctypes.c_void_p(0x7d0000000000)
    assert lib.adamw8_grad_norm_sq(fake_list8(1, 10, misalign=1), 1, 1, out, 0.0, 1.0, None, ws,
                                   1 << 30, None) == EINVAL      # bf16 gradient, odd address
    assert lib.adamw8_grad_norm_sq(arr, 1, 0, None, 1.0, 1.0, None, ws, 1 << 30, None) == EINVAL
    assert lib.adamw8_grad_norm_sq(arr, 1, 0, out, 0.0, 1.0, out, ws, 1 << 30, None) == EINVAL


def test_8bit_conversion_argument_errors(lib):
    p = ctypes.c_void_p(0x7d0000000000)
    assert lib.adamw8_quantize(p, -1, 0, p, p, None) == EINVAL
    assert lib.adamw8_quantize(p, 10, 2, p, p, None) == EINVAL
    assert lib.adamw8_quantize(None, 10, 0, p, p, None) == EINVAL
    assert lib.adamw8_dequantize(p, None, 10, 1, p, None) == EINVAL
    assert lib.adamw8_dequantize(p, p, 10, -1, p, None) == EINVAL
    # nothing to do: no pointer is needed and nothing is enqueued
    assert lib.adamw8_quantize(None, 0, 0, None, None, None) == 0
    assert lib.adamw8_dequantize(None, None, 0, 1, None, None) == 0


def test_header_is_plain_c(tmp_path):
    """The header compiles as C99 and C++17 on its own, with every warning,
    and its entry points have the declared C types."""
    src = tmp_path / "use.c"
    src.write_text(
        '#include "mps_adamw.h"\n'
        "size_t (*f0)(const mps_tensor*, int) = adamw_workspace_bytes;\n"
        "int (*f1)(const mps_tensor*, int, mps_dtype, double*, double, double, float*, void*,"
        " size_t, void*) = grad_norm_sq;\n"
        "int (*f2)(const double*, double, double, float*, void*) = clip_coef;\n"
        "int (*f3)(const mps_tensor8*, int, mps_dtype, const float*, const double*, int32_t*,"
        " double, double, double, double, double, void*, size_t, void*) = adamw8_multi_tensor_step;\n"
        "int (*f4)(const float*, int64_t, mps_q8_format, uint8_t*, uint8_t*, void*) = adamw8_quantize;\n"
        "const char* (*f5)(void) = adamw_last_error;\n"
        "typedef char size_check[(sizeof(mps_tensor) == 48 && sizeof(mps_tensor8) == 64 &&"
        " MPS_Q8_BLOCK == 32) ? 1 : -1];\n"
        "int main(void) { return (int)sizeof(size_check) - 1; }\n")
    inc = os.path.join(ROOT, "include")
    for compiler, std in (("gcc", "-std=c99"), ("g++", "-std=c++17")):
        args = [compiler, std, "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only",
                "-I", inc, str(src)]
        if compiler == "g++":
            args[-1:] = ["-x", "c++", str(src)]
        r = subprocess.run(args, capture_output=True, text=True)
        assert r.returncode == 0, (compiler, r.stderr)
    # the ctypes mirrors have the C layout
    assert ctypes.sizeof(binding.MpsTensor) == 48 and ctypes.sizeof(binding.MpsTensor8) == 64


def test_c_program_builds_against_the_header(lib, oracle_lib, tmp_path):
    """The C test program (tests/c_abi/step_from_c.c) compiles as C99 with
    every warning an error and links against the built library."""
    import importlib.util

    spec = importlib.util.spec_from_file_location(
        "c_abi_build", os.path.join(os.path.dirname(__file__), "c_abi", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    out = mod.build(str(tmp_path / "step_from_c"))
    assert os.path.getsize(out) > 0


def test_fused_status_rejects_bad_arguments(lib):
    P = ctypes.c_void_p
    assert lib.adamw_fused_status(P(0x7f0000000000), 4096, None, None) == EINVAL
    assert "d_error" in binding.last_error()
    assert lib.adamw_fused_status(None, 4096, P(0x1000), None) == EWORKSPACE
    assert lib.adamw_fused_status(P(0x7f0000000010), 4096, P(0x1000), None) == EWORKSPACE
    assert lib.adamw_fused_status(P(0x7f0000000000), 32, P(0x1000), None) == EWORKSPACE
    assert "too small" in binding.last_error()


def test_noalloc_step_checks_arguments_before_the_device(lib):
    arr = fake_list(2, 1000)
    args = [arr, 2, binding.MPS_DTYPE_F32, 1.0, 1.0, 0, None, None]
    hp = [3e-4, 0.9, 0.95, 1e-8, 0.1, None, None]
    assert lib.adamw_clipped_step_noalloc(*args, None, *hp) == EINVAL  # no step counter
    assert "d_step" in binding.last_error()
    bad_hp = [3e-4, 1.5, 0.95, 1e-8, 0.1, None, None]
    assert lib.adamw_clipped_step_noalloc(*args, ctypes.c_void_p(0x1000), *bad_hp) == EINVAL
    assert "beta1" in binding.last_error()
