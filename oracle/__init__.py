"""Python access to the scalar CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg, never by the GPU library or its binding.
Arrays are numpy; bf16 data is carried as uint16 bit patterns.

Every function is pinned by the CPU test suite (closed forms, torch's
AdamW and clip_grad_norm_ in fp64, exact rationals, brute force).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_c_f32p = ctypes.POINTER(ctypes.c_float)
_c_u16p = ctypes.POINTER(ctypes.c_uint16)
_c_u8p = ctypes.POINTER(ctypes.c_uint8)

E4M3, E5M2 = 0, 1   # 8-bit formats of the moment state: m, v
QBLOCK = 32         # elements per shared scale


class Scalars(ctypes.Structure):
    _fields_ = [(name, ctypes.c_float) for name in (
        "beta1", "beta2", "one_m_b1", "one_m_b2", "decay", "step_size",
        "bc2_sqrt", "eps")]

    def as_dict(self):
        return {name: np.float32(getattr(self, name)) for name, _ in self._fields_}


class Oracle:
    """ctypes wrapper around one build of oracle.c."""

    def __init__(self, lib_path: str = _build.LIB):
        if not os.path.exists(lib_path):
            _build.build(out=lib_path)
        lib = ctypes.CDLL(lib_path)
        self.lib = lib
        lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
        lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_bf16_array.restype = None
        lib.oracle_f32_to_bf16_array.argtypes = [_c_f32p, _c_u16p, ctypes.c_int64]
        lib.oracle_bf16_to_f32.restype = ctypes.c_float
        lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_sumsq_f32.restype = ctypes.c_double
        lib.oracle_sumsq_f32.argtypes = [_c_f32p, ctypes.c_int64, ctypes.c_double]
        lib.oracle_sumsq_bf16.restype = ctypes.c_double
        lib.oracle_sumsq_bf16.argtypes = [_c_u16p, ctypes.c_int64, ctypes.c_double]
        lib.oracle_clip_coef.restype = ctypes.c_float
        lib.oracle_clip_coef.argtypes = [ctypes.c_double, ctypes.c_double]
        lib.oracle_clip_coef_scaled.restype = ctypes.c_float
        lib.oracle_clip_coef_scaled.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double]
        lib.oracle_pow_int.restype = ctypes.c_double
        lib.oracle_pow_int.argtypes = [ctypes.c_double, ctypes.c_int64]
        lib.oracle_step_scalars.restype = None
        lib.oracle_step_scalars.argtypes = [
            ctypes.c_int64, ctypes.c_double, ctypes.c_double, ctypes.c_double,
            ctypes.c_double, ctypes.c_double, ctypes.POINTER(Scalars)]
        lib.oracle_adamw_step.restype = None
        lib.oracle_adamw_step.argtypes = [
            _c_f32p, _c_f32p, _c_f32p, ctypes.c_void_p, ctypes.c_int, _c_u16p,
            ctypes.c_int64, ctypes.c_float, ctypes.c_int64, ctypes.c_double,
            ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double]
        lib.oracle_fp8_value.restype = ctypes.c_double
        lib.oracle_fp8_value.argtypes = [ctypes.c_uint8, ctypes.c_int]
        lib.oracle_fp8_round.restype = ctypes.c_uint8
        lib.oracle_fp8_round.argtypes = [ctypes.c_double, ctypes.c_int]
        lib.oracle_fp8_round_array.restype = None
        lib.oracle_fp8_round_array.argtypes = [_c_f32p, ctypes.c_int64, ctypes.c_int, _c_u8p]
        lib.oracle_block_exponent.restype = ctypes.c_int
        lib.oracle_block_exponent.argtypes = [ctypes.c_double, ctypes.c_int]
        lib.oracle_quantize.restype = None
        lib.oracle_quantize.argtypes = [_c_f32p, ctypes.c_int64, ctypes.c_int, _c_u8p, _c_u8p]
        lib.oracle_dequantize.restype = None
        lib.oracle_dequantize.argtypes = [_c_u8p, _c_u8p, ctypes.c_int64, ctypes.c_int, _c_f32p]
        lib.oracle_adamw8_step.restype = None
        lib.oracle_adamw8_step.argtypes = [
            _c_f32p, _c_u8p, _c_u8p, _c_u8p, _c_u8p, ctypes.c_void_p, ctypes.c_int, _c_u16p,
            ctypes.c_int64, ctypes.c_float, ctypes.c_int64, ctypes.c_double,
            ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double]

    # -- bf16 -------------------------------------------------------------
    def f32_to_bf16(self, x) -> np.ndarray:
        """Round-to-nearest-even bf16 bit patterns (uint16) of float32 `x`."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_f32_to_bf16_array(_f32(x), _u16(out), x.size)
        return out

    def bf16_to_f32(self, h) -> np.ndarray:
        h = np.ascontiguousarray(h, dtype=np.uint16)
        return np.array([self.lib.oracle_bf16_to_f32(int(b)) for b in h.ravel()],
                        dtype=np.float32).reshape(h.shape)

    # -- norm and clip ------------------------------------------------------
    def grad_norm_sq(self, grads) -> float:
        """fp64 sum of squares over every gradient, sequential in list order.

        Each gradient is a float32 array or a uint16 array of bf16 words."""
        acc = 0.0
        for g in grads:
            g = np.ascontiguousarray(g)
            if g.dtype == np.float32:
                acc = self.lib.oracle_sumsq_f32(_f32(g), g.size, acc)
            elif g.dtype == np.uint16:
                acc = self.lib.oracle_sumsq_bf16(_u16(g), g.size, acc)
            else:
                raise TypeError("gradient must be float32 or bf16 words (uint16)")
        return acc

    def clip_coef(self, sumsq: float, max_norm: float, grad_scale: float = None) -> np.float32:
        """The clip coefficient; with grad_scale s, the multiplier for the
        stored gradient whose effective value is s * g."""
        if grad_scale is None:
            return np.float32(self.lib.oracle_clip_coef(sumsq, max_norm))
        return np.float32(self.lib.oracle_clip_coef_scaled(sumsq, max_norm, grad_scale))

    @staticmethod
    def skips(sumsq: float) -> bool:
        """A loss-scaled step is skipped when the gradients were not finite."""
        return not np.isfinite(sumsq)

    # -- scalars and update ---------------------------------------------------
    def pow_int(self, beta: float, t: int) -> float:
        return self.lib.oracle_pow_int(beta, t)

    def step_scalars(self, t, lr, beta1, beta2, eps, wd) -> dict:
        s = Scalars()
        self.lib.oracle_step_scalars(t, lr, beta1, beta2, eps, wd, ctypes.byref(s))
        return s.as_dict()

    def adamw_step(self, master, exp_avg, exp_avg_sq, grad, param_bf16, clip,
                   t, lr, beta1, beta2, eps, wd) -> None:
        """In-place step on one tensor (numpy float32 master/m/v, float32 or
        uint16-bf16 grad, optional uint16 copy out).  `t` is the step number
        after this update (1 for the first step)."""
        n = master.size
        for a in (master, exp_avg, exp_avg_sq):
            if a.dtype != np.float32 or not a.flags.c_contiguous or a.size != n:
                raise ValueError("master, exp_avg, exp_avg_sq: contiguous float32, same size")
        grad = np.ascontiguousarray(grad)
        if grad.size != n or grad.dtype not in (np.float32, np.uint16):
            raise ValueError("grad: float32 or uint16 (bf16), same size")
        if param_bf16 is not None and (param_bf16.dtype != np.uint16 or
                                       param_bf16.size != n or
                                       not param_bf16.flags.c_contiguous):
            raise ValueError("param_bf16: contiguous uint16 of the same size")
        self.lib.oracle_adamw_step(
            _f32(master), _f32(exp_avg), _f32(exp_avg_sq),
            grad.ctypes.data_as(ctypes.c_void_p), int(grad.dtype == np.uint16),
            _u16(param_bf16) if param_bf16 is not None else None,
            n, float(clip), int(t), lr, beta1, beta2, eps, wd)


    # -- 8-bit moment state -------------------------------------------------
    def fp8_value(self, codes, fmt) -> np.ndarray:
        """Values (float64) of 8-bit codes in format `fmt` (E4M3 or E5M2)."""
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        return np.array([self.lib.oracle_fp8_value(int(c), fmt) for c in codes.ravel()],
                        dtype=np.float64).reshape(codes.shape)

    def fp8_round(self, x, fmt) -> np.ndarray:
        """Nearest 8-bit code (ties to even) of each float32 in `x`."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint8)
        self.lib.oracle_fp8_round_array(_f32(x), x.size, fmt, _u8(out))
        return out

    def block_exponent(self, absmax: float, fmt) -> int:
        return self.lib.oracle_block_exponent(float(absmax), fmt)

    def quantize(self, x, fmt):
        """(codes uint8[n], scales uint8[ceil(n/32)]) of float32 `x`."""
        x = np.ascontiguousarray(x, dtype=np.float32).ravel()
        codes = np.empty(x.size, dtype=np.uint8)
        scales = np.empty((x.size + QBLOCK - 1) // QBLOCK, dtype=np.uint8)
        self.lib.oracle_quantize(_f32(x), x.size, fmt, _u8(codes), _u8(scales))
        return codes, scales

    def dequantize(self, codes, scales, fmt) -> np.ndarray:
        codes = np.ascontiguousarray(codes, dtype=np.uint8).ravel()
        scales = np.ascontiguousarray(scales, dtype=np.uint8).ravel()
        if scales.size != (codes.size + QBLOCK - 1) // QBLOCK:
            raise ValueError("scales: one byte per 32 codes")
        out = np.empty(codes.size, dtype=np.float32)
        self.lib.oracle_dequantize(_u8(codes), _u8(scales), codes.size, fmt, _f32(out))
        return out

    def adamw8_step(self, master, m_codes, m_scales, v_codes, v_scales, grad, param_bf16,
                    clip, t, lr, beta1, beta2, eps, wd) -> None:
        """In-place step on one tensor whose moments are 8-bit (m: E4M3,
        v: E5M2, one scale byte per 32 elements)."""
        n = master.size
        if master.dtype != np.float32 or not master.flags.c_contiguous:
            raise ValueError("master: contiguous float32")
        nb = (n + QBLOCK - 1) // QBLOCK
        for a, size in ((m_codes, n), (v_codes, n), (m_scales, nb), (v_scales, nb)):
            if a.dtype != np.uint8 or not a.flags.c_contiguous or a.size != size:
                raise ValueError("codes: contiguous uint8[n]; scales: contiguous uint8[ceil(n/32)]")
        grad = np.ascontiguousarray(grad)
        if grad.size != n or grad.dtype not in (np.float32, np.uint16):
            raise ValueError("grad: float32 or uint16 (bf16), same size")
        if param_bf16 is not None and (param_bf16.dtype != np.uint16 or
                                       param_bf16.size != n or
                                       not param_bf16.flags.c_contiguous):
            raise ValueError("param_bf16: contiguous uint16 of the same size")
        self.lib.oracle_adamw8_step(
            _f32(master), _u8(m_codes), _u8(m_scales), _u8(v_codes), _u8(v_scales),
            grad.ctypes.data_as(ctypes.c_void_p), int(grad.dtype == np.uint16),
            _u16(param_bf16) if param_bf16 is not None else None,
            n, float(clip), int(t), lr, beta1, beta2, eps, wd)


def _f32(a):
    return a.ctypes.data_as(_c_f32p)


def _u16(a):
    return a.ctypes.data_as(_c_u16p)


def _u8(a):
    return a.ctypes.data_as(_c_u8p)


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c (built on first use if missing)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
