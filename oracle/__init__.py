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


def _f32(a):
    return a.ctypes.data_as(_c_f32p)


def _u16(a):
    return a.ctypes.data_as(_c_u16p)


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c (built on first use if missing)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
