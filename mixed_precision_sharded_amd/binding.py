"""ctypes binding of libmps_adamw.so (C ABI in include/mps_adamw.h).

Argument marshalling only: every step of the optimizer runs in the HIP
kernels.  PyTorch supplies device memory and the stream.  If the library is
not built, every call raises; there is no fallback.
"""
import ctypes
import os
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmps_adamw.so")

MPS_OK = 0
MPS_DTYPE_F32 = 0
MPS_DTYPE_BF16 = 1
MPS_Q8_E4M3 = 0   # 8-bit format of m
MPS_Q8_E5M2 = 1   # 8-bit format of v
MPS_Q8_BLOCK = 32
WORKSPACE_ALIGN = 256


class MpsTensor(ctypes.Structure):
    """Mirror of `mps_tensor`."""
    _fields_ = [
        ("master", ctypes.c_void_p),
        ("exp_avg", ctypes.c_void_p),
        ("exp_avg_sq", ctypes.c_void_p),
        ("grad", ctypes.c_void_p),
        ("param_bf16", ctypes.c_void_p),
        ("numel", ctypes.c_int64),
    ]


class MpsTensor8(ctypes.Structure):
    """Mirror of `mps_tensor8`."""
    _fields_ = [
        ("master", ctypes.c_void_p),
        ("exp_avg_codes", ctypes.c_void_p),
        ("exp_avg_scales", ctypes.c_void_p),
        ("exp_avg_sq_codes", ctypes.c_void_p),
        ("exp_avg_sq_scales", ctypes.c_void_p),
        ("grad", ctypes.c_void_p),
        ("param_bf16", ctypes.c_void_p),
        ("numel", ctypes.c_int64),
    ]


class MpsError(RuntimeError):
    def __init__(self, code: int, where: str, message: str):
        super().__init__(f"{where} failed with code {code}: {message}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mixed_precision_sharded_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.adamw_workspace_bytes.restype = ctypes.c_size_t
        L.adamw_workspace_bytes.argtypes = [ctypes.POINTER(MpsTensor), ctypes.c_int]
        L.adamw_workspace_release.restype = ctypes.c_int
        L.adamw_workspace_release.argtypes = [P]
        L.grad_norm_sq.restype = ctypes.c_int
        L.grad_norm_sq.argtypes = [ctypes.POINTER(MpsTensor), ctypes.c_int, ctypes.c_int,
                                   P, ctypes.c_double, ctypes.c_double, P, P, ctypes.c_size_t, P]
        L.clip_coef.restype = ctypes.c_int
        L.clip_coef.argtypes = [P, ctypes.c_double, ctypes.c_double, P, P]
        L.adamw_multi_tensor_step.restype = ctypes.c_int
        L.adamw_multi_tensor_step.argtypes = [
            ctypes.POINTER(MpsTensor), ctypes.c_int, ctypes.c_int, P, P, P,
            ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double,
            ctypes.c_double, P, ctypes.c_size_t, P]
        whole_step = [
            ctypes.POINTER(MpsTensor), ctypes.c_int, ctypes.c_int, ctypes.c_double,
            ctypes.c_double, ctypes.c_int, P, P, P, ctypes.c_double, ctypes.c_double,
            ctypes.c_double, ctypes.c_double, ctypes.c_double, P, ctypes.c_size_t, P]
        L.adamw_clipped_step.restype = ctypes.c_int
        L.adamw_clipped_step.argtypes = whole_step + [P]
        L.adamw_clipped_step_noalloc.restype = ctypes.c_int
        L.adamw_clipped_step_noalloc.argtypes = whole_step[:-3] + [P, P]
        L.adamw_fused_step.restype = ctypes.c_int
        L.adamw_fused_step.argtypes = whole_step
        L.adamw_fused_status.restype = ctypes.c_int
        L.adamw_fused_status.argtypes = [P, ctypes.c_size_t, P, P]
        T8 = ctypes.POINTER(MpsTensor8)
        L.adamw8_workspace_bytes.restype = ctypes.c_size_t
        L.adamw8_workspace_bytes.argtypes = [T8, ctypes.c_int]
        L.adamw8_grad_norm_sq.restype = ctypes.c_int
        L.adamw8_grad_norm_sq.argtypes = [T8, ctypes.c_int, ctypes.c_int, P, ctypes.c_double,
                                          ctypes.c_double, P, P, ctypes.c_size_t, P]
        L.adamw8_multi_tensor_step.restype = ctypes.c_int
        L.adamw8_multi_tensor_step.argtypes = [
            T8, ctypes.c_int, ctypes.c_int, P, P, P, ctypes.c_double, ctypes.c_double,
            ctypes.c_double, ctypes.c_double, ctypes.c_double, P, ctypes.c_size_t, P]
        L.adamw8_clipped_step.restype = ctypes.c_int
        L.adamw8_clipped_step.argtypes = [T8] + whole_step[1:] + [P]
        L.adamw8_quantize.restype = ctypes.c_int
        L.adamw8_quantize.argtypes = [P, ctypes.c_int64, ctypes.c_int, P, P, P]
        L.adamw8_dequantize.restype = ctypes.c_int
        L.adamw8_dequantize.argtypes = [P, P, ctypes.c_int64, ctypes.c_int, P, P]
        L.adamw_last_error.restype = ctypes.c_char_p
        L.adamw_last_error.argtypes = []
        _lib = L
    return _lib


def last_error() -> str:
    return lib().adamw_last_error().decode()


def _check(rc: int, where: str) -> None:
    if rc != MPS_OK:
        raise MpsError(rc, where, last_error())


def _stream_handle(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


class TensorList:
    """A host array of `mps_tensor` records built from torch tensors, plus a
    device workspace sized for it.  Holds references to every tensor, so the
    buffers outlive the calls that use them.

    masters, exp_avgs, exp_avg_sqs: fp32 CUDA tensors; grads: fp32 or bf16
    (one dtype for the whole list); params_bf16: bf16 tensors or None entries.
    Each tensor must be contiguous; its storage offset may be anything.
    """

    def __init__(self, masters: Sequence[torch.Tensor], exp_avgs: Sequence[torch.Tensor],
                 exp_avg_sqs: Sequence[torch.Tensor], grads: Sequence[torch.Tensor],
                 params_bf16: Optional[Sequence[Optional[torch.Tensor]]] = None,
                 workspace: bool = True):
        n = len(masters)
        if not (len(exp_avgs) == len(exp_avg_sqs) == len(grads) == n) or n == 0:
            raise ValueError("masters, exp_avgs, exp_avg_sqs and grads: same non-zero length")
        if params_bf16 is None:
            params_bf16 = [None] * n
        if len(params_bf16) != n:
            raise ValueError("params_bf16 must have one entry per tensor")
        gdt = grads[0].dtype
        if gdt not in (torch.float32, torch.bfloat16):
            raise TypeError("grads must be float32 or bfloat16")
        self.grad_dtype = MPS_DTYPE_BF16 if gdt == torch.bfloat16 else MPS_DTYPE_F32
        self.device = masters[0].device
        self.array = (MpsTensor * n)()
        for i in range(n):
            w, m, v, g, p = masters[i], exp_avgs[i], exp_avg_sqs[i], grads[i], params_bf16[i]
            k = w.numel()
            for name, t, dt in (("master", w, torch.float32), ("exp_avg", m, torch.float32),
                                ("exp_avg_sq", v, torch.float32), ("grad", g, gdt)):
                _require(t, dt, k, self.device, f"{name}[{i}]")
            if p is not None:
                _require(p, torch.bfloat16, k, self.device, f"param_bf16[{i}]")
            self.array[i] = MpsTensor(_ptr(w), _ptr(m), _ptr(v), _ptr(g), _ptr(p), k)
        self.n = n
        self._refs = (list(masters), list(exp_avgs), list(exp_avg_sqs), list(grads),
                      list(params_bf16))
        if workspace:
            self._allocate_workspace(lib().adamw_workspace_bytes(self.array, n),
                                     "adamw_workspace_bytes")
        else:  # for adamw_clipped_step_noalloc, which brings its own
            self._ws_storage = None
            self.workspace_ptr, self.workspace_bytes = None, 0

    def _allocate_workspace(self, nbytes: int, where: str) -> None:
        if nbytes == 0:
            raise MpsError(-22, where, last_error())
        self.workspace_bytes = nbytes
        # Over-allocate so the base can be rounded up to 256 bytes.
        self._ws_storage = torch.empty(nbytes + WORKSPACE_ALIGN, dtype=torch.uint8,
                                       device=self.device)
        base = self._ws_storage.data_ptr()
        self.workspace_ptr = (base + WORKSPACE_ALIGN - 1) // WORKSPACE_ALIGN * WORKSPACE_ALIGN

    def release(self) -> None:
        """Tell the library the workspace is going away (see the header)."""
        if getattr(self, "_ws_storage", None) is not None:
            lib().adamw_workspace_release(self.workspace_ptr)
            self._ws_storage = None

    def __del__(self):
        try:
            self.release()
        except Exception:
            pass


def q8_scale_count(numel: int) -> int:
    """Scale bytes per moment of a tensor with 8-bit state."""
    return (numel + MPS_Q8_BLOCK - 1) // MPS_Q8_BLOCK


def zeros_q8_state(numel: int, device) -> tuple:
    """(m codes, m scales, v codes, v scales), all zero: m = v = 0."""
    nb = q8_scale_count(numel)
    return (torch.zeros(numel, dtype=torch.uint8, device=device),
            torch.zeros(nb, dtype=torch.uint8, device=device),
            torch.zeros(numel, dtype=torch.uint8, device=device),
            torch.zeros(nb, dtype=torch.uint8, device=device))


class TensorList8(TensorList):
    """The `mps_tensor8` records of a list whose moments are 8-bit, and its
    workspace.  states[i] = (m codes, m scales, v codes, v scales): uint8
    CUDA tensors of numel, ceil(numel / 32), numel, ceil(numel / 32)
    elements (see zeros_q8_state)."""

    def __init__(self, masters: Sequence[torch.Tensor], states: Sequence[tuple],
                 grads: Sequence[torch.Tensor],
                 params_bf16: Optional[Sequence[Optional[torch.Tensor]]] = None):
        n = len(masters)
        if not (len(states) == len(grads) == n) or n == 0:
            raise ValueError("masters, states and grads: same non-zero length")
        if params_bf16 is None:
            params_bf16 = [None] * n
        if len(params_bf16) != n:
            raise ValueError("params_bf16 must have one entry per tensor")
        gdt = grads[0].dtype
        if gdt not in (torch.float32, torch.bfloat16):
            raise TypeError("grads must be float32 or bfloat16")
        self.grad_dtype = MPS_DTYPE_BF16 if gdt == torch.bfloat16 else MPS_DTYPE_F32
        self.device = masters[0].device
        self.array = (MpsTensor8 * n)()
        for i in range(n):
            w, g, p = masters[i], grads[i], params_bf16[i]
            k = w.numel()
            if len(states[i]) != 4:
                raise ValueError(f"states[{i}]: (m codes, m scales, v codes, v scales)")
            mc, ms, vc, vs = states[i]
            _require(w, torch.float32, k, self.device, f"master[{i}]")
            _require(g, gdt, k, self.device, f"grad[{i}]")
            _require(mc, torch.uint8, k, self.device, f"m codes[{i}]")
            _require(vc, torch.uint8, k, self.device, f"v codes[{i}]")
            _require(ms, torch.uint8, q8_scale_count(k), self.device, f"m scales[{i}]")
            _require(vs, torch.uint8, q8_scale_count(k), self.device, f"v scales[{i}]")
            if p is not None:
                _require(p, torch.bfloat16, k, self.device, f"param_bf16[{i}]")
            self.array[i] = MpsTensor8(_ptr(w), _ptr(mc), _ptr(ms), _ptr(vc), _ptr(vs), _ptr(g),
                                       _ptr(p), k)
        self.n = n
        self._refs = (list(masters), [tuple(st) for st in states], list(grads), list(params_bf16))
        self._allocate_workspace(lib().adamw8_workspace_bytes(self.array, n), "adamw8_workspace_bytes")


def _require(t: torch.Tensor, dtype, numel: int, device, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device or t.device.type != "cuda":
        raise ValueError(f"{name}: must be on {device}")
    if t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def grad_norm_sq(tl: TensorList, out: torch.Tensor, max_norm: Optional[float] = None,
                 coef_out: Optional[torch.Tensor] = None, grad_scale: float = 1.0,
                 stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """out[0] (float64, on the device) = sum of g^2 over the list; with
    coef_out (float32) also the clip coefficient for max_norm and grad_scale,
    from the same launch."""
    if out.dtype != torch.float64 or out.device != tl.device or out.numel() < 1:
        raise ValueError("out: float64 tensor on the list's device")
    if coef_out is not None:
        if coef_out.dtype != torch.float32 or coef_out.device != tl.device:
            raise ValueError("coef_out: float32 tensor on the list's device")
        if max_norm is None:
            raise ValueError("coef_out needs max_norm")
    _check(lib().grad_norm_sq(tl.array, tl.n, tl.grad_dtype, out.data_ptr(),
                              float(max_norm) if max_norm is not None else 0.0, float(grad_scale),
                              _ptr(coef_out), tl.workspace_ptr, tl.workspace_bytes,
                              _stream_handle(stream)), "grad_norm_sq")
    return out


def clip_coef(sumsq: torch.Tensor, max_norm: float, out: torch.Tensor, grad_scale: float = 1.0,
              stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """out[0] (float32) = s * min(1, max_norm / (s * sqrt(sumsq[0]) + 1e-6)), s = grad_scale."""
    if sumsq.dtype != torch.float64 or sumsq.device.type != "cuda":
        raise ValueError("sumsq: float64 CUDA tensor")
    if out.dtype != torch.float32 or out.device != sumsq.device:
        raise ValueError("out: float32 tensor on sumsq's device")
    _check(lib().clip_coef(sumsq.data_ptr(), float(max_norm), float(grad_scale), out.data_ptr(),
                           _stream_handle(stream)), "clip_coef")
    return out


def adamw_multi_tensor_step(tl: TensorList, coef: Optional[torch.Tensor], step: torch.Tensor,
                            lr: float, beta1: float, beta2: float, eps: float,
                            weight_decay: float, skip_if_nonfinite: Optional[torch.Tensor] = None,
                            stream: Optional[torch.cuda.Stream] = None) -> None:
    """One AdamW step over the list; `step` (int32, device) counts completed
    steps and is incremented on the device.  With skip_if_nonfinite (a
    float64 device scalar, e.g. the sum of squares), a non-finite value skips
    the whole step."""
    if coef is not None and (coef.dtype != torch.float32 or coef.device != tl.device):
        raise ValueError("coef: float32 tensor on the list's device, or None")
    if step.dtype != torch.int32 or step.device != tl.device:
        raise ValueError("step: int32 tensor on the list's device")
    if skip_if_nonfinite is not None and (skip_if_nonfinite.dtype != torch.float64 or
                                          skip_if_nonfinite.device != tl.device):
        raise ValueError("skip_if_nonfinite: float64 tensor on the list's device, or None")
    _check(lib().adamw_multi_tensor_step(
        tl.array, tl.n, tl.grad_dtype, _ptr(coef), _ptr(skip_if_nonfinite), step.data_ptr(),
        float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), tl.workspace_ptr,
        tl.workspace_bytes, _stream_handle(stream)), "adamw_multi_tensor_step")


def _whole_step(name: str, tl: TensorList, step: torch.Tensor, lr: float, beta1: float,
                beta2: float, eps: float, weight_decay: float, max_norm: float, grad_scale: float,
                skip_if_nonfinite: bool, sumsq_out: Optional[torch.Tensor],
                coef_out: Optional[torch.Tensor], stream: Optional[torch.cuda.Stream],
                *extra) -> None:
    if step.dtype != torch.int32 or step.device != tl.device:
        raise ValueError("step: int32 tensor on the list's device")
    if sumsq_out is not None and (sumsq_out.dtype != torch.float64 or sumsq_out.device != tl.device):
        raise ValueError("sumsq_out: float64 tensor on the list's device, or None")
    if coef_out is not None and (coef_out.dtype != torch.float32 or coef_out.device != tl.device):
        raise ValueError("coef_out: float32 tensor on the list's device, or None")
    _check(getattr(lib(), name)(
        tl.array, tl.n, tl.grad_dtype, float(max_norm), float(grad_scale),
        1 if skip_if_nonfinite else 0, _ptr(sumsq_out), _ptr(coef_out), step.data_ptr(),
        float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), tl.workspace_ptr,
        tl.workspace_bytes, _stream_handle(stream), *extra), name)


def adamw_clipped_step(tl: TensorList, step: torch.Tensor, lr: float, beta1: float, beta2: float,
                       eps: float, weight_decay: float, max_norm: float, grad_scale: float = 1.0,
                       skip_if_nonfinite: bool = False, sumsq_out: Optional[torch.Tensor] = None,
                       coef_out: Optional[torch.Tensor] = None,
                       stream: Optional[torch.cuda.Stream] = None,
                       mid_event: Optional[torch.cuda.Event] = None) -> None:
    """Norm, clip and update in two plain launches, the clip finished inside
    the update (see adamw_clipped_step in the header).  `mid_event`, if given,
    is recorded between the two launches (it must have been recorded once
    before, so that it exists)."""
    if isinstance(tl, TensorList8):
        raise TypeError("adamw_clipped_step takes a TensorList (8-bit state: adamw8_clipped_step)")
    _whole_step("adamw_clipped_step", tl, step, lr, beta1, beta2, eps, weight_decay, max_norm,
                grad_scale, skip_if_nonfinite, sumsq_out, coef_out, stream,
                _event_handle(mid_event))


def adamw_clipped_step_noalloc(tl: TensorList, step: torch.Tensor, lr: float, beta1: float,
                               beta2: float, eps: float, weight_decay: float, max_norm: float,
                               grad_scale: float = 1.0, skip_if_nonfinite: bool = False,
                               sumsq_out: Optional[torch.Tensor] = None,
                               coef_out: Optional[torch.Tensor] = None,
                               stream: Optional[torch.cuda.Stream] = None,
                               mid_event: Optional[torch.cuda.Event] = None) -> None:
    """adamw_clipped_step on the library's own workspace (no allocation; see
    the header).  `tl` may be built with workspace=False."""
    if isinstance(tl, TensorList8):
        raise TypeError("adamw_clipped_step_noalloc takes a TensorList")
    if step.dtype != torch.int32 or step.device != tl.device:
        raise ValueError("step: int32 tensor on the list's device")
    if sumsq_out is not None and (sumsq_out.dtype != torch.float64 or sumsq_out.device != tl.device):
        raise ValueError("sumsq_out: float64 tensor on the list's device, or None")
    if coef_out is not None and (coef_out.dtype != torch.float32 or coef_out.device != tl.device):
        raise ValueError("coef_out: float32 tensor on the list's device, or None")
    _check(lib().adamw_clipped_step_noalloc(
        tl.array, tl.n, tl.grad_dtype, float(max_norm), float(grad_scale),
        1 if skip_if_nonfinite else 0, _ptr(sumsq_out), _ptr(coef_out), step.data_ptr(),
        float(lr), float(beta1), float(beta2), float(eps), float(weight_decay),
        _stream_handle(stream), _event_handle(mid_event)), "adamw_clipped_step_noalloc")


def _event_handle(event: Optional[torch.cuda.Event]):
    if event is None:
        return None
    if not event.cuda_event:
        raise ValueError("mid_event: record it once before passing it")
    return ctypes.c_void_p(event.cuda_event)


def adamw_fused_step(tl: TensorList, step: torch.Tensor, lr: float, beta1: float, beta2: float,
                     eps: float, weight_decay: float, max_norm: float, grad_scale: float = 1.0,
                     skip_if_nonfinite: bool = False, sumsq_out: Optional[torch.Tensor] = None,
                     coef_out: Optional[torch.Tensor] = None,
                     stream: Optional[torch.cuda.Stream] = None) -> None:
    """Norm, clip and update in one launch (see adamw_fused_step in the header)."""
    _whole_step("adamw_fused_step", tl, step, lr, beta1, beta2, eps, weight_decay, max_norm,
                grad_scale, skip_if_nonfinite, sumsq_out, coef_out, stream)


def adamw_fused_status(tl: TensorList, out: torch.Tensor,
                       stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """out[0] (int32 or uint32-sized tensor on the device) = the single-launch
    step's error flag of the list's workspace (1: a barrier wait ran out since
    the last query), which is then cleared."""
    if out.dtype != torch.int32 or out.device != tl.device or out.numel() < 1:
        raise ValueError("out: int32 tensor on the list's device")
    _check(lib().adamw_fused_status(tl.workspace_ptr, tl.workspace_bytes, out.data_ptr(),
                                    _stream_handle(stream)), "adamw_fused_status")
    return out


# ------------------------------------------------------ 8-bit moment state ---

def adamw8_grad_norm_sq(tl: TensorList8, out: torch.Tensor, max_norm: Optional[float] = None,
                        coef_out: Optional[torch.Tensor] = None, grad_scale: float = 1.0,
                        stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """grad_norm_sq for a TensorList8."""
    if not isinstance(tl, TensorList8):
        raise TypeError("adamw8_grad_norm_sq takes a TensorList8")
    if out.dtype != torch.float64 or out.device != tl.device or out.numel() < 1:
        raise ValueError("out: float64 tensor on the list's device")
    if coef_out is not None:
        if coef_out.dtype != torch.float32 or coef_out.device != tl.device:
            raise ValueError("coef_out: float32 tensor on the list's device")
        if max_norm is None:
            raise ValueError("coef_out needs max_norm")
    _check(lib().adamw8_grad_norm_sq(tl.array, tl.n, tl.grad_dtype, out.data_ptr(),
                                     float(max_norm) if max_norm is not None else 0.0,
                                     float(grad_scale), _ptr(coef_out), tl.workspace_ptr,
                                     tl.workspace_bytes, _stream_handle(stream)),
           "adamw8_grad_norm_sq")
    return out


def adamw8_multi_tensor_step(tl: TensorList8, coef: Optional[torch.Tensor], step: torch.Tensor,
                             lr: float, beta1: float, beta2: float, eps: float,
                             weight_decay: float, skip_if_nonfinite: Optional[torch.Tensor] = None,
                             stream: Optional[torch.cuda.Stream] = None) -> None:
    """adamw_multi_tensor_step with 8-bit moments."""
    if not isinstance(tl, TensorList8):
        raise TypeError("adamw8_multi_tensor_step takes a TensorList8")
    if coef is not None and (coef.dtype != torch.float32 or coef.device != tl.device):
        raise ValueError("coef: float32 tensor on the list's device, or None")
    if step.dtype != torch.int32 or step.device != tl.device:
        raise ValueError("step: int32 tensor on the list's device")
    if skip_if_nonfinite is not None and (skip_if_nonfinite.dtype != torch.float64 or
                                          skip_if_nonfinite.device != tl.device):
        raise ValueError("skip_if_nonfinite: float64 tensor on the list's device, or None")
    _check(lib().adamw8_multi_tensor_step(
        tl.array, tl.n, tl.grad_dtype, _ptr(coef), _ptr(skip_if_nonfinite), step.data_ptr(),
        float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), tl.workspace_ptr,
        tl.workspace_bytes, _stream_handle(stream)), "adamw8_multi_tensor_step")


def adamw8_clipped_step(tl: TensorList8, step: torch.Tensor, lr: float, beta1: float,
                        beta2: float, eps: float, weight_decay: float, max_norm: float,
                        grad_scale: float = 1.0, skip_if_nonfinite: bool = False,
                        sumsq_out: Optional[torch.Tensor] = None,
                        coef_out: Optional[torch.Tensor] = None,
                        stream: Optional[torch.cuda.Stream] = None,
                        mid_event: Optional[torch.cuda.Event] = None) -> None:
    """adamw_clipped_step with 8-bit moments."""
    if not isinstance(tl, TensorList8):
        raise TypeError("adamw8_clipped_step takes a TensorList8")
    _whole_step("adamw8_clipped_step", tl, step, lr, beta1, beta2, eps, weight_decay, max_norm,
                grad_scale, skip_if_nonfinite, sumsq_out, coef_out, stream,
                _event_handle(mid_event))


def adamw8_quantize(x: torch.Tensor, fmt: int, codes: torch.Tensor, scales: torch.Tensor,
                    stream: Optional[torch.cuda.Stream] = None) -> None:
    """Encode fp32 `x` into 8-bit codes and scale bytes (fmt MPS_Q8_E4M3 / _E5M2)."""
    n = x.numel()
    if x.dtype != torch.float32 or x.device.type != "cuda" or not x.is_contiguous():
        raise ValueError("x: contiguous float32 CUDA tensor")
    _require(codes, torch.uint8, n, x.device, "codes")
    _require(scales, torch.uint8, q8_scale_count(n), x.device, "scales")
    _check(lib().adamw8_quantize(_ptr(x), n, int(fmt), _ptr(codes), _ptr(scales),
                                 _stream_handle(stream)), "adamw8_quantize")


def adamw8_dequantize(codes: torch.Tensor, scales: torch.Tensor, fmt: int, out: torch.Tensor,
                      stream: Optional[torch.cuda.Stream] = None) -> None:
    """The fp32 values that 8-bit codes and scale bytes stand for."""
    n = codes.numel()
    if codes.device.type != "cuda":
        raise ValueError("codes: CUDA tensor")
    _require(codes, torch.uint8, n, codes.device, "codes")
    _require(scales, torch.uint8, q8_scale_count(n), codes.device, "scales")
    _require(out, torch.float32, n, codes.device, "out")
    _check(lib().adamw8_dequantize(_ptr(codes), _ptr(scales), n, int(fmt), _ptr(out),
                                   _stream_handle(stream)), "adamw8_dequantize")
