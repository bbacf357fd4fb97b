"""Fused, clipped, mixed-precision AdamW step for one GPU's shard (gfx950).

The compute path is the HIP library libmps_adamw.so (C ABI in
include/mps_adamw.h); `binding` marshals torch tensors into it.  `configs`
and `synth` describe and generate the seeded synthetic workloads.  Importing
the package does not load the library: the first call does, and raises if it
is not built.
"""
from .binding import (MPS_DTYPE_BF16, MPS_DTYPE_F32, MPS_Q8_E4M3, MPS_Q8_E5M2,  # noqa: F401
                      MpsError, TensorList, TensorList8, adamw8_clipped_step, adamw8_dequantize,
                      adamw8_grad_norm_sq, adamw8_multi_tensor_step, adamw8_quantize,
                      adamw_clipped_step, adamw_fused_step, adamw_multi_tensor_step, clip_coef,
                      grad_norm_sq, last_error, zeros_q8_state)
