// Launchers for the gfx950 kernels (defined in kernels.hip).
#pragma once

#include <hip/hip_runtime_api.h>

#include "layout.h"

namespace mps {

// The table entry of the one tensor of a list whose elements all sit in one
// tensor, passed with each launch (the fields of TensorEntry, without its
// 64-byte record alignment, which a kernel argument does not carry).
struct SoloEntry {
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
    const void* grad;
    uint16_t* param_bf16;
    int64_t numel;
    int32_t first_chunk;
    int32_t head;
};

// Pointers into one workspace, derived by the host library from its base.
struct WorkspaceView {
    WorkspaceHeader* header;
    const TensorEntry* tensors;
    const uint32_t* chunk_map;
    uint32_t* tickets;  // the update's step-ticket tree (kTicketGroups + 1 lines)
    double* partials;
    int n_tensors;    // entries in `tensors` (>= 1): a chunk-map value is clamped below it
    int n_chunks;
    int solo_tensor;  // the index every chunk maps to, or -1 (several tensors)
    int64_t chunk_elems;
    uint64_t tag;
    SoloEntry solo;          // that tensor's entry (when solo_tensor >= 0)
    QuantEntry solo_quant;   // and, for an 8-bit-moment list, its 8-bit state
};

// The norm launches take `cached_blocks`: blocks below it read their
// gradients with the default cache policy, the others nontemporally.
hipError_t launch_grad_norm(const WorkspaceView& ws, bool grad_bf16, int grid, int cached_blocks,
                            double* d_sumsq, double max_norm, double grad_scale,
                            float* d_coef, hipStream_t stream);

// The norm's first stage only: one partial sum per block, and the step
// number *d_step + 1, in the workspace for a following launch_clipped_step.
hipError_t launch_grad_norm_partials(const WorkspaceView& ws, bool grad_bf16, int grid,
                                     int cached_blocks, const int32_t* d_step,
                                     hipStream_t stream);

hipError_t launch_clip_coef(const double* d_sumsq, double max_norm, double grad_scale,
                            float* d_coef, hipStream_t stream);

// d_coef and d_skip_if_nonfinite are never NULL here: the library passes
// the workspace's constants (1 and 0) for inputs the caller left out.
// `large`: a whole-model list (MPS_LARGE_LIST_ELEMS elements or more), whose
// update takes MPS_LARGE_UNROLL groups of four per thread per tile.
hipError_t launch_adamw_step(const WorkspaceView& ws, bool grad_bf16, bool large, int grid,
                             const float* d_coef, const double* d_skip_if_nonfinite,
                             int32_t* d_step, const HyperParams& hp, hipStream_t stream);

// The update that finishes the norm from the `n_partials` partials a
// launch_grad_norm_partials of grid n_partials left in the workspace.
hipError_t launch_clipped_step(const WorkspaceView& ws, bool grad_bf16, bool large, int grid,
                               int n_partials, double max_norm, double grad_scale,
                               int skip_if_nonfinite, double* d_sumsq, float* d_coef,
                               int32_t* d_step, const HyperParams& hp, hipStream_t stream);

// Largest grid of the single-launch step whose blocks can all be resident.
hipError_t fused_grid_limit(bool grad_bf16, int* max_blocks);

// The single-launch step (cooperative launch; `grid` must not exceed
// fused_grid_limit nor kFusedMaxBlocks).  `spin_limit`: rounds of the
// barrier's bounded wait (0: the default, about 1 s).
hipError_t launch_fused_step(const WorkspaceView& ws, bool grad_bf16, int grid, int cached_blocks,
                             double max_norm, double grad_scale, int skip_if_nonfinite,
                             double* d_sumsq, float* d_coef, int32_t* d_step,
                             const HyperParams& hp, uint32_t spin_limit, hipStream_t stream);

// Copies the single-launch step's error flag from the header into *d_error
// and clears it.
hipError_t launch_fused_status(WorkspaceHeader* header, uint32_t* d_error, hipStream_t stream);

// The device address of the library-held workspace (kScratchBytes) on the
// current device, `device`: looked up once per device, with that device
// current, and kept.
hipError_t scratch_address(int device, void** ptr);

// 8-bit moment state (kernels_q8.hip).  `quant` is the QuantEntry table in
// the same workspace; d_coef and d_skip_if_nonfinite are never NULL (as in
// launch_adamw_step).
hipError_t launch_adamw8_step(const WorkspaceView& ws, const QuantEntry* quant, bool grad_bf16,
                              int grid, const float* d_coef, const double* d_skip_if_nonfinite,
                              int32_t* d_step, const HyperParams& hp, hipStream_t stream);

// The 8-bit update that finishes the norm (as launch_clipped_step).
hipError_t launch_adamw8_clipped(const WorkspaceView& ws, const QuantEntry* quant, bool grad_bf16,
                                 int grid, int n_partials, double max_norm, double grad_scale,
                                 int skip_if_nonfinite, double* d_sumsq, float* d_coef,
                                 int32_t* d_step, const HyperParams& hp, hipStream_t stream);

hipError_t launch_quantize(const float* x, int64_t n, bool e4m3, uint8_t* codes, uint8_t* scales,
                           hipStream_t stream);

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t n, bool e4m3,
                             float* x, hipStream_t stream);

}  // namespace mps
