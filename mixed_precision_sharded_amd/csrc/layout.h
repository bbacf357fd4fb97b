// Device-resident tables shared by the host library and the kernels.
//
// Workspace layout (256-byte aligned base):
//   [0, 64)                      WorkspaceHeader
//   [64, 64 + 64*T)              TensorEntry[T]
//   [.., + 4*K rounded to 8)     uint32 chunk -> tensor index, K chunks
//   [.., + 8*kNormMaxBlocks)     fp64 per-block partial sums of the norm
// Everything before the partials is written by one host-to-device copy when
// the list changes; the partials need no initial value.
#pragma once

#include <stdint.h>

namespace mps {

constexpr int kBlock = 256;               // threads per block, both kernels
constexpr int kNormMaxBlocks = 2048;      // norm grid cap (size of the partials)
constexpr int kStepMaxBlocks = 2048;      // update grid cap
constexpr int64_t kChunkQuantum = 2048;   // chunk sizes are multiples of this
constexpr int64_t kChunkMin = 2048;
constexpr int64_t kChunkMax = 65536;
constexpr int64_t kChunkTarget = 8192;    // aim for about this many chunks

struct alignas(64) WorkspaceHeader {
    uint32_t norm_ticket;   // blocks of the norm kernel that have finished
    uint32_t step_ticket;   // blocks of the update kernel that have finished
    uint64_t tag;           // identifies the uploaded tables
    int32_t n_tensors;
    int32_t n_chunks;
    int64_t chunk_elems;
    uint8_t reserved[32];
};
static_assert(sizeof(WorkspaceHeader) == 64, "header is one 64-byte record");

struct alignas(64) TensorEntry {
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
    const void* grad;
    uint16_t* param_bf16;   // may be null
    int64_t numel;
    int32_t first_chunk;    // global index of the tensor's first chunk
    int32_t head;           // elements before the first 16-byte-aligned group of
                            // four, 0..3; -1 when the streams share no alignment
};
static_assert(sizeof(TensorEntry) == 64, "tensor entry is one 64-byte record");

// Hyperparameters as passed by the caller (fp64, before rounding).
struct HyperParams {
    double lr;
    double beta1;
    double beta2;
    double eps;
    double weight_decay;
};

}  // namespace mps
