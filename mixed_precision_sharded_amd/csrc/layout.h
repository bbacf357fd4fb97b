// Device-resident tables shared by the host library and the kernels.
//
// Workspace layout (256-byte aligned base):
//   [0, 64)                      WorkspaceHeader
//   [64, 64 + 64*T)              TensorEntry[T]
//   [.., + 32*T)                 QuantEntry[T] (8-bit moment lists only)
//   [.., + 4*max(K, 1))          uint32 chunk -> tensor index, K chunks
//   [.. rounded to 128, + 128*(kTicketGroups + 1))  the update's step tickets,
//                                one uint32 per 128-byte line
//   [.., + 16)                   WorkspaceConstants
//   [.. rounded to 256, + 8*kPartials)  fp64 per-block partial sums of the norm
// Everything before the partials is written by one host-to-device copy when
// the list changes (the tickets start at zero and every complete launch
// brings them back to zero); the partials need no initial value.
#pragma once

#include <stdint.h>

namespace mps {

// Tuning knobs (compile-time; the defaults are the measured best on MI355X).
// Both kernels walk the chunks with a persistent grid (block b takes chunks
// b, b + G, ...): long-lived waves streaming neighbouring addresses beat one
// block per chunk on MI355X's HBM3E.  The update's grid, chunk size and tile
// depth were measured with library builds side by side in one process, on
// the workloads' own inputs (random values, one allocation per tensor), in
// three fresh processes each (the placement of the allocations moves every
// figure by up to 5 %, and the ranking of close variants with it):
//   - one GPU's shard (the 8B shard, the 70B and 405B shares): one block per
//     CU (256) with 4096-element chunks streamed 5.8-6.3 % faster than the
//     earlier 1280 blocks with 16384; 512, 768 and 1280 blocks and
//     8192-element chunks were slower on most shards;
//   - a whole model (the 8B-parameter list, 291 tensors): the wide walk wins
//     instead, 1280 blocks with 16384-element chunks, 1.0-2.0 % faster than
//     768 blocks and 3-5 % faster than 256 (on buffers carved from one
//     allocation the order was reversed, so the choice follows the
//     workloads' own layout);
//   - a small list, whose step is latency-bound, is spread one chunk per
//     block.
#ifndef MPS_NORM_MAX_BLOCKS
#define MPS_NORM_MAX_BLOCKS 256    // norm grid cap (= number of fp64 partials)
#endif
#ifndef MPS_STEP_MAX_BLOCKS
#define MPS_STEP_MAX_BLOCKS 256    // update grid cap for a shard: one block per CU
#endif
#ifndef MPS_STEP_SPREAD_CHUNKS
#define MPS_STEP_SPREAD_CHUNKS 1280  // lists of at most this many chunks: one block per chunk
#endif
// Lists of at least MPS_LARGE_LIST_ELEMS elements (a whole model rather
// than one GPU's shard of it) walk wider: at most MPS_LARGE_MAX_BLOCKS
// blocks, chunks of at most MPS_LARGE_CHUNK_MAX elements, tiles of
// MPS_LARGE_UNROLL groups of four per thread.
#ifndef MPS_LARGE_LIST_ELEMS
#define MPS_LARGE_LIST_ELEMS (1ll << 30)
#endif
#ifndef MPS_LARGE_MAX_BLOCKS
#define MPS_LARGE_MAX_BLOCKS 1280
#endif
#ifndef MPS_LARGE_CHUNK_MAX
#define MPS_LARGE_CHUNK_MAX 16384
#endif
#ifndef MPS_LARGE_UNROLL
#define MPS_LARGE_UNROLL 1
#endif
// Groups of four elements per thread per tile of a shard's update, by
// gradient type (two tiles are in flight): two for bf16 gradients (the 405B
// share 3.3 % faster than with one), one for fp32.
#ifndef MPS_STEP_UNROLL_BF16
#define MPS_STEP_UNROLL_BF16 2
#endif
#ifndef MPS_STEP_UNROLL_F32
#define MPS_STEP_UNROLL_F32 1
#endif
#ifndef MPS_CHUNK_MIN
#define MPS_CHUNK_MIN 2048
#endif
// Chunk sizes of a shard's fp32-state list (above) and of an 8-bit-moment
// list: those keep 16384 (4096 measured up to 3.4 % slower, 8192 and 32768
// mixed across the workloads).
#ifndef MPS_CHUNK_MAX
#define MPS_CHUNK_MAX 4096
#endif
#ifndef MPS_Q8_CHUNK_MAX
#define MPS_Q8_CHUNK_MAX 16384
#endif
#ifndef MPS_CHUNK_TARGET
#define MPS_CHUNK_TARGET 3072       // aim for about this many chunks
#endif

// Gradient bytes the norm reads with the default cache policy (the rest
// nontemporally).  What the default reads leave in the 256 MB Infinity Cache
// the update hits again; measured on MI355X, the whole step is equally fast
// for budgets from 320 to 768 MB and slower at 192 MB and below.
#ifndef MPS_NORM_CACHE_BUDGET
#define MPS_NORM_CACHE_BUDGET (384ll << 20)
#endif

// 8-bit-moment update grid cap.  Measured side by side on the workloads' own
// inputs in three fresh processes: 1280 blocks streamed 0.1-2.3 % faster
// than 768 on every workload; 512 and 1024 lost up to 11 % on the 8B shard,
// 256 (one per CU) 25-35 % on all of them.
#ifndef MPS_Q8_MAX_BLOCKS
#define MPS_Q8_MAX_BLOCKS 1280
#endif

#ifndef MPS_FUSED_MAX_BLOCKS
#define MPS_FUSED_MAX_BLOCKS 512   // single-launch step grid cap (all co-resident)
#endif

constexpr int kBlock = 256;                        // threads per block, all kernels
constexpr int kNormMaxBlocks = MPS_NORM_MAX_BLOCKS;
constexpr int kStepMaxBlocks = MPS_STEP_MAX_BLOCKS;
constexpr int kStepSpreadChunks = MPS_STEP_SPREAD_CHUNKS;
constexpr int64_t kLargeListElems = MPS_LARGE_LIST_ELEMS;
constexpr int kLargeMaxBlocks = MPS_LARGE_MAX_BLOCKS;
constexpr int64_t kLargeChunkMax = MPS_LARGE_CHUNK_MAX;
constexpr int kFusedMaxBlocks = MPS_FUSED_MAX_BLOCKS;
constexpr int kQ8MaxBlocks = MPS_Q8_MAX_BLOCKS;
constexpr int kPartials = kNormMaxBlocks > kFusedMaxBlocks ? kNormMaxBlocks : kFusedMaxBlocks;
constexpr int kTicketGroups = 8;                   // first level of the step-ticket tree
constexpr int kTicketStride = 32;                  // uint32s between tickets (128 B)
constexpr int64_t kChunkQuantum = 2048;            // chunk sizes are multiples of this
constexpr int64_t kChunkMin = MPS_CHUNK_MIN;
constexpr int64_t kChunkMax = MPS_CHUNK_MAX;
constexpr int64_t kQ8ChunkMax = MPS_Q8_CHUNK_MAX;
constexpr int64_t kChunkTarget = MPS_CHUNK_TARGET;
constexpr int64_t kNormCacheBudget = MPS_NORM_CACHE_BUDGET;

// The library-held workspace of adamw_clipped_step_noalloc: one array of
// this many bytes per GPU (enough for about 1M chunks — a shard of up to
// 2^30 parameters has at most 262K, a whole model of 17e9 parameters 1M —
// or 60K tensors; MPS_NOALLOC_WORKSPACE_BYTES in the C header).
constexpr size_t kScratchBytes = size_t{4} << 20;
constexpr int kScratchMaxDevices = 64;

struct alignas(64) WorkspaceHeader {
    // The single-launch step's outcome, decided once per launch k (low 32
    // bits of k) by whichever comes first: the last block to arrive at the
    // barrier (publish) or a waiter that gave up (abandon).  `fused_decided`
    // goes from k to k + 1 by compare-and-swap; `fused_abandoned` holds
    // k + 1 when launch k was abandoned.
    uint32_t fused_decided;
    uint32_t fused_abandoned;
    uint64_t tag;           // identifies the uploaded tables
    int32_t n_tensors;
    int32_t n_chunks;
    int64_t chunk_elems;
    // Grid barrier of the single-launch step.  Both counters only grow (from
    // zero at upload): launch k of a grid of G blocks takes arrivals
    // [kG, (k+1)G) and is released when `released` reaches k + 1.
    uint64_t fused_arrived;
    uint64_t fused_released;
    double fused_sumsq;     // S, published by the last block to arrive
    uint32_t fused_error;   // set when a barrier wait ran out (never expected); read
                            // and cleared by adamw_fused_status
    int32_t pending_step;   // the clipped step: t, written by its norm launch
                            // for its update launch
};
static_assert(sizeof(WorkspaceHeader) == 64, "header is one 64-byte record");

// Values the update kernels read where the caller passed no pointer: the
// skip value 0 (never skip) and the clip coefficient 1.  With a pointer
// always present, a kernel's first loads carry no branch and go out
// together.
struct alignas(16) WorkspaceConstants {
    double zero;
    float one;
    uint32_t unused;
};

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

// The 8-bit moment state of one tensor: codes (one byte per element; m in
// E4M3, v in E5M2) and one scale byte per 32 elements (2^(byte - 127); 255
// marks a block holding a non-finite value).
constexpr int kQuantBlock = 32;

struct QuantEntry {
    uint8_t* m_codes;
    uint8_t* m_scales;
    uint8_t* v_codes;
    uint8_t* v_scales;
};
static_assert(sizeof(QuantEntry) == 32, "quant entry is one 32-byte record");

// Hyperparameters as passed by the caller (fp64, before rounding).
struct HyperParams {
    double lr;
    double beta1;
    double beta2;
    double eps;
    double weight_decay;
};

}  // namespace mps
