// gfx950 kernels of the clipped mixed-precision AdamW step.
//
// The path is HBM-bound elementwise streaming plus one reduction (about
// 0.6 flop per byte), so there is no matrix-core work here: every kernel is
// built around 128-bit coalesced buffer loads and stores on 64-wide
// wavefronts.
//
//   grad_norm_kernel  sum of g^2 over the tensor list: exact squares summed in
//                     fp64 per thread, a DPP/cross-lane wavefront reduction, an
//                     LDS combine per block; then either a deterministic
//                     second stage run by the last block to finish (ticket
//                     tree), or, for the clipped step, nothing more: the
//                     per-block partials stay in the workspace.
//   clip_coef_kernel  c = min(1, max_norm / (sqrt(S) + 1e-6)), fp64, one lane.
//   adamw_clipped_kernel  the clipped step's update: every block first sums
//                     the norm's partials (the same order and bits as the
//                     second stage) and forms the clip coefficient; block 0
//                     stores the step counter.
//   adamw_step_kernel the three-call step's update, given the coefficient;
//                     the counter is stored by the block with the last ticket.
//                     Both updates share one body: clip scaling, both
//                     moments, decoupled weight decay, bias corrections
//                     derived on the device from the step counter, the
//                     optional bf16 copy.
//   adamw_fused_kernel the whole step in one cooperative launch.
//
// Memory access: each chunk's aligned body is addressed through buffer
// resources (base and size in scalar registers, 32-bit per-lane offsets).
// Lanes past the end of the body read zeros and their stores are dropped by
// the hardware range check, so the loops carry no per-load branches.  The
// streams are touched once, so loads and stores use the nontemporal policy.
//
// Build with -ffp-contract=off: every fp32 operation below must round once,
// in source order; division and sqrt are the correctly rounded defaults.
#include <hip/hip_runtime.h>

#include "device.h"
#include "kernels.h"

namespace mps {
namespace {

// ------------------------------------------------------------ grad norm ---

template <bool kBf16>
__device__ __forceinline__ double add_vector(double acc, u32x4 v)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (kBf16) {
            acc = add_square(acc, bf16_lo(v[k]));
            acc = add_square(acc, bf16_hi(v[k]));
        } else {
            acc = add_square(acc, __uint_as_float(v[k]));
        }
    }
    return acc;
}

// The run of chunks of block b among G: the first n % G blocks take
// n / G + 1 chunks, the others n / G (32-bit arithmetic only).
struct ChunkRun {
    int first, stop;
};

__device__ __forceinline__ ChunkRun block_run(int n_chunks)
{
    const uint32_t n = static_cast<uint32_t>(n_chunks);
    const uint32_t g = gridDim.x, b = blockIdx.x;
    const uint32_t per = n / g, rem = n % g;
    const uint32_t first = b * per + min(b, rem);
    return {static_cast<int>(first), static_cast<int>(first + per + (b < rem ? 1u : 0u))};
}

// The tensor index of chunk c.  A list whose chunks all belong to one tensor
// needs no chunk-map read.
__device__ __forceinline__ uint32_t tensor_of_chunk(const WorkspaceView& ws, int c)
{
    return ws.solo_tensor >= 0 ? static_cast<uint32_t>(ws.solo_tensor) : ws.chunk_map[c];
}

// The tensor index of chunk c for a kernel's prologue: c is clamped into the
// map, which has at least one slot (a block without chunks never uses the
// result).
__device__ __forceinline__ uint32_t prologue_tensor(const WorkspaceView& ws, int c)
{
    return tensor_of_chunk(ws, min(c, max(ws.n_chunks - 1, 0)));
}

// This thread's share of the sum of g^2 over the chunks [run_first,
// run_stop), in a fixed order.  Consecutive chunks of one tensor are one
// contiguous stretch of memory, streamed as a single body so the load
// pipeline only restarts at tensor boundaries.
template <bool kBf16, int kUnroll, int kPolicy>
__device__ __forceinline__ double norm_of_run(const WorkspaceView& ws, uint32_t first_tensor,
                                              int run_first, int run_stop)
{
    const TensorEntry* tensors = ws.tensors;
    const int64_t chunk_elems = ws.chunk_elems;
    constexpr int64_t kElemBytes = kBf16 ? 2 : 4;
    constexpr int64_t kPerVec = 16 / kElemBytes;
    const int tid = threadIdx.x;
    double acc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc[u] = 0.0;

    for (int c = run_first; c < run_stop;) {
        const TensorEntry te = tensors[c == run_first ? first_tensor : tensor_of_chunk(ws, c)];
        const int tensor_chunks = static_cast<int>((te.numel + chunk_elems - 1) / chunk_elems);
        const int c_lo = c;  // this body: chunks [c_lo, c_hi) of one tensor
        const int c_hi = min(run_stop, te.first_chunk + tensor_chunks);
        c = c_hi;
        const void* grad = te.grad;
        const int64_t begin = static_cast<int64_t>(c_lo - te.first_chunk) * chunk_elems;
        const int64_t end = min(static_cast<int64_t>(c_hi - te.first_chunk) * chunk_elems, te.numel);

        // Peel elements until the gradient address is 16-byte aligned.
        const uintptr_t addr = reinterpret_cast<uintptr_t>(grad) + begin * kElemBytes;
        int64_t head = static_cast<int64_t>((16 - (addr & 15)) & 15) / kElemBytes;
        head = min(head, end - begin);
        if (tid < head) acc[0] = add_square(acc[0], grad_at<kBf16>(grad, begin + tid));
        int64_t vbegin = begin + head;
        const int64_t nvec_all = (end - vbegin) / kPerVec;
        const int64_t tail = vbegin + nvec_all * kPerVec;

        // The body in pieces of at most 2^26 vectors (1 GiB), so that byte
        // offsets fit the 32-bit buffer addressing.
        for (int64_t done = 0; done < nvec_all;) {
            const int nvec = static_cast<int>(min(nvec_all - done, static_cast<int64_t>(1) << 26));
            const __amdgpu_buffer_rsrc_t g =
                rsrc(static_cast<const char*>(grad) + (vbegin + done * kPerVec) * kElemBytes,
                     static_cast<uint32_t>(nvec) * 16u);
            done += nvec;

            // Two register sets in turn: the loads of one are in flight while
            // the other is accumulated.  Offsets past the body read zeros
            // without touching memory, so the loop needs no bounds branches.
            constexpr int kStride = kBlock * kUnroll;
            u32x4 x[kUnroll], y[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) x[u] = load_u32x4<kPolicy>(g, (u * kBlock + tid) * 16u);
            for (int base = 0; base < nvec; base += 2 * kStride) {
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    y[u] = load_u32x4<kPolicy>(g, (base + kStride + u * kBlock + tid) * 16u);
                }
                __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the math
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) acc[u] = add_vector<kBf16>(acc[u], x[u]);
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    x[u] = load_u32x4<kPolicy>(g, (base + 2 * kStride + u * kBlock + tid) * 16u);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (base + kStride < nvec) {  // uniform: skip the math of an empty tile
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u) acc[u] = add_vector<kBf16>(acc[u], y[u]);
                }
            }
        }

        if (tid < end - tail) acc[0] = add_square(acc[0], grad_at<kBf16>(grad, tail + tid));
    }

    double mine = acc[0];
#pragma unroll
    for (int u = 1; u < kUnroll; ++u) mine = mine + acc[u];
    return mine;
}

// This block's share of S.  Blocks below `cached_blocks` read their
// gradients with the default cache policy, and what they read stays in the
// Infinity Cache for the update to hit again; the others stream theirs past
// the caches, which reads faster and does not fill the cache (a list larger
// than the cache cannot keep more than one cache's worth anyway).
template <bool kBf16, int kUnroll>
__device__ __forceinline__ double norm_share(const WorkspaceView& ws, int cached_blocks,
                                             uint32_t first_tensor, const ChunkRun& run)
{
    return static_cast<int>(blockIdx.x) < cached_blocks
               ? norm_of_run<kBf16, kUnroll, kPolicyDefault>(ws, first_tensor, run.first, run.stop)
               : norm_of_run<kBf16, kUnroll, kPolicyStream>(ws, first_tensor, run.first, run.stop);
}

// kFinish: the last block to finish sums the partials and writes S (and the
// clip coefficient).  Otherwise the launch ends with one partial per block in
// the workspace, and the step number t = *d_step + 1 in the header, for the
// clipped update to finish.
template <bool kBf16, int kUnroll, bool kFinish>
__global__ __launch_bounds__(kBlock) void grad_norm_kernel(
    WorkspaceView ws, int cached_blocks, double* d_sumsq, double max_norm, double grad_scale,
    float* d_coef, const int32_t* d_step)
{
    const int tid = threadIdx.x;
    const ChunkRun run = block_run(ws.n_chunks);
    // The tag and the first chunk's tensor index are independent loads, in
    // flight together.
    const uint64_t seen = ws.header->tag;
    const uint32_t first_tensor = prologue_tensor(ws, run.first);
    if (seen != ws.tag) {  // tables overwritten: touch nothing, report NaN
        if (kFinish && blockIdx.x == 0 && tid == 0) {
            *d_sumsq = __builtin_nan("");
            if (d_coef) *d_coef = __builtin_nanf("");
        }
        return;
    }

    const double mine = norm_share<kBf16, kUnroll>(ws, cached_blocks, first_tensor, run);

    __shared__ double lds[kWavesPerBlock];
    __shared__ bool is_last;
    const double block_total = block_sum(mine, lds);
    if (!kFinish) {
        if (tid == 0) ws.partials[blockIdx.x] = block_total;
        // The step the following clipped update will take (it reads t here,
        // so its own block 0 may store the counter at any time).
        if (blockIdx.x == 0 && tid == 0) ws.header->pending_step = *d_step + 1;
        return;
    }
    // Hand-off to the last block.  The partial is written with an agent-scope
    // atomic store, which goes through to the device's coherence point, and
    // the ticket is taken only once that store is acknowledged (s_waitcnt on
    // every counter).  That is all the release the partial needs; a general
    // release fence would also write back the whole L2, dirty with the
    // previous update's state.  The last block reads the partials with
    // agent-scope atomic loads, after an acquire fence.
    if (tid == 0) {
        __hip_atomic_store(&ws.partials[blockIdx.x], block_total, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        is_last = last_ticket(ws.tickets);
    }
    __syncthreads();
    if (!is_last) return;

    // Second stage: the last block sums the partials in block-index order.
    const double total = sum_partials<true>(ws.partials, gridDim.x, lds);
    if (tid == 0) {
        *d_sumsq = total;
        if (d_coef) *d_coef = clip_from_sumsq(total, max_norm, grad_scale);
    }
}

// ----------------------------------------------------------------- clip ---

__global__ __launch_bounds__(kWave) void clip_coef_kernel(const double* d_sumsq, double max_norm,
                                                          double grad_scale, float* d_coef)
{
    if (threadIdx.x != 0) return;
    *d_coef = clip_from_sumsq(*d_sumsq, max_norm, grad_scale);
}


// ---------------------------------------------------------------- update ---


template <bool kBf16>
__device__ __forceinline__ void adamw_scalar_at(const TensorEntry* te, int64_t i, const StepScalars& s)
{
    const float grad = grad_at<kBf16>(te->grad, i);
    float w = te->master[i], m = te->exp_avg[i], v = te->exp_avg_sq[i];
    adamw_element(w, m, v, grad, s);
    te->master[i] = w;
    te->exp_avg[i] = m;
    te->exp_avg_sq[i] = v;
    if (te->param_bf16) te->param_bf16[i] = bf16_one(w);
}

// The aligned body of one chunk: `nquad` groups of four elements starting at
// element `q0` of the tensor, every stream 16-byte (fp32) or 8-byte (bf16)
// aligned there.
template <bool kBf16, int kUnroll>
__device__ __forceinline__ void adamw_body(const TensorEntry* te, int64_t q0, int nquad,
                                           const StepScalars& s)
{
    const int tid = threadIdx.x;
    const __amdgpu_buffer_rsrc_t W = rsrc(te->master + q0, nquad * 16u);
    const __amdgpu_buffer_rsrc_t M = rsrc(te->exp_avg + q0, nquad * 16u);
    const __amdgpu_buffer_rsrc_t V = rsrc(te->exp_avg_sq + q0, nquad * 16u);
    const __amdgpu_buffer_rsrc_t G = rsrc(static_cast<const char*>(te->grad) + q0 * (kBf16 ? 2 : 4),
                                          nquad * (kBf16 ? 8u : 16u));
    const bool copy = te->param_bf16 != nullptr;
    const __amdgpu_buffer_rsrc_t P = rsrc(copy ? te->param_bf16 + q0 : nullptr, copy ? nquad * 8u : 0u);

    // One tile = kUnroll groups of four per thread.  Two tiles are held in
    // registers in turn: the loads of the next tile are in flight while the
    // current one is computed and stored.  Lanes past the body read zeros and
    // their stores are dropped, so the tail needs no branches.
    struct Tile {
        f32x4 w[kUnroll], m[kUnroll], v[kUnroll], g[kUnroll];
    };
    auto load_tile = [&](Tile& t, int base) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t q = base + u * kBlock + tid;
            t.w[u] = load_f32x4(W, q * 16u);
            t.m[u] = load_f32x4(M, q * 16u);
            t.v[u] = load_f32x4(V, q * 16u);
            if (kBf16) {
                const u32x2 h = load_u32x2(G, q * 8u);
                t.g[u] = f32x4{bf16_lo(h[0]), bf16_hi(h[0]), bf16_lo(h[1]), bf16_hi(h[1])};
            } else {
                t.g[u] = load_f32x4(G, q * 16u);
            }
        }
    };
    auto update_tile = [&](Tile& t, int base) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t q = base + u * kBlock + tid;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float wk = t.w[u][k], mk = t.m[u][k], vk = t.v[u][k];
                adamw_element(wk, mk, vk, t.g[u][k], s);
                t.w[u][k] = wk;
                t.m[u][k] = mk;
                t.v[u][k] = vk;
            }
            store_f32x4(t.w[u], W, q * 16u);
            store_f32x4(t.m[u], M, q * 16u);
            store_f32x4(t.v[u], V, q * 16u);
            if (copy) {
                u32x2 packed;
                packed[0] = bf16_pack2(t.w[u][0], t.w[u][1]);
                packed[1] = bf16_pack2(t.w[u][2], t.w[u][3]);
                store_u32x2(packed, P, q * 8u);
            }
        }
    };

    constexpr int kStride = kBlock * kUnroll;
    Tile a, b;
    load_tile(a, 0);
    for (int base = 0; base < nquad; base += 2 * kStride) {
        load_tile(b, base + kStride);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the math
        update_tile(a, base);
        if (base + kStride >= nquad) break;  // uniform: the other tile is empty
        load_tile(a, base + 2 * kStride);
        __builtin_amdgcn_sched_barrier(0);
        update_tile(b, base + kStride);
    }
}

// Update the chunks b, b + G, b + 2G, ... of this block (G = gridDim.x): at
// any moment the blocks stream neighbouring chunks.  `next` is the table
// entry of chunk b, fetched by the caller's prologue; the entry of each
// following chunk is fetched before the current chunk streams, so the two
// dependent scalar lookups overlap the data loads.
template <bool kBf16, int kUnroll>
__device__ __forceinline__ void update_chunks(const WorkspaceView& ws, TensorEntry next,
                                              const StepScalars& s)
{
    const int tid = threadIdx.x;
    const int n_chunks = ws.n_chunks;
    const int64_t chunk_elems = ws.chunk_elems;
    for (int c = blockIdx.x; c < n_chunks; c += gridDim.x) {
        const TensorEntry entry = next;
        const int c_next = c + static_cast<int>(gridDim.x);
        if (ws.solo_tensor < 0 && c_next < n_chunks) next = ws.tensors[ws.chunk_map[c_next]];
        const TensorEntry* te = &entry;
        const int64_t begin = static_cast<int64_t>(c - te->first_chunk) * chunk_elems;
        const int64_t end = min(begin + chunk_elems, te->numel);

        if (te->head < 0) {  // streams share no alignment: element-wise
            for (int64_t i = begin + tid; i < end; i += kBlock) adamw_scalar_at<kBf16>(te, i, s);
            continue;
        }
        const int64_t qbegin = min(begin + te->head, end);
        if (tid < qbegin - begin) adamw_scalar_at<kBf16>(te, begin + tid, s);
        const int nquad = static_cast<int>((end - qbegin) / 4);
        adamw_body<kBf16, kUnroll>(te, qbegin, nquad, s);
        const int64_t tail = qbegin + static_cast<int64_t>(nquad) * 4;
        if (tid < end - tail) adamw_scalar_at<kBf16>(te, tail + tid, s);
    }
}

template <bool kBf16, int kUnroll>
__global__ __launch_bounds__(kBlock) void adamw_step_kernel(
    WorkspaceView ws, const float* d_coef, const double* d_skip_if_nonfinite, int32_t* d_step,
    HyperParams hp)
{
    // Independent loads, in flight together (the first chunk is chunk
    // blockIdx.x of the strided walk).
    const uint64_t seen = ws.header->tag;
    const int32_t count = *d_step;
    const float coef = d_coef ? *d_coef : 1.0f;
    const double skip_value = d_skip_if_nonfinite ? *d_skip_if_nonfinite : 0.0;
    const TensorEntry first = ws.tensors[prologue_tensor(ws, blockIdx.x)];
    if (seen != ws.tag) return;  // tables overwritten: touch nothing
    // A skipped step writes nothing and leaves the counter.  The value is
    // uniform, so every block makes the same choice.
    if (!__builtin_isfinite(skip_value)) return;

    const int64_t t = static_cast<int64_t>(count) + 1;
    update_chunks<kBf16, kUnroll>(ws, first, step_scalars(t, hp, coef));
    advance_step(ws.tickets, d_step, t);
}

// The update with the end of the norm folded in.  A norm launch without the
// finish left one partial per block (n_partials of them) and the step number
// in the workspace; every block here sums the partials exactly as the norm's
// own last block would (same order, same tree: S is the same bits), forms the
// clip coefficient, and skips a step whose S is not finite if asked to.
// Block 0 publishes S, the coefficient and the new step count: the blocks
// take t from the header, not from the counter, so the store needs no ticket.
// Against the three-call step this saves the norm's hand-off between its
// blocks (a store, an atomic and a load, each a trip to the device's
// coherence point) and the update's end-of-launch tickets (on a
// 2^20-parameter shard, whose blocks all finish at about the same moment,
// 4 us of 17 with a single counter); it costs a 2 KB read per block that
// overlaps the other prologue loads.
template <bool kBf16, int kUnroll>
__global__ __launch_bounds__(kBlock) void adamw_clipped_kernel(
    WorkspaceView ws, int n_partials, double max_norm, double grad_scale, int skip_if_nonfinite,
    double* d_sumsq, float* d_coef, int32_t* d_step, HyperParams hp)
{
    const int tid = threadIdx.x;
    const uint64_t seen = ws.header->tag;
    const int32_t t = ws.header->pending_step;
    const TensorEntry first = ws.tensors[prologue_tensor(ws, blockIdx.x)];
    if (seen != ws.tag) {  // tables overwritten: touch nothing, report NaN
        if (blockIdx.x == 0 && tid == 0) {
            if (d_sumsq) *d_sumsq = __builtin_nan("");
            if (d_coef) *d_coef = __builtin_nanf("");
        }
        return;
    }
    __shared__ double lds[kWavesPerBlock];
    const double total = sum_partials<false>(ws.partials, n_partials, lds);
    const float clip = clip_from_sumsq(total, max_norm, grad_scale);
    const bool skip = skip_if_nonfinite && !__builtin_isfinite(total);
    if (blockIdx.x == 0 && tid == 0) {
        if (d_sumsq) *d_sumsq = total;
        if (d_coef) *d_coef = clip;
        if (!skip) *d_step = t;
    }
    if (skip) return;
    update_chunks<kBf16, kUnroll>(ws, first, step_scalars(t, hp, clip));
}

// ------------------------------------------------------ single launch ---

constexpr uint32_t kSpinLimit = 1u << 23;  // x s_sleep(2): about 1 s, never reached

// The whole step in one launch: norm, grid barrier, clip, update.  Launched
// cooperatively, so every block is resident and the barrier completes; the
// bounded wait only guards against a broken launch (it then flags the error
// and the waiting block stops without writing state).
template <bool kBf16, int kNormUnroll, int kStepUnroll>
__global__ __launch_bounds__(kBlock) void adamw_fused_kernel(
    WorkspaceView ws, int cached_blocks, double max_norm, double grad_scale, int skip_if_nonfinite,
    double* d_sumsq, float* d_coef, int32_t* d_step, HyperParams hp)
{
    const int tid = threadIdx.x;
    const int grid = gridDim.x;
    WorkspaceHeader* header = ws.header;
    const ChunkRun run = block_run(ws.n_chunks);
    const uint64_t seen = header->tag;
    const uint32_t first_tensor = prologue_tensor(ws, run.first);
    if (seen != ws.tag) {  // tables overwritten: touch nothing, report NaN
        if (blockIdx.x == 0 && tid == 0) {
            if (d_sumsq) *d_sumsq = __builtin_nan("");
            if (d_coef) *d_coef = __builtin_nanf("");
        }
        return;
    }
    // Every block reads the step count before it arrives at the barrier; the
    // last block to arrive is therefore free to store the new count.
    const int64_t t = static_cast<int64_t>(*d_step) + 1;

    // Phase 1: this block's partial of S.
    const double mine = norm_share<kBf16, kNormUnroll>(ws, cached_blocks, first_tensor, run);
    __shared__ double lds[kWavesPerBlock];
    __shared__ uint64_t launch;
    __shared__ bool last, failed;
    const double block_total = block_sum(mine, lds);
    if (tid == 0) {
        __hip_atomic_store(&ws.partials[blockIdx.x], block_total, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);  // the partial is visible device-wide
        const uint64_t arrival = __hip_atomic_fetch_add(&header->fused_arrived, uint64_t{1},
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        launch = arrival / grid;
        last = arrival % grid == static_cast<uint64_t>(grid - 1);
        failed = false;
    }
    __syncthreads();

    // Barrier.  The last block to arrive sums the partials in block order,
    // publishes S and the new step count, then releases the others.
    if (last) {
        const double total = sum_partials<true>(ws.partials, grid, lds);
        if (tid == 0) {
            const bool skip = skip_if_nonfinite && !__builtin_isfinite(total);
            __hip_atomic_store(&header->fused_sumsq, total, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            if (d_sumsq) *d_sumsq = total;
            if (d_coef) *d_coef = clip_from_sumsq(total, max_norm, grad_scale);
            if (!skip) *d_step = static_cast<int32_t>(t);
            __builtin_amdgcn_s_waitcnt(0);  // S is visible before the release
            __hip_atomic_store(&header->fused_released, launch + 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    } else if (tid == 0) {
        uint32_t spins = 0;
        while (__hip_atomic_load(&header->fused_released, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT) < launch + 1) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins == kSpinLimit) {
                __hip_atomic_store(&header->fused_error, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                failed = true;
                break;
            }
        }
    }
    __syncthreads();
    if (failed) return;

    // Phase 2: every block sees the same S, hence the same coefficient.
    const double total = __hip_atomic_load(&header->fused_sumsq, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    if (skip_if_nonfinite && !__builtin_isfinite(total)) return;
    const StepScalars s = step_scalars(t, hp, clip_from_sumsq(total, max_norm, grad_scale));
    update_chunks<kBf16, kStepUnroll>(ws, ws.tensors[prologue_tensor(ws, blockIdx.x)], s);
}

}  // namespace

// --------------------------------------------------------------- launchers ---

namespace {

template <bool kFinish>
void grad_norm_launch(const WorkspaceView& ws, bool grad_bf16, int grid, int cached_blocks,
                      double* d_sumsq, double max_norm, double grad_scale, float* d_coef,
                      const int32_t* d_step, hipStream_t stream)
{
    if (grad_bf16) {
        grad_norm_kernel<true, MPS_NORM_UNROLL, kFinish><<<grid, kBlock, 0, stream>>>(
            ws, cached_blocks, d_sumsq, max_norm, grad_scale, d_coef, d_step);
    } else {
        grad_norm_kernel<false, MPS_NORM_UNROLL, kFinish><<<grid, kBlock, 0, stream>>>(
            ws, cached_blocks, d_sumsq, max_norm, grad_scale, d_coef, d_step);
    }
}

}  // namespace

hipError_t launch_grad_norm(const WorkspaceView& ws, bool grad_bf16, int grid, int cached_blocks,
                            double* d_sumsq, double max_norm, double grad_scale, float* d_coef,
                            hipStream_t stream)
{
    grad_norm_launch<true>(ws, grad_bf16, grid, cached_blocks, d_sumsq, max_norm, grad_scale,
                           d_coef, nullptr, stream);
    return hipGetLastError();
}

hipError_t launch_grad_norm_partials(const WorkspaceView& ws, bool grad_bf16, int grid,
                                     int cached_blocks, const int32_t* d_step, hipStream_t stream)
{
    grad_norm_launch<false>(ws, grad_bf16, grid, cached_blocks, nullptr, 0.0, 0.0, nullptr, d_step,
                            stream);
    return hipGetLastError();
}

hipError_t launch_clip_coef(const double* d_sumsq, double max_norm, double grad_scale,
                            float* d_coef, hipStream_t stream)
{
    clip_coef_kernel<<<1, kWave, 0, stream>>>(d_sumsq, max_norm, grad_scale, d_coef);
    return hipGetLastError();
}

hipError_t launch_adamw_step(const WorkspaceView& ws, bool grad_bf16, int grid,
                             const float* d_coef, const double* d_skip_if_nonfinite,
                             int32_t* d_step, const HyperParams& hp, hipStream_t stream)
{
    if (grad_bf16) {
        adamw_step_kernel<true, MPS_STEP_UNROLL><<<grid, kBlock, 0, stream>>>(
            ws, d_coef, d_skip_if_nonfinite, d_step, hp);
    } else {
        adamw_step_kernel<false, MPS_STEP_UNROLL><<<grid, kBlock, 0, stream>>>(
            ws, d_coef, d_skip_if_nonfinite, d_step, hp);
    }
    return hipGetLastError();
}

hipError_t launch_clipped_step(const WorkspaceView& ws, bool grad_bf16, int grid, int n_partials,
                               double max_norm, double grad_scale, int skip_if_nonfinite,
                               double* d_sumsq, float* d_coef, int32_t* d_step,
                               const HyperParams& hp, hipStream_t stream)
{
    if (grad_bf16) {
        adamw_clipped_kernel<true, MPS_STEP_UNROLL><<<grid, kBlock, 0, stream>>>(
            ws, n_partials, max_norm, grad_scale, skip_if_nonfinite, d_sumsq, d_coef, d_step, hp);
    } else {
        adamw_clipped_kernel<false, MPS_STEP_UNROLL><<<grid, kBlock, 0, stream>>>(
            ws, n_partials, max_norm, grad_scale, skip_if_nonfinite, d_sumsq, d_coef, d_step, hp);
    }
    return hipGetLastError();
}

namespace {

template <bool kBf16>
auto fused_kernel()
{
    return adamw_fused_kernel<kBf16, MPS_NORM_UNROLL, MPS_STEP_UNROLL>;
}

}  // namespace

hipError_t fused_grid_limit(bool grad_bf16, int* max_blocks)
{
    int device = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&device);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e == hipSuccess) {
        e = grad_bf16 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                            &per_cu, reinterpret_cast<const void*>(fused_kernel<true>()), kBlock, 0)
                      : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                            &per_cu, reinterpret_cast<const void*>(fused_kernel<false>()), kBlock, 0);
    }
    *max_blocks = (e == hipSuccess) ? cus * per_cu : 0;
    return e;
}

hipError_t launch_fused_step(const WorkspaceView& ws, bool grad_bf16, int grid, int cached_blocks,
                             double max_norm, double grad_scale, int skip_if_nonfinite,
                             double* d_sumsq, float* d_coef, int32_t* d_step,
                             const HyperParams& hp, hipStream_t stream)
{
    WorkspaceView view = ws;
    HyperParams params = hp;
    void* args[] = {&view,    &cached_blocks, &max_norm, &grad_scale, &skip_if_nonfinite,
                    &d_sumsq, &d_coef,        &d_step,   &params};
    const void* fn = grad_bf16 ? reinterpret_cast<const void*>(fused_kernel<true>())
                               : reinterpret_cast<const void*>(fused_kernel<false>());
    // Cooperative: the runtime refuses the launch unless every block can be
    // resident, which the barrier needs.  (Measured on MI355X: this launch
    // costs about 20 us more than a plain one, so the single-launch step is
    // slower than the two-launch step even on a 2^20-parameter shard.)
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kBlock), args, 0, stream);
}

}  // namespace mps