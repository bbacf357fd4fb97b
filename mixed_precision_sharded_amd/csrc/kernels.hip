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
// Memory access: every access of the updates to the tensors goes through a
// buffer resource (base and size in scalar registers, 32-bit per-lane
// offsets): the vector bodies, and the per-element heads, tails and
// unaligned tensors, one element per lane.  Lanes past the end read zeros
// and their stores are dropped by the hardware range check, so the loops
// carry no per-load branches.  The workspace tables are read with scalar
// loads (a constant-address-space view).  Both matter to the compiler's
// waits: with only buffer operations in flight it counts them in issue
// order and keeps the next tile's loads in flight while a tile is computed;
// one flat access, a descriptor it cannot prove uniform or a branch inside
// the tile loop made it wait for everything.  The streams are touched once,
// so their loads and stores use the nontemporal policy.
//
// Build with -ffp-contract=off: every fp32 operation below must round once,
// in source order; division and sqrt are the correctly rounded defaults.
#include <hip/hip_runtime.h>

#include <mutex>

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
// needs no chunk-map read.  The value read from the map is clamped into the
// tensor table, whose size comes with the launch: the prologues read the
// entry before the header's tag has been compared, and a map overwritten
// behind the library's back must not send that read past the table.
__device__ __forceinline__ uint32_t tensor_of_chunk(const WorkspaceView& ws, int c)
{
    return ws.solo_tensor >= 0 ? static_cast<uint32_t>(ws.solo_tensor)
                               : table_index(constant_view(ws.chunk_map)[c], ws.n_tensors);
}

// The tensor index of chunk c for a kernel's prologue: c is clamped into the
// map, which has at least one slot (a block without chunks never uses the
// result).
__device__ __forceinline__ uint32_t prologue_tensor(const WorkspaceView& ws, int c)
{
    return tensor_of_chunk(ws, min(c, max(ws.n_chunks - 1, 0)));
}

// Adds this thread's share of the sum of g^2 over elements [begin, end) of
// one gradient to acc: a peel to 16-byte alignment, the vector body, the
// tail.
template <bool kBf16, int kUnroll, int kPolicy>
__device__ __forceinline__ void norm_stretch(const void* grad, int64_t begin, int64_t end,
                                             double (&acc)[kUnroll])
{
    constexpr int64_t kElemBytes = kBf16 ? 2 : 4;
    constexpr int64_t kPerVec = 16 / kElemBytes;
    const int tid = threadIdx.x;

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

template <int kUnroll>
__device__ __forceinline__ double sum_of(const double (&acc)[kUnroll])
{
    double mine = acc[0];
#pragma unroll
    for (int u = 1; u < kUnroll; ++u) mine = mine + acc[u];
    return mine;
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
    double acc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc[u] = 0.0;

    for (int c = run_first; c < run_stop;) {
        const TensorEntry te =
            read_entry(tensors, c == run_first ? first_tensor : tensor_of_chunk(ws, c));
        const int tensor_chunks = static_cast<int>((te.numel + chunk_elems - 1) / chunk_elems);
        const int c_lo = c;  // this stretch: chunks [c_lo, c_hi) of one tensor
        const int c_hi = min(run_stop, te.first_chunk + tensor_chunks);
        c = c_hi;
        const int64_t begin = static_cast<int64_t>(c_lo - te.first_chunk) * chunk_elems;
        const int64_t end = min(static_cast<int64_t>(c_hi - te.first_chunk) * chunk_elems, te.numel);
        norm_stretch<kBf16, kUnroll, kPolicy>(te.grad, begin, end, acc);
    }
    return sum_of(acc);
}

// The same when every chunk belongs to the one tensor `te` that came with
// the launch: the run is one stretch, and no table is read.
template <bool kBf16, int kUnroll, int kPolicy>
__device__ __forceinline__ double norm_of_solo_run(const SoloEntry& te, int64_t chunk_elems,
                                                   int run_first, int run_stop)
{
    double acc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc[u] = 0.0;
    const int64_t begin = static_cast<int64_t>(run_first - te.first_chunk) * chunk_elems;
    const int64_t end =
        max(begin, min(static_cast<int64_t>(run_stop - te.first_chunk) * chunk_elems, te.numel));
    norm_stretch<kBf16, kUnroll, kPolicy>(te.grad, begin, end, acc);
    return sum_of(acc);
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

template <bool kBf16, int kUnroll>
__device__ __forceinline__ double norm_solo_share(const WorkspaceView& ws, int cached_blocks,
                                                  const ChunkRun& run)
{
    return static_cast<int>(blockIdx.x) < cached_blocks
               ? norm_of_solo_run<kBf16, kUnroll, kPolicyDefault>(ws.solo, ws.chunk_elems,
                                                                   run.first, run.stop)
               : norm_of_solo_run<kBf16, kUnroll, kPolicyStream>(ws.solo, ws.chunk_elems,
                                                                  run.first, run.stop);
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
    const uint64_t seen = ws.header->tag;
    auto report_stale = [&] {  // tables overwritten: write nothing but a NaN S
        if (kFinish && blockIdx.x == 0 && tid == 0) {
            *d_sumsq = __builtin_nan("");
            if (d_coef) *d_coef = __builtin_nanf("");
        }
    };
    double mine;
    if (ws.solo_tensor >= 0) {
        // One tensor, which came with the launch: its reads need no table and
        // start at once; the tag is checked below, before anything is written.
        mine = norm_solo_share<kBf16, kUnroll>(ws, cached_blocks, run);
    } else {
        // The tag and the first chunk's tensor index are independent loads,
        // in flight together; the table's pointers are used only once the tag
        // has matched.
        const uint32_t first_tensor = prologue_tensor(ws, run.first);
        if (seen != ws.tag) {
            report_stale();
            return;
        }
        mine = norm_share<kBf16, kUnroll>(ws, cached_blocks, first_tensor, run);
    }

    __shared__ double lds[kWavesPerBlock];
    __shared__ bool is_last;
    const double block_total = block_sum(mine, lds);
    if (seen != ws.tag) {
        report_stale();
        return;
    }
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


// Elements [base, base + count) of one tensor (0 <= count <= kBlock), one
// per lane, through buffer resources like the vector body: lanes past count
// read zeros and their stores are dropped.  Plain pointer accesses here
// would be flat memory operations, which the compiler cannot order against
// the body's buffer operations; it then waited for every load in flight
// before each tile, the next tile's loads included.
template <bool kBf16, class Entry>
__device__ __forceinline__ void adamw_elements_at(const Entry* te, int64_t base, int64_t count,
                                                  const StepScalars& s)
{
    if (count <= 0) return;  // uniform
    const uint32_t n = static_cast<uint32_t>(count);
    const __amdgpu_buffer_rsrc_t W = rsrc(te->master + base, n * 4u);
    const __amdgpu_buffer_rsrc_t M = rsrc(te->exp_avg + base, n * 4u);
    const __amdgpu_buffer_rsrc_t V = rsrc(te->exp_avg_sq + base, n * 4u);
    const __amdgpu_buffer_rsrc_t G = rsrc(static_cast<const char*>(te->grad) + base * (kBf16 ? 2 : 4),
                                          n * (kBf16 ? 2u : 4u));
    const __amdgpu_buffer_rsrc_t P = rsrc(te->param_bf16 ? te->param_bf16 + base : nullptr,
                                          te->param_bf16 ? n * 2u : 0u);
    const uint32_t o = threadIdx.x;
    float w = load_f32(W, o * 4u), m = load_f32(M, o * 4u), v = load_f32(V, o * 4u);
    const float g = kBf16 ? __uint_as_float(static_cast<uint32_t>(load_u16(G, o * 2u)) << 16)
                          : load_f32(G, o * 4u);
    adamw_element(w, m, v, g, s);
    store_f32(w, W, o * 4u);
    store_f32(m, M, o * 4u);
    store_f32(v, V, o * 4u);
    store_u16(bf16_one(w), P, o * 2u);
}

// The aligned body of one chunk: `nquad` groups of four elements starting at
// element `q0` of the tensor, every stream 16-byte (fp32) or 8-byte (bf16)
// aligned there.  One tile = kUnroll groups of four per thread.  Two tiles
// are held in registers in turn: the loads of the next tile are in flight
// while the current one is computed and stored.  Lanes past the body read
// zeros and their stores are dropped, so the tail needs no branches.
template <bool kBf16, int kUnroll>
struct Body {
    // The gradient stays in its loaded bits until the arithmetic: converting
    // bf16 in load() would wait for the load right after issuing it.
    struct Tile {
        f32x4 w[kUnroll], m[kUnroll], v[kUnroll];
        u32x4 g[kUnroll];  // fp32: four values; bf16: g[0..1] hold four
    };
    __amdgpu_buffer_rsrc_t W, M, V, G, P;
    bool copy;
    int nquad;

    template <class Entry>
    __device__ __forceinline__ Body(const Entry* te, int64_t q0, int n)
        : W(rsrc(te->master + q0, static_cast<uint32_t>(n) * 16u)),
          M(rsrc(te->exp_avg + q0, static_cast<uint32_t>(n) * 16u)),
          V(rsrc(te->exp_avg_sq + q0, static_cast<uint32_t>(n) * 16u)),
          G(rsrc(static_cast<const char*>(te->grad) + q0 * (kBf16 ? 2 : 4),
                 static_cast<uint32_t>(n) * (kBf16 ? 8u : 16u))),
          P(rsrc(te->param_bf16 ? te->param_bf16 + q0 : nullptr,
                 te->param_bf16 ? static_cast<uint32_t>(n) * 8u : 0u)),
          copy(te->param_bf16 != nullptr),
          nquad(n)
    {
    }

    __device__ __forceinline__ void load(Tile& t, int base) const
    {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t q = base + u * kBlock + threadIdx.x;
            t.w[u] = load_f32x4(W, q * 16u);
            t.m[u] = load_f32x4(M, q * 16u);
            t.v[u] = load_f32x4(V, q * 16u);
            if (kBf16) {
                const u32x2 h = load_u32x2(G, q * 8u);
                t.g[u] = u32x4{h[0], h[1], 0u, 0u};
            } else {
                t.g[u] = __builtin_bit_cast(u32x4, load_f32x4(G, q * 16u));
            }
        }
    }

    template <bool kCopy>
    __device__ __forceinline__ void update(Tile& t, int base, const StepScalars& s) const
    {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t q = base + u * kBlock + threadIdx.x;
            const f32x4 g = kBf16 ? f32x4{bf16_lo(t.g[u][0]), bf16_hi(t.g[u][0]),
                                          bf16_lo(t.g[u][1]), bf16_hi(t.g[u][1])}
                                  : __builtin_bit_cast(f32x4, t.g[u]);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float wk = t.w[u][k], mk = t.m[u][k], vk = t.v[u][k];
                adamw_element(wk, mk, vk, g[k], s);
                t.w[u][k] = wk;
                t.m[u][k] = mk;
                t.v[u][k] = vk;
            }
            store_f32x4(t.w[u], W, q * 16u);
            store_f32x4(t.m[u], M, q * 16u);
            store_f32x4(t.v[u], V, q * 16u);
            if (kCopy) {
                u32x2 packed;
                packed[0] = bf16_pack2(t.w[u][0], t.w[u][1]);
                packed[1] = bf16_pack2(t.w[u][2], t.w[u][3]);
                store_u32x2(packed, P, q * 8u);
            }
        }
    }

    // Streams the body; `a` already holds the loads of its first tile.
    // The copy is decided once per body: a branch inside the loop would make
    // the compiler wait for every load in flight, the next tile's included,
    // before each tile's arithmetic.
    __device__ __forceinline__ void run(Tile& a, const StepScalars& s) const
    {
        if (copy) {
            run_tiles<true>(a, s);
        } else {
            run_tiles<false>(a, s);
        }
    }

    template <bool kCopy>
    __device__ __forceinline__ void run_tiles(Tile& a, const StepScalars& s) const
    {
        constexpr int kStride = kBlock * kUnroll;
        Tile b;
        for (int base = 0; base < nquad; base += 2 * kStride) {
            load(b, base + kStride);
            __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the math
            update<kCopy>(a, base, s);
            if (base + kStride >= nquad) break;  // uniform: the other tile is empty
            load(a, base + 2 * kStride);
            __builtin_amdgcn_sched_barrier(0);
            update<kCopy>(b, base + kStride, s);
        }
    }
};

// The element ranges of chunk c of a tensor whose streams share an
// alignment (head >= 0): scalar [begin, qbegin), nquad groups of four from
// qbegin, scalar [tail, end).
struct ChunkSpan {
    int64_t begin, qbegin, tail, end;
    int nquad;
};

template <class Entry>
__device__ __forceinline__ ChunkSpan chunk_span(const Entry* te, int c, int64_t chunk_elems)
{
    ChunkSpan k;
    k.begin = static_cast<int64_t>(c - te->first_chunk) * chunk_elems;
    k.end = min(k.begin + chunk_elems, te->numel);
    k.qbegin = min(k.begin + te->head, k.end);
    k.nquad = static_cast<int>((k.end - k.qbegin) / 4);
    k.tail = k.qbegin + static_cast<int64_t>(k.nquad) * 4;
    return k;
}

// Chunk c of tensor te in full.
template <bool kBf16, int kUnroll, class Entry>
__device__ __forceinline__ void adamw_chunk(const Entry* te, int c, int64_t chunk_elems,
                                            const StepScalars& s)
{
    if (te->head < 0) {  // streams share no alignment: element-wise
        const int64_t begin = static_cast<int64_t>(c - te->first_chunk) * chunk_elems;
        const int64_t end = min(begin + chunk_elems, te->numel);
        for (int64_t b = begin; b < end; b += kBlock) {
            adamw_elements_at<kBf16>(te, b, min(static_cast<int64_t>(kBlock), end - b), s);
        }
        return;
    }
    const ChunkSpan k = chunk_span(te, c, chunk_elems);
    adamw_elements_at<kBf16>(te, k.begin, k.qbegin - k.begin, s);
    const Body<kBf16, kUnroll> body(te, k.qbegin, k.nquad);
    typename Body<kBf16, kUnroll>::Tile a;
    body.load(a, 0);
    body.run(a, s);
    adamw_elements_at<kBf16>(te, k.tail, k.end - k.tail, s);
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
    const int n_chunks = ws.n_chunks;
    for (int c = blockIdx.x; c < n_chunks; c += gridDim.x) {
        const TensorEntry entry = uniform_entry(next);
        const int c_next = c + static_cast<int>(gridDim.x);
        if (ws.solo_tensor < 0 && c_next < n_chunks) {
            next = read_entry(ws.tensors, tensor_of_chunk(ws, c_next));
        }
        adamw_chunk<kBf16, kUnroll>(&entry, c, ws.chunk_elems, s);
    }
}

// A block's walk over a one-tensor list, whose tensor came with the launch
// (no table is read).  The constructor does the address arithmetic of the
// block's first chunk (chunk blockIdx.x of the strided walk); load_first()
// issues the loads of its first tile, so that a kernel can put them in
// flight before it waits for anything; finish() streams that chunk and the
// block's later ones.  A block whose first chunk has no vector body loads
// nothing there (an empty range).
template <bool kBf16, int kUnroll>
struct SoloWalk {
    const SoloEntry* te;
    int n_chunks;
    int64_t chunk_elems;
    ChunkSpan k;
    bool whole, vector;
    Body<kBf16, kUnroll> body;
    typename Body<kBf16, kUnroll>::Tile a;

    __device__ __forceinline__ explicit SoloWalk(const WorkspaceView& ws)
        : te(&ws.solo),
          n_chunks(ws.n_chunks),
          chunk_elems(ws.chunk_elems),
          k(chunk_span(&ws.solo, min(static_cast<int>(blockIdx.x), ws.n_chunks - 1),
                       ws.chunk_elems)),
          whole(static_cast<int>(blockIdx.x) < ws.n_chunks),
          vector(whole && ws.solo.head >= 0),
          body(&ws.solo, vector ? k.qbegin : k.begin, vector ? k.nquad : 0)
    {
    }

    __device__ __forceinline__ void load_first() { body.load(a, 0); }

    __device__ __forceinline__ void finish(const StepScalars& s)
    {
        if (vector) {
            adamw_elements_at<kBf16>(te, k.begin, k.qbegin - k.begin, s);
            body.run(a, s);
            adamw_elements_at<kBf16>(te, k.tail, k.end - k.tail, s);
        } else if (whole) {
            adamw_chunk<kBf16, kUnroll>(te, static_cast<int>(blockIdx.x), chunk_elems, s);
        }
        for (int c = blockIdx.x + gridDim.x; c < n_chunks; c += gridDim.x) {
            adamw_chunk<kBf16, kUnroll>(te, c, chunk_elems, s);
        }
    }
};

template <bool kBf16, int kUnroll>
__global__ __launch_bounds__(kBlock) void adamw_step_kernel(
    WorkspaceView ws, const float* d_coef, const double* d_skip_if_nonfinite, int32_t* d_step,
    HyperParams hp)
{
    if (ws.solo_tensor >= 0) {
        // The address arithmetic of the first tile from the kernel
        // arguments, then the scalar loads and that tile's loads, all in
        // flight together; the tag is compared before anything is stored.
        SoloWalk<kBf16, kUnroll> walk(ws);
        const uint64_t seen = ws.header->tag;
        const int32_t count = *d_step;
        const float coef = *d_coef;
        const double skip_value = *d_skip_if_nonfinite;
        walk.load_first();
        __builtin_amdgcn_sched_barrier(0);
        if (seen != ws.tag) return;                  // tables overwritten: touch nothing
        if (!__builtin_isfinite(skip_value)) return;  // a skipped step writes nothing
        const int64_t t = static_cast<int64_t>(count) + 1;
        walk.finish(step_scalars(t, hp, coef));
        advance_step(ws.tickets, d_step, t);
        return;
    }

    // Independent loads, in flight together (the first chunk is chunk
    // blockIdx.x of the strided walk).
    const uint64_t seen = ws.header->tag;
    const int32_t count = *d_step;
    const float coef = *d_coef;
    const double skip_value = *d_skip_if_nonfinite;
    const int64_t t = static_cast<int64_t>(count) + 1;
    const TensorEntry first = read_entry(ws.tensors, prologue_tensor(ws, blockIdx.x));
    if (seen != ws.tag) return;  // tables overwritten: touch nothing
    // A skipped step writes nothing and leaves the counter.  The value is
    // uniform, so every block makes the same choice.
    if (!__builtin_isfinite(skip_value)) return;

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
//
// A list with one tensor brings that tensor's entry with the launch, and
// the kernel starts by issuing the loads of its first tile, before it reads
// the tag or the partials: on a small shard the update then waits for one
// memory round trip before its data moves instead of three.  The tag is
// checked before anything is stored.
template <bool kBf16, int kUnroll>
__global__ __launch_bounds__(kBlock) void adamw_clipped_kernel(
    WorkspaceView ws, int n_partials, double max_norm, double grad_scale, int skip_if_nonfinite,
    double* d_sumsq, float* d_coef, int32_t* d_step, HyperParams hp)
{
    // The header first: read before anything else, these are scalar loads,
    // which the vector-memory counter does not wait for.
    const uint64_t seen = ws.header->tag;
    const int32_t t = ws.header->pending_step;
    __shared__ double lds[kWavesPerBlock];

    if (ws.solo_tensor >= 0) {
        SoloWalk<kBf16, kUnroll> walk(ws);
        // The vector-memory counter is waited for in issue order.  All the
        // address arithmetic comes first, then the loads of the partials,
        // then the tile's: the sum of the partials can start while the tile
        // is still in flight.
        __builtin_amdgcn_sched_barrier(0);
        const PartialSlots slots = load_partials<false>(ws.partials);
        __builtin_amdgcn_sched_barrier(0);
        walk.load_first();
        __builtin_amdgcn_sched_barrier(0);
        const double total = block_sum(partial_share(slots, n_partials), lds);
        if (seen != ws.tag) {
            report_stale_clip(d_sumsq, d_coef);
            return;
        }
        const float clip = clip_from_sumsq(total, max_norm, grad_scale);
        if (publish_clip(total, clip, t, skip_if_nonfinite, d_sumsq, d_coef, d_step)) return;
        walk.finish(step_scalars(t, hp, clip));
        return;
    }

    const TensorEntry first = read_entry(ws.tensors, prologue_tensor(ws, blockIdx.x));
    if (seen != ws.tag) {
        report_stale_clip(d_sumsq, d_coef);
        return;
    }
    const double total = sum_partials<false>(ws.partials, n_partials, lds);
    const float clip = clip_from_sumsq(total, max_norm, grad_scale);
    if (publish_clip(total, clip, t, skip_if_nonfinite, d_sumsq, d_coef, d_step)) return;
    update_chunks<kBf16, kUnroll>(ws, first, step_scalars(t, hp, clip));
}

// ------------------------------------------------------ single launch ---

// The barrier's wait is bounded: kSpinLimit rounds of s_sleep(2), about 1 s,
// never reached in a launch whose blocks are all resident.  The host may pass
// a smaller limit (the library's test hook), so that the give-up path can be
// exercised with every block still ending normally.
constexpr uint32_t kSpinLimit = 1u << 23;

// A waiter gives launch k up: it takes the launch's one decision (k -> k + 1)
// if the last block has not taken it yet.  True if this call decided.
__device__ __forceinline__ bool take_decision(WorkspaceHeader* header, uint32_t k)
{
    uint32_t expected = k;
    return __hip_atomic_compare_exchange_strong(&header->fused_decided, &expected, k + 1u,
                                                __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
}

// The whole step in one launch: norm, grid barrier, clip, update.  Launched
// cooperatively, so every block is resident and the barrier completes.  The
// bounded wait guards against a broken launch: the first waiter to run out
// abandons the launch (if the last block has not already published), and an
// abandoned launch writes no element, leaves the counter, and reports NaN for
// S and the coefficient, with the workspace's error flag set.  A waiter that
// runs out after the last block has published keeps waiting for the release
// (it is on its way), again bounded; running out a second time only sets the
// flag.
template <bool kBf16, int kNormUnroll, int kStepUnroll>
__global__ __launch_bounds__(kBlock) void adamw_fused_kernel(
    WorkspaceView ws, int cached_blocks, double max_norm, double grad_scale, int skip_if_nonfinite,
    double* d_sumsq, float* d_coef, int32_t* d_step, HyperParams hp, uint32_t spin_limit)
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
    const uint32_t k = static_cast<uint32_t>(launch);

    // Barrier.  The last block to arrive sums the partials in block order and,
    // unless a waiter gave the launch up first, publishes S and the new step
    // count; either way it then releases the others.
    if (last) {
        const double total = sum_partials<true>(ws.partials, grid, lds);
        if (tid == 0) {
            if (take_decision(header, k)) {
                const bool skip = skip_if_nonfinite && !__builtin_isfinite(total);
                __hip_atomic_store(&header->fused_sumsq, total, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                if (d_sumsq) *d_sumsq = total;
                if (d_coef) *d_coef = clip_from_sumsq(total, max_norm, grad_scale);
                if (!skip) *d_step = static_cast<int32_t>(t);
            } else {
                __hip_atomic_store(&header->fused_abandoned, k + 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                if (d_sumsq) *d_sumsq = __builtin_nan("");
                if (d_coef) *d_coef = __builtin_nanf("");
            }
            __builtin_amdgcn_s_waitcnt(0);  // all of it is visible before the release
            __hip_atomic_store(&header->fused_released, launch + 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    } else if (tid == 0) {
        uint32_t spins = 0;
        bool gave_up_once = false;
        while (__hip_atomic_load(&header->fused_released, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT) < launch + 1) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins < spin_limit) continue;
            if (!gave_up_once && !take_decision(header, k)) {
                gave_up_once = true;  // the last block has published: wait for its release
                spins = 0;
                continue;
            }
            __hip_atomic_store(&header->fused_error, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            if (!gave_up_once) {  // this block abandoned the launch
                if (d_sumsq) *d_sumsq = __builtin_nan("");
                if (d_coef) *d_coef = __builtin_nanf("");
            }
            failed = true;
            break;
        }
    }
    __syncthreads();
    if (failed) return;
    // An abandoned launch (the last block recorded it before the release)
    // writes no element.
    if (__hip_atomic_load(&header->fused_abandoned, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        k + 1u) {
        return;
    }

    // Phase 2: every block sees the same S, hence the same coefficient.
    const double total = __hip_atomic_load(&header->fused_sumsq, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    if (skip_if_nonfinite && !__builtin_isfinite(total)) return;
    const StepScalars s = step_scalars(t, hp, clip_from_sumsq(total, max_norm, grad_scale));
    update_chunks<kBf16, kStepUnroll>(
        ws, read_entry(ws.tensors, prologue_tensor(ws, blockIdx.x)), s);
}

// The single-launch step's error flag: copied out and cleared (one lane).
__global__ __launch_bounds__(kWave) void fused_status_kernel(WorkspaceHeader* header,
                                                             uint32_t* d_error)
{
    if (threadIdx.x != 0) return;
    *d_error = __hip_atomic_exchange(&header->fused_error, 0u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
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

namespace {

// The update kernels' tile depth (groups of four per thread): a whole-model
// list's, or a shard's by gradient type.
template <bool kBf16, bool kLarge>
constexpr int step_unroll()
{
    return kLarge ? MPS_LARGE_UNROLL : (kBf16 ? MPS_STEP_UNROLL_BF16 : MPS_STEP_UNROLL_F32);
}

template <bool kBf16, bool kLarge>
void step_launch(const WorkspaceView& ws, int grid, const float* d_coef,
                 const double* d_skip_if_nonfinite, int32_t* d_step, const HyperParams& hp,
                 hipStream_t stream)
{
    adamw_step_kernel<kBf16, step_unroll<kBf16, kLarge>()><<<grid, kBlock, 0, stream>>>(
        ws, d_coef, d_skip_if_nonfinite, d_step, hp);
}

template <bool kBf16, bool kLarge>
void clipped_launch(const WorkspaceView& ws, int grid, int n_partials, double max_norm,
                    double grad_scale, int skip_if_nonfinite, double* d_sumsq, float* d_coef,
                    int32_t* d_step, const HyperParams& hp, hipStream_t stream)
{
    adamw_clipped_kernel<kBf16, step_unroll<kBf16, kLarge>()><<<grid, kBlock, 0, stream>>>(
        ws, n_partials, max_norm, grad_scale, skip_if_nonfinite, d_sumsq, d_coef, d_step, hp);
}

}  // namespace

hipError_t launch_adamw_step(const WorkspaceView& ws, bool grad_bf16, bool large, int grid,
                             const float* d_coef, const double* d_skip_if_nonfinite,
                             int32_t* d_step, const HyperParams& hp, hipStream_t stream)
{
    if (grad_bf16) {
        (large ? step_launch<true, true> : step_launch<true, false>)(
            ws, grid, d_coef, d_skip_if_nonfinite, d_step, hp, stream);
    } else {
        (large ? step_launch<false, true> : step_launch<false, false>)(
            ws, grid, d_coef, d_skip_if_nonfinite, d_step, hp, stream);
    }
    return hipGetLastError();
}

hipError_t launch_clipped_step(const WorkspaceView& ws, bool grad_bf16, bool large, int grid,
                               int n_partials, double max_norm, double grad_scale,
                               int skip_if_nonfinite, double* d_sumsq, float* d_coef,
                               int32_t* d_step, const HyperParams& hp, hipStream_t stream)
{
    if (grad_bf16) {
        (large ? clipped_launch<true, true> : clipped_launch<true, false>)(
            ws, grid, n_partials, max_norm, grad_scale, skip_if_nonfinite, d_sumsq, d_coef,
            d_step, hp, stream);
    } else {
        (large ? clipped_launch<false, true> : clipped_launch<false, false>)(
            ws, grid, n_partials, max_norm, grad_scale, skip_if_nonfinite, d_sumsq, d_coef,
            d_step, hp, stream);
    }
    return hipGetLastError();
}

namespace {

template <bool kBf16>
auto fused_kernel()
{
    return adamw_fused_kernel<kBf16, MPS_NORM_UNROLL, MPS_FUSED_STEP_UNROLL>;
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
                             const HyperParams& hp, uint32_t spin_limit, hipStream_t stream)
{
    WorkspaceView view = ws;
    HyperParams params = hp;
    if (spin_limit == 0) spin_limit = kSpinLimit;
    void* args[] = {&view,    &cached_blocks, &max_norm, &grad_scale, &skip_if_nonfinite,
                    &d_sumsq, &d_coef,        &d_step,   &params,     &spin_limit};
    const void* fn = grad_bf16 ? reinterpret_cast<const void*>(fused_kernel<true>())
                               : reinterpret_cast<const void*>(fused_kernel<false>());
    // Cooperative: the runtime refuses the launch unless every block can be
    // resident, which the barrier needs.  (Measured on MI355X: this launch
    // costs about 20 us more than a plain one, so the single-launch step is
    // slower than the two-launch step even on a 2^20-parameter shard.)
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kBlock), args, 0, stream);
}

hipError_t launch_fused_status(WorkspaceHeader* header, uint32_t* d_error, hipStream_t stream)
{
    fused_status_kernel<<<1, kWave, 0, stream>>>(header, d_error);
    return hipGetLastError();
}

// ------------------------------------------------ library-held workspace ---

// The workspace of adamw_clipped_step_noalloc, for callers that cannot
// allocate device memory: a file-scope device array, one copy on every GPU
// the library runs on, held until the process ends.  In host code its name
// only stands for the symbol; its device address on each GPU comes from
// hipGetSymbolAddress, called once per device with that device current, and
// only that address is ever passed to a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(int device, void** ptr)
{
    static std::mutex mutex;
    static void* address[kScratchMaxDevices] = {};
    if (device < 0 || device >= kScratchMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mutex);
    if (!address[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        address[device] = p;
    }
    *ptr = address[device];
    return hipSuccess;
}

}  // namespace mps
