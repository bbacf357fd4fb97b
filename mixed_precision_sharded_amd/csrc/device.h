// Device helpers shared by the gfx950 kernels of the AdamW step: buffer
// resources and vector loads/stores, bf16 rounding, fp64 wavefront and block
// reductions, the norm's second stage, the step counter, the clip
// multiplier, the step scalars and the per-element update.  Included by
// kernels.hip and kernels_q8.hip only.
//
// Build with -ffp-contract=off: every fp32 operation below must round once,
// in source order; division and sqrt are the correctly rounded defaults.
#pragma once

#include <hip/hip_runtime.h>

#include "layout.h"

#ifndef MPS_FUSED_STEP_UNROLL
#define MPS_FUSED_STEP_UNROLL 1   // the single-launch step: groups of four per thread per tile
#endif
#ifndef MPS_NORM_UNROLL
#define MPS_NORM_UNROLL 4   // 16-byte vectors per thread per tile (two tiles in flight)
#endif
// Buffer cache policies (the aux operand of buffer loads and stores):
// 0 = default, 2 = nontemporal.
#ifndef MPS_LOAD_POLICY
#define MPS_LOAD_POLICY 2   // update: master, m, v, gradient
#endif
#ifndef MPS_STORE_POLICY
#define MPS_STORE_POLICY 2  // update: master, m, v, bf16 copy
#endif


namespace mps {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kLoadPolicy = MPS_LOAD_POLICY;
constexpr int kStorePolicy = MPS_STORE_POLICY;
constexpr int kPolicyDefault = 0;  // the norm's gradient reads, cached blocks
constexpr int kPolicyStream = 2;   // the norm's gradient reads, the other blocks
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

// ------------------------------------------------------ buffer resources ---

// Table entries in scalar registers.  An entry read from the workspace with
// vector loads is the same in every lane, but the compiler cannot prove it:
// buffer resources built from it would then run every load and store in a
// loop over the lanes' distinct descriptors (one pass, but a branch and an
// exec-mask change around each access, and a full wait for memory where the
// next tile's loads should stay in flight).  readfirstlane states the fact.
__device__ __forceinline__ uint64_t uniform64(uint64_t x)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p)
{
    return reinterpret_cast<T*>(uniform64(reinterpret_cast<uintptr_t>(p)));
}

// A view of workspace tables for reading them with scalar loads: the tables
// do not change while a kernel runs, so the constant address space is
// correct for them, and its loads are counted apart from the vector memory
// operations (reading the next chunk's entry then does not wait for the
// stores of the chunk before).
template <class T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* constant_view(const T* p)
{
    return (const __attribute__((address_space(4))) T*)p;
}

// Entry i of a table, read field by field through the constant view.
__device__ __forceinline__ TensorEntry read_entry(const TensorEntry* table, uint32_t i)
{
    const __attribute__((address_space(4))) TensorEntry* e = constant_view(table) + i;
    TensorEntry r;
    r.master = e->master;
    r.exp_avg = e->exp_avg;
    r.exp_avg_sq = e->exp_avg_sq;
    r.grad = e->grad;
    r.param_bf16 = e->param_bf16;
    r.numel = e->numel;
    r.first_chunk = e->first_chunk;
    r.head = e->head;
    return r;
}

__device__ __forceinline__ QuantEntry read_entry(const QuantEntry* table, uint32_t i)
{
    const __attribute__((address_space(4))) QuantEntry* e = constant_view(table) + i;
    QuantEntry r;
    r.m_codes = e->m_codes;
    r.m_scales = e->m_scales;
    r.v_codes = e->v_codes;
    r.v_scales = e->v_scales;
    return r;
}

// A tensor index read from the chunk map, clamped into a table of n >= 1
// entries (one scalar min: a map in its uploaded state is never changed).
__device__ __forceinline__ uint32_t table_index(uint32_t raw, int n)
{
    return min(raw, static_cast<uint32_t>(n - 1));
}

__device__ __forceinline__ TensorEntry uniform_entry(const TensorEntry& e)
{
    TensorEntry u;
    u.master = uniform_ptr(e.master);
    u.exp_avg = uniform_ptr(e.exp_avg);
    u.exp_avg_sq = uniform_ptr(e.exp_avg_sq);
    u.grad = uniform_ptr(e.grad);
    u.param_bf16 = uniform_ptr(e.param_bf16);
    u.numel = static_cast<int64_t>(uniform64(static_cast<uint64_t>(e.numel)));
    u.first_chunk = __builtin_amdgcn_readfirstlane(e.first_chunk);
    u.head = __builtin_amdgcn_readfirstlane(e.head);
    return u;
}

__device__ __forceinline__ QuantEntry uniform_entry(const QuantEntry& e)
{
    QuantEntry u;
    u.m_codes = uniform_ptr(e.m_codes);
    u.m_scales = uniform_ptr(e.m_scales);
    u.v_codes = uniform_ptr(e.v_codes);
    u.v_scales = uniform_ptr(e.v_scales);
    return u;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                             kRsrcWord3);
}

__device__ __forceinline__ f32x4 load_f32x4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kLoadPolicy));
}

template <int kAux>
__device__ __forceinline__ u32x4 load_u32x4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAux);
}

__device__ __forceinline__ u32x2 load_u32x2(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kLoadPolicy);
}

__device__ __forceinline__ void store_f32x4(f32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kStorePolicy);
}

__device__ __forceinline__ void store_u32x2(u32x2 v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kStorePolicy);
}

__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kLoadPolicy));
}

__device__ __forceinline__ uint16_t load_u16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kLoadPolicy);
}

__device__ __forceinline__ void store_f32(float v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, kStorePolicy);
}

__device__ __forceinline__ void store_u16(uint16_t v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, kStorePolicy);
}

// ----------------------------------------------------------------- bf16 ---

__device__ __forceinline__ float bf16_lo(uint32_t word) { return __uint_as_float(word << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t word) { return __uint_as_float(word & 0xffff0000u); }

// bf16 copies use the chip's conversion (v_cvt_pk_bf16_f32 on gfx950): round
// to nearest, ties to even, two values per instruction.  A NaN stays a NaN.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// a in the low half, b in the high half.
__device__ __forceinline__ uint32_t bf16_pack2(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2));
}

__device__ __forceinline__ uint16_t bf16_one(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// ------------------------------------------------------ reductions (fp64) ---

template <int kCtrl>
__device__ __forceinline__ double dpp_move(double x)
{
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(x), kCtrl, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(x), kCtrl, 0xf, 0xf, false);
    return __hiloint2double(hi, lo);
}

// Sum over the 64 lanes of a wavefront; every lane ends with the total.
// Within each row of 16 lanes the exchange uses DPP (quad permutes, then the
// half-row and row mirrors); the two cross-row steps use lane shuffles.
// All lanes must be active.
__device__ __forceinline__ double wave_sum(double x)
{
    constexpr int kQuadSwap1 = 0xb1;   // quad_perm [1,0,3,2]
    constexpr int kQuadSwap2 = 0x4e;   // quad_perm [2,3,0,1]
    constexpr int kHalfMirror = 0x141; // row_half_mirror
    constexpr int kRowMirror = 0x140;  // row_mirror
    x = x + dpp_move<kQuadSwap1>(x);
    x = x + dpp_move<kQuadSwap2>(x);
    x = x + dpp_move<kHalfMirror>(x);
    x = x + dpp_move<kRowMirror>(x);
    x = x + __shfl_xor(x, 16, kWave);
    x = x + __shfl_xor(x, 32, kWave);
    return x;
}

// Sum over the block in a fixed order, returned to every thread (each
// computes the same bits).  `lds` holds one double per wavefront.  Ends with
// a barrier so that `lds` may be reused right away.
__device__ __forceinline__ double block_sum(double x, double* lds)
{
    x = wave_sum(x);
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    if (lane == 0) lds[wave] = x;
    __syncthreads();
    double r = 0.0;
    for (int w = 0; w < kWavesPerBlock; ++w) r = r + lds[w];
    __syncthreads();
    return r;
}

__device__ __forceinline__ double add_square(double acc, float x)
{
    const double d = static_cast<double>(x);
    return __builtin_fma(d, d, acc);  // d*d is exact in fp64: one rounding
}

// The multiplier the update applies to the stored gradient g, whose value
// for the step is s*g (s: 1/K accumulation, 1/world averaging, 1/loss scale):
//     s * min(1, max_norm / (s * sqrt(S) + 1e-6))
// in fp64, rounded once to fp32.  With s = 1 it is the plain clip
// coefficient.  A NaN S gives NaN (the comparison is false), an infinite S
// gives 0.
__device__ __forceinline__ float clip_from_sumsq(double sumsq, double max_norm, double grad_scale)
{
    const double norm = grad_scale * __builtin_sqrt(sumsq);
    double clip = max_norm / (norm + 1e-6);
    clip = (clip > 1.0) ? 1.0 : clip;
    return static_cast<float>(grad_scale * clip);
}

// The two partial slots of this thread, tid and tid + kBlock of the
// workspace's kPartials, loaded without a condition (no loop, no branch: a
// kernel can issue these loads early and wait for them alone).  kAtomic:
// the partials were written by other blocks of this launch (agent-scope
// loads after an acquire fence); otherwise by an earlier launch.
static_assert(kPartials <= 2 * kBlock, "at most two partials per thread");
struct PartialSlots {
    double first, second;
};

template <bool kAtomic>
__device__ __forceinline__ PartialSlots load_partials(const double* partials)
{
    const int i = threadIdx.x;
    if (kAtomic) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        return {__hip_atomic_load(&partials[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                __hip_atomic_load(&partials[i + kBlock], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)};
    }
    // Buffer loads (default cache policy), the same kind as the update's
    // streams: the compiler counts loads of one kind in issue order, so a
    // wait for these leaves later stream loads in flight.
    const __amdgpu_buffer_rsrc_t r = rsrc(partials, sizeof(double) * kPartials);
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, i * 8u, 0, 0);
    const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(r, (i + kBlock) * 8u, 0, 0);
    return {__builtin_bit_cast(double, a), __builtin_bit_cast(double, b)};
}

// This thread's strided share of the first n partials: 0 + the slots below
// n.  A slot at or past n is added as +0, which leaves the sum's bits as they
// are (the share is never -0).
__device__ __forceinline__ double partial_share(const PartialSlots& p, int n)
{
    const int i = threadIdx.x;
    double q = 0.0;
    q = q + (i < n ? p.first : 0.0);
    q = q + (i + kBlock < n ? p.second : 0.0);
    return q;
}

// S from the n per-block partials, in block-index order: each thread sums
// its strided share, then the block combines the threads in a fixed tree.
// Every thread returns the same bits, and so does every block that calls
// this on the same partials.
template <bool kAtomic>
__device__ __forceinline__ double sum_partials(const double* partials, int n, double* lds)
{
    return block_sum(partial_share(load_partials<kAtomic>(partials), n), lds);
}

// A clipped update that finds the workspace tables overwritten writes a NaN
// S and coefficient (block 0) and nothing else.
__device__ __forceinline__ void report_stale_clip(double* d_sumsq, float* d_coef)
{
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (d_sumsq) *d_sumsq = __builtin_nan("");
        if (d_coef) *d_coef = __builtin_nanf("");
    }
}

// Block 0 of a clipped update publishes S, the coefficient and, unless the
// step is skipped (S not finite and skipping asked for), the new count t.
// Returns whether the step is skipped (the same in every block).
__device__ __forceinline__ bool publish_clip(double total, float clip, int32_t t,
                                             int skip_if_nonfinite, double* d_sumsq,
                                             float* d_coef, int32_t* d_step)
{
    const bool skip = skip_if_nonfinite && !__builtin_isfinite(total);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (d_sumsq) *d_sumsq = total;
        if (d_coef) *d_coef = clip;
        if (!skip) *d_step = t;
    }
    return skip;
}

// One ticket per block (called by one thread of each block of a launch);
// true in the block that takes the last one.  Two levels, each counter on
// its own 128-byte line: block b counts in group b mod 8, and the last block
// of each group then counts at the top.  With a single counter, a small
// shard's blocks all reach it at about the same moment and their atomics
// queue (measured on 2^20 parameters: the update took 12.5 us with one
// counter, 9.7 us with the tree).  Every counter wraps back to zero once per
// complete launch, so launches that follow each other on a stream share the
// tree.  What a block wrote before its ticket (and waited for) is visible to
// the block that takes the last one: every ticket of a group precedes the
// group's top ticket.
__device__ __forceinline__ bool last_ticket(uint32_t* tickets)
{
    const uint32_t grid = gridDim.x, b = blockIdx.x;
    const uint32_t groups = grid < kTicketGroups ? grid : kTicketGroups;
    const uint32_t g = b % groups;
    const uint32_t members = grid / groups + (g < grid % groups ? 1u : 0u);
    return atomicInc(&tickets[kTicketStride * g], members - 1) == members - 1 &&
           atomicInc(&tickets[kTicketStride * kTicketGroups], groups - 1) == groups - 1;
}

// The step counter.  Every wave reads the completed-step count in its
// prologue; at its end each block takes a ticket, and the block that takes
// the last one stores the new count.  The only order this needs is that
// every read comes before that store: the barrier puts all of a block's waves
// (each past its read) before its ticket, and the last block stores only
// after seeing every other ticket.  No block reads data that another block of
// the launch wrote, so there is no release fence (on this chip an agent-scope
// release writes back the whole L2, which cost ~20 us per launch on a
// 62.7M-parameter shard).  Taking the tickets at the start of the block
// instead was measured slower: the atomics then queue before any data moves.
__device__ __forceinline__ void advance_step(uint32_t* tickets, int32_t* d_step, int64_t t)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);  // the compiler keeps the ticket last
        if (last_ticket(tickets)) *d_step = static_cast<int32_t>(t);
    }
}

// ------------------------------------------------------------ gradients ---

template <bool kBf16>
__device__ __forceinline__ float grad_at(const void* p, int64_t i)
{
    if (kBf16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
    return static_cast<const float*>(p)[i];
}

// ---------------------------------------------------------------- update ---

struct StepScalars {
    float beta1, beta2, one_m_b1, one_m_b2, decay, step_size, bc2_sqrt, eps, clip;
};

// beta^t, squaring the base and multiplying in the set bits from the lowest.
__device__ __forceinline__ double power_by_squaring(double beta, int64_t t)
{
    double result = 1.0;
    double base = beta;
    for (; t > 0; t >>= 1) {
        if (t & 1) result = result * base;
        base = base * base;
    }
    return result;
}

__device__ __forceinline__ StepScalars step_scalars(int64_t t, const HyperParams& hp, float clip)
{
    StepScalars s;
    const double p1 = power_by_squaring(hp.beta1, t);
    const double p2 = power_by_squaring(hp.beta2, t);
    s.beta1 = static_cast<float>(hp.beta1);
    s.beta2 = static_cast<float>(hp.beta2);
    s.one_m_b1 = static_cast<float>(1.0 - hp.beta1);
    s.one_m_b2 = static_cast<float>(1.0 - hp.beta2);
    s.decay = static_cast<float>(1.0 - hp.lr * hp.weight_decay);
    s.step_size = static_cast<float>(hp.lr / (1.0 - p1));
    s.bc2_sqrt = static_cast<float>(__builtin_sqrt(1.0 - p2));
    s.eps = static_cast<float>(hp.eps);
    s.clip = clip;
    return s;
}

// One element; each statement is a single correctly rounded fp32 operation.
__device__ __forceinline__ void adamw_element(float& w, float& m, float& v, float grad,
                                              const StepScalars& s)
{
    const float g = grad * s.clip;
    const float m_keep = s.beta1 * m;
    const float m_add = s.one_m_b1 * g;
    m = m_keep + m_add;
    const float v_keep = s.beta2 * v;
    const float g_sq = g * g;
    const float v_add = s.one_m_b2 * g_sq;
    v = v_keep + v_add;
    const float root = __builtin_sqrtf(v);
    const float root_hat = root / s.bc2_sqrt;
    const float den = root_hat + s.eps;
    const float w_decayed = w * s.decay;
    const float ratio = m / den;
    const float delta = s.step_size * ratio;
    w = w_decayed - delta;
}

}  // namespace
}  // namespace mps
