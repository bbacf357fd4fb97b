// gfx950 kernels of the AdamW step with 8-bit moment state.
//
// m and v are stored as one byte per element: m as OCP FP8 E4M3 codes, v as
// OCP FP8 E5M2 codes, every run of 32 consecutive elements of a tensor with
// one power-of-two scale byte (value = code * 2^(byte - 127); 255 marks a
// run that held a NaN or an infinity and reads back as NaN).  A step decodes
// the moments, runs the same fp32 update as the fp32-state kernel, takes the
// new largest magnitude of each run, picks the smallest exponent that fits
// it under the format's largest code, and re-encodes with the hardware's
// round-to-nearest-even conversions.
//
//   adamw8_clipped_kernel / adamw8_step_kernel
//                       the update, in the clipped step (finishing the norm's
//                       partials first) or given the coefficient, as the
//                       fp32-state pair.  A thread takes four consecutive
//                       elements, so eight lanes hold one run of 32 and its
//                       largest magnitude is three DPP exchanges away, and
//                       every access of an instruction is contiguous across
//                       the wavefront.  Streams per element: master 4 B in and out,
//                       codes 1 + 1 B in and out, gradient 2 or 4 B in, bf16
//                       copy 2 B out, scales 2 B per 32 elements each way.
//   quantize_kernel /   conversion between fp32 moments and the 8-bit
//   dequantize_kernel   state (checkpoints, switching a run over).
//
// Tensors whose streams are not all aligned for the vector loads, and the
// last partial run of every tensor, go through an element-per-lane path in
// which 32 lanes hold one run and reduce it with lane shuffles.
#include <hip/hip_runtime.h>

#include "device.h"
#include "kernels.h"

// Cache policies of the 8-bit update's streams (aux operand: 0 default,
// 2 nontemporal).  A tile reads 32 scale bytes per moment, a fraction of a
// cache line that the next tile reads too: read nontemporally, each line
// came from memory again for every tile that touched it (1 % more bytes
// read than the algorithm needs, on the 70B share); cached, it comes once.
#ifndef MPS_Q8_W_POLICY
#define MPS_Q8_W_POLICY 2       // master and gradient loads
#endif
#ifndef MPS_Q8_CODE_POLICY
#define MPS_Q8_CODE_POLICY 2    // code loads
#endif
#ifndef MPS_Q8_SCALE_POLICY
#define MPS_Q8_SCALE_POLICY 0   // scale-byte loads (cached: consecutive tiles share a line)
#endif
#ifndef MPS_Q8_STORE_POLICY
#define MPS_Q8_STORE_POLICY 2   // every store
#endif

namespace mps {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kQ8WPolicy = MPS_Q8_W_POLICY;
constexpr int kQ8CodePolicy = MPS_Q8_CODE_POLICY;
constexpr int kQ8ScalePolicy = MPS_Q8_SCALE_POLICY;
constexpr int kQ8StorePolicy = MPS_Q8_STORE_POLICY;

// Largest finite code of each format is 1.75 * 2^k: 448 (E4M3), 57344 (E5M2).
constexpr int kE4M3TopExp = 8;
constexpr int kE5M2TopExp = 15;
constexpr uint32_t kNonFinite = 255;

// ------------------------------------------------------ scales and codes ---

// 2^(byte - 127); byte 0 is the subnormal 2^-127; 255 gives NaN.
__device__ __forceinline__ float scale_value(uint32_t byte)
{
    uint32_t bits = byte << 23;
    bits = byte == 0 ? 0x00400000u : bits;
    bits = byte == kNonFinite ? 0x7fc00000u : bits;
    return __uint_as_float(bits);
}

// The scale byte of a run whose largest magnitude has the bit pattern
// `absbits` (sign cleared): the smallest e >= -127 with
// absmax <= 1.75 * 2^(kTopExp + e), or 255 when the run is not finite.
template <int kTopExp>
__device__ __forceinline__ uint32_t scale_byte(uint32_t absbits)
{
    if (absbits >= 0x7f800000u) return kNonFinite;
    int e = static_cast<int>(absbits >> 23) - 127 - kTopExp + ((absbits & 0x7fffffu) > 0x600000u ? 1 : 0);
    e = e < -127 ? -127 : e;
    return static_cast<uint32_t>(e + 127);
}

// 2^-e for a finite scale byte (exact: e <= 120 for any finite fp32 run).
__device__ __forceinline__ float inverse_scale(uint32_t byte)
{
    return __uint_as_float((254u - byte) << 23);
}

__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7fffffffu; }

// The two codes in the low (kHigh false) or high half of `word`, widened.
template <bool kE4M3, bool kHigh>
__device__ __forceinline__ f32x2 decode_pair(uint32_t word)
{
    return kE4M3 ? __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(word), kHigh)
                 : __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(word), kHigh);
}

// Four codes (one word) to values times `scale`.
template <bool kE4M3>
__device__ __forceinline__ void decode4(uint32_t codes, float scale, float (&out)[4])
{
    const f32x2 lo = decode_pair<kE4M3, false>(codes);
    const f32x2 hi = decode_pair<kE4M3, true>(codes);
    out[0] = lo[0] * scale;
    out[1] = lo[1] * scale;
    out[2] = hi[0] * scale;
    out[3] = hi[1] * scale;
}

// Round a and b to codes (nearest, ties to even) into the low (kHigh false)
// or high half of `old`, keeping the other half.
template <bool kE4M3, bool kHigh>
__device__ __forceinline__ uint32_t encode_pair(float a, float b, uint32_t old)
{
    return static_cast<uint32_t>(kE4M3 ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, static_cast<int>(old), kHigh)
                                       : __builtin_amdgcn_cvt_pk_bf8_f32(a, b, static_cast<int>(old), kHigh));
}

// Four values to codes at the run's scale byte (all 0xFF for a non-finite
// run).
template <bool kE4M3>
__device__ __forceinline__ uint32_t encode4(const float (&x)[4], uint32_t byte)
{
    const float inv = inverse_scale(byte);
    uint32_t word = encode_pair<kE4M3, false>(x[0] * inv, x[1] * inv, 0u);
    word = encode_pair<kE4M3, true>(x[2] * inv, x[3] * inv, word);
    return byte == kNonFinite ? 0xffffffffu : word;
}

template <bool kE4M3>
__device__ __forceinline__ uint32_t encode1(float x, uint32_t byte)
{
    const uint32_t word = encode_pair<kE4M3, false>(x * inverse_scale(byte), 0.0f, 0u);
    return byte == kNonFinite ? 0xffu : (word & 0xffu);
}

template <bool kE4M3>
__device__ __forceinline__ float decode1(uint32_t code, float scale)
{
    return decode_pair<kE4M3, false>(code)[0] * scale;
}

// Largest over the eight lanes 8k .. 8k+7 (one run of 32 elements): two
// exchanges within each quad, then the half-row mirror (lane i with lane
// 7 - i of the eight), which meets the other quad.
__device__ __forceinline__ uint32_t run_max(uint32_t x)
{
    constexpr int kQuadSwap1 = 0xb1;   // quad_perm [1,0,3,2]
    constexpr int kQuadSwap2 = 0x4e;   // quad_perm [2,3,0,1]
    constexpr int kHalfMirror = 0x141; // row_half_mirror
    x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kQuadSwap1, 0xf, 0xf, false)));
    x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kQuadSwap2, 0xf, 0xf, false)));
    x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kHalfMirror, 0xf, 0xf, false)));
    return x;
}

// Largest over the 32 lanes of this half wavefront.  All lanes must be active.
__device__ __forceinline__ uint32_t half_wave_max(uint32_t x)
{
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) x = max(x, static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), off, kWave)));
    return x;
}

template <int kAux>
__device__ __forceinline__ uint32_t load_byte(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, kAux);
}

template <int kAux>
__device__ __forceinline__ u32x2 load_u32x2_policy(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kAux);
}

template <int kAux>
__device__ __forceinline__ uint32_t load_u32(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kAux);
}

__device__ __forceinline__ void store_byte(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(v), r, off, 0, kQ8StorePolicy);
}

__device__ __forceinline__ void store8_u32x2(u32x2 v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kQ8StorePolicy);
}

__device__ __forceinline__ void store8_u32x4(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kQ8StorePolicy);
}

__device__ __forceinline__ void store8_u32(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kQ8StorePolicy);
}

// ---------------------------------------------------------------- update ---

// Elements [begin, end) of one tensor, one element per lane; `begin` is a
// multiple of 32, so each half wavefront holds one run.  Every access goes
// through a buffer resource, like the vector body's (lanes past the end read
// zeros and their stores are dropped): flat accesses here would keep the
// compiler from counting the body's loads in issue order.
template <bool kBf16, class Entry>
__device__ __forceinline__ void adamw8_elements(const Entry* te, const QuantEntry* qe,
                                                int64_t begin, int64_t end, const StepScalars& s)
{
    for (int64_t base = begin; base < end; base += kBlock) {
        const uint32_t n = static_cast<uint32_t>(min(static_cast<int64_t>(kBlock), end - base));
        const int64_t r0 = base / kQuantBlock;
        const uint32_t runs = (n + kQuantBlock - 1) / kQuantBlock;
        const __amdgpu_buffer_rsrc_t W = rsrc(te->master + base, n * 4u);
        const __amdgpu_buffer_rsrc_t G = rsrc(static_cast<const char*>(te->grad) + base * (kBf16 ? 2 : 4),
                                              n * (kBf16 ? 2u : 4u));
        const __amdgpu_buffer_rsrc_t P = rsrc(te->param_bf16 ? te->param_bf16 + base : nullptr,
                                              te->param_bf16 ? n * 2u : 0u);
        const __amdgpu_buffer_rsrc_t MC = rsrc(qe->m_codes + base, n);
        const __amdgpu_buffer_rsrc_t VC = rsrc(qe->v_codes + base, n);
        const __amdgpu_buffer_rsrc_t MS = rsrc(qe->m_scales + r0, runs);
        const __amdgpu_buffer_rsrc_t VS = rsrc(qe->v_scales + r0, runs);
        const uint32_t o = threadIdx.x;
        const uint32_t run = o / kQuantBlock;
        const bool valid = o < n;
        float w = load_f32(W, o * 4u);
        const float g = kBf16 ? __uint_as_float(static_cast<uint32_t>(load_u16(G, o * 2u)) << 16)
                              : load_f32(G, o * 4u);
        float m = decode1<true>(load_byte<kQ8CodePolicy>(MC, o),
                                scale_value(load_byte<kQ8ScalePolicy>(MS, run)));
        float v = decode1<false>(load_byte<kQ8CodePolicy>(VC, o),
                                 scale_value(load_byte<kQ8ScalePolicy>(VS, run)));
        adamw_element(w, m, v, g, s);
        const uint32_t mb = scale_byte<kE4M3TopExp>(half_wave_max(valid ? abs_bits(m) : 0u));
        const uint32_t vb = scale_byte<kE5M2TopExp>(half_wave_max(valid ? abs_bits(v) : 0u));
        store_f32(w, W, o * 4u);
        store_byte(encode1<true>(m, mb), MC, o);
        store_byte(encode1<false>(v, vb), VC, o);
        store_u16(bf16_one(w), P, o * 2u);
        if (o % kQuantBlock == 0) {
            store_byte(mb, MS, run);
            store_byte(vb, VS, run);
        }
    }
}

// Scale bytes of one body are collected in LDS (a run's quad leader writes
// its byte) and stored after the body's last tile by consecutive threads, so
// each wavefront writes 64 contiguous bytes per moment instead of 16-byte
// pieces.  Two buffers alternate between consecutive bodies of a block: the
// barrier that ends one body also separates the readers of a buffer from the
// writers of the body after next.  A body is at most one chunk of an 8-bit
// list, whose chunks are at most kQ8ChunkMax elements (the host's plan).
constexpr int kMaxRunsPerBody = static_cast<int>(kQ8ChunkMax / kQuantBlock);
static_assert(kQ8ChunkMax % kQuantBlock == 0, "a chunk of an 8-bit list holds whole runs");

// The two pairs of scale-byte buffers (m, v) that consecutive bodies of a
// block alternate between, one LDS allocation however often this is inlined.
__device__ __forceinline__ uint8_t (*scale_lds())[2][kMaxRunsPerBody]
{
    __shared__ uint8_t buffers[2][2][kMaxRunsPerBody];
    return buffers;
}

// Whole runs [e0, e0 + 4 * ngroups) of one tensor (ngroups a multiple of 8,
// at most one chunk), every stream aligned for its vector width there.
// Thread q of a tile takes elements 4q .. 4q+3, so eight consecutive lanes
// hold one run of 32 and every load and store of a tile is contiguous across
// the wavefront.  Two tiles are held in registers in turn, as in the fp32
// kernel: the next tile's loads are in flight while this one is computed.
// Groups past the end read zeros and their stores are dropped; the eight
// lanes of a run are either all inside or all past the end.
template <bool kBf16>
struct Body8 {
    struct Tile {
        f32x4 w;
        u32x4 g;  // bf16: g[0..1] hold the four gradients; fp32: all four
        uint32_t mq, vq, ms, vs;
    };
    __amdgpu_buffer_rsrc_t W, G, P, MQ, VQ, MS, VS;
    bool copy;
    uint32_t ng;

    template <class Entry>
    __device__ __forceinline__ Body8(const Entry* te, const QuantEntry* qe, int64_t e0, int ngroups)
        : W(rsrc(te->master + e0, static_cast<uint32_t>(ngroups) * 16u)),
          G(rsrc(static_cast<const char*>(te->grad) + e0 * (kBf16 ? 2 : 4),
                 static_cast<uint32_t>(ngroups) * (kBf16 ? 8u : 16u))),
          P(rsrc(te->param_bf16 ? te->param_bf16 + e0 : nullptr,
                 te->param_bf16 ? static_cast<uint32_t>(ngroups) * 8u : 0u)),
          MQ(rsrc(qe->m_codes + e0, static_cast<uint32_t>(ngroups) * 4u)),
          VQ(rsrc(qe->v_codes + e0, static_cast<uint32_t>(ngroups) * 4u)),
          MS(rsrc(qe->m_scales + e0 / kQuantBlock, static_cast<uint32_t>(ngroups) / 8u)),
          VS(rsrc(qe->v_scales + e0 / kQuantBlock, static_cast<uint32_t>(ngroups) / 8u)),
          copy(te->param_bf16 != nullptr),
          ng(static_cast<uint32_t>(ngroups))
    {
    }

    __device__ __forceinline__ void load(Tile& t, int base) const
    {
        const uint32_t q = base + threadIdx.x;
        t.w = __builtin_bit_cast(f32x4, load_u32x4<kQ8WPolicy>(W, q * 16u));
        if (kBf16) {
            const u32x2 h = load_u32x2_policy<kQ8WPolicy>(G, q * 8u);
            t.g = u32x4{h[0], h[1], 0u, 0u};
        } else {
            t.g = load_u32x4<kQ8WPolicy>(G, q * 16u);
        }
        t.mq = load_u32<kQ8CodePolicy>(MQ, q * 4u);
        t.vq = load_u32<kQ8CodePolicy>(VQ, q * 4u);
        t.ms = load_byte<kQ8ScalePolicy>(MS, q / 8u);
        t.vs = load_byte<kQ8ScalePolicy>(VS, q / 8u);
    }

    // A run's quad leader leaves its two scale bytes in lds_m / lds_v.
    template <bool kCopy>
    __device__ __forceinline__ void update(Tile& t, int base, const StepScalars& s, uint8_t* lds_m,
                                           uint8_t* lds_v) const
    {
        const int tid = threadIdx.x;
        const uint32_t q = base + tid;
        float w[4], m[4], v[4], g[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = t.w[k];
        if (kBf16) {
            g[0] = bf16_lo(t.g[0]);
            g[1] = bf16_hi(t.g[0]);
            g[2] = bf16_lo(t.g[1]);
            g[3] = bf16_hi(t.g[1]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) g[k] = __uint_as_float(t.g[k]);
        }
        decode4<true>(t.mq, scale_value(t.ms), m);
        decode4<false>(t.vq, scale_value(t.vs), v);
        uint32_t am = 0, av = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            adamw_element(w[k], m[k], v[k], g[k], s);
            am = max(am, abs_bits(m[k]));
            av = max(av, abs_bits(v[k]));
        }
        const uint32_t mb = scale_byte<kE4M3TopExp>(run_max(am));
        const uint32_t vb = scale_byte<kE5M2TopExp>(run_max(av));
        store8_u32x4(u32x4{__float_as_uint(w[0]), __float_as_uint(w[1]), __float_as_uint(w[2]),
                           __float_as_uint(w[3])}, W, q * 16u);
        store8_u32(encode4<true>(m, mb), MQ, q * 4u);
        store8_u32(encode4<false>(v, vb), VQ, q * 4u);
        if (kCopy) store8_u32x2(u32x2{bf16_pack2(w[0], w[1]), bf16_pack2(w[2], w[3])}, P, q * 8u);
        if ((tid & 7) == 0 && q < ng) {
            lds_m[q / 8u] = static_cast<uint8_t>(mb);
            lds_v[q / 8u] = static_cast<uint8_t>(vb);
        }
    }

    // Streams the body (`a` already holds its first tile's loads), then
    // stores the scale bytes from lds_m / lds_v (kMaxRunsPerBody bytes
    // each) with consecutive threads.  The copy is decided once per body,
    // not per tile, for the compiler's waits (as in the fp32 body).
    __device__ __forceinline__ void run(Tile& a, const StepScalars& s, uint8_t* lds_m,
                                        uint8_t* lds_v) const
    {
        if (copy) {
            run_tiles<true>(a, s, lds_m, lds_v);
        } else {
            run_tiles<false>(a, s, lds_m, lds_v);
        }
        __syncthreads();
        for (uint32_t r = threadIdx.x; r < ng / 8u; r += kBlock) {
            store_byte(lds_m[r], MS, r);
            store_byte(lds_v[r], VS, r);
        }
    }

    template <bool kCopy>
    __device__ __forceinline__ void run_tiles(Tile& a, const StepScalars& s, uint8_t* lds_m,
                                              uint8_t* lds_v) const
    {
        const int ngroups = static_cast<int>(ng);
        Tile b;
        for (int base = 0; base < ngroups; base += 2 * kBlock) {
            load(b, base + kBlock);
            __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the math
            update<kCopy>(a, base, s, lds_m, lds_v);
            if (base + kBlock >= ngroups) break;  // uniform: the other tile is empty
            load(a, base + 2 * kBlock);
            __builtin_amdgcn_sched_barrier(0);
            update<kCopy>(b, base + kBlock, s, lds_m, lds_v);
        }
    }
};

// The element range of chunk c of a tensor and the end of its vector part:
// the whole runs of an aligned tensor take the vector body, the tensor's
// last partial run (and every element of an unaligned tensor) the element
// path.
struct Chunk8 {
    int64_t begin, vend, end;
};

template <class Entry>
__device__ __forceinline__ Chunk8 chunk8_span(const Entry* te, int c, int64_t chunk_elems)
{
    Chunk8 k;
    k.begin = static_cast<int64_t>(c - te->first_chunk) * chunk_elems;
    k.end = min(k.begin + chunk_elems, te->numel);
    const int64_t whole = te->numel - te->numel % kQuantBlock;
    k.vend = te->head < 0 ? k.begin : max(k.begin, min(k.end, whole));
    return k;
}

// Chunk c of one tensor in full.  `parity` picks this block's pair of scale
// buffers and flips after each body: the barrier that ends one body also
// separates the readers of a pair from the writers of the body after next.
template <bool kBf16, class Entry>
__device__ __forceinline__ void adamw8_chunk(const Entry* te, const QuantEntry* qe, int c,
                                             int64_t chunk_elems, const StepScalars& s,
                                             int& parity)
{
    const Chunk8 k = chunk8_span(te, c, chunk_elems);
    if (k.vend > k.begin) {
        const Body8<kBf16> body(te, qe, k.begin, static_cast<int>((k.vend - k.begin) / 4));
        typename Body8<kBf16>::Tile a;
        body.load(a, 0);
        body.run(a, s, scale_lds()[parity][0], scale_lds()[parity][1]);
        parity ^= 1;
    }
    if (k.end > k.vend) adamw8_elements<kBf16>(te, qe, k.vend, k.end, s);
}

// Chunks b, b + G, ... of this block, as in the fp32 kernel (the next
// chunk's table entries are fetched before this chunk streams).
template <bool kBf16>
__device__ __forceinline__ void update8_chunks(const TensorEntry* __restrict__ tensors,
                                               const QuantEntry* __restrict__ quant,
                                               const uint32_t* __restrict__ chunk_map,
                                               int n_tensors, int n_chunks, int64_t chunk_elems,
                                               const StepScalars& s)
{
    int parity = 0;
    TensorEntry next{};
    QuantEntry next_q{};
    if (static_cast<int>(blockIdx.x) < n_chunks) {
        const uint32_t k = table_index(constant_view(chunk_map)[blockIdx.x], n_tensors);
        next = read_entry(tensors, k);
        next_q = read_entry(quant, k);
    }
    for (int c = blockIdx.x; c < n_chunks; c += gridDim.x) {
        const TensorEntry te = uniform_entry(next);
        const QuantEntry qe = uniform_entry(next_q);
        if (c + static_cast<int>(gridDim.x) < n_chunks) {
            const uint32_t k = table_index(constant_view(chunk_map)[c + gridDim.x], n_tensors);
            next = read_entry(tensors, k);
            next_q = read_entry(quant, k);
        }
        adamw8_chunk<kBf16>(&te, &qe, c, chunk_elems, s, parity);
    }
}

// A block's walk over a one-tensor list whose entries came with the launch,
// as SoloWalk in the fp32 kernels: the constructor does the address
// arithmetic of the block's first chunk, load_first() issues the loads of
// its first tile, finish() streams that chunk and the block's later ones.
template <bool kBf16>
struct Solo8Walk {
    const SoloEntry* te;
    const QuantEntry* qe;
    int n_chunks;
    int64_t chunk_elems;
    Chunk8 k;
    bool whole, vector;
    Body8<kBf16> body;
    typename Body8<kBf16>::Tile a;

    __device__ __forceinline__ explicit Solo8Walk(const WorkspaceView& ws)
        : te(&ws.solo),
          qe(&ws.solo_quant),
          n_chunks(ws.n_chunks),
          chunk_elems(ws.chunk_elems),
          k(chunk8_span(&ws.solo, min(static_cast<int>(blockIdx.x), ws.n_chunks - 1),
                        ws.chunk_elems)),
          whole(static_cast<int>(blockIdx.x) < ws.n_chunks),
          vector(whole && k.vend > k.begin),
          // A block without a vector body loads nothing (an empty range).
          body(&ws.solo, &ws.solo_quant, k.begin,
               vector ? static_cast<int>((k.vend - k.begin) / 4) : 0)
    {
    }

    __device__ __forceinline__ void load_first() { body.load(a, 0); }

    __device__ __forceinline__ void finish(const StepScalars& s)
    {
        int parity = 0;
        if (vector) {
            body.run(a, s, scale_lds()[0][0], scale_lds()[0][1]);
            parity = 1;
            if (k.end > k.vend) adamw8_elements<kBf16>(te, qe, k.vend, k.end, s);
        } else if (whole) {
            adamw8_chunk<kBf16>(te, qe, static_cast<int>(blockIdx.x), chunk_elems, s, parity);
        }
        for (int c = blockIdx.x + gridDim.x; c < n_chunks; c += gridDim.x) {
            adamw8_chunk<kBf16>(te, qe, c, chunk_elems, s, parity);
        }
    }
};

template <bool kBf16>
__global__ __launch_bounds__(kBlock) void adamw8_step_kernel(
    WorkspaceView ws, const QuantEntry* __restrict__ quant, const float* d_coef,
    const double* d_skip_if_nonfinite, int32_t* d_step, HyperParams hp)
{
    if (ws.solo_tensor >= 0) {
        // As in the fp32 step kernel: the first tile's addresses from the
        // kernel arguments, then the scalar loads and the tile's loads
        // together; the tag is compared before anything is stored.
        Solo8Walk<kBf16> walk(ws);
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

    // Independent scalar loads, in flight together.
    const uint64_t seen = ws.header->tag;
    const int32_t count = *d_step;
    const float coef = *d_coef;
    const double skip_value = *d_skip_if_nonfinite;
    const int64_t t = static_cast<int64_t>(count) + 1;
    if (seen != ws.tag) return;  // tables overwritten: touch nothing
    if (!__builtin_isfinite(skip_value)) return;
    update8_chunks<kBf16>(ws.tensors, quant, ws.chunk_map, ws.n_tensors, ws.n_chunks, ws.chunk_elems,
                          step_scalars(t, hp, coef));
    advance_step(ws.tickets, d_step, t);
}

// The update with the end of the norm folded in, as the fp32 state's clipped
// kernel: every block sums the norm launch's partials in block order (the
// same bits as the norm's own second stage), forms the coefficient, and takes
// t from the header, where the norm launch left it; block 0 publishes S, the
// coefficient and the new count.  A list with one tensor brings that
// tensor's entries with the launch, and the loads of each block's first
// tile are issued before the tag and the partials are waited for, as in the
// fp32 kernel; nothing is stored before the tag has matched.
template <bool kBf16>
__global__ __launch_bounds__(kBlock) void adamw8_clipped_kernel(
    WorkspaceView ws, const QuantEntry* __restrict__ quant, int n_partials, double max_norm,
    double grad_scale, int skip_if_nonfinite, double* d_sumsq, float* d_coef, int32_t* d_step,
    HyperParams hp)
{
    // The header first: scalar loads, which the vector-memory counter does
    // not wait for.
    const uint64_t seen = ws.header->tag;
    const int32_t t = ws.header->pending_step;
    __shared__ double lds[kWavesPerBlock];

    if (ws.solo_tensor >= 0) {
        Solo8Walk<kBf16> walk(ws);
        // Loads in issue order: the partials, then the tile, so the sum of
        // the partials can start while the tile is still in flight.
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

    if (seen != ws.tag) {
        report_stale_clip(d_sumsq, d_coef);
        return;
    }
    const double total = sum_partials<false>(ws.partials, n_partials, lds);
    const float clip = clip_from_sumsq(total, max_norm, grad_scale);
    if (publish_clip(total, clip, t, skip_if_nonfinite, d_sumsq, d_coef, d_step)) return;
    update8_chunks<kBf16>(ws.tensors, quant, ws.chunk_map, ws.n_tensors, ws.n_chunks, ws.chunk_elems,
                          step_scalars(t, hp, clip));
}

// ------------------------------------------------------------ conversion ---

// One element per lane; each half wavefront holds one run of 32.
template <bool kE4M3>
__global__ __launch_bounds__(kBlock) void quantize_kernel(const float* x, int64_t n, uint8_t* codes,
                                                          uint8_t* scales)
{
    constexpr int kTop = kE4M3 ? kE4M3TopExp : kE5M2TopExp;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kBlock; base < n; base += stride) {
        const int64_t i = base + threadIdx.x;
        const bool valid = i < n;
        const float xi = valid ? x[i] : 0.0f;
        const uint32_t byte = scale_byte<kTop>(half_wave_max(abs_bits(xi)));
        if (valid) {
            codes[i] = static_cast<uint8_t>(encode1<kE4M3>(xi, byte));
            if (i % kQuantBlock == 0) scales[i / kQuantBlock] = static_cast<uint8_t>(byte);
        }
    }
}

template <bool kE4M3>
__global__ __launch_bounds__(kBlock) void dequantize_kernel(const uint8_t* codes, const uint8_t* scales,
                                                            int64_t n, float* x)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride) {
        x[i] = decode1<kE4M3>(codes[i], scale_value(scales[i / kQuantBlock]));
    }
}

}  // namespace

// --------------------------------------------------------------- launchers ---

hipError_t launch_adamw8_step(const WorkspaceView& ws, const QuantEntry* quant, bool grad_bf16,
                              int grid, const float* d_coef, const double* d_skip_if_nonfinite,
                              int32_t* d_step, const HyperParams& hp, hipStream_t stream)
{
    if (grad_bf16) {
        adamw8_step_kernel<true><<<grid, kBlock, 0, stream>>>(ws, quant, d_coef,
                                                              d_skip_if_nonfinite, d_step, hp);
    } else {
        adamw8_step_kernel<false><<<grid, kBlock, 0, stream>>>(ws, quant, d_coef,
                                                               d_skip_if_nonfinite, d_step, hp);
    }
    return hipGetLastError();
}

hipError_t launch_adamw8_clipped(const WorkspaceView& ws, const QuantEntry* quant, bool grad_bf16,
                                 int grid, int n_partials, double max_norm, double grad_scale,
                                 int skip_if_nonfinite, double* d_sumsq, float* d_coef,
                                 int32_t* d_step, const HyperParams& hp, hipStream_t stream)
{
    if (grad_bf16) {
        adamw8_clipped_kernel<true><<<grid, kBlock, 0, stream>>>(
            ws, quant, n_partials, max_norm, grad_scale, skip_if_nonfinite, d_sumsq, d_coef,
            d_step, hp);
    } else {
        adamw8_clipped_kernel<false><<<grid, kBlock, 0, stream>>>(
            ws, quant, n_partials, max_norm, grad_scale, skip_if_nonfinite, d_sumsq, d_coef,
            d_step, hp);
    }
    return hipGetLastError();
}

hipError_t launch_quantize(const float* x, int64_t n, bool e4m3, uint8_t* codes, uint8_t* scales,
                           hipStream_t stream)
{
    const int64_t blocks = (n + kBlock - 1) / kBlock;
    const int grid = static_cast<int>(blocks < 4096 ? blocks : 4096);
    if (e4m3) quantize_kernel<true><<<grid, kBlock, 0, stream>>>(x, n, codes, scales);
    else quantize_kernel<false><<<grid, kBlock, 0, stream>>>(x, n, codes, scales);
    return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t n, bool e4m3,
                             float* x, hipStream_t stream)
{
    const int64_t blocks = (n + kBlock - 1) / kBlock;
    const int grid = static_cast<int>(blocks < 4096 ? blocks : 4096);
    if (e4m3) dequantize_kernel<true><<<grid, kBlock, 0, stream>>>(codes, scales, n, x);
    else dequantize_kernel<false><<<grid, kBlock, 0, stream>>>(codes, scales, n, x);
    return hipGetLastError();
}

}  // namespace mps
