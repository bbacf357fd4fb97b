// The practical streaming ceiling that bench.py reports beside the AdamW
// update's roofline, measured in the same process on the same GPU: a plain
// kernel with exactly the update's streams (the same loads, stores and
// access widths: fp32 master, m and v read and written as 16-byte vectors,
// the gradient read as fp32 16-byte or bf16 8-byte vectors, the bf16 copy
// written as 8-byte vectors) and a few multiply-adds in place of the
// update's arithmetic.  Not part of the optimizer library: a measuring
// instrument for the benchmark.
//
// C ABI (loaded with ctypes by bench.py):
//   double stream_ceiling_us(int grad_bf16, float* w, float* m, float* v,
//                            const void* g, uint16_t* p, int64_t n, int grid,
//                            int unroll, int reps, void* stream)
// times `reps` launches (after two untimed ones) over n elements (n a
// multiple of 4; p may be NULL: no copy) with `grid` blocks of 256 threads
// and `unroll` groups of four elements per thread per tile (1, 2 or 4);
// returns the mean microseconds per launch, or a negative number if a HIP
// call failed or an argument is out of range.  Every access is a buffer
// access bounded to the tile, so lanes past the end read zeros and their
// stores are dropped.
//   double stream_ceiling8_us(int grad_bf16, float* w, const void* g,
//                             uint16_t* p, uint8_t* m_codes,
//                             uint8_t* m_scales, uint8_t* v_codes,
//                             uint8_t* v_scales, int64_t n, int grid,
//                             int reps, void* stream)
// the same for the 8-bit-moment update's streams: fp32 master read and
// written as 16-byte vectors, the gradient as in the fp32 kernel, m and v
// codes read and written as 4-byte words (four per thread), one scale byte
// per 32 elements read per thread (cached, as the update reads them) and
// written after each 16384-element chunk by consecutive threads from LDS,
// the bf16 copy written as 8-byte vectors.  n must be a multiple of 16384.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kNontemporal = 2;  // the update's policy for its streams

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                             0x00020000);
}

// Tiles of kUnroll * 256 groups of four elements; block b takes tiles b,
// b + G, ... (all blocks stream neighbouring addresses).
template <bool kBf16, bool kCopy, int kUnroll>
__global__ __launch_bounds__(kThreads) void same_streams(float* w, float* m, float* v,
                                                         const void* g, uint16_t* p, int64_t nq)
{
    const int64_t tile = static_cast<int64_t>(kThreads) * kUnroll;
    const int64_t ntiles = (nq + tile - 1) / tile;
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const int64_t q0 = t * tile;
        const uint32_t groups = static_cast<uint32_t>(nq - q0 < tile ? nq - q0 : tile);
        const auto W = rsrc(w + 4 * q0, groups * 16u);
        const auto M = rsrc(m + 4 * q0, groups * 16u);
        const auto V = rsrc(v + 4 * q0, groups * 16u);
        const auto G = rsrc(static_cast<const char*>(g) + q0 * (kBf16 ? 8 : 16),
                            groups * (kBf16 ? 8u : 16u));
        const auto P = rsrc(kCopy ? p + 4 * q0 : nullptr, kCopy ? groups * 8u : 0u);
        u32x4 a[kUnroll], b[kUnroll], c[kUnroll], d[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t o = u * kThreads + threadIdx.x;
            a[u] = __builtin_amdgcn_raw_buffer_load_b128(W, o * 16u, 0, kNontemporal);
            b[u] = __builtin_amdgcn_raw_buffer_load_b128(M, o * 16u, 0, kNontemporal);
            c[u] = __builtin_amdgcn_raw_buffer_load_b128(V, o * 16u, 0, kNontemporal);
            if (kBf16) {
                const u32x2 h = __builtin_amdgcn_raw_buffer_load_b64(G, o * 8u, 0, kNontemporal);
                d[u] = u32x4{h[0], h[1], 0u, 0u};
            } else {
                d[u] = __builtin_amdgcn_raw_buffer_load_b128(G, o * 16u, 0, kNontemporal);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t o = u * kThreads + threadIdx.x;
            const f32x4 gr = kBf16 ? f32x4{__uint_as_float(d[u][0] << 16),
                                           __uint_as_float(d[u][0] & 0xffff0000u),
                                           __uint_as_float(d[u][1] << 16),
                                           __uint_as_float(d[u][1] & 0xffff0000u)}
                                   : __builtin_bit_cast(f32x4, d[u]);
            const f32x4 mm = __builtin_bit_cast(f32x4, b[u]) * 0.9f + gr * 0.1f;
            const f32x4 vv = __builtin_bit_cast(f32x4, c[u]) * 0.95f + gr * gr * 0.05f;
            const f32x4 ww = __builtin_bit_cast(f32x4, a[u]) - mm * 0.001f;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ww), W, o * 16u, 0,
                                                   kNontemporal);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, mm), M, o * 16u, 0,
                                                   kNontemporal);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, vv), V, o * 16u, 0,
                                                   kNontemporal);
            if (kCopy) {
                const u32x2 packed{(__float_as_uint(ww[0]) >> 16) | (__float_as_uint(ww[1]) & 0xffff0000u),
                                   (__float_as_uint(ww[2]) >> 16) | (__float_as_uint(ww[3]) & 0xffff0000u)};
                __builtin_amdgcn_raw_buffer_store_b64(packed, P, o * 8u, 0, kNontemporal);
            }
        }
    }
}

template <bool kBf16, bool kCopy>
void launch(int unroll, int grid, float* w, float* m, float* v, const void* g, uint16_t* p,
            int64_t nq, hipStream_t s)
{
    if (unroll == 1) same_streams<kBf16, kCopy, 1><<<grid, kThreads, 0, s>>>(w, m, v, g, p, nq);
    if (unroll == 2) same_streams<kBf16, kCopy, 2><<<grid, kThreads, 0, s>>>(w, m, v, g, p, nq);
    if (unroll == 4) same_streams<kBf16, kCopy, 4><<<grid, kThreads, 0, s>>>(w, m, v, g, p, nq);
}

// The 8-bit update's streams, one 16384-element chunk per block at a time
// (block b takes chunks b, b + G, ...), one tile of 256 groups of four per
// step; the scale bytes of a chunk are gathered in LDS and stored at its end.
constexpr int kChunk8 = 16384;
constexpr int kRuns8 = kChunk8 / 32;
constexpr int kScalePolicy = 0;  // the update's scale loads are cached

template <bool kBf16, bool kCopy>
__global__ __launch_bounds__(kThreads) void same_streams8(float* w, const void* g, uint16_t* p,
                                                          uint8_t* mq, uint8_t* ms, uint8_t* vq,
                                                          uint8_t* vs, int64_t nchunks)
{
    __shared__ uint8_t lm[kRuns8], lv[kRuns8];
    const uint32_t tid = threadIdx.x;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t e0 = c * kChunk8;
        const auto W = rsrc(w + e0, kChunk8 * 4u);
        const auto G = rsrc(static_cast<const char*>(g) + e0 * (kBf16 ? 2 : 4), kChunk8 * (kBf16 ? 2u : 4u));
        const auto P = rsrc(kCopy ? p + e0 : nullptr, kCopy ? kChunk8 * 2u : 0u);
        const auto MQ = rsrc(mq + e0, kChunk8);
        const auto VQ = rsrc(vq + e0, kChunk8);
        const auto MS = rsrc(ms + e0 / 32, kRuns8);
        const auto VS = rsrc(vs + e0 / 32, kRuns8);
        for (uint32_t t = 0; t < kChunk8 / (4 * kThreads); ++t) {
            const uint32_t q = t * kThreads + tid;
            const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(W, q * 16u, 0, kNontemporal);
            u32x4 d;
            if (kBf16) {
                const u32x2 h = __builtin_amdgcn_raw_buffer_load_b64(G, q * 8u, 0, kNontemporal);
                d = u32x4{h[0], h[1], 0u, 0u};
            } else {
                d = __builtin_amdgcn_raw_buffer_load_b128(G, q * 16u, 0, kNontemporal);
            }
            const uint32_t mc = __builtin_amdgcn_raw_buffer_load_b32(MQ, q * 4u, 0, kNontemporal);
            const uint32_t vc = __builtin_amdgcn_raw_buffer_load_b32(VQ, q * 4u, 0, kNontemporal);
            const uint32_t mb = __builtin_amdgcn_raw_buffer_load_b8(MS, q / 8u, 0, kScalePolicy);
            const uint32_t vb = __builtin_amdgcn_raw_buffer_load_b8(VS, q / 8u, 0, kScalePolicy);
            const f32x4 gr = kBf16 ? f32x4{__uint_as_float(d[0] << 16), __uint_as_float(d[0] & 0xffff0000u),
                                           __uint_as_float(d[1] << 16), __uint_as_float(d[1] & 0xffff0000u)}
                                   : __builtin_bit_cast(f32x4, d);
            const f32x4 ww = __builtin_bit_cast(f32x4, a) * 0.999f - gr * 1e-6f;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ww), W, q * 16u, 0,
                                                   kNontemporal);
            __builtin_amdgcn_raw_buffer_store_b32(mc ^ 0x01010101u, MQ, q * 4u, 0, kNontemporal);
            __builtin_amdgcn_raw_buffer_store_b32(vc ^ 0x01010101u, VQ, q * 4u, 0, kNontemporal);
            if (kCopy) {
                const u32x2 packed{(__float_as_uint(ww[0]) >> 16) | (__float_as_uint(ww[1]) & 0xffff0000u),
                                   (__float_as_uint(ww[2]) >> 16) | (__float_as_uint(ww[3]) & 0xffff0000u)};
                __builtin_amdgcn_raw_buffer_store_b64(packed, P, q * 8u, 0, kNontemporal);
            }
            if ((tid & 7u) == 0u) {
                lm[q / 8u] = static_cast<uint8_t>(mb + 1u);
                lv[q / 8u] = static_cast<uint8_t>(vb + 1u);
            }
        }
        __syncthreads();
        for (uint32_t r = tid; r < kRuns8; r += kThreads) {
            __builtin_amdgcn_raw_buffer_store_b8(lm[r], MS, r, 0, kNontemporal);
            __builtin_amdgcn_raw_buffer_store_b8(lv[r], VS, r, 0, kNontemporal);
        }
        __syncthreads();  // the next chunk writes lm / lv again
    }
}

template <bool kBf16, bool kCopy>
void launch8(int grid, float* w, const void* g, uint16_t* p, uint8_t* mq, uint8_t* ms, uint8_t* vq,
             uint8_t* vs, int64_t nchunks, hipStream_t s)
{
    same_streams8<kBf16, kCopy><<<grid, kThreads, 0, s>>>(w, g, p, mq, ms, vq, vs, nchunks);
}

// Times `reps` calls of `once` between two events on `s`, after two
// untimed ones: mean microseconds per call, or a negative number on error.
template <class F>
double time_launches(F once, int reps, hipStream_t s)
{
    hipEvent_t start = nullptr, end = nullptr;
    if (hipEventCreate(&start) != hipSuccess) return -2.0;
    if (hipEventCreate(&end) != hipSuccess) {
        (void)hipEventDestroy(start);
        return -2.0;
    }
    once();
    once();
    float ms = -1.0f;
    bool good = hipGetLastError() == hipSuccess && hipEventRecord(start, s) == hipSuccess;
    for (int i = 0; good && i < reps; ++i) once();
    good = good && hipGetLastError() == hipSuccess && hipEventRecord(end, s) == hipSuccess &&
           hipEventSynchronize(end) == hipSuccess &&
           hipEventElapsedTime(&ms, start, end) == hipSuccess;
    (void)hipEventDestroy(start);
    (void)hipEventDestroy(end);
    return good ? ms * 1e3 / reps : -3.0;
}

}  // namespace

extern "C" double stream_ceiling8_us(int grad_bf16, float* w, const void* g, uint16_t* p,
                                     uint8_t* m_codes, uint8_t* m_scales, uint8_t* v_codes,
                                     uint8_t* v_scales, int64_t n, int grid, int reps, void* stream)
{
    if (!w || !g || !m_codes || !m_scales || !v_codes || !v_scales || n <= 0 || n % kChunk8 ||
        grid < 1 || grid > 65536 || reps < 1) {
        return -1.0;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t nchunks = n / kChunk8;
    auto once = [&] {
        if (grad_bf16 && p) launch8<true, true>(grid, w, g, p, m_codes, m_scales, v_codes, v_scales, nchunks, s);
        if (grad_bf16 && !p) launch8<true, false>(grid, w, g, p, m_codes, m_scales, v_codes, v_scales, nchunks, s);
        if (!grad_bf16 && p) launch8<false, true>(grid, w, g, p, m_codes, m_scales, v_codes, v_scales, nchunks, s);
        if (!grad_bf16 && !p) launch8<false, false>(grid, w, g, p, m_codes, m_scales, v_codes, v_scales, nchunks, s);
    };
    return time_launches(once, reps, s);
}

extern "C" double stream_ceiling_us(int grad_bf16, float* w, float* m, float* v, const void* g,
                                    uint16_t* p, int64_t n, int grid, int unroll, int reps,
                                    void* stream)
{
    if (!w || !m || !v || !g || n <= 0 || n % 4 || grid < 1 || grid > 65536 || reps < 1 ||
        (unroll != 1 && unroll != 2 && unroll != 4)) {
        return -1.0;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t nq = n / 4;
    auto once = [&] {
        if (grad_bf16 && p) launch<true, true>(unroll, grid, w, m, v, g, p, nq, s);
        if (grad_bf16 && !p) launch<true, false>(unroll, grid, w, m, v, g, p, nq, s);
        if (!grad_bf16 && p) launch<false, true>(unroll, grid, w, m, v, g, p, nq, s);
        if (!grad_bf16 && !p) launch<false, false>(unroll, grid, w, m, v, g, p, nq, s);
    };
    return time_launches(once, reps, s);
}
