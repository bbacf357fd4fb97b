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

}  // namespace

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
