// Practical HBM ceilings for the roofline of the AdamW step: plain streaming
// kernels with the same access patterns and trivial arithmetic — read only,
// copy, and 4 reads / 3 writes (master, m, v, gradient in; master, m, v out).
// Usage: stream_ceiling [floats per buffer]   (default 62,736,416: one
// 8B-parameter model's FSDP shard at 128-way).  Prints GB/s per variant.
// Every kernel is a grid-stride loop with i < n guards; buffers hold n f32x4.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <vector>
#include <string>

typedef float f4 __attribute__((ext_vector_type(4)));

#define CHECK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e), __LINE__); exit(1);} } while (0)

template <int U, bool NT>
__global__ __launch_bounds__(256) void read_kernel(const f4* __restrict__ a, long n, float* out) {
  float acc = 0.f;
  long stride = (long)gridDim.x * 256 * U;
  for (long base = (long)blockIdx.x * 256 * U + threadIdx.x; base < n; base += stride) {
    f4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) { long i = base + u * 256; x[u] = i < n ? (NT ? __builtin_nontemporal_load(&a[i]) : a[i]) : f4(0); }
#pragma unroll
    for (int u = 0; u < U; ++u) acc += x[u][0] + x[u][1] + x[u][2] + x[u][3];
  }
  if (acc == 123.456f) out[0] = acc;
}

template <int U, bool NT>
__global__ __launch_bounds__(256) void copy_kernel(const f4* __restrict__ a, f4* __restrict__ b, long n) {
  long stride = (long)gridDim.x * 256 * U;
  for (long base = (long)blockIdx.x * 256 * U + threadIdx.x; base < n; base += stride) {
    f4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) { long i = base + u * 256; if (i < n) x[u] = NT ? __builtin_nontemporal_load(&a[i]) : a[i]; }
#pragma unroll
    for (int u = 0; u < U; ++u) { long i = base + u * 256; if (i < n) { if (NT) __builtin_nontemporal_store(x[u], &b[i]); else b[i] = x[u]; } }
  }
}

// 4 reads (w, m, v, g), 3 writes (w, m, v).
template <int U, bool NT>
__global__ __launch_bounds__(256) void adam_like(f4* __restrict__ w, f4* __restrict__ m, f4* __restrict__ v, const f4* __restrict__ g, long n) {
  long stride = (long)gridDim.x * 256 * U;
  for (long base = (long)blockIdx.x * 256 * U + threadIdx.x; base < n; base += stride) {
    f4 W[U], M[U], V[U], G[U];
#pragma unroll
    for (int u = 0; u < U; ++u) { long i = base + u * 256; if (i < n) {
      W[u] = NT ? __builtin_nontemporal_load(&w[i]) : w[i];
      M[u] = NT ? __builtin_nontemporal_load(&m[i]) : m[i];
      V[u] = NT ? __builtin_nontemporal_load(&v[i]) : v[i];
      G[u] = NT ? __builtin_nontemporal_load(&g[i]) : g[i]; } }
#pragma unroll
    for (int u = 0; u < U; ++u) { long i = base + u * 256; if (i < n) {
      f4 mm = M[u] * 0.9f + G[u] * 0.1f; f4 vv = V[u] * 0.95f + G[u] * G[u] * 0.05f; f4 ww = W[u] - mm * 0.001f;
      if (NT) { __builtin_nontemporal_store(ww, &w[i]); __builtin_nontemporal_store(mm, &m[i]); __builtin_nontemporal_store(vv, &v[i]); }
      else { w[i] = ww; m[i] = mm; v[i] = vv; } } }
  }
}

// The same bytes with w, m and v interleaved per group of four (48 B per
// thread, three 16 B loads and stores of one contiguous piece): one
// read-write state stream and the gradient stream instead of four streams.
template <bool NT>
__global__ __launch_bounds__(256) void adam_aos(f4* __restrict__ s, const f4* __restrict__ g, long n) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    f4 W = NT ? __builtin_nontemporal_load(&s[3 * i]) : s[3 * i];
    f4 M = NT ? __builtin_nontemporal_load(&s[3 * i + 1]) : s[3 * i + 1];
    f4 V = NT ? __builtin_nontemporal_load(&s[3 * i + 2]) : s[3 * i + 2];
    f4 G = NT ? __builtin_nontemporal_load(&g[i]) : g[i];
    f4 mm = M * 0.9f + G * 0.1f; f4 vv = V * 0.95f + G * G * 0.05f; f4 ww = W - mm * 0.001f;
    if (NT) { __builtin_nontemporal_store(ww, &s[3 * i]); __builtin_nontemporal_store(mm, &s[3 * i + 1]); __builtin_nontemporal_store(vv, &s[3 * i + 2]); }
    else { s[3 * i] = ww; s[3 * i + 1] = mm; s[3 * i + 2] = vv; }
  }
}

typedef unsigned int u2 __attribute__((ext_vector_type(2)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

// The bf16-gradient update's streams, four elements per lane: fp32 w, m, v
// (16 B loads and stores), bf16 g in (8 B), bf16 copy out (8 B).
template <bool NT>
__global__ __launch_bounds__(256) void adam_bf16_quads(f4* __restrict__ w, f4* __restrict__ m, f4* __restrict__ v,
                                                       const u2* __restrict__ g, u2* __restrict__ p, long n) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    f4 W = NT ? __builtin_nontemporal_load(&w[i]) : w[i];
    f4 M = NT ? __builtin_nontemporal_load(&m[i]) : m[i];
    f4 V = NT ? __builtin_nontemporal_load(&v[i]) : v[i];
    u2 G = NT ? __builtin_nontemporal_load(&g[i]) : g[i];
    f4 gf = f4{__uint_as_float(G[0] << 16), __uint_as_float(G[0] & 0xffff0000u), __uint_as_float(G[1] << 16), __uint_as_float(G[1] & 0xffff0000u)};
    f4 mm = M * 0.9f + gf * 0.1f; f4 vv = V * 0.95f + gf * gf * 0.05f; f4 ww = W - mm * 0.001f;
    u2 P = u2{(__float_as_uint(ww[0]) >> 16) | (__float_as_uint(ww[1]) & 0xffff0000u), (__float_as_uint(ww[2]) >> 16) | (__float_as_uint(ww[3]) & 0xffff0000u)};
    if (NT) { __builtin_nontemporal_store(ww, &w[i]); __builtin_nontemporal_store(mm, &m[i]); __builtin_nontemporal_store(vv, &v[i]); __builtin_nontemporal_store(P, &p[i]); }
    else { w[i] = ww; m[i] = mm; v[i] = vv; p[i] = P; }
  }
}

// bf16_quads with the library's work split: block b walks chunks b, b + G,
// ... of `kChunk` groups of four, each chunk streamed front to back.
template <int kChunk>
__global__ __launch_bounds__(256) void adam_bf16_quads_chunked(f4* __restrict__ w, f4* __restrict__ m, f4* __restrict__ v,
                                                               const u2* __restrict__ g, u2* __restrict__ p, long n) {
  const long n_chunks = (n + kChunk - 1) / kChunk;
  for (long c = blockIdx.x; c < n_chunks; c += gridDim.x) {
    const long end = c * kChunk + kChunk < n ? c * kChunk + kChunk : n;
    for (long i = c * kChunk + threadIdx.x; i < end; i += 256) {
      f4 W = __builtin_nontemporal_load(&w[i]), M = __builtin_nontemporal_load(&m[i]), V = __builtin_nontemporal_load(&v[i]);
      u2 G = __builtin_nontemporal_load(&g[i]);
      f4 gf = f4{__uint_as_float(G[0] << 16), __uint_as_float(G[0] & 0xffff0000u), __uint_as_float(G[1] << 16), __uint_as_float(G[1] & 0xffff0000u)};
      f4 mm = M * 0.9f + gf * 0.1f; f4 vv = V * 0.95f + gf * gf * 0.05f; f4 ww = W - mm * 0.001f;
      u2 P = u2{(__float_as_uint(ww[0]) >> 16) | (__float_as_uint(ww[1]) & 0xffff0000u), (__float_as_uint(ww[2]) >> 16) | (__float_as_uint(ww[3]) & 0xffff0000u)};
      __builtin_nontemporal_store(ww, &w[i]); __builtin_nontemporal_store(mm, &m[i]); __builtin_nontemporal_store(vv, &v[i]); __builtin_nontemporal_store(P, &p[i]);
    }
  }
}

// Same streams, eight elements per lane: bf16 g and copy as 16 B accesses,
// fp32 w, m, v as two 16 B accesses each (lanes 32 B apart).
template <bool NT>
__global__ __launch_bounds__(256) void adam_bf16_octets(f4* __restrict__ w, f4* __restrict__ m, f4* __restrict__ v,
                                                        const u4* __restrict__ g, u4* __restrict__ p, long n8) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256) {
    f4 W0 = NT ? __builtin_nontemporal_load(&w[2 * i]) : w[2 * i], W1 = NT ? __builtin_nontemporal_load(&w[2 * i + 1]) : w[2 * i + 1];
    f4 M0 = NT ? __builtin_nontemporal_load(&m[2 * i]) : m[2 * i], M1 = NT ? __builtin_nontemporal_load(&m[2 * i + 1]) : m[2 * i + 1];
    f4 V0 = NT ? __builtin_nontemporal_load(&v[2 * i]) : v[2 * i], V1 = NT ? __builtin_nontemporal_load(&v[2 * i + 1]) : v[2 * i + 1];
    u4 G = NT ? __builtin_nontemporal_load(&g[i]) : g[i];
    f4 g0 = f4{__uint_as_float(G[0] << 16), __uint_as_float(G[0] & 0xffff0000u), __uint_as_float(G[1] << 16), __uint_as_float(G[1] & 0xffff0000u)};
    f4 g1 = f4{__uint_as_float(G[2] << 16), __uint_as_float(G[2] & 0xffff0000u), __uint_as_float(G[3] << 16), __uint_as_float(G[3] & 0xffff0000u)};
    f4 m0 = M0 * 0.9f + g0 * 0.1f, m1 = M1 * 0.9f + g1 * 0.1f;
    f4 v0 = V0 * 0.95f + g0 * g0 * 0.05f, v1 = V1 * 0.95f + g1 * g1 * 0.05f;
    f4 w0 = W0 - m0 * 0.001f, w1 = W1 - m1 * 0.001f;
    u4 P = u4{(__float_as_uint(w0[0]) >> 16) | (__float_as_uint(w0[1]) & 0xffff0000u), (__float_as_uint(w0[2]) >> 16) | (__float_as_uint(w0[3]) & 0xffff0000u),
              (__float_as_uint(w1[0]) >> 16) | (__float_as_uint(w1[1]) & 0xffff0000u), (__float_as_uint(w1[2]) >> 16) | (__float_as_uint(w1[3]) & 0xffff0000u)};
    if (NT) {
      __builtin_nontemporal_store(w0, &w[2 * i]); __builtin_nontemporal_store(w1, &w[2 * i + 1]);
      __builtin_nontemporal_store(m0, &m[2 * i]); __builtin_nontemporal_store(m1, &m[2 * i + 1]);
      __builtin_nontemporal_store(v0, &v[2 * i]); __builtin_nontemporal_store(v1, &v[2 * i + 1]);
      __builtin_nontemporal_store(P, &p[i]);
    } else {
      w[2 * i] = w0; w[2 * i + 1] = w1; m[2 * i] = m0; m[2 * i + 1] = m1; v[2 * i] = v0; v[2 * i + 1] = v1; p[i] = P;
    }
  }
}

// The 8-bit-moment update's streams, eight elements per lane: fp32 w in and
// out (two 16 B accesses), bf16 g in (16 B), bf16 copy out (16 B), m and v
// codes in and out (8 B each), one scale byte per 32 elements for each
// moment in (every lane) and out (one lane in four).  16.125 B per element.
template <bool NT>
__global__ __launch_bounds__(256) void adam_q8_octets(f4* __restrict__ w, const u4* __restrict__ g, u4* __restrict__ p,
                                                      u2* __restrict__ mq, u2* __restrict__ vq,
                                                      unsigned char* __restrict__ ms, unsigned char* __restrict__ vs, long n8) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256) {
    f4 W0 = NT ? __builtin_nontemporal_load(&w[2 * i]) : w[2 * i], W1 = NT ? __builtin_nontemporal_load(&w[2 * i + 1]) : w[2 * i + 1];
    u4 G = NT ? __builtin_nontemporal_load(&g[i]) : g[i];
    u2 M = NT ? __builtin_nontemporal_load(&mq[i]) : mq[i];
    u2 V = NT ? __builtin_nontemporal_load(&vq[i]) : vq[i];
    unsigned sm = ms[i / 4], sv = vs[i / 4];
    f4 g0 = f4{__uint_as_float(G[0] << 16), __uint_as_float(G[0] & 0xffff0000u), __uint_as_float(G[1] << 16), __uint_as_float(G[1] & 0xffff0000u)};
    f4 g1 = f4{__uint_as_float(G[2] << 16), __uint_as_float(G[2] & 0xffff0000u), __uint_as_float(G[3] << 16), __uint_as_float(G[3] & 0xffff0000u)};
    f4 w0 = W0 - g0 * 0.001f, w1 = W1 - g1 * 0.001f;
    u2 M2 = M ^ (u2)(sm * 0x01010101u), V2 = V ^ (u2)(sv * 0x01010101u);
    u4 P = u4{(__float_as_uint(w0[0]) >> 16) | (__float_as_uint(w0[1]) & 0xffff0000u), (__float_as_uint(w0[2]) >> 16) | (__float_as_uint(w0[3]) & 0xffff0000u),
              (__float_as_uint(w1[0]) >> 16) | (__float_as_uint(w1[1]) & 0xffff0000u), (__float_as_uint(w1[2]) >> 16) | (__float_as_uint(w1[3]) & 0xffff0000u)};
    if (NT) {
      __builtin_nontemporal_store(w0, &w[2 * i]); __builtin_nontemporal_store(w1, &w[2 * i + 1]);
      __builtin_nontemporal_store(M2, &mq[i]); __builtin_nontemporal_store(V2, &vq[i]); __builtin_nontemporal_store(P, &p[i]);
    } else {
      w[2 * i] = w0; w[2 * i + 1] = w1; mq[i] = M2; vq[i] = V2; p[i] = P;
    }
    if ((threadIdx.x & 3) == 0) { ms[i / 4] = (unsigned char)(sm + 1); vs[i / 4] = (unsigned char)(sv + 1); }
  }
}

// The 8-bit-moment streams with four elements per lane: fp32 w in and out
// (16 B), bf16 g in and bf16 copy out (8 B), m and v codes (4 B each), a
// scale byte per 32 elements (eight lanes) per moment.  Every access of one
// instruction is contiguous across the wavefront.
template <bool NT>
__global__ __launch_bounds__(256) void adam_q8_quads(f4* __restrict__ w, const u2* __restrict__ g, u2* __restrict__ p,
                                                     unsigned* __restrict__ mq, unsigned* __restrict__ vq,
                                                     unsigned char* __restrict__ ms, unsigned char* __restrict__ vs, long n4) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long)gridDim.x * 256) {
    f4 W = NT ? __builtin_nontemporal_load(&w[i]) : w[i];
    u2 G = NT ? __builtin_nontemporal_load(&g[i]) : g[i];
    unsigned M = NT ? __builtin_nontemporal_load(&mq[i]) : mq[i];
    unsigned V = NT ? __builtin_nontemporal_load(&vq[i]) : vq[i];
    unsigned sm = ms[i / 8], sv = vs[i / 8];
    f4 gf = f4{__uint_as_float(G[0] << 16), __uint_as_float(G[0] & 0xffff0000u), __uint_as_float(G[1] << 16), __uint_as_float(G[1] & 0xffff0000u)};
    f4 ww = W - gf * 0.001f;
    unsigned M2 = M ^ (sm * 0x01010101u), V2 = V ^ (sv * 0x01010101u);
    u2 P = u2{(__float_as_uint(ww[0]) >> 16) | (__float_as_uint(ww[1]) & 0xffff0000u), (__float_as_uint(ww[2]) >> 16) | (__float_as_uint(ww[3]) & 0xffff0000u)};
    if (NT) {
      __builtin_nontemporal_store(ww, &w[i]); __builtin_nontemporal_store(M2, &mq[i]); __builtin_nontemporal_store(V2, &vq[i]); __builtin_nontemporal_store(P, &p[i]);
    } else {
      w[i] = ww; mq[i] = M2; vq[i] = V2; p[i] = P;
    }
    if ((threadIdx.x & 7) == 0) { ms[i / 8] = (unsigned char)(sm + 1); vs[i / 8] = (unsigned char)(sv + 1); }
  }
}

// The same bytes with the codes of m and v interleaved per eight elements
// (16 B per thread, one load and one store) and the two scale bytes of a run
// side by side (2 B per 32 elements): four read and four write streams.
template <bool NT>
__global__ __launch_bounds__(256) void adam_q8_interleaved(f4* __restrict__ w, const u4* __restrict__ g, u4* __restrict__ p,
                                                           u4* __restrict__ mv, unsigned short* __restrict__ sc, long n8) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256) {
    f4 W0 = NT ? __builtin_nontemporal_load(&w[2 * i]) : w[2 * i], W1 = NT ? __builtin_nontemporal_load(&w[2 * i + 1]) : w[2 * i + 1];
    u4 G = NT ? __builtin_nontemporal_load(&g[i]) : g[i];
    u4 C = NT ? __builtin_nontemporal_load(&mv[i]) : mv[i];
    unsigned s = sc[i / 4];
    f4 g0 = f4{__uint_as_float(G[0] << 16), __uint_as_float(G[0] & 0xffff0000u), __uint_as_float(G[1] << 16), __uint_as_float(G[1] & 0xffff0000u)};
    f4 g1 = f4{__uint_as_float(G[2] << 16), __uint_as_float(G[2] & 0xffff0000u), __uint_as_float(G[3] << 16), __uint_as_float(G[3] & 0xffff0000u)};
    f4 w0 = W0 - g0 * 0.001f, w1 = W1 - g1 * 0.001f;
    u4 C2 = C ^ (u4)(s * 0x00010001u);
    u4 P = u4{(__float_as_uint(w0[0]) >> 16) | (__float_as_uint(w0[1]) & 0xffff0000u), (__float_as_uint(w0[2]) >> 16) | (__float_as_uint(w0[3]) & 0xffff0000u),
              (__float_as_uint(w1[0]) >> 16) | (__float_as_uint(w1[1]) & 0xffff0000u), (__float_as_uint(w1[2]) >> 16) | (__float_as_uint(w1[3]) & 0xffff0000u)};
    if (NT) {
      __builtin_nontemporal_store(w0, &w[2 * i]); __builtin_nontemporal_store(w1, &w[2 * i + 1]);
      __builtin_nontemporal_store(C2, &mv[i]); __builtin_nontemporal_store(P, &p[i]);
    } else {
      w[2 * i] = w0; w[2 * i + 1] = w1; mv[i] = C2; p[i] = P;
    }
    if ((threadIdx.x & 3) == 0) sc[i / 4] = (unsigned short)(s + 1);
  }
}

template <typename F>
float time_ms(F launch, int reps) {
  hipEvent_t a, b; CHECK(hipEventCreate(&a)); CHECK(hipEventCreate(&b));
  for (int i = 0; i < 3; ++i) launch();
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(a));
  for (int i = 0; i < reps; ++i) launch();
  CHECK(hipEventRecord(b)); CHECK(hipEventSynchronize(b));
  float ms; CHECK(hipEventElapsedTime(&ms, a, b));
  CHECK(hipEventDestroy(a)); CHECK(hipEventDestroy(b));
  return ms / reps;
}

int main(int argc, char** argv) {
  long n = 62736416 / 4;  // f32x4 per buffer (the 8B / 128 shard)
  if (argc > 1) n = atol(argv[1]) / 4;
  f4 *w, *m, *v, *g, *b; float* out;
  // w, m and v in one allocation, back to back, so the interleaved pattern
  // can use all three as one 3n-vector state buffer.
  CHECK(hipMalloc(&w, n * 48)); m = w + n; v = w + 2 * n;
  CHECK(hipMalloc(&g, n * 16)); CHECK(hipMalloc(&b, n * 16)); CHECK(hipMalloc(&out, 16));
  CHECK(hipMemset(w, 0, n * 16)); CHECK(hipMemset(m, 0, n * 16)); CHECK(hipMemset(v, 0, n * 16));
  CHECK(hipMemset(g, 0, n * 16)); CHECK(hipMemset(b, 0, n * 16));
  hipDeviceProp_t prop; CHECK(hipGetDeviceProperties(&prop, 0));
  printf("device %s CUs %d clock %d kHz L2 %d MB, n=%ld floats per buffer\n", prop.gcnArchName, prop.multiProcessorCount, prop.clockRate, prop.l2CacheSize >> 20, n * 4);
  int cus = prop.multiProcessorCount;
  const int reps = 20;
  for (int bpc : {2, 4, 8, 16, 32}) {
    int grid = cus * bpc;
#define RUN(NAME, U, NT, BYTES, ...) { float ms = time_ms([&]{ NAME<U, NT><<<grid, 256>>>(__VA_ARGS__); }, reps); \
      printf("%-10s U=%d NT=%d blocks/CU=%2d  %8.1f us  %7.0f GB/s\n", #NAME, U, (int)NT, bpc, ms * 1e3, (double)(BYTES) / (ms * 1e-3) / 1e9); fflush(stdout); }
    RUN(read_kernel, 4, false, n * 16.0, g, n, out);
    RUN(read_kernel, 8, false, n * 16.0, g, n, out);
    RUN(read_kernel, 4, true, n * 16.0, g, n, out);
    RUN(copy_kernel, 2, false, n * 32.0, g, b, n);
    RUN(copy_kernel, 4, false, n * 32.0, g, b, n);
    RUN(copy_kernel, 4, true, n * 32.0, g, b, n);
    RUN(adam_like, 1, false, n * 112.0, w, m, v, g, n);
    RUN(adam_like, 2, false, n * 112.0, w, m, v, g, n);
    RUN(adam_like, 2, true, n * 112.0, w, m, v, g, n);
    RUN(adam_like, 4, false, n * 112.0, w, m, v, g, n);
    // interleaved state: n groups of four in the 3n f32x4 of w, m, v
    for (int nt = 0; nt < 2; ++nt) {
      float ms = time_ms([&]{ if (nt) adam_aos<true><<<grid, 256>>>(w, g, n); else adam_aos<false><<<grid, 256>>>(w, g, n); }, reps);
      printf("%-10s NT=%d blocks/CU=%2d  %8.1f us  %7.0f GB/s\n", "adam_aos", nt, bpc, ms * 1e3, n * 112.0 / (ms * 1e-3) / 1e9); fflush(stdout);
    }
    // bf16 gradient + copy: n f32x4 groups of w, m, v; g and the copy reuse
    // the first halves of the g and b buffers (8 B per group of four).
    {
      float ms = time_ms([&]{ adam_bf16_quads<true><<<grid, 256>>>(w, m, v, (const u2*)g, (u2*)b, n); }, reps);
      printf("%-10s NT=1 blocks/CU=%2d  %8.1f us  %7.0f GB/s\n", "bf16_quads", bpc, ms * 1e3, n * 4 * 30.0 / (ms * 1e-3) / 1e9); fflush(stdout);
      ms = time_ms([&]{ adam_bf16_quads_chunked<512><<<grid, 256>>>(w, m, v, (const u2*)g, (u2*)b, n); }, reps);
      printf("%-10s NT=1 blocks/CU=%2d  %8.1f us  %7.0f GB/s\n", "bf16_ch2k", bpc, ms * 1e3, n * 4 * 30.0 / (ms * 1e-3) / 1e9); fflush(stdout);
      ms = time_ms([&]{ adam_bf16_quads_chunked<4096><<<grid, 256>>>(w, m, v, (const u2*)g, (u2*)b, n); }, reps);
      printf("%-10s NT=1 blocks/CU=%2d  %8.1f us  %7.0f GB/s\n", "bf16_ch16k", bpc, ms * 1e3, n * 4 * 30.0 / (ms * 1e-3) / 1e9); fflush(stdout);
      ms = time_ms([&]{ adam_bf16_octets<true><<<grid, 256>>>(w, m, v, (const u4*)g, (u4*)b, n / 2); }, reps);
      printf("%-10s NT=1 blocks/CU=%2d  %8.1f us  %7.0f GB/s\n", "bf16_octets", bpc, ms * 1e3, n * 4 * 30.0 / (ms * 1e-3) / 1e9); fflush(stdout);
    }
    // 8-bit moments: 4n elements; codes in the m and v buffers (4n bytes
    // each), scale bytes after them (n/2 bytes each).
    for (int nt = 0; nt < 2; ++nt) {
      unsigned char* mb = (unsigned char*)m; unsigned char* vb = (unsigned char*)v;
      auto launch = [&]{
        if (nt) adam_q8_octets<true><<<grid, 256>>>(w, (const u4*)g, (u4*)b, (u2*)mb, (u2*)vb, mb + 4 * n, vb + 4 * n, n / 2);
        else adam_q8_octets<false><<<grid, 256>>>(w, (const u4*)g, (u4*)b, (u2*)mb, (u2*)vb, mb + 4 * n, vb + 4 * n, n / 2);
      };
      float ms = time_ms(launch, reps);
      printf("%-10s NT=%d blocks/CU=%2d  %8.1f us  %7.0f GB/s\n", "q8_octets", nt, bpc, ms * 1e3, n * 4 * 16.125 / (ms * 1e-3) / 1e9); fflush(stdout);
      // interleaved codes (8n bytes) in the m buffer, scale pairs after them
      auto launch2 = [&]{
        if (nt) adam_q8_interleaved<true><<<grid, 256>>>(w, (const u4*)g, (u4*)b, (u4*)mb, (unsigned short*)(mb + 8 * n), n / 2);
        else adam_q8_interleaved<false><<<grid, 256>>>(w, (const u4*)g, (u4*)b, (u4*)mb, (unsigned short*)(mb + 8 * n), n / 2);
      };
      ms = time_ms(launch2, reps);
      printf("%-10s NT=%d blocks/CU=%2d  %8.1f us  %7.0f GB/s\n", "q8_interl", nt, bpc, ms * 1e3, n * 4 * 16.125 / (ms * 1e-3) / 1e9); fflush(stdout);
      auto launch3 = [&]{
        if (nt) adam_q8_quads<true><<<grid, 256>>>(w, (const u2*)g, (u2*)b, (unsigned*)mb, (unsigned*)vb, mb + 4 * n, vb + 4 * n, n);
        else adam_q8_quads<false><<<grid, 256>>>(w, (const u2*)g, (u2*)b, (unsigned*)mb, (unsigned*)vb, mb + 4 * n, vb + 4 * n, n);
      };
      ms = time_ms(launch3, reps);
      printf("%-10s NT=%d blocks/CU=%2d  %8.1f us  %7.0f GB/s\n", "q8_quads", nt, bpc, ms * 1e3, n * 4 * 16.125 / (ms * 1e-3) / 1e9); fflush(stdout);
    }
  }
  return 0;
}
