/*
 * Test infrastructure: a plain C program that drives the optimizer library
 * through its C ABI alone, as a C or C++ training framework would -- the HIP
 * runtime for device memory and one stream, no Python and no torch.  On two
 * ragged lists (one element-misaligned view among them) it runs
 *   - the clipped step twice (bf16 gradients, bf16 copy, clipping active),
 *   - the three-call step (fp32 gradients: grad_norm_sq with the clip
 *     output, then adamw_multi_tensor_step),
 *   - the same clipped step on the library's own workspace (no-alloc entry),
 * and checks every element of master, m, v and the copy against the CPU
 * oracle stepped with the device's clip coefficient (bitwise), the sum of
 * squares against the oracle's (relative 1e-5), the coefficient against the
 * oracle's for the device's sum, and the step counter.  The oracle is linked
 * in because this program is a checker, not part of the library.
 *
 * Prints "c abi ok" and exits 0 when everything matches; otherwise prints
 * the first mismatch and exits 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "mps_adamw.h"

/* The oracle's entry points (oracle/oracle.c). */
double oracle_sumsq_f32(const float* g, int64_t n, double acc);
double oracle_sumsq_bf16(const uint16_t* g, int64_t n, double acc);
float oracle_clip_coef(double sumsq, double max_norm);
void oracle_adamw_step(float* master, float* exp_avg, float* exp_avg_sq, const void* grad,
                       int grad_is_bf16, uint16_t* param_bf16, int64_t n, float clip, int64_t t,
                       double lr, double beta1, double beta2, double eps, double wd);

#define CHECK_HIP(call)                                                                     \
    do {                                                                                    \
        hipError_t e_ = (call);                                                             \
        if (e_ != hipSuccess) {                                                             \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #call,                     \
                    hipGetErrorString(e_));                                                 \
            exit(1);                                                                        \
        }                                                                                   \
    } while (0)

#define CHECK_MPS(call)                                                                     \
    do {                                                                                    \
        int r_ = (call);                                                                    \
        if (r_ != 0) {                                                                      \
            fprintf(stderr, "%s:%d %s returned %d: %s\n", __FILE__, __LINE__, #call, r_,    \
                    adamw_last_error());                                                    \
            exit(1);                                                                        \
        }                                                                                   \
    } while (0)

#define LR 3e-4
#define BETA1 0.9
#define BETA2 0.95
#define EPS 1e-8
#define WD 0.1

/* splitmix64, and an approximate normal from twelve uniforms. */
static uint64_t rng_state = 0x4d505343ull;

static uint64_t next_u64(void)
{
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

static float normal(double std)
{
    double s = 0.0;
    for (int i = 0; i < 12; ++i) s += (double)(next_u64() >> 11) * 0x1.0p-53;
    return (float)((s - 6.0) * std);
}

static uint16_t to_bf16_bits(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16); /* truncation: any bf16 value is a valid input */
}

/* One tensor: host copies (what the oracle steps) and its device views,
 * `offset` elements into device buffers of numel + offset elements. */
typedef struct {
    int64_t n, offset;
    float *w, *m, *v;
    void* g;
    uint16_t* p;
    float *dw_buf, *dm_buf, *dv_buf;
    void* dg_buf;
    uint16_t* dp_buf;
} tensor;

static void* dmalloc(size_t bytes)
{
    void* p = NULL;
    CHECK_HIP(hipMalloc(&p, bytes > 0 ? bytes : 1));
    return p;
}

static void make_tensor(tensor* t, int64_t n, int64_t offset, int bf16, int copy)
{
    const size_t gsz = bf16 ? 2 : 4;
    const size_t alloc = (size_t)(n + offset);
    t->n = n;
    t->offset = offset;
    t->w = malloc(4 * alloc + 4);
    t->m = malloc(4 * alloc + 4);
    t->v = malloc(4 * alloc + 4);
    t->g = malloc(gsz * alloc + 4);
    t->p = copy ? calloc(alloc + 1, 2) : NULL;
    for (int64_t i = 0; i < n; ++i) {
        t->w[i] = normal(0.02);
        t->m[i] = normal(1e-4);
        t->v[i] = fabsf(normal(1e-8));
        const float g = normal(1e-3);
        if (bf16) {
            ((uint16_t*)t->g)[i] = to_bf16_bits(g);
        } else {
            ((float*)t->g)[i] = g;
        }
    }
    t->dw_buf = dmalloc(4 * alloc);
    t->dm_buf = dmalloc(4 * alloc);
    t->dv_buf = dmalloc(4 * alloc);
    t->dg_buf = dmalloc(gsz * alloc);
    t->dp_buf = copy ? dmalloc(2 * alloc) : NULL;
    CHECK_HIP(hipMemcpy(t->dw_buf + offset, t->w, 4 * (size_t)n, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(t->dm_buf + offset, t->m, 4 * (size_t)n, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(t->dv_buf + offset, t->v, 4 * (size_t)n, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy((char*)t->dg_buf + gsz * (size_t)offset, t->g, gsz * (size_t)n,
                        hipMemcpyHostToDevice));
    if (copy) CHECK_HIP(hipMemset(t->dp_buf, 0, 2 * alloc));
}

static mps_tensor describe(const tensor* t, int bf16)
{
    mps_tensor d;
    d.master = t->dw_buf + t->offset;
    d.exp_avg = t->dm_buf + t->offset;
    d.exp_avg_sq = t->dv_buf + t->offset;
    d.grad = (const char*)t->dg_buf + (size_t)t->offset * (bf16 ? 2 : 4);
    d.param_bf16 = t->dp_buf ? t->dp_buf + t->offset : NULL;
    d.numel = t->n;
    return d;
}

static int equal_bits(const void* a, const void* b, size_t bytes, const char* what, int tensor_i)
{
    if (memcmp(a, b, bytes) == 0) return 1;
    const unsigned char *x = a, *y = b;
    size_t k = 0;
    while (x[k] == y[k]) ++k;
    fprintf(stderr, "%s of tensor %d differs first at byte %zu\n", what, tensor_i, k);
    return 0;
}

/* Device results after a step against the oracle stepped on the host copies
 * with the device's coefficient; S and the coefficient checked first. */
static int check_step(tensor* ts, int nt, int bf16, double S_dev, float c_dev, int32_t step_dev,
                      int64_t t, double max_norm, const char* what)
{
    double S_ref = 0.0;
    for (int i = 0; i < nt; ++i) {
        S_ref = bf16 ? oracle_sumsq_bf16(ts[i].g, ts[i].n, S_ref)
                     : oracle_sumsq_f32(ts[i].g, ts[i].n, S_ref);
    }
    if (!(fabs(S_dev - S_ref) <= 1e-5 * S_ref)) {
        fprintf(stderr, "%s: sum of squares %.17g, oracle %.17g\n", what, S_dev, S_ref);
        return 0;
    }
    const float c_ref = oracle_clip_coef(S_dev, max_norm);
    if (memcmp(&c_ref, &c_dev, 4) != 0) {
        fprintf(stderr, "%s: coefficient %.9g, oracle %.9g\n", what, c_dev, c_ref);
        return 0;
    }
    if (step_dev != t) {
        fprintf(stderr, "%s: step counter %d, expected %lld\n", what, step_dev, (long long)t);
        return 0;
    }
    for (int i = 0; i < nt; ++i) {
        tensor* x = &ts[i];
        const size_t n = (size_t)x->n;
        oracle_adamw_step(x->w, x->m, x->v, x->g, bf16, x->p, x->n, c_dev, t, LR, BETA1, BETA2,
                          EPS, WD);
        float* got = malloc(4 * n + 4);
        uint16_t* gotp = malloc(2 * n + 2);
        CHECK_HIP(hipMemcpy(got, x->dw_buf + x->offset, 4 * n, hipMemcpyDeviceToHost));
        if (!equal_bits(got, x->w, 4 * n, "master", i)) return 0;
        CHECK_HIP(hipMemcpy(got, x->dm_buf + x->offset, 4 * n, hipMemcpyDeviceToHost));
        if (!equal_bits(got, x->m, 4 * n, "exp_avg", i)) return 0;
        CHECK_HIP(hipMemcpy(got, x->dv_buf + x->offset, 4 * n, hipMemcpyDeviceToHost));
        if (!equal_bits(got, x->v, 4 * n, "exp_avg_sq", i)) return 0;
        if (x->p) {
            CHECK_HIP(hipMemcpy(gotp, x->dp_buf + x->offset, 2 * n, hipMemcpyDeviceToHost));
            if (!equal_bits(gotp, x->p, 2 * n, "param_bf16", i)) return 0;
        }
        free(got);
        free(gotp);
    }
    printf("%s: S %.9e (oracle %.9e), coefficient %.9g, step %d, every element bitwise\n", what,
           S_dev, S_ref, c_dev, step_dev);
    return 1;
}

typedef struct {
    double* sumsq;
    float* coef;
    int32_t* step;
} scalars;

static void read_scalars(scalars d, double* S, float* c, int32_t* step, hipStream_t s)
{
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(S, d.sumsq, 8, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(c, d.coef, 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(step, d.step, 4, hipMemcpyDeviceToHost));
}

int main(void)
{
    hipStream_t stream;
    CHECK_HIP(hipSetDevice(0));
    CHECK_HIP(hipStreamCreate(&stream));
    scalars d = {dmalloc(8), dmalloc(4), dmalloc(4)};
    double S;
    float c;
    int32_t step;

    /* List A: bf16 gradients and a bf16 copy; tensor 2 is a view one element
     * into its buffers (every stream shares that misalignment); an empty
     * tensor in the middle.  max_norm 0.1 keeps clipping active. */
    const int64_t sizes_a[] = {1000, 4097, 33, 0, 65539};
    enum { NA = 5 };
    tensor a[NA];
    mps_tensor da[NA];
    for (int i = 0; i < NA; ++i) {
        make_tensor(&a[i], sizes_a[i], i == 2 ? 1 : 0, 1, 1);
        da[i] = describe(&a[i], 1);
    }
    const size_t ws_bytes = adamw_workspace_bytes(da, NA);
    if (ws_bytes == 0) {
        fprintf(stderr, "adamw_workspace_bytes: %s\n", adamw_last_error());
        return 1;
    }
    void* ws = dmalloc(ws_bytes);
    int32_t completed = 3;
    CHECK_HIP(hipMemcpy(d.step, &completed, 4, hipMemcpyHostToDevice));
    for (int64_t t = 4; t <= 5; ++t) {
        CHECK_MPS(adamw_clipped_step(da, NA, MPS_DTYPE_BF16, 0.1, 1.0, 0, d.sumsq, d.coef, d.step,
                                     LR, BETA1, BETA2, EPS, WD, ws, ws_bytes, stream, NULL));
        read_scalars(d, &S, &c, &step, stream);
        if (!check_step(a, NA, 1, S, c, step, t, 0.1, "clipped step, bf16 list")) return 1;
    }

    /* The same list through the no-alloc entry point (library workspace). */
    CHECK_MPS(adamw_clipped_step_noalloc(da, NA, MPS_DTYPE_BF16, 0.1, 1.0, 0, d.sumsq, d.coef,
                                         d.step, LR, BETA1, BETA2, EPS, WD, stream, NULL));
    read_scalars(d, &S, &c, &step, stream);
    if (!check_step(a, NA, 1, S, c, step, 6, 0.1, "no-alloc clipped step, bf16 list")) return 1;

    /* List B: fp32 gradients, no copy, through the three-call form (the
     * norm with its clip output, then the update), on the same workspace. */
    const int64_t sizes_b[] = {7, 2048, 100003};
    enum { NB = 3 };
    tensor b[NB];
    mps_tensor db[NB];
    for (int i = 0; i < NB; ++i) {
        make_tensor(&b[i], sizes_b[i], 0, 0, 0);
        db[i] = describe(&b[i], 0);
    }
    const size_t ws_b = adamw_workspace_bytes(db, NB);
    if (ws_b == 0 || ws_b > ws_bytes) {
        fprintf(stderr, "workspace for list B: %zu bytes (list A's: %zu)\n", ws_b, ws_bytes);
        return 1;
    }
    completed = 0;
    CHECK_HIP(hipMemcpy(d.step, &completed, 4, hipMemcpyHostToDevice));
    CHECK_MPS(grad_norm_sq(db, NB, MPS_DTYPE_F32, d.sumsq, 0.1, 1.0, d.coef, ws, ws_bytes, stream));
    CHECK_MPS(adamw_multi_tensor_step(db, NB, MPS_DTYPE_F32, d.coef, NULL, d.step, LR, BETA1,
                                      BETA2, EPS, WD, ws, ws_bytes, stream));
    read_scalars(d, &S, &c, &step, stream);
    if (!check_step(b, NB, 0, S, c, step, 1, 0.1, "three-call step, fp32 list")) return 1;

    CHECK_MPS(adamw_workspace_release(ws));
    CHECK_HIP(hipFree(ws));
    CHECK_HIP(hipStreamDestroy(stream));
    printf("c abi ok\n");
    return 0;
}
