/*
 * Scalar CPU oracle for the clipped, mixed-precision AdamW step on one
 * GPU's parameter shard.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, includes or calls it, and it shares no source with that library.
 *
 * What it computes, and where that comes from:
 *   - "TorchTitan: a one-stop PyTorch-native solution for production LLM
 *     pre-training" (zenmind digest), section 3.3 (mixed-precision bullet)
 *     and section 4, steps 5 and 7: parameters are gathered and used in
 *     BF16, gradients are reduce-scattered in FP32, and the sharded optimizer
 *     state is updated in FP32.  Hence the update arithmetic below is fp32.
 *   - Lecture 9 exercises page, answer deriving the 16N state accounting and
 *     its three-basis table: bf16 params (2N) and grads (2N), fp32 m and v
 *     (8N), fp32 master weights (4N); the pure-fp32 basis has fp32 grads and
 *     no separate master.  Hence: grads arrive as bf16 or fp32, m, v and the
 *     master are fp32, and the bf16 parameter is a rounded copy of the master.
 *   - The same page's ZeRO-2 + AdamW scenario answer names AdamW with bf16
 *     params and grads, an fp32 master and no loss scaling.
 *
 * The pages give no AdamW formula, no eps placement, no clipping rule and no
 * summation precision.  The readings taken here (all listed in the design
 * notes):
 *   - AdamW with decoupled, multiplicative weight decay applied to the
 *     pre-update master, and Adam's bias corrections; eps is added to the
 *     bias-corrected sqrt(v).
 *   - Global-norm clipping: c = min(1, max_norm / (||g|| + 1e-6)), with the
 *     norm over every gradient of the call; c scales the gradient in fp32
 *     inside the update.
 *   - The norm is accumulated in fp64 (each product g*g is exact in fp64),
 *     sequentially in list order.
 *   - Derived scalars are formed in fp64 from the hyperparameters and rounded
 *     once to fp32; beta^t by binary exponentiation.
 *   - Each fp32 operation rounds once (build with -ffp-contract=off, no
 *     fast-math), in the order written below.
 *   - bf16 copy: round to nearest, ties to even; NaN stays a NaN of the same
 *     sign with the quiet bit set.
 *   - A gradient scale s (1/K accumulation, 1/world averaging, 1/loss scale)
 *     is folded into the coefficient: the step sees s*g, clipped by the norm
 *     of s*g.  A step with non-finite gradients may be skipped whole (the
 *     caller's choice), as a loss-scaled step is.
 *
 * Parity status: every function here is pinned by CPU tests against library
 * routines, closed forms, exact rational arithmetic or brute force.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------- bf16 --- */

/* bf16 is the upper half of an IEEE binary32 word; widening is exact. */
float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Narrow binary32 to bf16 by round-to-nearest, ties to even. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) {
        /* NaN: keep sign and the top payload bits, force the quiet bit. */
        return (uint16_t)((u >> 16) | 0x0040u);
    }
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) {
        kept += 1u; /* may carry into the exponent, up to infinity */
    }
    return (uint16_t)kept;
}

void oracle_f32_to_bf16_array(const float* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(x[i]);
}

/* ------------------------------------------------------------ grad norm --- */

/* Continue the running fp64 sum of squares `acc` over one fp32 gradient. */
double oracle_sumsq_f32(const float* g, int64_t n, double acc)
{
    for (int64_t i = 0; i < n; ++i) {
        double x = (double)g[i];
        acc = acc + x * x;
    }
    return acc;
}

/* Same for a bf16 gradient. */
double oracle_sumsq_bf16(const uint16_t* g, int64_t n, double acc)
{
    for (int64_t i = 0; i < n; ++i) {
        double x = (double)oracle_bf16_to_f32(g[i]);
        acc = acc + x * x;
    }
    return acc;
}

/* ----------------------------------------------------------------- clip --- */

/* c = min(1, max_norm / (sqrt(S) + 1e-6)) in fp64, rounded once to fp32.
 * The comparison is written so that a NaN norm gives a NaN coefficient and
 * an infinite norm gives 0. */
float oracle_clip_coef(double sumsq, double max_norm)
{
    double norm = sqrt(sumsq);
    double c = max_norm / (norm + 1e-6);
    if (c > 1.0) c = 1.0;
    return (float)c;
}

/* Gradient scaling folded into the coefficient.  The gradient the step should
 * see is s * g (s = 1/K after K accumulated micro-batches, 1/world for an
 * average over ranks, 1/loss_scale to undo loss scaling).  Its norm is
 * s * sqrt(S); the clip factor of that norm times s is the single multiplier
 * the update applies to the stored g:
 *     c = s * min(1, max_norm / (s * sqrt(S) + 1e-6))   (fp64, rounded once). */
float oracle_clip_coef_scaled(double sumsq, double max_norm, double grad_scale)
{
    double norm = grad_scale * sqrt(sumsq);
    double clip = max_norm / (norm + 1e-6);
    if (clip > 1.0) clip = 1.0;
    return (float)(grad_scale * clip);
}

/* ------------------------------------------------------- step scalars --- */

typedef struct {
    float beta1;      /* b1                                  */
    float beta2;      /* b2                                  */
    float one_m_b1;   /* 1 - b1                              */
    float one_m_b2;   /* 1 - b2                              */
    float decay;      /* 1 - lr * wd                         */
    float step_size;  /* lr / (1 - b1^t)                     */
    float bc2_sqrt;   /* sqrt(1 - b2^t)                      */
    float eps;        /* eps                                 */
} oracle_scalars;

/* beta^t by binary exponentiation, low bit first. */
double oracle_pow_int(double beta, int64_t t)
{
    double r = 1.0;
    double b = beta;
    while (t > 0) {
        if (t & 1) r = r * b;
        b = b * b;
        t >>= 1;
    }
    return r;
}

void oracle_step_scalars(int64_t t, double lr, double beta1, double beta2,
                         double eps, double wd, oracle_scalars* s)
{
    double p1 = oracle_pow_int(beta1, t);
    double p2 = oracle_pow_int(beta2, t);
    s->beta1 = (float)beta1;
    s->beta2 = (float)beta2;
    s->one_m_b1 = (float)(1.0 - beta1);
    s->one_m_b2 = (float)(1.0 - beta2);
    s->decay = (float)(1.0 - lr * wd);
    s->step_size = (float)(lr / (1.0 - p1));
    s->bc2_sqrt = (float)sqrt(1.0 - p2);
    s->eps = (float)eps;
}

/* ---------------------------------------------------------------- update --- */

/* One element of the step.  `g_raw` is the unclipped gradient widened to
 * fp32; every line is one correctly rounded fp32 operation. */
static void oracle_update_one(float* w, float* m, float* v, float g_raw,
                              float c, const oracle_scalars* s)
{
    float g = g_raw * c;

    float m_old = s->beta1 * *m;
    float m_in = s->one_m_b1 * g;
    float m_new = m_old + m_in;

    float v_old = s->beta2 * *v;
    float g2 = g * g;
    float v_in = s->one_m_b2 * g2;
    float v_new = v_old + v_in;

    float root = sqrtf(v_new);
    float root_hat = root / s->bc2_sqrt;
    float den = root_hat + s->eps;

    float w_decayed = *w * s->decay;
    float ratio = m_new / den;
    float delta = s->step_size * ratio;
    float w_new = w_decayed - delta;

    *m = m_new;
    *v = v_new;
    *w = w_new;
}

/* The step over one tensor.  grad_is_bf16 selects the gradient's type
 * (uint16_t bf16 words or float).  param_bf16 may be NULL (no copy). */
void oracle_adamw_step(float* master, float* exp_avg, float* exp_avg_sq,
                       const void* grad, int grad_is_bf16, uint16_t* param_bf16,
                       int64_t n, float clip, int64_t t, double lr,
                       double beta1, double beta2, double eps, double wd)
{
    oracle_scalars s;
    oracle_step_scalars(t, lr, beta1, beta2, eps, wd, &s);
    for (int64_t i = 0; i < n; ++i) {
        float g = grad_is_bf16 ? oracle_bf16_to_f32(((const uint16_t*)grad)[i])
                               : ((const float*)grad)[i];
        oracle_update_one(&master[i], &exp_avg[i], &exp_avg_sq[i], g, clip, &s);
        if (param_bf16) param_bf16[i] = oracle_f32_to_bf16(master[i]);
    }
}

/* ------------------------------------------------- 8-bit moment state --- */

/* The 10N variant of the state (Lecture 9 exercises page: the third row of
 * the three-basis table and the 7B answer, where 8-bit optimizer state takes
 * the 16N of mixed-precision Adam down to 10N, 112 GB to 70 GB): m and v are
 * stored in one byte per element.  The page names no encoding.  The reading
 * taken here:
 *   - element codes are OCP 8-bit floats: E4M3 (finite only, largest 448)
 *     for m and E5M2 (largest finite 57344) for v, whose wider exponent range
 *     holds v's squared magnitudes;
 *   - each run of 32 consecutive elements of a tensor (the last run may be
 *     shorter) shares a power-of-two scale 2^e, stored as the byte e + 127;
 *     an element's value is code * 2^e;
 *   - e is the smallest integer >= -127 for which the run's largest magnitude
 *     is at most the format's largest finite value times 2^e, so scaling
 *     never overflows and is exact;
 *   - a scaled value is rounded to the nearest code, ties to the even code;
 *   - a run holding a NaN or an infinity is stored as scale byte 255 with
 *     every code 255 and reads back as NaN;
 *   - a step decodes m and v, applies the fp32 update above unchanged (the
 *     new master comes from the unrounded fp32 moments) and stores the new
 *     moments re-encoded with fresh scales. */

#define ORACLE_QBLOCK 32
#define ORACLE_E4M3 0
#define ORACLE_E5M2 1

/* Value of one 8-bit code (sign, exponent field, mantissa field). */
double oracle_fp8_value(uint8_t code, int format)
{
    const int mbits = format == ORACLE_E4M3 ? 3 : 2;
    const int ebits = 7 - mbits;
    const int bias = (1 << (ebits - 1)) - 1;
    const int E = (code >> mbits) & ((1 << ebits) - 1);
    const int M = code & ((1 << mbits) - 1);
    double mag;
    if (format == ORACLE_E4M3 && E == 15 && M == 7) return NAN;
    if (format == ORACLE_E5M2 && E == 31) {
        if (M != 0) return NAN;
        mag = INFINITY;
    } else if (E == 0) {
        mag = ldexp((double)M, 1 - bias - mbits);            /* subnormal */
    } else {
        mag = ldexp((double)((1 << mbits) + M), E - bias - mbits);
    }
    return (code & 0x80) ? -mag : mag;
}

/* Nearest code to x, ties to the even code.  The candidates are every finite
 * non-negative code and the code one above the largest, standing for the
 * next step of the grid: in E4M3 that code is NaN (480), in E5M2 infinity
 * (65536), so values past the halfway point to it overflow the way the
 * format's own conversion rule says. */
uint8_t oracle_fp8_round(double x, int format)
{
    if (isnan(x)) return signbit(x) ? 0xFF : 0x7F;
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    const int top = format == ORACLE_E4M3 ? 0x7E : 0x7B;
    const double next = format == ORACLE_E4M3 ? 480.0 : 65536.0;
    const double a = fabs(x);
    /* At or past the next grid point, that point is the nearest candidate
     * (the test keeps the distances below exact in double). */
    if (a >= next) return (uint8_t)(sign | (top + 1));
    int best = 0;
    double best_d = a;
    for (int c = 1; c <= top + 1; ++c) {
        const double v = c <= top ? oracle_fp8_value((uint8_t)c, format) : next;
        const double d = fabs(a - v);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(sign | best);
}

void oracle_fp8_round_array(const float* x, int64_t n, int format, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp8_round((double)x[i], format);
}

/* Smallest e >= -127 with absmax <= largest * 2^e. */
int oracle_block_exponent(double absmax, int format)
{
    const double largest = format == ORACLE_E4M3 ? 448.0 : 57344.0;
    int e = -127;
    while (ldexp(largest, e) < absmax) ++e;
    return e;
}

/* Encode x[0..n) run by run: codes[n], scales[ceil(n / 32)]. */
void oracle_quantize(const float* x, int64_t n, int format, uint8_t* codes, uint8_t* scales)
{
    for (int64_t b0 = 0; b0 < n; b0 += ORACLE_QBLOCK) {
        const int64_t len = n - b0 < ORACLE_QBLOCK ? n - b0 : ORACLE_QBLOCK;
        int finite = 1;
        double absmax = 0.0;
        for (int64_t i = 0; i < len; ++i) {
            const double a = fabs((double)x[b0 + i]);
            if (!isfinite(a)) finite = 0;
            else if (a > absmax) absmax = a;
        }
        if (!finite) {
            scales[b0 / ORACLE_QBLOCK] = 255;
            memset(codes + b0, 255, (size_t)len);
            continue;
        }
        const int e = oracle_block_exponent(absmax, format);
        scales[b0 / ORACLE_QBLOCK] = (uint8_t)(e + 127);
        for (int64_t i = 0; i < len; ++i) {
            codes[b0 + i] = oracle_fp8_round(ldexp((double)x[b0 + i], -e), format);
        }
    }
}

void oracle_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t n, int format, float* x)
{
    for (int64_t i = 0; i < n; ++i) {
        const int s = scales[i / ORACLE_QBLOCK];
        x[i] = s == 255 ? NAN : (float)ldexp(oracle_fp8_value(codes[i], format), s - 127);
    }
}

/* The step over one tensor with 8-bit moments, run by run. */
void oracle_adamw8_step(float* master, uint8_t* m_codes, uint8_t* m_scales, uint8_t* v_codes,
                        uint8_t* v_scales, const void* grad, int grad_is_bf16,
                        uint16_t* param_bf16, int64_t n, float clip, int64_t t, double lr,
                        double beta1, double beta2, double eps, double wd)
{
    oracle_scalars s;
    oracle_step_scalars(t, lr, beta1, beta2, eps, wd, &s);
    float m[ORACLE_QBLOCK], v[ORACLE_QBLOCK];
    for (int64_t b0 = 0; b0 < n; b0 += ORACLE_QBLOCK) {
        const int64_t len = n - b0 < ORACLE_QBLOCK ? n - b0 : ORACLE_QBLOCK;
        const int64_t blk = b0 / ORACLE_QBLOCK;
        oracle_dequantize(m_codes + b0, m_scales + blk, len, ORACLE_E4M3, m);
        oracle_dequantize(v_codes + b0, v_scales + blk, len, ORACLE_E5M2, v);
        for (int64_t i = 0; i < len; ++i) {
            const int64_t k = b0 + i;
            const float g = grad_is_bf16 ? oracle_bf16_to_f32(((const uint16_t*)grad)[k])
                                         : ((const float*)grad)[k];
            oracle_update_one(&master[k], &m[i], &v[i], g, clip, &s);
            if (param_bf16) param_bf16[k] = oracle_f32_to_bf16(master[k]);
        }
        oracle_quantize(m, len, ORACLE_E4M3, m_codes + b0, m_scales + blk);
        oracle_quantize(v, len, ORACLE_E5M2, v_codes + b0, v_scales + blk);
    }
}
