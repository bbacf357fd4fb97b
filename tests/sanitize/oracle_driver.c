/* Drives the oracle over ragged sizes, non-finite values and both 8-bit
 * formats with every buffer allocated to its exact size, so that a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer reports any access
 * past an array or any undefined operation.  Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_bf16_to_f32(uint16_t h);
uint16_t oracle_f32_to_bf16(float f);
void oracle_f32_to_bf16_array(const float* x, uint16_t* out, int64_t n);
double oracle_sumsq_f32(const float* g, int64_t n, double acc);
double oracle_sumsq_bf16(const uint16_t* g, int64_t n, double acc);
float oracle_clip_coef(double sumsq, double max_norm);
float oracle_clip_coef_scaled(double sumsq, double max_norm, double grad_scale);
double oracle_pow_int(double beta, int64_t t);
void oracle_adamw_step(float* master, float* exp_avg, float* exp_avg_sq, const void* grad,
                       int grad_is_bf16, uint16_t* param_bf16, int64_t n, float clip, int64_t t,
                       double lr, double beta1, double beta2, double eps, double wd);
double oracle_fp8_value(uint8_t code, int format);
uint8_t oracle_fp8_round(double x, int format);
int oracle_block_exponent(double absmax, int format);
void oracle_quantize(const float* x, int64_t n, int format, uint8_t* codes, uint8_t* scales);
void oracle_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t n, int format,
                       float* x);
void oracle_adamw8_step(float* master, uint8_t* m_codes, uint8_t* m_scales, uint8_t* v_codes,
                        uint8_t* v_scales, const void* grad, int grad_is_bf16,
                        uint16_t* param_bf16, int64_t n, float clip, int64_t t, double lr,
                        double beta1, double beta2, double eps, double wd);

static uint64_t state = 0x9E3779B97F4A7C15ull;

static double uniform(void)  /* xorshift64*, in [0, 1) */
{
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (double)((state * 2685821657736338717ull) >> 11) / 9007199254740992.0;
}

static float value(int k)  /* mostly small normals, with special values mixed in */
{
    switch (k % 97) {
        case 3: return NAN;
        case 5: return INFINITY;
        case 7: return -INFINITY;
        case 11: return 1e-40f; /* subnormal */
        case 13: return -0.0f;
        case 17: return 3e38f;
        default: return (float)((uniform() - 0.5) * 0.02);
    }
}

static double checksum = 0.0;

static void add(double x)  /* keeps the results live; non-finite ones are counted apart */
{
    checksum += isfinite(x) ? x : 1.0;
}

static void* exact(size_t bytes)  /* exactly the bytes asked for (at least one) */
{
    void* p = malloc(bytes ? bytes : 1);
    if (!p) exit(2);
    return p;
}

int main(void)
{
    const int64_t sizes[] = {0, 1, 5, 31, 32, 33, 63, 64, 65, 100, 1000, 4099};
    for (size_t si = 0; si < sizeof sizes / sizeof sizes[0]; ++si) {
        const int64_t n = sizes[si];
        const int64_t runs = (n + 31) / 32;
#ifdef PLANTED_OVERRUN  /* one element short: the sanitizer must report it */
        float* w = exact(sizeof(float) * (n > 1 ? n - 1 : n));
#else
        float* w = exact(sizeof(float) * n);
#endif
        float* m = exact(sizeof(float) * n);
        float* v = exact(sizeof(float) * n);
        float* g = exact(sizeof(float) * n);
        uint16_t* gb = exact(sizeof(uint16_t) * n);
        uint16_t* p = exact(sizeof(uint16_t) * n);
        uint8_t* mc = exact(n);
        uint8_t* vc = exact(n);
        uint8_t* ms = exact(runs);
        uint8_t* vs = exact(runs);
        for (int64_t i = 0; i < n; ++i) {
            w[i] = value((int)i + 1);
            m[i] = value((int)i + 2) * 0.01f;
            v[i] = fabsf(value((int)i + 3)) * 1e-4f;
            g[i] = value((int)i);
        }
        oracle_f32_to_bf16_array(g, gb, n);
        add(oracle_sumsq_f32(g, n, 0.0));
        add(oracle_sumsq_bf16(gb, n, 0.0));
        const double S = oracle_sumsq_f32(g, n, 0.0);
        const float c = oracle_clip_coef(S, 1.0);
        add(oracle_clip_coef_scaled(S, 1.0, 0.125));
        for (int64_t t = 1; t <= 3; ++t) {
            oracle_adamw_step(w, m, v, g, 0, NULL, n, c, t, 3e-4, 0.9, 0.95, 1e-8, 0.1);
            oracle_adamw_step(w, m, v, gb, 1, p, n, c, t, 3e-4, 0.9, 0.95, 1e-8, 0.1);
        }
        for (int format = 0; format < 2; ++format) {
            oracle_quantize(m, n, format, mc, ms);
            oracle_dequantize(mc, ms, n, format, m);
        }
        oracle_quantize(m, n, 0, mc, ms);
        oracle_quantize(v, n, 1, vc, vs);
        oracle_adamw8_step(w, mc, ms, vc, vs, gb, 1, p, n, c, 7, 3e-4, 0.9, 0.95, 1e-8, 0.1);
        oracle_adamw8_step(w, mc, ms, vc, vs, g, 0, NULL, n, c, 8, 3e-4, 0.9, 0.95, 1e-8, 0.1);
        for (int64_t i = 0; i < n; ++i) add(w[i]);
        free(w); free(m); free(v); free(g); free(gb); free(p);
        free(mc); free(vc); free(ms); free(vs);
    }
    const int64_t steps[] = {1, 2, 1000, 123456, 2147483646};
    for (size_t i = 0; i < sizeof steps / sizeof steps[0]; ++i) {
        add(oracle_pow_int(0.9, steps[i]) + oracle_pow_int(0.95, steps[i]));
    }
    const double specials[] = {0.0, -0.0, 1e-45, 1e-30, 0.5, 448.0, 464.0, 57344.0, 61440.0,
                               1e30, INFINITY, -INFINITY, NAN};
    for (size_t i = 0; i < sizeof specials / sizeof specials[0]; ++i) {
        for (int format = 0; format < 2; ++format) {
            add(oracle_fp8_round(specials[i], format));
            add(oracle_block_exponent(fabs(specials[i]), format));
        }
        add(oracle_bf16_to_f32(oracle_f32_to_bf16((float)specials[i])));
    }
    for (int code = 0; code < 256; ++code) {
        for (int format = 0; format < 2; ++format) {
            add(oracle_fp8_value((uint8_t)code, format));
        }
    }
    printf("oracle driver ok %g\n", checksum);
    return 0;
}
