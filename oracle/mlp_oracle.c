/*
 * mlp_oracle.c -- plain CPU oracle for the tile-synchronized MLP GEMM chain.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table
 * or constant with the GPU library.
 *
 * What it computes (the plain definition, written out):
 *
 *   The chain is the transformer MLP whose first GEMM carries the pointwise
 *   activation and whose second GEMM consumes the activated intermediate
 *   (CuSync README, github.com/microsoft/cusync, paragraph on the GPT-3 and
 *   LLaMA MLP graphs: GeLU is fused with the first GeMM).  Synchronizing
 *   tiles instead of kernels changes when tiles run, not what they compute
 *   (CuSync README, opening paragraph), so the oracle is the unsynchronized
 *   definition:
 *
 *     h[m,i]  = sum_{k=0..H-1} x[m,k] * w1[k,i]        fp32, k ascending
 *     a[m,i]  = act(h[m,i])                             fp32
 *     t[m,i]  = RNE_dtype(a[m,i])                       storage dtype
 *     y[m,n]  = RNE_dtype( sum_{i=0..I-1} t[m,i] * w2[i,n] )   fp32, i ascending
 *
 *   act is one of
 *     none      : a = h
 *     gelu_tanh : a = 0.5 h (1 + tanh( sqrt(2/pi) (h + 0.044715 h^3) ))
 *     swiglu    : a = silu(g) * u,  silu(g) = g / (1 + exp(-g)),
 *                 g from w1[:, 0:I] and u from w1[:, I:2I]  (w1 is [H, 2I])
 *
 *   Inputs are fp16 or bf16 bit patterns, widened exactly to fp32.  Every
 *   fp16*fp16 and bf16*bf16 product is exact in fp32, so only the additions
 *   round.  The intermediate is rounded once, after the activation.
 *
 * Loop order: each output row is one OpenMP task.  Inside a row the k loop
 * is outermost and the column loop innermost, which streams the weight rows
 * contiguously; each accumulator still sees its terms in ascending k (and
 * ascending i for the second GEMM), exactly as the definition states.
 * Compiled with -ffp-contract=off and without fast-math.
 *
 * Readings where the pages are silent (GeLU variant, SwiGLU packing, no
 * bias, RNE rounding, activation on the unrounded fp32 accumulator) are the
 * plainest ones and are listed in the project's design notes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_ACT_NONE = 0, ORACLE_ACT_GELU_TANH = 1, ORACLE_ACT_SWIGLU = 2 };
enum { ORACLE_F16 = 0, ORACLE_BF16 = 1 };

/* ---- storage formats (IEEE 754 binary16, and bfloat16 = top half of binary32) ---- */

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
 * normal:    (-1)^s * 2^(e-15) * (1 + f/1024)
 * subnormal: (-1)^s * 2^-14    * (f/1024)          (e == 0)
 * e == 31:   inf (f == 0) or NaN                                      */
static float widen_f16(uint16_t h) {
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    float v;
    if (e == 0) {
        v = ldexpf((float)f, -24);                 /* f/1024 * 2^-14, exact */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexpf((float)(1024 + f), e - 25);     /* (1024+f) * 2^(e-15-10), exact */
    }
    return s ? -v : v;
}

/* bfloat16 is the upper 16 bits of a binary32 value. */
static float widen_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float v;
    memcpy(&v, &u, sizeof v);
    return v;
}

static float widen(uint16_t v, int dtype) {
    return dtype == ORACLE_BF16 ? widen_bf16(v) : widen_f16(v);
}

/* Round a finite, non-negative fp32 value a to a format with `man` stored
 * fraction bits and minimum normal exponent `emin`, ties to even, and
 * return the encoding (exponent field << man) + fraction, which may carry
 * into the next binade.  The value is scaled by a power of two (exact) so
 * that one unit of the result's last place becomes 1.0, then rounded to an
 * integer with nearbyintf under the default round-to-nearest-even mode. */
static uint32_t round_magnitude(float a, int man, int emin, int bias) {
    if (a == 0.0f) return 0;
    int ex;
    frexpf(a, &ex);                                   /* a = fr * 2^ex, fr in [0.5,1) */
    int e = ex - 1;                                   /* a in [2^e, 2^(e+1)) */
    if (e < emin) {
        /* subnormal range: fixed quantum 2^(emin - man) */
        float q = nearbyintf(ldexpf(a, man - emin));
        return (uint32_t)q;                           /* 2^man here means the smallest normal */
    }
    float q = nearbyintf(ldexpf(a, man - e));         /* in [2^man, 2^(man+1)] */
    return ((uint32_t)(e + bias) << man) + ((uint32_t)q - (1u << man));
}

static uint16_t round_f16(float v) {
    uint16_t s = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return s | 0x7e00;
    float a = fabsf(v);
    if (isinf(a) || a >= 131072.0f) return s | 0x7c00;   /* far beyond the largest finite value */
    uint32_t enc = round_magnitude(a, 10, -14, 15);
    if (enc >= 0x7c00) return s | 0x7c00;                 /* rounded past 65504: overflow to inf */
    return (uint16_t)(s | enc);
}

static uint16_t round_bf16(float v) {
    uint16_t s = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return s | 0x7fc0;
    float a = fabsf(v);
    if (isinf(a)) return s | 0x7f80;
    uint32_t enc = round_magnitude(a, 7, -126, 127);
    if (enc >= 0x7f80) return s | 0x7f80;
    return (uint16_t)(s | enc);
}

static uint16_t round_to(float v, int dtype) {
    return dtype == ORACLE_BF16 ? round_bf16(v) : round_f16(v);
}

/* ---- activations, fp32, host libm ---- */

/* tanh form of GeLU (the GeLU that the CuSync README fuses into the first
 * GeMM; the pages give no formula, so this is the common tanh variant). */
static float gelu_tanh(float h) {
    const float c = 0.7978845608028654f;   /* sqrt(2/pi) */
    const float k = 0.044715f;
    float inner = c * (h + k * (h * h * h));
    return 0.5f * h * (1.0f + tanhf(inner));
}

static float silu(float g) {
    return g / (1.0f + expf(-g));
}

static float activate(float g, float u, int act) {
    switch (act) {
    case ORACLE_ACT_GELU_TANH: return gelu_tanh(g);
    case ORACLE_ACT_SWIGLU:    return silu(g) * u;
    default:                   return g;
    }
}

/* ---- exported pieces, so the test suite can pin each one ---- */

void oracle_widen(const uint16_t* in, float* out, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) out[i] = widen(in[i], dtype);
}

void oracle_round(const float* in, uint16_t* out, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) out[i] = round_to(in[i], dtype);
}

/* u may be NULL unless act is swiglu */
void oracle_act(const float* g, const float* u, float* out, int64_t n, int act) {
    for (int64_t i = 0; i < n; ++i) out[i] = activate(g[i], u ? u[i] : 0.0f, act);
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- the chain ----
 *
 * x  : [M, H]      row-major, dtype bits
 * w1 : [H, g*I]    row-major (g = 2 for swiglu: gate columns 0..I-1, up columns I..2I-1)
 * w2 : [I, H]      row-major
 * t  : [M, I]      optional (may be NULL): receives the rounded intermediate
 * y  : [M, H]      receives the rounded output
 * nthreads <= 0 uses the OpenMP default.
 * Returns 0, -1 for bad arguments, -2 if memory runs out. */
int oracle_mlp_chain(const uint16_t* x, const uint16_t* w1, const uint16_t* w2,
                     uint16_t* t, uint16_t* y, int64_t M, int64_t H, int64_t I,
                     int act, int dtype, int nthreads) {
    if (M < 0 || H <= 0 || I <= 0) return -1;
    if (act < ORACLE_ACT_NONE || act > ORACLE_ACT_SWIGLU) return -1;
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    if (M == 0) return 0;
    if (!x || !w1 || !w2 || !y) return -1;

    const int64_t g = (act == ORACLE_ACT_SWIGLU) ? 2 : 1;
    const int64_t n1 = g * I;                  /* columns of w1 */

    float* w1f = (float*)malloc(sizeof(float) * (size_t)(H * n1));
    float* w2f = (float*)malloc(sizeof(float) * (size_t)(I * H));
    if (!w1f || !w2f) { free(w1f); free(w2f); return -2; }
    oracle_widen(w1, w1f, H * n1, dtype);
    oracle_widen(w2, w2f, I * H, dtype);

    int failed = 0;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
    {
        float* acc1 = (float*)malloc(sizeof(float) * (size_t)n1);
        float* tf = (float*)malloc(sizeof(float) * (size_t)I);
        float* acc2 = (float*)malloc(sizeof(float) * (size_t)H);
        if (!acc1 || !tf || !acc2) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int64_t m = 0; m < M; ++m) {
                const uint16_t* xr = x + m * H;
                /* first GEMM: acc1[c] = sum_k x[m,k] * w1[k,c], k ascending */
                for (int64_t c = 0; c < n1; ++c) acc1[c] = 0.0f;
                for (int64_t k = 0; k < H; ++k) {
                    const float xv = widen(xr[k], dtype);
                    const float* wr = w1f + k * n1;
                    for (int64_t c = 0; c < n1; ++c) acc1[c] = acc1[c] + xv * wr[c];
                }
                /* activation on the fp32 accumulator(s), one rounding to dtype */
                for (int64_t i = 0; i < I; ++i) {
                    const float a = activate(acc1[i], g == 2 ? acc1[I + i] : 0.0f, act);
                    const uint16_t tb = round_to(a, dtype);
                    if (t) t[m * I + i] = tb;
                    tf[i] = widen(tb, dtype);
                }
                /* second GEMM: acc2[n] = sum_i t[m,i] * w2[i,n], i ascending */
                for (int64_t n = 0; n < H; ++n) acc2[n] = 0.0f;
                for (int64_t i = 0; i < I; ++i) {
                    const float tv = tf[i];
                    const float* wr = w2f + i * H;
                    for (int64_t n = 0; n < H; ++n) acc2[n] = acc2[n] + tv * wr[n];
                }
                for (int64_t n = 0; n < H; ++n) y[m * H + n] = round_to(acc2[n], dtype);
            }
        }
        free(acc1);
        free(tf);
        free(acc2);
    }
    free(w1f);
    free(w2f);
    return failed ? -2 : 0;
}
