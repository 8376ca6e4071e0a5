/*
 * mxfp4_oracle.c -- plain CPU oracle (TEST INFRASTRUCTURE ONLY; see the
 * header for the source passages and the readings R1-R5).
 *
 * Written for clarity, not speed: each value is decoded from its bit fields,
 * every rounding is spelled out, fp64 is used wherever the method does not
 * itself fix a narrower type.  Rows are independent, so the outer loops carry
 * an OpenMP pragma; nothing else is reordered.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared
 *        -fPIC mxfp4_oracle.c -o _liboracle.so -lm
 */
#include "mxfp4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------- */
/* Scalar codecs                                                           */
/* ---------------------------------------------------------------------- */

/* E2M1 ([P2] Overview: float4_e2m1fn): 1 sign bit, 2 exponent bits with
   bias 1, 1 mantissa bit; exponent field 0 is subnormal (0.5 * mantissa).
   The magnitudes are therefore {0, 0.5, 1, 1.5, 2, 3, 4, 6}; max 6 as the
   single-scale section of [P2] states. */
double orc_e2m1_value(unsigned code)
{
    unsigned sign = (code >> 3) & 1u;
    unsigned exp  = (code >> 1) & 3u;
    unsigned man  = code & 1u;
    double mag;
    if (exp == 0)
        mag = 0.5 * (double)man;
    else
        mag = ldexp(1.0 + 0.5 * (double)man, (int)exp - 1);
    return sign ? -mag : mag;
}

/* float8_e4m3fn ([P3] section 4: the NVFP4 per-16 group scale type):
   1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinities,
   S.1111.111 is NaN, max finite 448. */
double orc_e4m3_value(unsigned byte)
{
    unsigned sign = (byte >> 7) & 1u;
    unsigned exp  = (byte >> 3) & 15u;
    unsigned man  = byte & 7u;
    double mag;
    if (exp == 15 && man == 7)
        return NAN;
    if (exp == 0)
        mag = ldexp((double)man / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)man / 8.0, (int)exp - 7);
    return sign ? -mag : mag;
}

/* float8_e8m0fnu ([P2] Overview; Validation and Notes item 4: raw bytes):
   an unsigned biased exponent, value 2^(b-127), 0xFF is NaN. */
double orc_e8m0_value(unsigned byte)
{
    if ((byte & 0xFFu) == 0xFFu)
        return NAN;
    return ldexp(1.0, (int)(byte & 0xFFu) - 127);
}

double orc_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bfloat16 (8 significant bits, exponent range
   of fp32, subnormals down to 2^-133), ties to even, overflow to infinity. */
uint16_t orc_bf16_from_double(double v)
{
    if (isnan(v))
        return 0x7FC0u;
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v);
    double r;
    if (isinf(a)) {
        r = INFINITY;
    } else if (a == 0.0) {
        r = 0.0;
    } else {
        int x;
        frexp(a, &x);                 /* a = f * 2^x, f in [0.5, 1)      */
        int e = x - 1;                /* floor(log2 a)                    */
        int quantum_exp = (e < -126) ? -133 : e - 7;
        double n = nearbyint(ldexp(a, -quantum_exp));   /* half-to-even */
        r = ldexp(n, quantum_exp);
        if (r >= ldexp(1.0, 128))
            r = INFINITY;
    }
    float f = (float)r;               /* exact: r is bf16-representable  */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t bits = (uint16_t)(u >> 16);
    return neg ? (uint16_t)(bits | 0x8000u) : bits;
}

uint16_t orc_bf16_from_float(float v) { return orc_bf16_from_double((double)v); }

/* R4 -- element encode ([P2] single-scale section: round_mode="rint", E2M1
   maximum 6).  The E2M1 value nearest to q is chosen; when q lies exactly
   half-way between two neighbours the one with the even code (mantissa bit
   0) wins.  Magnitudes of 6 and above saturate to 6 (E2M1 has no Inf); the
   test comes first because for |q| beyond about 2^53 the fp64 distances to
   4 and 6 are no longer exact and would tie.  The sign bit is copied from q.
   Below 6 the distances are exact in fp64 (q has at most 24 significant
   bits), so no false ties arise. */
unsigned orc_e2m1_encode(double q)
{
    static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double a = fabs(q);
    if (a >= 6.0)
        return (signbit(q) ? 8u : 0u) | 7u;
    unsigned best = 0;
    double bestd = a;
    for (unsigned i = 1; i < 8; ++i) {
        double d = fabs(a - grid[i]);
        if (d < bestd || (d == bestd && (i % 2u) == 0u)) {
            best = i;
            bestd = d;
        }
    }
    return (signbit(q) ? 8u : 0u) | best;
}

/* R4 applied to bf16 values at one fixed scale byte: the element step of
   the block quantizer below (q = v / 2^(byte - 127), exact by ldexp, then the
   nearest E2M1 code), one code per input in the low nibble of codes[i].
   Exposed so that the encoder can be swept over every (bf16 value, scale
   byte) pair; NaN and Inf inputs are the block rule's business and get 0. */
void orc_e2m1_encode_bf16_at_scale(const uint16_t* x, int64_t n, unsigned byte,
                                   uint8_t* codes)
{
    int e = (int)byte - 127;
    for (int64_t i = 0; i < n; ++i) {
        double v = orc_bf16_value(x[i]);
        codes[i] = (isnan(v) || isinf(v)) ? 0u : (uint8_t)orc_e2m1_encode(ldexp(v, -e));
    }
}

/* R3 -- shared exponent of an OCP MX block ([P2] single-scale section:
   setting 0 = OCP MX; Overview: one E8M0 exponent per 32 K-elements).  The
   block scale is 2^(floor(log2 amax) - emax) with emax = 2, the exponent of
   the largest E2M1 binade (6 = 1.5 * 2^2), clamped to E8M0's range. */
unsigned orc_shared_exponent(double amax)
{
    if (isnan(amax) || isinf(amax))
        return 0xFFu;
    int e;
    if (amax == 0.0) {
        e = -127;
    } else {
        int x;
        frexp(amax, &x);
        e = (x - 1) - 2;
    }
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return (unsigned)(e + 127);
}

/* R9: the smallest e with amax <= 7.25 * 2^e, found by counting up from an
   e that is certainly too small (7.25 * 2^(x-5) < 2^(x-1) <= amax); 7.25 * 2^e
   and the comparison are exact in fp64. */
unsigned orc_shared_exponent_uos(double amax)
{
    if (isnan(amax) || isinf(amax))
        return 0xFFu;
    int e;
    if (amax == 0.0) {
        e = -127;
    } else {
        int x;
        frexp(amax, &x);
        e = (x - 1) - 4;
        while (amax > 7.25 * ldexp(1.0, e))
            ++e;
    }
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return (unsigned)(e + 127);
}

/* R3 + R4 on one block of 32 values, packed per R1. */
void orc_mx_quantize_block(const double v[32], uint8_t codes[16], uint8_t* scale)
{
    orc_mx_quantize_block_rule(v, codes, scale, ORC_RULE_OCP);
}

/* R3 (or R9) + R4 on one block of 32 values, packed per R1. */
void orc_mx_quantize_block_rule(const double v[32], uint8_t codes[16], uint8_t* scale,
                                int rule)
{
    double amax = 0.0;
    int bad = 0;
    for (int i = 0; i < 32; ++i) {
        if (isnan(v[i]) || isinf(v[i]))
            bad = 1;
        else if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    }
    unsigned b = bad ? 0xFFu
                     : (rule == ORC_RULE_UOS ? orc_shared_exponent_uos(amax)
                                             : orc_shared_exponent(amax));
    *scale = (uint8_t)b;
    if (b == 0xFFu) {
        memset(codes, 0, 16);
        return;
    }
    int e = (int)b - 127;
    for (int j = 0; j < 16; ++j) {
        unsigned lo = orc_e2m1_encode(ldexp(v[2 * j], -e));
        unsigned hi = orc_e2m1_encode(ldexp(v[2 * j + 1], -e));
        codes[j] = (uint8_t)(lo | (hi << 4));
    }
}

/* ---------------------------------------------------------------------- */
/* NVFP4 dequantization (R2)                                               */
/* ---------------------------------------------------------------------- */

static unsigned nibble(const uint8_t* row, int64_t k)
{
    uint8_t byte = row[k / 2];
    return (k % 2 == 0) ? (byte & 15u) : (byte >> 4);
}

/* [P1] introduction: NVFP4 = packed E2M1, an FP8 scale per block, an FP32
   per-tensor scale.  [P3] sections 3-4: codes [N, K/2], E4M3 scales
   [N, K/16], fp32 global.  The product code * block scale is exact in fp32
   (at most 6 significant bits); multiplying by g rounds once (RNE). */
static void nvfp4_dequant_row(const uint8_t* codes_row, const uint8_t* scales_row,
                              float g, int64_t K, int bf16_intermediate, float* out)
{
    for (int64_t k = 0; k < K; ++k) {
        double cs = orc_e2m1_value(nibble(codes_row, k)) *
                    orc_e4m3_value(scales_row[k / 16]);
        float p = (float)cs;          /* exact                              */
        float w = p * g;              /* one IEEE fp32 rounding             */
        if (bf16_intermediate) {
            uint32_t u = (uint32_t)orc_bf16_from_float(w) << 16;
            memcpy(&w, &u, sizeof w);
        }
        out[k] = w;
    }
}

void orc_nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, float g,
                       int64_t N, int64_t K, int bf16_intermediate, float* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        nvfp4_dequant_row(codes + n * (K / 2), scales + n * (K / 16), g, K,
                          bf16_intermediate, out + n * K);
}

/* ---------------------------------------------------------------------- */
/* The four operations                                                     */
/* ---------------------------------------------------------------------- */

/* [P1] pipeline section: dequantize a layer, quantize the intermediate to
   MXFP4, write it into the preallocated destination.  MX block j along K
   covers NVFP4 blocks 2j and 2j+1. */
void orc_requant(const uint8_t* nv_codes, const uint8_t* nv_scales,
                 const float* nv_global, int64_t T, int64_t N, int64_t K,
                 int bf16_intermediate, uint8_t* mx_codes, uint8_t* mx_scales)
{
    orc_requant_rule(nv_codes, nv_scales, nv_global, T, N, K, bf16_intermediate,
                     ORC_RULE_OCP, mx_codes, mx_scales);
}

void orc_requant_rule(const uint8_t* nv_codes, const uint8_t* nv_scales,
                      const float* nv_global, int64_t T, int64_t N, int64_t K,
                      int bf16_intermediate, int rule, uint8_t* mx_codes,
                      uint8_t* mx_scales)
{
    for (int64_t t = 0; t < T; ++t) {
#pragma omp parallel
        {
            float* row = (float*)malloc((size_t)K * sizeof(float));
            double blk[32];
#pragma omp for schedule(static)
            for (int64_t n = 0; n < N; ++n) {
                int64_t r = t * N + n;
                nvfp4_dequant_row(nv_codes + r * (K / 2), nv_scales + r * (K / 16),
                                  nv_global[t], K, bf16_intermediate, row);
                for (int64_t j = 0; j < K / 32; ++j) {
                    for (int i = 0; i < 32; ++i)
                        blk[i] = (double)row[32 * j + i];
                    orc_mx_quantize_block_rule(blk, mx_codes + r * (K / 2) + 16 * j,
                                               mx_scales + r * (K / 32) + j, rule);
                }
            }
            free(row);
        }
    }
}

/* [P1] closing list: activations are quantized to MXFP4 per batch, with no
   stored scales; [P2] single-scale section: axis=-1, block 32. */
void orc_quantize_act(const uint16_t* x, int64_t ldx, const int32_t* row_index,
                      int64_t M, int64_t K, uint8_t* codes, uint8_t* scales)
{
    orc_quantize_act_rule(x, ldx, row_index, M, K, ORC_RULE_OCP, codes, scales);
}

void orc_quantize_act_rule(const uint16_t* x, int64_t ldx, const int32_t* row_index,
                           int64_t M, int64_t K, int rule, uint8_t* codes,
                           uint8_t* scales)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        int64_t src = row_index ? (int64_t)row_index[m] : m;
        const uint16_t* xr = x + src * ldx;
        double blk[32];
        for (int64_t j = 0; j < K / 32; ++j) {
            for (int i = 0; i < 32; ++i)
                blk[i] = orc_bf16_value(xr[32 * j + i]);
            orc_mx_quantize_block_rule(blk, codes + m * (K / 2) + 16 * j,
                                       scales + m * (K / 32) + j, rule);
        }
    }
}

/* Dequantized MXFP4 element: e2m1(code) * 2^(byte - 127), exact in fp64. */
static double mx_value(const uint8_t* codes, const uint8_t* scales, int64_t row,
                       int64_t K, int64_t k)
{
    return orc_e2m1_value(nibble(codes + row * (K / 2), k)) *
           orc_e8m0_value(scales[row * (K / 32) + k / 32]);
}

static void mx_row(const uint8_t* codes, const uint8_t* scales, int64_t row,
                   int64_t K, double* out)
{
    for (int64_t k = 0; k < K; ++k)
        out[k] = mx_value(codes, scales, row, K, k);
}

static void dot_row(const double* a, const double* b, int64_t K, double* y, double* s)
{
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = a[k] * b[k];
        acc += p;
        mag += fabs(p);
    }
    *y = acc;
    *s = mag;
}

/* [P1] closing list: both GEMM operands are MXFP4; FP32 accumulation is the
   hardware's, the oracle sums the exact products in fp64 (R5). */
void orc_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
              const uint8_t* b_codes, const uint8_t* b_scales,
              int64_t M, int64_t N, int64_t K, double* y, double* s)
{
    double* bd = (double*)malloc((size_t)(N * K) * sizeof(double));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        mx_row(b_codes, b_scales, n, K, bd + n * K);
#pragma omp parallel
    {
        double* ad = (double*)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            mx_row(a_codes, a_scales, m, K, ad);
            for (int64_t n = 0; n < N; ++n) {
                double yy, ss;
                dot_row(ad, bd + n * K, K, &yy, &ss);
                if (y) y[m * N + n] = yy;
                if (s) s[m * N + n] = ss;
            }
        }
        free(ad);
    }
    free(bd);
}

void orc_gemm_at(const uint8_t* a_codes, const uint8_t* a_scales,
                 const uint8_t* b_codes, const uint8_t* b_scales,
                 int64_t M, int64_t N, int64_t K,
                 const int64_t* pm, const int64_t* pn, int64_t P,
                 double* y, double* s)
{
    (void)M; (void)N;
#pragma omp parallel
    {
        double* ad = (double*)malloc((size_t)K * sizeof(double));
        double* bd = (double*)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t p = 0; p < P; ++p) {
            mx_row(a_codes, a_scales, pm[p], K, ad);
            mx_row(b_codes, b_scales, pn[p], K, bd);
            double yy, ss;
            dot_row(ad, bd, K, &yy, &ss);
            if (y) y[p] = yy;
            if (s) s[p] = ss;
        }
        free(ad);
        free(bd);
    }
}

/* [P1] closing list: MoE experts run on MXFP4 kernels; one GEMM per expert
   over its contiguous block of (already expert-sorted) rows. */
void orc_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                      const uint8_t* b_codes, const uint8_t* b_scales,
                      const int32_t* offsets, int64_t E, int64_t N, int64_t K,
                      double* y, double* s)
{
    for (int64_t e = 0; e < E; ++e) {
        int64_t r0 = offsets[e], r1 = offsets[e + 1];
        if (r1 <= r0)
            continue;
        orc_gemm(a_codes + r0 * (K / 2), a_scales + r0 * (K / 32),
                 b_codes + e * N * (K / 2), b_scales + e * N * (K / 32),
                 r1 - r0, N, K,
                 y ? y + r0 * N : NULL, s ? s + r0 * N : NULL);
    }
}

/* ---- Smooth pre-scale ------------------------------------------------------ */

/* R17: the per-channel product in fp32 (contraction off), rounded to bf16. */
void orc_smooth_rows(const uint16_t* x, int64_t ldx, const int32_t* row_index,
                     const uint16_t* smooth, int64_t M, int64_t K, uint16_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        int64_t src = row_index ? (int64_t)row_index[m] : m;
        for (int64_t k = 0; k < K; ++k) {
            float v = (float)orc_bf16_value(x[src * ldx + k]);
            float s = (float)orc_bf16_value(smooth[k]);
            float p = v * s;
            out[m * K + k] = orc_bf16_from_float(p);
        }
    }
}

/* ---- W4A8: MXFP8 activations x MXFP4 weights ------------------------------ */

/* R14: the float8_e4m3fn value nearest to q, found by scanning the 127
   non-negative finite codes (values increase with the code); on an exact tie
   the even code (mantissa bit 0) wins.  448 (0x7E) is the largest, so larger
   q saturate to it.  Distances are exact in fp64 for the q the path forms
   (a bf16 value times a power of two, |q| < 512). */
unsigned orc_e4m3_encode(double q)
{
    double a = fabs(q);
    unsigned best = 0;
    double bestd = a;
    for (unsigned c = 1; c < 0x7Fu; ++c) {
        double d = fabs(a - orc_e4m3_value(c));
        if (d < bestd || (d == bestd && (c % 2u) == 0u)) {
            best = c;
            bestd = d;
        }
    }
    return (signbit(q) ? 0x80u : 0u) | best;
}

/* R13: 2^(floor(log2 amax) - 8), clamped to E8M0's range. */
unsigned orc_shared_exponent_fp8(double amax)
{
    if (isnan(amax) || isinf(amax))
        return 0xFFu;
    int e;
    if (amax == 0.0) {
        e = -127;
    } else {
        int x;
        frexp(amax, &x);
        e = (x - 1) - 8;
    }
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return (unsigned)(e + 127);
}

void orc_mx8_quantize_block(const double v[32], uint8_t codes[32], uint8_t* scale)
{
    double amax = 0.0;
    int bad = 0;
    for (int i = 0; i < 32; ++i) {
        if (isnan(v[i]) || isinf(v[i]))
            bad = 1;
        else if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    }
    unsigned b = bad ? 0xFFu : orc_shared_exponent_fp8(amax);
    *scale = (uint8_t)b;
    if (b == 0xFFu) {
        memset(codes, 0, 32);
        return;
    }
    int e = (int)b - 127;
    for (int i = 0; i < 32; ++i)
        codes[i] = (uint8_t)orc_e4m3_encode(ldexp(v[i], -e));
}

void orc_quantize_act_fp8(const uint16_t* x, int64_t ldx, const int32_t* row_index,
                          int64_t M, int64_t K, uint8_t* codes, uint8_t* scales)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        int64_t src = row_index ? (int64_t)row_index[m] : m;
        const uint16_t* xr = x + src * ldx;
        double blk[32];
        for (int64_t j = 0; j < K / 32; ++j) {
            for (int i = 0; i < 32; ++i)
                blk[i] = orc_bf16_value(xr[32 * j + i]);
            orc_mx8_quantize_block(blk, codes + m * K + 32 * j, scales + m * (K / 32) + j);
        }
    }
}

/* R15: the products e4m3 * e2m1 are exact in fp64, as are their scaled sums
   within the GEMM's parity domain; summed in fp64 like orc_gemm. */
void orc_gemm_w4a8_at(const uint8_t* a_codes, const uint8_t* a_scales,
                      const uint8_t* b_codes, const uint8_t* b_scales,
                      int64_t M, int64_t N, int64_t K,
                      const int64_t* pm, const int64_t* pn, int64_t P,
                      double* y, double* s)
{
    (void)M;   /* positions are given; M only bounds them (checked by the caller) */
#pragma omp parallel
    {
        double* ad = (double*)malloc((size_t)K * sizeof(double));
        double* bd = (double*)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < P; ++i) {
            int64_t m = pm ? pm[i] : i / N;
            int64_t n = pn ? pn[i] : i % N;
            for (int64_t k = 0; k < K; ++k)
                ad[k] = orc_e4m3_value(a_codes[m * K + k]) *
                        orc_e8m0_value(a_scales[m * (K / 32) + k / 32]);
            mx_row(b_codes, b_scales, n, K, bd);
            double yy, ss;
            dot_row(ad, bd, K, &yy, &ss);
            y[i] = yy;
            if (s) s[i] = ss;
        }
        free(ad);
        free(bd);
    }
}

/* ---- MoE expert epilogues ----------------------------------------------- */

/* R10: silu(g) = g * sigma(g), sigma(g) = 1 / (1 + exp(-g)), times the up
   value, each operation rounded to fp32 (the oracle's exp is the C library's
   double exp rounded to fp32). */
float orc_silu_mul_f32(float g, float u)
{
    float e = (float)exp(-(double)g);
    float d = 1.0f + e;
    float r = 1.0f / d;
    float sg = g * r;
    return sg * u;
}

void orc_silu_mul(const uint16_t* gate_up, int64_t ldg, int64_t M, int64_t I,
                  uint16_t* h_bf16, float* h_f32)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* row = gate_up + m * ldg;
        for (int64_t i = 0; i < I; ++i) {
            float g = (float)orc_bf16_value(row[i]);
            float u = (float)orc_bf16_value(row[I + i]);
            float h = orc_silu_mul_f32(g, u);
            if (h_f32) h_f32[m * I + i] = h;
            if (h_bf16) h_bf16[m * I + i] = orc_bf16_from_float(h);
        }
    }
}

/* R10 then the activation quantization of the down projection's input. */
void orc_silu_mul_quantize(const uint16_t* gate_up, int64_t ldg, int64_t M, int64_t I,
                           int rule, uint8_t* codes, uint8_t* scales)
{
    uint16_t* h = malloc((size_t)(M * I > 0 ? M * I : 1) * sizeof(uint16_t));
    if (!h) abort();
    orc_silu_mul(gate_up, ldg, M, I, h, NULL);
    orc_quantize_act_rule(h, I, NULL, M, I, rule, codes, scales);
    free(h);
}

/* R11: each output element is a sum of topk exact fp64 products (a bf16
   value times an fp32 weight needs 32 significant bits), added in fp64. */
void orc_moe_combine(const uint16_t* y, int64_t ldy, const int32_t* rows, const float* w,
                     int64_t T, int64_t topk, int64_t H, double* out, double* s)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t n = 0; n < H; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t j = 0; j < topk; ++j) {
                double p = (double)w[t * topk + j] *
                           orc_bf16_value(y[(int64_t)rows[t * topk + j] * ldy + n]);
                acc += p;
                mag += fabs(p);
            }
            out[t * H + n] = acc;
            if (s) s[t * H + n] = mag;
        }
    }
}

/* R12: the row bias joins the exact sum before any rounding (one fp64 add of
   a bf16 value; its rounding error is far below the output's). */
void orc_add_row_bias(double* y, double* s, int64_t M, int64_t N, const uint16_t* bias)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double b = orc_bf16_value(bias[n]);
            y[m * N + n] += b;
            if (s) s[m * N + n] += fabs(b);
        }
    }
}

/* Elementwise helper for the tests: RNE of n doubles to bf16 bit patterns. */
void orc_bf16_from_double_array(const double* v, int64_t n, uint16_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_from_double(v[i]);
}

/* Threads the OpenMP loops use from now on (n >= 1); for timing the oracle
   on one core beside all of them. */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
