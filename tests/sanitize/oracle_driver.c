/* Host sanitizer run of the oracle (test infrastructure): every function of
 * oracle/mxfp4_oracle.h on small inputs in buffers of exactly the size its
 * contract names, built with AddressSanitizer and UndefinedBehaviorSanitizer
 * (no recovery), so that any out-of-bounds access, use after free or
 * undefined arithmetic aborts the run.  A few
 * results are checked against values fixed by the formats themselves. */
#include "mxfp4_oracle.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static int failures = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static uint64_t lcg_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
    lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(lcg_state >> 33);
}
static void* exact(size_t n) {           /* n may be 0: a 1-byte block, never read */
    void* p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}
static void fill(uint8_t* p, size_t n, unsigned lo, unsigned hi) {
    for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)(lo + rnd() % (hi - lo + 1));
}
static void fill_bf16(uint16_t* p, size_t n) {   /* finite values, |v| < 64 */
    for (size_t i = 0; i < n; ++i) p[i] = orc_bf16_from_double(((double)(rnd() % 20001) - 10000.0) / 160.0);
}

int main(void) {
    /* codecs: the E2M1 grid, E8M0 powers of two, E4M3 one and NaN */
    static const double grid[8] = {0, 0.5, 1, 1.5, 2, 3, 4, 6};
    for (unsigned c = 0; c < 16; ++c) CHECK(orc_e2m1_value(c) == (c & 8 ? -grid[c & 7] : grid[c & 7]));
    CHECK(orc_e8m0_value(127) == 1.0 && orc_e8m0_value(0) == ldexp(1.0, -127));
    CHECK(isnan(orc_e8m0_value(255)));
    CHECK(orc_e4m3_value(0x38) == 1.0 && isnan(orc_e4m3_value(0x7F)));
    for (unsigned b = 0; b < 256; ++b) (void)orc_e4m3_value(b);
    CHECK(orc_bf16_value(orc_bf16_from_double(1.5)) == 1.5 && orc_bf16_from_float(NAN) == 0x7FC0);
    CHECK(orc_e2m1_encode(6.0) == 7 && orc_e2m1_encode(-0.25) == 8);
    CHECK(orc_shared_exponent(6.0) == 127);            /* 6 = 1.5 * 2^2, E2M1's top binade */
    (void)orc_shared_exponent_uos(6.0);
    {
        const int64_t n = 65536;
        uint16_t* x = exact(n * 2);
        uint8_t* codes = exact(n);
        for (int64_t i = 0; i < n; ++i) x[i] = (uint16_t)i;
        orc_e2m1_encode_bf16_at_scale(x, n, 127, codes);
        CHECK(codes[0x3F80] == 2);               /* 1.0 at scale 1 */
        free(x), free(codes);
    }
    /* one block under both scale rules, and its error bound */
    {
        double v[32];
        uint8_t codes[16], scale;
        for (int i = 0; i < 32; ++i) v[i] = (i - 15.5) * 0.37;
        for (int rule = 0; rule < 2; ++rule) {
            orc_mx_quantize_block_rule(v, codes, &scale, rule);
            const double s = orc_e8m0_value(scale);
            for (int i = 0; i < 32; ++i) {
                const unsigned c = (codes[i / 2] >> (4 * (i % 2))) & 15;
                CHECK(fabs(orc_e2m1_value(c) * s - v[i]) <= 1.0 * s);
            }
        }
        orc_mx_quantize_block(v, codes, &scale);
    }
    /* NVFP4 dequant and requant, T = 2 tensors [3][64] */
    const int64_t T = 2, N = 3, K = 64;
    {
        uint8_t* nc = exact(T * N * K / 2);
        uint8_t* ns = exact(T * N * K / 16);
        float* g = exact(T * 4);
        float* out = exact(N * K * 4);
        uint8_t* mc = exact(T * N * K / 2);
        uint8_t* ms = exact(T * N * K / 32);
        fill(nc, T * N * K / 2, 0, 255);
        fill(ns, T * N * K / 16, 0x20, 0x50);
        g[0] = 0.75f, g[1] = 1.0f / 3.0f;
        for (int b = 0; b < 2; ++b) orc_nvfp4_dequant(nc, ns, g[0], N, K, b, out);
        for (int rule = 0; rule < 2; ++rule)
            for (int b = 0; b < 2; ++b) orc_requant_rule(nc, ns, g, T, N, K, b, rule, mc, ms);
        orc_requant(nc, ns, g, T, N, K, 0, mc, ms);
        free(nc), free(ns), free(g), free(out), free(mc), free(ms);
    }
    /* activations: 5 rows gathered from 7, ldx 80 > K */
    const int64_t M = 5, ldx = 80, rows = 7;
    uint16_t* x = exact(rows * ldx * 2);
    int32_t* ri = exact(M * 4);
    fill_bf16(x, rows * ldx);
    for (int i = 0; i < M; ++i) ri[i] = (int32_t)((i * 3) % rows);
    uint8_t* ac = exact(M * K / 2);
    uint8_t* as = exact(M * K / 32);
    orc_quantize_act(x, ldx, ri, M, K, ac, as);
    orc_quantize_act_rule(x, ldx, NULL, M, K, ORC_RULE_UOS, ac, as);
    orc_quantize_act(x, ldx, NULL, M, K, ac, as);
    /* GEMM three ways: whole, sampled, grouped (every expert the same B) */
    const int64_t Nb = 6, E = 3;
    uint8_t* bc = exact(E * Nb * K / 2);
    uint8_t* bs = exact(E * Nb * K / 32);
    fill(bc, Nb * K / 2, 0, 255);
    fill(bs, Nb * K / 32, 120, 132);
    for (int e = 1; e < E; ++e) {
        memcpy(bc + e * Nb * K / 2, bc, Nb * K / 2);
        memcpy(bs + e * Nb * K / 32, bs, Nb * K / 32);
    }
    double* y = exact(M * Nb * 8);
    double* s = exact(M * Nb * 8);
    double* yg = exact(M * Nb * 8);
    orc_gemm(ac, as, bc, bs, M, Nb, K, y, s);
    orc_gemm(ac, as, bc, bs, M, Nb, K, NULL, NULL);
    int64_t pm[4] = {0, 4, 2, 3}, pn[4] = {5, 0, 3, 3};
    double ya[4], sa[4];
    orc_gemm_at(ac, as, bc, bs, M, Nb, K, pm, pn, 4, ya, sa);
    for (int p = 0; p < 4; ++p) CHECK(fabs(ya[p] - y[pm[p] * Nb + pn[p]]) <= 1e-12 * (1 + sa[p]));
    int32_t off[4] = {0, 2, 2, 5};
    orc_grouped_gemm(ac, as, bc, bs, off, E, Nb, K, yg, NULL);
    for (int i = 0; i < M * Nb; ++i) CHECK(fabs(yg[i] - y[i]) <= 1e-12 * (1 + s[i]));
    uint16_t* bias = exact(Nb * 2);
    fill_bf16(bias, Nb);
    orc_add_row_bias(y, s, M, Nb, bias);
    orc_add_row_bias(y, NULL, M, Nb, bias);
    uint16_t* yb = exact(M * Nb * 2);
    orc_bf16_from_double_array(y, M * Nb, yb);
    /* Smooth pre-scale, W4A8 */
    uint16_t* sm = exact(K * 2);
    uint16_t* xs = exact(M * K * 2);
    fill_bf16(sm, K);
    orc_smooth_rows(x, ldx, ri, sm, M, K, xs);
    orc_smooth_rows(x, ldx, NULL, sm, M, K, xs);
    CHECK(orc_e4m3_encode(1.0) == 0x38);
    (void)orc_shared_exponent_fp8(448.0);
    {
        double v[32];
        uint8_t c8[32], sc;
        for (int i = 0; i < 32; ++i) v[i] = (i - 16) * 13.0;
        orc_mx8_quantize_block(v, c8, &sc);
    }
    uint8_t* a8 = exact(M * K);
    orc_quantize_act_fp8(x, ldx, ri, M, K, a8, as);
    double* y8 = exact(M * Nb * 8);
    orc_gemm_w4a8_at(a8, as, bc, bs, M, Nb, K, NULL, NULL, M * Nb, y8, NULL);
    orc_gemm_w4a8_at(a8, as, bc, bs, M, Nb, K, pm, pn, 4, ya, sa);
    for (int p = 0; p < 4; ++p) CHECK(ya[p] == y8[pm[p] * Nb + pn[p]]);
    /* the MoE epilogues: gate_up [3][ldg 136], I = 64; combine T=3, topk=2 */
    const int64_t I = 64, ldg = 136, Mg = 3;
    uint16_t* gu = exact(Mg * ldg * 2);
    fill_bf16(gu, Mg * ldg);
    uint16_t* h = exact(Mg * I * 2);
    float* hf = exact(Mg * I * 4);
    orc_silu_mul(gu, ldg, Mg, I, h, hf);
    orc_silu_mul(gu, ldg, Mg, I, NULL, hf);
    uint8_t* hc = exact(Mg * I / 2);
    uint8_t* hs = exact(Mg * I / 32);
    orc_silu_mul_quantize(gu, ldg, Mg, I, ORC_RULE_OCP, hc, hs);
    orc_silu_mul_quantize(gu, ldg, Mg, I, ORC_RULE_UOS, hc, hs);
    CHECK(orc_silu_mul_f32(0.0f, 5.0f) == 0.0f);
    const int64_t Tk = 3, topk = 2, H = 16, ldy = 24, R = 6;
    uint16_t* ym = exact(R * ldy * 2);
    fill_bf16(ym, R * ldy);
    int32_t* rw = exact(Tk * topk * 4);
    float* wt = exact(Tk * topk * 4);
    for (int i = 0; i < Tk * topk; ++i) rw[i] = (int32_t)(R - 1 - i), wt[i] = 0.25f * (float)(i + 1);
    double* co = exact(Tk * H * 8);
    double* cs = exact(Tk * H * 8);
    orc_moe_combine(ym, ldy, rw, wt, Tk, topk, H, co, cs);
    orc_moe_combine(ym, ldy, rw, wt, Tk, topk, H, co, NULL);
    CHECK(co[0] == 0.25 * orc_bf16_value(ym[rw[0] * ldy]) + 0.5 * orc_bf16_value(ym[rw[1] * ldy]));
    /* threads */
    orc_set_num_threads(2);
    CHECK(orc_num_threads() == 2);
    orc_gemm(ac, as, bc, bs, M, Nb, K, y, s);
    /* empty shapes */
    orc_gemm(ac, as, bc, bs, 0, Nb, K, y, s);
    orc_quantize_act(x, ldx, NULL, 0, K, ac, as);
    int32_t off0[4] = {0, 0, 0, 0};
    orc_grouped_gemm(ac, as, bc, bs, off0, E, Nb, K, yg, NULL);
    free(x), free(ri), free(ac), free(as), free(bc), free(bs), free(y), free(s), free(yg);
    free(bias), free(yb), free(sm), free(xs), free(a8), free(y8), free(gu), free(h), free(hf);
    free(hc), free(hs), free(ym), free(rw), free(wt), free(co), free(cs);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run ok\n");
    return 0;
}
