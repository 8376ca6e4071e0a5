/*
 * mxfp4_oracle.h -- plain, slow, obviously-correct CPU oracle for the
 * block-scaled 4-bit (E2M1) linear-layer path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this library: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no code, header, table or
 * constant generator with the HIP library.
 *
 * All arithmetic that is not exact integer work is carried out in fp64 (or,
 * where the method itself fixes fp32, in IEEE fp32 with contraction off).
 * Every function names the passage of the source pages it follows:
 *
 *   [P1] AMD blog "Efficiently Serving NVFP4 Models on AMD Instinct
 *        MI350X/MI355X Accelerators via Online NVFP4 to Quark MXFP4
 *        Requantization" -- introduction (NVFP4 = packed E2M1 + FP8 per-block
 *        scale + FP32 per-tensor scale), the pipeline section under Figure 1
 *        (dequantize one layer, quantize to MXFP4, write into a preallocated
 *        destination), and the closing list (dynamic per-batch activation
 *        quantization; both GEMM operands MXFP4 on the scaled MFMA).
 *   [P2] vLLM-Omni user guide "W4A4 MXFP4 Quantization" -- Overview (OCP MX:
 *        32 K-elements share one float8_e8m0fnu exponent, E2M1 packed two per
 *        byte), "mxfp4 -- Single-Scale Block Scaling (OCP / UOS)" (setting 0 =
 *        OCP MX, axis=-1, block_size=32, round_mode="rint", E2M1 max 6),
 *        "Validation and Notes" item 4 (scale bytes are raw E8M0 bytes).
 *   [P3] SGLang FP4 post ("[SGLang] FP4 ..."), sections 3-4: NVFP4 weight
 *        layout weight_packed [N, K/2] u8, weight_scale [N, K/16]
 *        float8_e4m3fn, fp32 global scale.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   R1 nibble order: element 2j in bits 3:0 of byte j, element 2j+1 in 7:4.
 *   R2 NVFP4 value = fl32( fl32(e2m1 * e4m3) * g ), g multiplies on dequant.
 *      The requant's materialised intermediate is fp32 unless the caller asks
 *      for bf16 (RNE of that fp32 value).
 *   R3 shared exponent (OCP MX): e = floor(log2(amax)) - 2, clamped to
 *      [-127, 127]; byte = e + 127.  amax NaN/Inf -> byte 0xFF, codes 0.
 *   R4 element encode: round-half-to-even onto the E2M1 grid, saturating at
 *      +-6, sign bit copied from the input (so -0.1 * 2^e encodes as 0x8).
 *   R5 GEMM output: fp64 sum of exact products, rounded once (RNE) to the
 *      output type.
 *   R9 shared exponent, UOS variant (vLLM-Omni guide, "Single-Scale Block
 *      Scaling", setting 2, Qmax = 7.25): e = ceil(log2(amax / 7.25)), i.e.
 *      the smallest e with amax <= 7.25 * 2^e, clamped to [-127, 127];
 *      elements are encoded as in R4 (still saturating at 6).
 *   R10 expert activation between the two grouped GEMMs ([P1] closing list:
 *      the MoE experts run as fused-MoE kernels; the expert weights are a
 *      gate/up pair and a down projection): the gate_up output row holds the
 *      gate half in columns [0, I) and the up half in [I, 2I); the down
 *      projection's input is h = bf16(silu(gate) * up), quantized like any
 *      activation (R3/R9 + R4).  The value decides quantized codes, so it is
 *      computed in the kernel's precision, fp32 with every step rounded once:
 *      e = fl32(exp(-g)), d = fl32(1 + e), r = fl32(1 / d), s = fl32(g * r),
 *      h = fl32(s * u).  A GPU exp or reciprocal that is not correctly
 *      rounded can move h by a few fp32 ulps, so where h lies that close to
 *      a bf16 rounding midpoint either neighbour is a correct result.
 *   R13 W4A8 activations ([P2] "W4A8 fallback": MXFP8 activations,
 *      float8_e4m3fn with scale_alg=0, the same block-32 grouping and "rint"
 *      rounding, no UOS; the weights stay the MXFP4 ones): the OCP MX shared
 *      exponent for E4M3 elements is e = floor(log2 amax) - 8 (8 is the
 *      exponent of E4M3's largest binade, 448 = 1.75 * 2^8), clamped to
 *      [-127, 127]; a NaN/Inf block gets byte 0xFF and all-zero codes.
 *   R14 E4M3 element encode: the float8_e4m3fn value nearest to q = v / 2^e,
 *      ties to the even code, saturating at +-448 (beyond it 448 is nearest;
 *      the NaN code 0x7F is never produced), sign bit copied.  Codes are one
 *      byte per element, row-major [M][K].
 *   R15 W4A8 GEMM: y[m][n] = sum_k A[m,k] * B[n,k] with A = e4m3 * 2^(sa-127)
 *      and B = e2m1 * 2^(sb-127), exact, rounded once (as R5), plus the
 *      optional row bias (R12) ([P2]: the mixed FP8/FP4 GEMM gives bf16
 *      output with a bf16 row bias).
 *   R17 Smooth pre-scale ([P2] pre-quantized single-scale weights: both
 *      W4A4 and W4A8 quantize x * mul_scale, the per-input-channel Smooth
 *      tensor converted to the activation dtype): the quantized values are
 *      h_k = bf16(fl32(x_k * s_k)) with s = the bf16 Smooth vector [K] (a
 *      product of two bf16 values is exact in fp32 except in fp32's
 *      subnormal range), then quantized as R3/R9 + R4 or R13 + R14.
 *   R12 row bias ([P3] NVFP4 apply_weights: the GEMM output plus an optional
 *      bias; [P2] W4A8 notes: bf16 output with a matching bf16 row bias): y
 *      gains bias[n] on every row, one bias per weight row (output column),
 *      added to the exact sum before the single rounding to the output type.
 *   R11 top-k combine ([P1] closing list, MoE experts): each token's output
 *      row is the sum over its k routed rows of weight * expert output row,
 *      computed exactly (fp64) and rounded once to the output type.  The
 *      weights and the token -> sorted-row map are inputs.
 */
#ifndef MXFP4_ORACLE_H
#define MXFP4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- scalar codecs ---------------------------------------------------- */
double   orc_e2m1_value(unsigned code);          /* code in [0,15]          */
double   orc_e4m3_value(unsigned byte);          /* float8_e4m3fn           */
double   orc_e8m0_value(unsigned byte);          /* float8_e8m0fnu          */
double   orc_bf16_value(uint16_t bits);
uint16_t orc_bf16_from_double(double v);         /* RNE, NaN -> 0x7FC0      */
uint16_t orc_bf16_from_float(float v);           /* RNE, NaN -> 0x7FC0      */
unsigned orc_e2m1_encode(double q);              /* R4                      */
/* R4 at one scale byte over n bf16 values (the block quantizer's element
   step); NaN/Inf inputs give 0. */
void     orc_e2m1_encode_bf16_at_scale(const uint16_t* x, int64_t n, unsigned byte,
                                       uint8_t* codes);
unsigned orc_shared_exponent(double amax);       /* R3, amax >= 0 or NaN    */
unsigned orc_shared_exponent_uos(double amax);   /* R9, amax >= 0 or NaN    */

/* Scale rule of the _rule variants below: R3 (OCP MX) or R9 (UOS). */
enum { ORC_RULE_OCP = 0, ORC_RULE_UOS = 1 };

/* ---- MX quantization of one 32-element block (R3 + R4) ---------------- */
void orc_mx_quantize_block(const double v[32], uint8_t codes[16], uint8_t* scale);
void orc_mx_quantize_block_rule(const double v[32], uint8_t codes[16], uint8_t* scale,
                                int rule);

/* ---- NVFP4 dequantization of one tensor into fp32 (R2) ---------------- */
void orc_nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, float g,
                       int64_t N, int64_t K, int bf16_intermediate, float* out);

/* ---- the four operations of the path ---------------------------------- */
/* NVFP4 -> MXFP4 requant of T same-shape tensors [T][N][K]. */
void orc_requant(const uint8_t* nv_codes, const uint8_t* nv_scales,
                 const float* nv_global, int64_t T, int64_t N, int64_t K,
                 int bf16_intermediate, uint8_t* mx_codes, uint8_t* mx_scales);
void orc_requant_rule(const uint8_t* nv_codes, const uint8_t* nv_scales,
                      const float* nv_global, int64_t T, int64_t N, int64_t K,
                      int bf16_intermediate, int rule, uint8_t* mx_codes,
                      uint8_t* mx_scales);

/* bf16 [*, ldx] -> MXFP4 codes [M][K/2] + E8M0 [M][K/32]; optional gather. */
void orc_quantize_act(const uint16_t* x, int64_t ldx, const int32_t* row_index,
                      int64_t M, int64_t K, uint8_t* codes, uint8_t* scales);
void orc_quantize_act_rule(const uint16_t* x, int64_t ldx, const int32_t* row_index,
                           int64_t M, int64_t K, int rule, uint8_t* codes,
                           uint8_t* scales);

/* y[m][n] = sum_k A[m,k] * B[n,k] over dequantized MXFP4 (fp64), and
   s[m][n] = sum_k |A[m,k] * B[n,k]|.  Either output may be NULL. */
void orc_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
              const uint8_t* b_codes, const uint8_t* b_scales,
              int64_t M, int64_t N, int64_t K, double* y, double* s);

/* The same quantities at P sampled (m, n) positions only. */
void orc_gemm_at(const uint8_t* a_codes, const uint8_t* a_scales,
                 const uint8_t* b_codes, const uint8_t* b_scales,
                 int64_t M, int64_t N, int64_t K,
                 const int64_t* pm, const int64_t* pn, int64_t P,
                 double* y, double* s);

/* Per expert e, rows [off[e], off[e+1]) times expert e's weights. */
void orc_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                      const uint8_t* b_codes, const uint8_t* b_scales,
                      const int32_t* offsets, int64_t E, int64_t N, int64_t K,
                      double* y, double* s);

/* ---- Smooth pre-scale (R17) ---------------------------------------------- */
/* x bf16 [*][ldx] (optional gather) times the bf16 Smooth vector [K], each
   product rounded to fp32 then to bf16: out bf16 [M][K]. */
void orc_smooth_rows(const uint16_t* x, int64_t ldx, const int32_t* row_index,
                     const uint16_t* smooth, int64_t M, int64_t K, uint16_t* out);

/* ---- W4A8: MXFP8 (E4M3) activations x MXFP4 weights (R13-R15) --------- */
unsigned orc_e4m3_encode(double q);              /* R14: float8_e4m3fn byte  */
unsigned orc_shared_exponent_fp8(double amax);   /* R13                      */

/* R13 + R14 on one block of 32 values: 32 code bytes and the scale byte. */
void orc_mx8_quantize_block(const double v[32], uint8_t codes[32], uint8_t* scale);

/* bf16 [*, ldx] -> MXFP8 codes [M][K] (one byte each) + E8M0 [M][K/32];
   optional gather as orc_quantize_act. */
void orc_quantize_act_fp8(const uint16_t* x, int64_t ldx, const int32_t* row_index,
                          int64_t M, int64_t K, uint8_t* codes, uint8_t* scales);

/* R15 at P sampled (m, n) positions (P = M*N with pm/pn NULL gives the whole
   [M][N] result, row-major): A is MXFP8 [M][K] + [M][K/32], B is MXFP4
   [N][K/2] + [N][K/32].  y and s as for orc_gemm. */
void orc_gemm_w4a8_at(const uint8_t* a_codes, const uint8_t* a_scales,
                      const uint8_t* b_codes, const uint8_t* b_scales,
                      int64_t M, int64_t N, int64_t K,
                      const int64_t* pm, const int64_t* pn, int64_t P,
                      double* y, double* s);

/* ---- MoE expert epilogues (R10, R11) ---------------------------------- */
/* silu(g) * u in fp32, every step rounded once (R10). */
float orc_silu_mul_f32(float g, float u);

/* gate_up bf16 [M][ldg] -> h = bf16(silu(gate) * up) [M][I] (h_bf16) and the
   fp32 value before that rounding (h_f32); either output may be NULL. */
void orc_silu_mul(const uint16_t* gate_up, int64_t ldg, int64_t M, int64_t I,
                  uint16_t* h_bf16, float* h_f32);

/* h as above, then quantized by orc_quantize_act_rule: codes [M][I/2],
   E8M0 [M][I/32]. */
void orc_silu_mul_quantize(const uint16_t* gate_up, int64_t ldg, int64_t M, int64_t I,
                           int rule, uint8_t* codes, uint8_t* scales);

/* out[t][n] = sum_{j<topk} w[t*topk+j] * y[rows[t*topk+j]][n] (fp64) and
   s[t][n] = sum_j |w * y| (R11); y is bf16 [*][ldy]; s may be NULL. */
void orc_moe_combine(const uint16_t* y, int64_t ldy, const int32_t* rows, const float* w,
                     int64_t T, int64_t topk, int64_t H, double* out, double* s);

/* R12: y[m][n] += bf16 bias[n] and s[m][n] += |bias[n]| (s may be NULL), over
   an [M][N] result of orc_gemm. */
void orc_add_row_bias(double* y, double* s, int64_t M, int64_t N, const uint16_t* bias);

void orc_bf16_from_double_array(const double* v, int64_t n, uint16_t* out);
int  orc_num_threads(void);
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
