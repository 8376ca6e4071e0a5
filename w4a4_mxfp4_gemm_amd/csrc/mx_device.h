// mx_device.h -- gfx950 device helpers for E2M1 / E4M3 / E8M0 / bf16 codes.
//
// Everything here is integer or exactly-rounded fp32 work, so results do not
// depend on FMA contraction or the order of evaluation.  fp32 denormals are
// kept (the kernels are built with the default IEEE denormal mode).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// bf16 bit pattern (low 16 bits of b) -> fp32, exact.
__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 -> packed bf16 (RNE), a in the low half: one v_cvt_pk_bf16_f32.
// (Two scalar casts compile to two of them, each with a zero partner, plus a
// shift and an OR.)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
    typedef float f32x2_v __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{a, b}, bf16x2_v));
}

// float8_e4m3fn byte -> fp32 (exact): bias 7, exponent field 0 subnormal,
// S.1111.111 NaN, no infinities.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    uint32_t e = (b >> 3) & 15u, m = b & 7u;
    float mag;
    if (e == 0) mag = (float)m * 0.001953125f;                 // m * 2^-9
    else mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
    if (e == 15u && m == 7u) mag = __uint_as_float(0x7FC00000u);
    return (b & 0x80u) ? -mag : mag;
}

// E2M1 code (low 4 bits) -> fp32 (exact).
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
    uint32_t e = (c >> 1) & 3u, m = c & 1u;
    float mag = e ? __uint_as_float(((e + 126u) << 23) | (m << 22)) : 0.5f * (float)m;
    return (c & 8u) ? -mag : mag;
}

// OCP MX shared-exponent byte from the fp32 bit pattern of a block's amax
// (sign bit clear).  floor(log2 amax) - 2 + 127 is the biased exponent field
// minus 2, clamped at 0; NaN or Inf anywhere in the block gives 0xFF.
__device__ __forceinline__ uint32_t mx_scale_from_amax_bits(uint32_t amax_bits) {
    uint32_t E = amax_bits >> 23;
    if (E >= 255u) return 255u;
    return E >= 2u ? E - 2u : 0u;
}

// UOS shared-exponent byte (the single-scale setting with Qmax = 7.25): the
// smallest e with amax <= 7.25 * 2^e.  With amax = f * 2^p (f in [1, 2)),
// amax / 2^(p-2) = 4f is at most 7.25 exactly when f <= 1.8125, so this is the
// OCP byte plus one when the fraction bits exceed 0x680000, clamped at 0 the
// same way (subnormal amax included).  NaN or Inf gives 0xFF.
__device__ __forceinline__ uint32_t mx_scale_uos_from_amax_bits(uint32_t amax_bits) {
    const uint32_t E = amax_bits >> 23;
    if (E >= 255u) return 255u;
    const uint32_t e = E + ((amax_bits & 0x7FFFFFu) > 0x680000u ? 1u : 0u);
    return e >= 2u ? e - 2u : 0u;
}

template <bool UOS>
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits) {
    return UOS ? mx_scale_uos_from_amax_bits(amax_bits) : mx_scale_from_amax_bits(amax_bits);
}

// E2M1 magnitude code (0..7) of q >= 0: the nearest of {0, .5, 1, 1.5, 2, 3,
// 4, 6}, exact half-way points going to the even code, anything past 5
// saturating to 6.  Each term counts one decision threshold: strict '>' where
// the tie belongs to the lower (even) neighbour, '>=' where it belongs to the
// upper one.
__device__ __forceinline__ uint32_t e2m1_mag_rne(float q) {
    return (uint32_t)(q > 0.25f) + (uint32_t)(q >= 0.75f) + (uint32_t)(q > 1.25f) +
           (uint32_t)(q >= 1.75f) + (uint32_t)(q > 2.5f) + (uint32_t)(q >= 3.5f) +
           (uint32_t)(q > 5.0f);
}

// E2M1 code of v under the block scale 2^(byte-127) (byte != 0xFF).
// v * 2^(127-byte) is exact whenever it is at least 2^-126; smaller results
// round to code 0 either way.  The sign bit of v is kept.
__device__ __forceinline__ uint32_t e2m1_encode(float v, int neg_exp) {
    float q = __builtin_amdgcn_ldexpf(__builtin_fabsf(v), neg_exp);
    return e2m1_mag_rne(q) | ((__float_as_uint(v) >> 28) & 8u);
}

// E8M0 byte (0..254) -> its scale 2^(byte-127) as fp32.  Byte 0 is the fp32
// subnormal 2^-127.
__device__ __forceinline__ float e8m0_to_f32(uint32_t byte) {
    return __uint_as_float(byte ? byte << 23 : 0x00400000u);
}

// gfx950 v_cvt_scalef32_pk_fp4_*: two values divided by the scale, rounded to
// the nearest E2M1 code (ties to the even code), saturated at +-6, sign of
// zero kept, written into byte SEL of OLD.  For scale = 2^(byte-127) with any
// byte 0..254 this is bit-identical to e2m1_encode on every finite input
// whose quotient stays below 8 -- checked exhaustively on the hardware for
// all such fp32 and bf16 inputs.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float a, float b, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Same for a packed pair of bf16 values (low half -> low nibble).
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2_bf16(uint32_t old, uint32_t pair, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, __builtin_bit_cast(bf16x2_t, pair),
                                                     scale, SEL);
}

// The expert activation h = bf16(silu(gate) * up) of an MoE layer, shared by
// the act-quant kernel's GLU mode and the grouped GEMM's fused epilogue.
// e^-g to within about 2 ulp in seven operations: e^x = 2^(x log2 e), with
// the product split into ph = fl(x * L) and its rounding error pl (recovered
// exactly by an fma, plus the part of log2 e below fp32), so that
// 2^(ph + pl) = exp2(ph) * (1 + pl ln 2) to second order in pl (|pl| < 2^-17).
// x is clamped to [-104, 89], beyond which e^x is 0 or Inf in fp32 anyway, to
// keep pl meaningful; a NaN g gives some finite value here, and NaN in the
// caller's g * r.
__device__ __forceinline__ float exp_neg(float g) {
    constexpr float LOG2E_HI = 1.44269502162933349609375f;      // fp32(log2 e)
    constexpr float LOG2E_LO = 1.925963033500011e-08f;          // log2 e - LOG2E_HI
    constexpr float LN2 = 0.693147180559945309f;
    const float x = __builtin_amdgcn_fmed3f(-g, -104.0f, 89.0f);
    const float ph = x * LOG2E_HI;
    const float pl = __builtin_fmaf(x, LOG2E_LO, __builtin_fmaf(x, LOG2E_HI, -ph));
    return __builtin_amdgcn_exp2f(ph) * __builtin_fmaf(pl, LN2, 1.0f);
}

// silu(g) * u for the two bf16 pairs packed in gw / uw, rounded to bf16 (RNE),
// packed the same way.  fp32 steps: e = exp(-g), d = 1 + e, r = 1/d (v_rcp,
// 1 ulp), s = g * r, h = s * u; d >= 1 or Inf, so the reciprocal never sees
// a denormal, and g = -Inf gives -Inf * 0 = NaN.
__device__ __forceinline__ uint32_t glu_pair(uint32_t gw, uint32_t uw) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const float g[2] = {__uint_as_float(gw << 16), __uint_as_float(gw & 0xFFFF0000u)};
    const float u[2] = {__uint_as_float(uw << 16), __uint_as_float(uw & 0xFFFF0000u)};
    float h[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float d = 1.0f + exp_neg(g[i]);
        h[i] = (g[i] * __builtin_amdgcn_rcpf(d)) * u[i];
    }
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{h[0], h[1]}, bf16x2_t));
}

// One whole 32-element MX block of bf16 values held by one lane (16 packed
// pairs, element 2i in the low half of w[i]) -> its E8M0 byte and 16 code
// bytes (element 2i in the low nibble of byte i).  The activation rule: amax
// over the bf16 magnitudes (compared as integers, so NaN and Inf patterns
// rank above every finite value), the OCP MX exponent, each value divided by
// the scale and rounded to E2M1; a NaN or Inf block gives 0xFF and zero codes.
// UOS: the Qmax = 7.25 exponent rule instead of the OCP one.
template <bool UOS = false>
__device__ __forceinline__ uint32_t quant_block32_bf16(const uint32_t (&w)[16], uint32_t (&c)[4]) {
    typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
    u16x2_t a = __builtin_bit_cast(u16x2_t, w[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int i = 1; i < 16; ++i)
        a = __builtin_elementwise_max(a, __builtin_bit_cast(u16x2_t, w[i] & 0x7FFF7FFFu));
    const uint32_t amax = a[0] > a[1] ? a[0] : a[1];
    const uint32_t byte = mx_scale_byte<UOS>(amax << 16);
    const float scale = e8m0_to_f32(byte);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t v = cvt_fp4x2_bf16<0>(0u, w[4 * d], scale);
        v = cvt_fp4x2_bf16<1>(v, w[4 * d + 1], scale);
        v = cvt_fp4x2_bf16<2>(v, w[4 * d + 2], scale);
        v = cvt_fp4x2_bf16<3>(v, w[4 * d + 3], scale);
        c[d] = byte == 255u ? 0u : v;
    }
    return byte;
}

// E4M3 codes of four packed bf16 pairs under scale byte `byte` (< 255), 8
// bytes, element 2i+h in byte 2i+h.  gfx950's v_cvt_scalef32_pk_fp8_bf16
// divides by the scale and rounds to the nearest E4M3 value (ties to even,
// subnormals included) but turns quotients of 464 and more into the NaN code
// instead of saturating -- measured against the nearest-value encoder over
// every bf16 magnitude and scale byte.  So each magnitude is first clamped to
// 448 * 2^(byte-127), whose bf16 pattern is exponent field byte + 8 with
// mantissa 0x60 (448 = 1.75 * 2^8); quotients up to 464 round to 448 anyway.
__device__ __forceinline__ uint2 e4m3_codes8(const uint32_t (&w)[4], uint32_t byte) {
    typedef short s16x2_t __attribute__((ext_vector_type(2)));
    const uint32_t lim = ((byte + 8u) << 7) | 0x60u;
    typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
    const u16x2_t limv = {(unsigned short)lim, (unsigned short)lim};
    const float scale = e8m0_to_f32(byte);
    auto clamp = [&](uint32_t x) {
        const u16x2_t mag =
            __builtin_elementwise_min(__builtin_bit_cast(u16x2_t, x & 0x7FFF7FFFu), limv);
        return __builtin_bit_cast(bf16x2_t, __builtin_bit_cast(uint32_t, mag) | (x & 0x80008000u));
    };
    uint32_t out[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        s16x2_t v = {0, 0};
        v = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(v, clamp(w[2 * i]), scale, false);
        v = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(v, clamp(w[2 * i + 1]), scale, true);
        out[i] = __builtin_bit_cast(uint32_t, v);
    }
    return make_uint2(out[0], out[1]);
}

// MXFP8 (E4M3) scale byte of a block whose bf16 magnitude maximum has bits
// `amax` (16-bit pattern): the exponent field E minus 8 (448 = 1.75 * 2^8),
// clamped at 0; 0xFF for NaN or Inf.
__device__ __forceinline__ uint32_t mx8_scale_from_bf16_amax(uint32_t amax) {
    const uint32_t E = amax >> 7;
    return E >= 255u ? 255u : (E > 8u ? E - 8u : 0u);
}

// Byte permute (v_perm_b32): selector byte k in 0..3 picks byte k of lo,
// 4..7 picks byte k-4 of hi.
__device__ __forceinline__ uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Max over the 4 lanes of an aligned quad (DPP quad permutations).
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
    uint32_t x = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
    v = v > x ? v : x;
    x = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);           // [2,3,0,1]
    return v > x ? v : x;
}

}  // namespace mx
