// quant_kernels.hip -- NVFP4 -> MXFP4 requant and bf16 -> MXFP4 activation
// quantization for gfx950.
//
// Both are streaming kernels bound by HBM bandwidth: every byte is read once
// with 16-byte loads that are contiguous across a wavefront and written once
// with contiguous stores.  No LDS, no atomics.  The E2M1 rounding itself is
// done by gfx950's scaled FP4 converter (two values per instruction), which
// matches the exact round-half-to-even rule of the OCP MX format.
#include "mx_device.h"
#include "launch.h"

namespace mx {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Activation quantization.  One thread owns 8 consecutive bf16 values of a
// row (one 16-byte load); the 4 lanes of an aligned quad own one 32-element
// MX block and share its amax through DPP.  Threads along x walk one row's K,
// so a wavefront reads 1 KiB of a row contiguously; blockIdx.y walks rows,
// ROWS rows per thread per pass with every load issued before any math.
// ---------------------------------------------------------------------------
// NT_OUT: codes and scales stored non-temporally (outputs too large to stay
// cached for the GEMM that reads them next).
//
// GLU: x is an MoE expert's gate_up output, gate in columns [0, K) and up in
// [K, 2K) of each row (row_index unused), and the values quantized are
// h = bf16(silu(gate) * up), the down projection's input (glu_pair).

// Two packed bf16 values times two packed bf16 Smooth factors, each product in
// fp32 rounded to bf16 (RNE), packed the same way.
__device__ __forceinline__ uint32_t smooth_pair(uint32_t xw, uint32_t sw) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const float p0 = __uint_as_float(xw << 16) * __uint_as_float(sw << 16);
    const float p1 = __uint_as_float(xw & 0xFFFF0000u) * __uint_as_float(sw & 0xFFFF0000u);
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{p0, p1}, bf16x2_t));
}

// SMOOTH: the values quantized are bf16(x * smooth[k]) (smooth: bf16 [K], the
// per-channel Smooth pre-scale), each product in fp32 (exact for two bf16
// values outside fp32's subnormal range) rounded to bf16.
// SCATTER: row m of x is quantized once and its codes and scale bytes are
// written to output rows dest[m * fan + j], j < fan, each clamped to [0, R)
// (the MoE dispatch: a token's row to each of its routed expert rows).
template <int ROWS, bool NT_OUT, bool UOS, bool GLU = false, bool SMOOTH = false,
          bool SCATTER = false>
__global__ __launch_bounds__(256) void act_quant_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const int32_t* __restrict__ row_index,
    int64_t M, int64_t K, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ smooth, const int32_t* __restrict__ dest = nullptr,
    int fan = 0, int64_t R = 0) {
    const int64_t chunks = K / 8;                     // 16-byte chunks per row; multiple of 4
    const int64_t kq = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (kq >= chunks) return;                         // whole quads leave together
    uint4 sm = make_uint4(0, 0, 0, 0);
    if constexpr (SMOOTH) sm = *reinterpret_cast<const uint4*>(smooth + kq * 8);
    for (int64_t m0 = (int64_t)blockIdx.y * ROWS; m0 < M; m0 += (int64_t)gridDim.y * ROWS) {
        uint4 raw[ROWS];
        uint4 up[GLU ? ROWS : 1];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const int64_t m = m0 + r;
            if (m < M) {
                const int64_t src = row_index ? (int64_t)row_index[m] : m;
                const uint16_t* p = x + src * ldx + kq * 8;
                if constexpr (GLU) {
                    // gate and up, both read once
                    const v4u_t c = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(p));
                    const v4u_t d =
                        __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(p + K));
                    raw[r] = make_uint4(c[0], c[1], c[2], c[3]);
                    up[r] = make_uint4(d[0], d[1], d[2], d[3]);
                } else if (row_index) {
                    // a gather reads rows several times: keep them cached
                    raw[r] = *reinterpret_cast<const uint4*>(p);
                } else {
                    // each row read once: stream it past the Infinity Cache
                    // (with the GEMMs' non-temporal Y, the prefill step 10% faster)
                    const v4u_t c = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(p));
                    raw[r] = make_uint4(c[0], c[1], c[2], c[3]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const int64_t m = m0 + r;
            if (m >= M) break;                        // uniform across the workgroup
            uint32_t w[4] = {raw[r].x, raw[r].y, raw[r].z, raw[r].w};
            if constexpr (GLU) {
                const uint32_t uv[4] = {up[r].x, up[r].y, up[r].z, up[r].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = glu_pair(w[i], uv[i]);
            }
            if constexpr (SMOOTH) {
                const uint32_t sv[4] = {sm.x, sm.y, sm.z, sm.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = smooth_pair(w[i], sv[i]);
            }
            // amax over the 8 values as bf16 magnitudes (monotone as integers;
            // NaN and Inf patterns sort above every finite value).
            u16x2 a = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
            for (int i = 1; i < 4; ++i)
                a = __builtin_elementwise_max(a, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
            const uint32_t amax = quad_max_u32(max((uint32_t)a[0], (uint32_t)a[1]));
            const uint32_t byte = mx_scale_byte<UOS>(amax << 16);
            const float scale = e8m0_to_f32(byte);
            uint32_t packed = cvt_fp4x2_bf16<0>(0u, w[0], scale);
            packed = cvt_fp4x2_bf16<1>(packed, w[1], scale);
            packed = cvt_fp4x2_bf16<2>(packed, w[2], scale);
            packed = cvt_fp4x2_bf16<3>(packed, w[3], scale);
            if (byte == 255u) packed = 0u;            // NaN/Inf block: codes are zero
            if constexpr (SCATTER) {
                for (int j = 0; j < fan; ++j) {
                    int64_t d = dest[m * fan + j];
                    d = d < 0 ? 0 : (d >= R ? R - 1 : d);
                    *reinterpret_cast<uint32_t*>(codes + d * (K / 2) + kq * 4) = packed;
                    if ((kq & 3) == 0) scales[d * (K / 32) + kq / 4] = (uint8_t)byte;
                }
                continue;
            }
            uint32_t* cdst = reinterpret_cast<uint32_t*>(codes + m * (K / 2) + kq * 4);
            uint8_t* sdst = scales + m * (K / 32) + kq / 4;
            if (NT_OUT) {
                __builtin_nontemporal_store(packed, cdst);
                if ((kq & 3) == 0) __builtin_nontemporal_store((uint8_t)byte, sdst);
            } else {
                *cdst = packed;
                if ((kq & 3) == 0) *sdst = (uint8_t)byte;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// MXFP8 activation quantization (the W4A8 activations): E4M3 elements, one
// byte each, OCP MX scale 2^(floor(log2 amax) - 8).  Same thread layout as
// act_quant_kernel: a thread owns 8 bf16 values (one 16-byte load, one 8-byte
// store of codes), an aligned quad owns the 32-element block.
// ---------------------------------------------------------------------------

template <int ROWS, bool SMOOTH = false>
__global__ __launch_bounds__(256) void act_quant_fp8_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const int32_t* __restrict__ row_index,
    int64_t M, int64_t K, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ smooth) {
    const int64_t chunks = K / 8;
    const int64_t kq = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (kq >= chunks) return;                         // whole quads leave together
    uint4 sm = make_uint4(0, 0, 0, 0);
    if constexpr (SMOOTH) sm = *reinterpret_cast<const uint4*>(smooth + kq * 8);
    for (int64_t m0 = (int64_t)blockIdx.y * ROWS; m0 < M; m0 += (int64_t)gridDim.y * ROWS) {
        uint4 raw[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const int64_t m = m0 + r;
            if (m < M) {
                const int64_t src = row_index ? (int64_t)row_index[m] : m;
                raw[r] = *reinterpret_cast<const uint4*>(x + src * ldx + kq * 8);
            }
        }
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const int64_t m = m0 + r;
            if (m >= M) break;                        // uniform across the workgroup
            uint32_t w[4] = {raw[r].x, raw[r].y, raw[r].z, raw[r].w};
            if constexpr (SMOOTH) {
                const uint32_t sv[4] = {sm.x, sm.y, sm.z, sm.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = smooth_pair(w[i], sv[i]);
            }
            u16x2 a = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
            for (int i = 1; i < 4; ++i)
                a = __builtin_elementwise_max(a, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
            const uint32_t amax = quad_max_u32(max((uint32_t)a[0], (uint32_t)a[1]));
            const uint32_t byte = mx8_scale_from_bf16_amax(amax);
            const uint2 out = byte == 255u ? make_uint2(0u, 0u) : e4m3_codes8(w, byte);
            *reinterpret_cast<uint2*>(codes + m * K + kq * 8) = out;
            if ((kq & 3) == 0) scales[m * (K / 32) + kq / 4] = (uint8_t)byte;
        }
    }
}

hipError_t launch_act_quant_fp8(const uint16_t* x, int64_t ldx, const int32_t* row_index,
                                int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                                hipStream_t stream, const uint16_t* smooth) {
    constexpr int ROWS = 2;
    const int64_t gx = (K / 8 + 255) / 256;
    int64_t gy = (M + ROWS - 1) / ROWS;
    if (gy > 65535) gy = 65535;
    const dim3 grid((unsigned)gx, (unsigned)gy);
    if (smooth)
        hipLaunchKernelGGL((act_quant_fp8_kernel<ROWS, true>), grid, dim3(256), 0, stream, x, ldx,
                           row_index, M, K, codes, scales, smooth);
    else
        hipLaunchKernelGGL((act_quant_fp8_kernel<ROWS, false>), grid, dim3(256), 0, stream, x,
                           ldx, row_index, M, K, codes, scales, smooth);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// NVFP4 -> MXFP4 requant.  One thread owns one 32-element MX block: 16 code
// bytes (one 16-byte load) and the E4M3 scales of its two NVFP4 blocks.
//
// Inside an NVFP4 block every element is v = fl32(fl32(e2m1 * s) * g), a
// function of its 4-bit code alone, and |v| grows with the code's magnitude
// (rounding is monotone).  So per half-block the thread
//   1. forms the 8 magnitudes |v(c)|, c = 0..7 (the sign of v is the code's
//      sign bit xor the signs of s and g, also for zeros),
//   2. finds the largest code magnitude present; the MX block's amax is the
//      larger of the two halves' |v(cmax)|, which gives the E8M0 byte,
//   3. encodes the 8 magnitudes once with the hardware converter into an
//      8-entry byte table, and
//   4. maps every code through that table with byte permutes (v_perm_b32),
//      eight codes per two permutes, restoring the sign bits afterwards.
// A NaN or Inf anywhere in the NVFP4 block shows up in |v(cmax)| (0 * Inf,
// NaN scales and Inf products all surface there), giving byte 0xFF and zero
// codes.
// ---------------------------------------------------------------------------
template <bool BF16_INTERMEDIATE>
__device__ __forceinline__ float nv_mag(float e2m1_mag, float s_abs, float g_abs) {
    float v = (e2m1_mag * s_abs) * g_abs;    // first product exact, second rounded once
    if (BF16_INTERMEDIATE) v = bf16_to_f32(f32_to_bf16_rne(v));
    return v;
}

// Bytes 0..7 of {hi:lo} hold one-hot masks 1 << c: permuting by code
// magnitudes marks which magnitudes occur.
constexpr uint32_t ONEHOT_LO = 0x08040201u, ONEHOT_HI = 0x80402010u;

template <bool BF16_INTERMEDIATE, bool UOS>
__device__ __forceinline__ void requant_block(uint4 raw, uint32_t sc, float g_abs,
                                              uint32_t g_sign, uint4& out, uint32_t& byte_out) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t sel_lo[4], sel_hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sel_lo[i] = w[i] & 0x07070707u;            // even elements' code magnitudes
        sel_hi[i] = (w[i] >> 4) & 0x07070707u;     // odd elements'
    }
    float tab_mag[2][8];
    uint32_t amax_bits = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t s8 = (sc >> (8 * h)) & 0xFFu;
        const float s_abs = e4m3_to_f32(s8 & 0x7Fu);
        constexpr float E[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
#pragma unroll
        for (int c = 0; c < 8; ++c) tab_mag[h][c] = nv_mag<BF16_INTERMEDIATE>(E[c], s_abs, g_abs);
        uint32_t seen = 0;
#pragma unroll
        for (int i = 2 * h; i < 2 * h + 2; ++i)
            seen |= byte_perm(ONEHOT_HI, ONEHOT_LO, sel_lo[i]) |
                    byte_perm(ONEHOT_HI, ONEHOT_LO, sel_hi[i]);
        seen |= seen >> 16;
        seen |= seen >> 8;
        const uint32_t cmax = 31u - (uint32_t)__builtin_clz(seen & 0xFFu);
        const float top = nv_mag<BF16_INTERMEDIATE>(e2m1_to_f32(cmax), s_abs, g_abs);
        amax_bits = max(amax_bits, __float_as_uint(top) & 0x7FFFFFFFu);
    }
    const uint32_t byte = mx_scale_byte<UOS>(amax_bits);
    const float scale = e8m0_to_f32(byte);
    uint32_t res[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float* m = tab_mag[h];
        uint32_t t = cvt_fp4x2<0>(0u, m[0], m[4], scale);
        t = cvt_fp4x2<1>(t, m[1], m[5], scale);
        t = cvt_fp4x2<2>(t, m[2], m[6], scale);
        t = cvt_fp4x2<3>(t, m[3], m[7], scale);
        const uint32_t tab_lo = t & 0x0F0F0F0Fu;          // codes of magnitudes 0..3
        const uint32_t tab_hi = (t >> 4) & 0x0F0F0F0Fu;   // codes of magnitudes 4..7
        const uint32_t s8 = (sc >> (8 * h)) & 0xFFu;
        const uint32_t flip = ((s8 >> 7) ^ g_sign) ? 0x88888888u : 0u;
#pragma unroll
        for (int i = 2 * h; i < 2 * h + 2; ++i)
            res[i] = byte_perm(tab_hi, tab_lo, sel_lo[i]) |
                     (byte_perm(tab_hi, tab_lo, sel_hi[i]) << 4) |
                     ((w[i] ^ flip) & 0x88888888u);
    }
    if (byte == 255u) res[0] = res[1] = res[2] = res[3] = 0u;
    out = make_uint4(res[0], res[1], res[2], res[3]);
    byte_out = byte;
}

// Grid: x walks the MX blocks of one tensor, 2 * 256 per workgroup pass;
// y walks tensors (each with its own global scale).  Source and destination
// are touched exactly once and are far larger than the caches, so loads and
// stores are non-temporal (measured: about 12% more bandwidth on a layer).
// Tensors of a subset requant, chosen on the host and passed by value in
// the kernel arguments (no device memory): up to NSEL per launch.  NSEL = 1
// is the whole-batch form, where the list is unused.
template <int NSEL>
struct TensorSel {
    int32_t t[NSEL];
};
constexpr int REQUANT_SEL = 512;

// `count` tensors: tensor i of the launch is sel.t[i] (NSEL > 1) or i.
template <bool BF16_INTERMEDIATE, int NSEL, bool UOS>
__global__ __launch_bounds__(256) void requant_kernel(
    const uint8_t* __restrict__ nv_codes, const uint8_t* __restrict__ nv_scales,
    const float* __restrict__ nv_global, int64_t count, const TensorSel<NSEL> sel,
    int64_t blocks_per_tensor, uint8_t* __restrict__ mx_codes, uint8_t* __restrict__ mx_scales) {
    constexpr int UNROLL = 2;
    for (int64_t i = blockIdx.y; i < count; i += gridDim.y) {
        const int64_t t = NSEL > 1 ? (int64_t)sel.t[i] : i;
        const float g = nv_global[t];
        const float g_abs = __builtin_fabsf(g);
        const uint32_t g_sign = __float_as_uint(g) >> 31;
        const int64_t base = t * blocks_per_tensor;
        for (int64_t b0 = (int64_t)blockIdx.x * (UNROLL * 256) + threadIdx.x;
             b0 < blocks_per_tensor; b0 += (int64_t)gridDim.x * (UNROLL * 256)) {
            uint4 raw[UNROLL];
            uint32_t sc[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int64_t b = b0 + u * 256;
                if (b < blocks_per_tensor) {
                    const v4u_t c = __builtin_nontemporal_load(
                        reinterpret_cast<const v4u_t*>(nv_codes + (base + b) * 16));
                    raw[u] = make_uint4(c[0], c[1], c[2], c[3]);
                    sc[u] = __builtin_nontemporal_load(
                        reinterpret_cast<const uint16_t*>(nv_scales + (base + b) * 2));
                }
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int64_t b = b0 + u * 256;
                if (b < blocks_per_tensor) {
                    uint4 out;
                    uint32_t byte;
                    requant_block<BF16_INTERMEDIATE, UOS>(raw[u], sc[u], g_abs, g_sign, out, byte);
                    __builtin_nontemporal_store(v4u_t{out.x, out.y, out.z, out.w},
                                                reinterpret_cast<v4u_t*>(mx_codes + (base + b) * 16));
                    __builtin_nontemporal_store((uint8_t)byte, mx_scales + base + b);
                }
            }
        }
    }
}

// 256-thread workgroups of `kernel` resident on the current device at once
// (0 if the runtime cannot say; the failed query's error is then cleared,
// so that the launch that follows reports only its own).
static int64_t resident_workgroups(const void* kernel) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return (int64_t)cus * per_cu;
}

hipError_t launch_act_quant(const uint16_t* x, int64_t ldx, const int32_t* row_index,
                            int64_t M, int64_t K, uint8_t* codes, uint8_t* scales, bool uos,
                            hipStream_t stream, const uint16_t* smooth) {
    constexpr int ROWS = 2;            // 1 and 4 measured slower
    const int64_t chunks = K / 8;
    const int64_t gx = (chunks + 255) / 256;
    int64_t gy = (M + ROWS - 1) / ROWS;
    if (gy > 65535) gy = 65535;
    // Between one and two rounds of resident workgroups: three quarters of
    // one round, each walking more rows, rather than a second partial round
    // ([4096, 4096]: 8.82 -> 8.37 us; one quarter of a round, or capping the
    // seven rounds of [4096, 14336], measured slower).
    {
        static const int64_t resident = resident_workgroups(
            reinterpret_cast<const void*>(act_quant_kernel<ROWS, false, false>));
        if (resident > 0 && gx * gy > resident && gx * gy <= 2 * resident)
            gy = (resident * 3 / 4 + gx - 1) / gx;
    }
    // codes past 16 MiB (more than the next GEMM finds in L2) go out
    // non-temporally unless gathered (a gathered batch is the MoE one, whose
    // GEMM re-reads each expert's rows): measured 7% faster at [4096,14336],
    // slower for the decode and [4096,4096] sizes
    const bool nt_out = !row_index && M * (K / 2) >= ((int64_t)16 << 20);
    const dim3 grid((unsigned)gx, (unsigned)gy);
    const int32_t* no_dest = nullptr;
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, x, ldx, row_index, M, K, codes,
                           scales, smooth, no_dest, 0, (int64_t)0);
    };
    if (smooth) {
        if (uos)
            nt_out ? go(act_quant_kernel<ROWS, true, true, false, true>)
                   : go(act_quant_kernel<ROWS, false, true, false, true>);
        else
            nt_out ? go(act_quant_kernel<ROWS, true, false, false, true>)
                   : go(act_quant_kernel<ROWS, false, false, false, true>);
    } else if (uos) {
        nt_out ? go(act_quant_kernel<ROWS, true, true>) : go(act_quant_kernel<ROWS, false, true>);
    } else {
        nt_out ? go(act_quant_kernel<ROWS, true, false>)
               : go(act_quant_kernel<ROWS, false, false>);
    }
    return hipGetLastError();
}

hipError_t launch_act_quant_scatter(const uint16_t* x, int64_t ldx, int64_t T, int64_t K,
                                    const int32_t* dest, int64_t fan, int64_t R,
                                    uint8_t* codes, uint8_t* scales, bool uos,
                                    hipStream_t stream) {
    constexpr int ROWS = 2;
    const int64_t gx = (K / 8 + 255) / 256;
    int64_t gy = (T + ROWS - 1) / ROWS;
    if (gy > 65535) gy = 65535;
    const dim3 grid((unsigned)gx, (unsigned)gy);
    const uint16_t* none = nullptr;
    const int32_t* no_index = nullptr;
    if (uos)
        hipLaunchKernelGGL((act_quant_kernel<ROWS, false, true, false, false, true>), grid,
                           dim3(256), 0, stream, x, ldx, no_index, T, K, codes, scales, none,
                           dest, (int)fan, R);
    else
        hipLaunchKernelGGL((act_quant_kernel<ROWS, false, false, false, false, true>), grid,
                           dim3(256), 0, stream, x, ldx, no_index, T, K, codes, scales, none,
                           dest, (int)fan, R);
    return hipGetLastError();
}

hipError_t launch_silu_mul_quantize(const uint16_t* gate_up, int64_t ldg, int64_t M, int64_t I,
                                   uint8_t* codes, uint8_t* scales, bool uos,
                                   hipStream_t stream) {
    constexpr int ROWS = 2;
    const int64_t gx = (I / 8 + 255) / 256;
    int64_t gy = (M + ROWS - 1) / ROWS;
    if (gy > 65535) gy = 65535;
    const dim3 grid((unsigned)gx, (unsigned)gy);
    // the codes feed the down GEMM next: normal stores
    const int32_t* no_index = nullptr;
    const uint16_t* none = nullptr;
    if (uos)
        hipLaunchKernelGGL((act_quant_kernel<ROWS, false, true, true>), grid, dim3(256), 0,
                           stream, gate_up, ldg, no_index, M, I, codes, scales, none, no_index, 0,
                           (int64_t)0);
    else
        hipLaunchKernelGGL((act_quant_kernel<ROWS, false, false, true>), grid, dim3(256), 0,
                           stream, gate_up, ldg, no_index, M, I, codes, scales, none, no_index, 0,
                           (int64_t)0);
    return hipGetLastError();
}

hipError_t launch_requant(const uint8_t* nv_codes, const uint8_t* nv_scales,
                          const float* nv_global, int64_t T, int64_t N, int64_t K,
                          const int32_t* tensors, int64_t n_tensors, uint8_t* mx_codes,
                          uint8_t* mx_scales, bool bf16_intermediate, bool uos,
                          hipStream_t stream) {
    const int64_t bpt = N * (K / 32);
    int64_t gx = (bpt + 511) / 512;
    if (gx > 8192) gx = 8192;
    // One tensor: at most one round of resident workgroups, each walking
    // the tensor's blocks, rather than a second, partly filled round.  For
    // a [12288, 4096] weight (3072 workgroup steps of 512 blocks) measured
    // 12.9 -> 11.9 us.
    if (!tensors && T == 1) {
        static const int64_t resident =
            resident_workgroups(reinterpret_cast<const void*>(requant_kernel<false, 1, false>));
        if (resident > 0 && gx > resident) gx = resident;
    }
    auto grid = [&](int64_t count) {
        return dim3((unsigned)gx, (unsigned)(count > 65535 ? 65535 : count));
    };
    // the four variants of the kernel for one tensor-list size
    auto go = [&](auto sel, dim3 g, int64_t count) {
        constexpr int NSEL = sizeof(sel.t) / sizeof(int32_t);
        if (bf16_intermediate && uos)
            hipLaunchKernelGGL((requant_kernel<true, NSEL, true>), g, dim3(256), 0, stream,
                               nv_codes, nv_scales, nv_global, count, sel, bpt, mx_codes,
                               mx_scales);
        else if (bf16_intermediate)
            hipLaunchKernelGGL((requant_kernel<true, NSEL, false>), g, dim3(256), 0, stream,
                               nv_codes, nv_scales, nv_global, count, sel, bpt, mx_codes,
                               mx_scales);
        else if (uos)
            hipLaunchKernelGGL((requant_kernel<false, NSEL, true>), g, dim3(256), 0, stream,
                               nv_codes, nv_scales, nv_global, count, sel, bpt, mx_codes,
                               mx_scales);
        else
            hipLaunchKernelGGL((requant_kernel<false, NSEL, false>), g, dim3(256), 0, stream,
                               nv_codes, nv_scales, nv_global, count, sel, bpt, mx_codes,
                               mx_scales);
        return hipGetLastError();
    };
    if (!tensors) return go(TensorSel<1>{{0}}, grid(T), T);
    for (int64_t c0 = 0; c0 < n_tensors; c0 += REQUANT_SEL) {
        const int64_t count = n_tensors - c0 < REQUANT_SEL ? n_tensors - c0 : REQUANT_SEL;
        TensorSel<REQUANT_SEL> sel{};
        for (int64_t i = 0; i < count; ++i) sel.t[i] = tensors[c0 + i];
        const hipError_t e = go(sel, grid(count), count);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mx
