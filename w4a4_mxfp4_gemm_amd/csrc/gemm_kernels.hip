// gemm_kernels.hip -- MXFP4 x MXFP4 GEMM (dense and grouped by expert) on
// gfx950's block-scaled MFMA, v_mfma_scale_f32_16x16x128_f8f6f4 with both
// operands in E2M1 (format code 4).
//
// Operand mapping.  One 16x16x128 MFMA takes, per lane l, 32 E2M1 values
// (16 bytes) of row l%16 of each operand and one E8M0 scale for them; lanes
// l/16 = 0..3 hold four different 32-element K-chunks.  A 32-element chunk is
// exactly one MX block, so each lane's scale is that block's scale byte.
// The dot product does not care which K-chunk sits in which MFMA, only that
// A and B agree, so a "super-step" of 512 K (16 MX blocks) is split as: lane
// group g feeds blocks 4g..4g+3 to MFMAs 0..3.  Each lane then reads 64
// contiguous code bytes and 4 contiguous scale bytes per operand row, and the
// MFMA's scale op_sel picks the byte for each of the four MFMAs.
//
// Output mapping of the 16x16 accumulator: lane l, register r holds row
// 4*(l/16) + r of the A tile and column l%16 of the B tile.
#include "mx_device.h"
#include "launch.h"

#include <type_traits>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int S>
__device__ __forceinline__ v4f mfma_e2m1(const uint4& a, const uint4& b, v4f acc, uint32_t sa,
                                         uint32_t sb) {
    const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4, 4, S, (int)sa, S,
                                                            (int)sb);
}

// One operand row's share of a 512-K super-step: 4 MX blocks of codes plus
// their 4 scale bytes packed into one register.  Blocks past K (and rows
// outside the tile) read as code 0 with scale 2^0, contributing nothing.
struct Frag {
    uint4 c[4];
    uint32_t s;
};

__device__ __forceinline__ void load_frag(const uint8_t* __restrict__ codes,
                                          const uint8_t* __restrict__ scales, int64_t row,
                                          bool row_ok, int kb_first, int nkb, Frag& f) {
    const uint8_t* crow = codes + row * (int64_t)nkb * 16;
    const uint8_t* srow = scales + row * (int64_t)nkb;
    uint32_t s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int kb = kb_first + q;
        const bool ok = row_ok && kb < nkb;
        f.c[q] = ok ? *reinterpret_cast<const uint4*>(crow + (int64_t)kb * 16)
                    : make_uint4(0, 0, 0, 0);
        s |= (ok ? (uint32_t)srow[kb] : 127u) << (8 * q);
    }
    f.s = s;
}

// W4A8: an MXFP8 operand row's share of a super-step.  An E4M3 operand is 32
// bytes a lane (8 registers), but not one MX block: in lane group g, bytes
// 0..15 are K 16g..16g+15 of the 128 and bytes 16..31 are K 64+16g..64+16g+15
// (measured), while an E2M1 operand's lane group g holds K 32g..32g+31, and
// the scale of lane group j applies to K 32j..32j+31 for both.  So the MX
// block that MFMA q takes at K 32j.. (block 4j+q of the super-step, as for
// E2M1) is split: its first half goes to lane group 2(j%2), its second half to
// 2(j%2)+1, in bytes 0..15 for j < 2 and 16..31 for j >= 2.  Lane group g
// therefore loads half g%2 of blocks 4(g/2)+q and 4(2+g/2)+q; its scale byte
// stays block 4g+q's.  Rows are K bytes long.
struct Frag8 {
    uint4 c[4][2];
    uint32_t s;
};

__device__ __forceinline__ void load_frag8(const uint8_t* __restrict__ codes,
                                           const uint8_t* __restrict__ scales, int64_t row,
                                           bool row_ok, int base, int g, int nkb, Frag8& f) {
    const uint8_t* crow = codes + row * (int64_t)nkb * 32 + 16 * (g & 1);
    const uint8_t* srow = scales + row * (int64_t)nkb;
    uint32_t s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int k0 = base + 4 * (g >> 1) + q, k1 = k0 + 8;
        const bool ok0 = row_ok && k0 < nkb, ok1 = row_ok && k1 < nkb;
        f.c[q][0] = ok0 ? *reinterpret_cast<const uint4*>(crow + (int64_t)k0 * 32)
                        : make_uint4(0, 0, 0, 0);
        f.c[q][1] = ok1 ? *reinterpret_cast<const uint4*>(crow + (int64_t)k1 * 32)
                        : make_uint4(0, 0, 0, 0);
        const int ks = base + 4 * g + q;
        s |= (row_ok && ks < nkb ? (uint32_t)srow[ks] : 127u) << (8 * q);
    }
    f.s = s;
}

// E4M3 A (format code 0) times E2M1 B (format code 4)
template <int S>
__device__ __forceinline__ v4f mfma_e4m3_e2m1(const uint4 (&a)[2], const uint4& b, v4f acc,
                                              uint32_t sa, uint32_t sb) {
    const v8i av = {(int)a[0].x, (int)a[0].y, (int)a[0].z, (int)a[0].w,
                    (int)a[1].x, (int)a[1].y, (int)a[1].z, (int)a[1].w};
    const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 4, S, (int)sa, S,
                                                            (int)sb);
}

template <int WM, int WN>
__device__ __forceinline__ void mfma_superstep(const Frag8 (&fa)[WM], const Frag (&fb)[WN],
                                               v4f (&acc)[WM][WN]) {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            acc[i][j] = mfma_e4m3_e2m1<0>(fa[i].c[0], fb[j].c[0], acc[i][j], fa[i].s, fb[j].s);
            acc[i][j] = mfma_e4m3_e2m1<1>(fa[i].c[1], fb[j].c[1], acc[i][j], fa[i].s, fb[j].s);
            acc[i][j] = mfma_e4m3_e2m1<2>(fa[i].c[2], fb[j].c[2], acc[i][j], fa[i].s, fb[j].s);
            acc[i][j] = mfma_e4m3_e2m1<3>(fa[i].c[3], fb[j].c[3], acc[i][j], fa[i].s, fb[j].s);
        }
}

template <int WM, int WN>
__device__ __forceinline__ void mfma_superstep(const Frag (&fa)[WM], const Frag (&fb)[WN],
                                               v4f (&acc)[WM][WN]) {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            acc[i][j] = mfma_e2m1<0>(fa[i].c[0], fb[j].c[0], acc[i][j], fa[i].s, fb[j].s);
            acc[i][j] = mfma_e2m1<1>(fa[i].c[1], fb[j].c[1], acc[i][j], fa[i].s, fb[j].s);
            acc[i][j] = mfma_e2m1<2>(fa[i].c[2], fb[j].c[2], acc[i][j], fa[i].s, fb[j].s);
            acc[i][j] = mfma_e2m1<3>(fa[i].c[3], fb[j].c[3], acc[i][j], fa[i].s, fb[j].s);
        }
}

// A workgroup of 4 wavefronts.  KSPLIT of them share one output tile and
// split its K super-steps round-robin (their partial tiles are summed through
// LDS in a fixed order); the other factor tiles N.  Each wavefront owns a
// (16*WM) x (16*WN) tile of 16x16 MFMA blocks.
// A8: A is MXFP8 (W4A8 activations), else MXFP4.
template <int WM, int WN, int KSPLIT, bool OUT_BF16, bool A8 = false>
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ a_codes,
                                          const uint8_t* __restrict__ a_scales,
                                          const uint8_t* __restrict__ b_codes,
                                          const uint8_t* __restrict__ b_scales, int64_t m0,
                                          int64_t m_end, int64_t n0_wg, int64_t N, int64_t K,
                                          void* __restrict__ y,
                                          const uint16_t* __restrict__ bias) {
    constexpr int WAVES_N = 4 / KSPLIT;
    static_assert(WAVES_N * KSPLIT == 4, "4 wavefronts per workgroup");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kw = wave % KSPLIT;
    const int wn = wave / KSPLIT;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int nkb = (int)(K / 32);
    const int nss = (nkb + 15) / 16;
    const int64_t n0 = n0_wg + (int64_t)wn * 16 * WN;

    v4f acc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int ss = kw; ss < nss; ss += KSPLIT) {
        const int kb_first = ss * 16 + 4 * g;
        std::conditional_t<A8, Frag8, Frag> fa[WM];
        Frag fb[WN];
#pragma unroll
        for (int i = 0; i < WM; ++i) {
            const int64_t row = m0 + 16 * i + r16;
            if constexpr (A8)
                load_frag8(a_codes, a_scales, row, row < m_end, ss * 16, g, nkb, fa[i]);
            else
                load_frag(a_codes, a_scales, row, row < m_end, kb_first, nkb, fa[i]);
        }
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            const int64_t row = n0 + 16 * j + r16;
            load_frag(b_codes, b_scales, row, row < N, kb_first, nkb, fb[j]);
        }
        mfma_superstep<WM, WN>(fa, fb, acc);
    }

    if constexpr (KSPLIT > 1) {
        __shared__ float red[(KSPLIT > 1 ? 4 - WAVES_N : 1)][WM * WN * 4][64];
        if (kw > 0) {
            const int slot = wave - wn * KSPLIT - 1 + wn * (KSPLIT - 1);
#pragma unroll
            for (int i = 0; i < WM; ++i)
#pragma unroll
                for (int j = 0; j < WN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) red[slot][(i * WN + j) * 4 + r][lane] = acc[i][j][r];
        }
        __syncthreads();
        if (kw > 0) return;
#pragma unroll
        for (int q = 1; q < KSPLIT; ++q) {
            const int slot = wn * (KSPLIT - 1) + (q - 1);
#pragma unroll
            for (int i = 0; i < WM; ++i)
#pragma unroll
                for (int j = 0; j < WN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] += red[slot][(i * WN + j) * 4 + r][lane];
        }
    }

#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            const int64_t n = n0 + 16 * j + r16;
            if (n >= N) continue;
            // the row bias joins the fp32 sum before its one rounding
            const float bn = bias ? __uint_as_float((uint32_t)bias[n] << 16) : 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + 16 * i + 4 * g + r;
                if (m >= m_end) continue;
                const float v = bias ? acc[i][j][r] + bn : acc[i][j][r];
                if (OUT_BF16)
                    reinterpret_cast<uint16_t*>(y)[m * N + n] = (uint16_t)f32_to_bf16_rne(v);
                else
                    reinterpret_cast<float*>(y)[m * N + n] = v;
            }
        }
}

template <int WM, int WN, int KSPLIT, bool OUT_BF16, bool A8 = false>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* __restrict__ a_codes,
                                                   const uint8_t* __restrict__ a_scales,
                                                   const uint8_t* __restrict__ b_codes,
                                                   const uint8_t* __restrict__ b_scales,
                                                   int64_t M, int64_t N, int64_t K,
                                                   void* __restrict__ y,
                                                   const uint16_t* __restrict__ bias) {
    constexpr int TN = 16 * WN * (4 / KSPLIT);
    const int64_t m0 = (int64_t)blockIdx.y * 16 * WM;
    const int64_t n0 = (int64_t)blockIdx.x * TN;
    gemm_tile<WM, WN, KSPLIT, OUT_BF16, A8>(a_codes, a_scales, b_codes, b_scales, m0, M, n0, N,
                                            K, y, bias);
}

// Grouped variant: blockIdx.y enumerates the row tiles of all experts in
// order; each workgroup walks the offset table to find its expert.  Row
// ranges are clamped to [0, total_M), so a malformed table never causes an
// access outside A or y.
template <int WM, int WN, int KSPLIT, bool OUT_BF16>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales,
    const int32_t* __restrict__ offsets, int64_t E, int64_t total_M, int64_t N, int64_t K,
    void* __restrict__ y) {
    constexpr int TM = 16 * WM;
    constexpr int TN = 16 * WN * (4 / KSPLIT);
    const int64_t t = blockIdx.y;
    int64_t base = 0, r0 = 0, r1 = 0, e = -1;
    for (int64_t ee = 0; ee < E; ++ee) {
        int64_t a0 = offsets[ee], a1 = offsets[ee + 1];
        a0 = a0 < 0 ? 0 : (a0 > total_M ? total_M : a0);
        a1 = a1 < a0 ? a0 : (a1 > total_M ? total_M : a1);
        const int64_t nt = (a1 - a0 + TM - 1) / TM;
        if (t < base + nt) {
            e = ee;
            r0 = a0 + (t - base) * TM;
            r1 = a1;
            break;
        }
        base += nt;
    }
    if (e < 0) return;
    const int64_t n0 = (int64_t)blockIdx.x * TN;
    const int64_t nkb = K / 32;
    gemm_tile<WM, WN, KSPLIT, OUT_BF16>(a_codes, a_scales, b_codes + e * N * nkb * 16,
                                        b_scales + e * N * nkb, r0, r1, n0, N, K, y, nullptr);
}

template <int WM, int WN, int KSPLIT, bool A8 = false>
static hipError_t launch_dense(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                               const uint8_t* bs, int64_t M, int64_t N, int64_t K, void* y,
                               const uint16_t* bias, bool out_bf16, hipStream_t stream) {
    constexpr int TM = 16 * WM;
    constexpr int TN = 16 * WN * (4 / KSPLIT);
    const dim3 grid((unsigned)((N + TN - 1) / TN), (unsigned)((M + TM - 1) / TM));
    if (out_bf16)
        hipLaunchKernelGGL((gemm_kernel<WM, WN, KSPLIT, true, A8>), grid, dim3(256), 0, stream, a,
                           as, b, bs, M, N, K, y, bias);
    else
        hipLaunchKernelGGL((gemm_kernel<WM, WN, KSPLIT, false, A8>), grid, dim3(256), 0, stream,
                           a, as, b, bs, M, N, K, y, bias);
    return hipGetLastError();
}

// W4A8: A MXFP8 [M][K] + [M][K/32], B MXFP4.  The skinny weight-streaming
// kernel for decode shapes, the LDS-staged tiled kernel from 128 rows, the
// 16x16x128 tile kernel otherwise.
hipError_t launch_gemm_w4a8(const uint8_t* a_codes, const uint8_t* a_scales,
                            const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N,
                            int64_t K, void* y, const uint16_t* bias, bool out_bf16,
                            hipStream_t stream) {
    if (skinny_gemm_supported(M, N, K, a_codes, a_scales, b_scales))
        return launch_gemm_skinny_w4a8(a_codes, a_scales, b_codes, b_scales, M, N, K, y, bias,
                                       out_bf16, stream);
    if (tiled_w4a8_supported(M, N, K, a_scales, b_scales))
        return launch_gemm_tiled_w4a8(a_codes, a_scales, b_codes, b_scales, M, N, K, y, bias,
                                      out_bf16, stream);
    if (M <= 16)
        return launch_dense<1, 1, 4, true>(a_codes, a_scales, b_codes, b_scales, M, N, K, y, bias,
                                           out_bf16, stream);
    if (M <= 32)
        return launch_dense<2, 1, 4, true>(a_codes, a_scales, b_codes, b_scales, M, N, K, y, bias,
                                           out_bf16, stream);
    return launch_dense<2, 2, 1, true>(a_codes, a_scales, b_codes, b_scales, M, N, K, y, bias,
                                       out_bf16, stream);
}

// M just past the decode kernel's 64 rows: that kernel once per 64-row slice
// (each row's result is that of one launch), while the 256-row tiles would
// leave most CUs idle.  Measured at K = 4096: M = 96, N = 12288 19.6 us
// against 59.3 on the generic kernel; at M = 128 the tiles win from about 64
// tiles (N = 28672: 31.8 against 37.1 us for two slices).
static bool sliced_rows(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                        const uint8_t* a_scales, const uint8_t* b_scales) {
    if (M <= 64 || M > 128) return false;
    if (M == 128 && ((N + 255) / 256) >= 64) return false;
    const int64_t ldc = K / 2, lds_ = K / 32;
    const uint8_t* c2 = a_codes + 64 * ldc;
    const uint8_t* s2 = a_scales + 64 * lds_;
    return (skinny_gemm_supported(64, N, K, a_codes, a_scales, b_scales) &&
            skinny_gemm_supported(64, N, K, c2, s2, b_scales)) ||
           (skinny_any_k_supported(64, N, K, a_codes, a_scales, b_scales) &&
            skinny_any_k_supported(64, N, K, c2, s2, b_scales));
}

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                       const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* y,
                       const uint16_t* bias, bool out_bf16, hipStream_t stream) {
    if (sliced_rows(M, N, K, a_codes, a_scales, b_scales)) {
        const int64_t esize = out_bf16 ? 2 : 4;
        for (int64_t m0 = 0; m0 < M; m0 += 64) {
            const hipError_t e = launch_gemm(a_codes + m0 * (K / 2), a_scales + m0 * (K / 32),
                                             b_codes, b_scales, M - m0 < 64 ? M - m0 : 64, N, K,
                                             static_cast<uint8_t*>(y) + m0 * N * esize, bias,
                                             out_bf16, stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    if (skinny_gemm_supported(M, N, K, a_codes, a_scales, b_scales))
        return launch_gemm_skinny(a_codes, a_scales, b_codes, b_scales, M, N, K, y, bias,
                                  out_bf16, stream);
    if (skinny_any_k_supported(M, N, K, a_codes, a_scales, b_scales))
        return launch_gemm_skinny_any_k(a_codes, a_scales, b_codes, b_scales, M, N, K, y, bias,
                                        out_bf16, stream);
    if (tiled_gemm_supported(M, N, K, a_scales, b_scales))
        return launch_gemm_tiled(a_codes, a_scales, b_codes, b_scales, M, N, K, y, bias,
                                 out_bf16, stream);
    if (M <= 16)
        return launch_dense<1, 1, 4>(a_codes, a_scales, b_codes, b_scales, M, N, K, y, bias,
                                     out_bf16, stream);
    if (M <= 32)
        return launch_dense<2, 1, 4>(a_codes, a_scales, b_codes, b_scales, M, N, K, y, bias,
                                     out_bf16, stream);
    if (M <= 64)
        return launch_dense<4, 1, 4>(a_codes, a_scales, b_codes, b_scales, M, N, K, y, bias,
                                     out_bf16, stream);
    return launch_dense<2, 2, 1>(a_codes, a_scales, b_codes, b_scales, M, N, K, y, bias,
                                 out_bf16, stream);
}

hipError_t launch_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                               const uint8_t* b_codes, const uint8_t* b_scales,
                               const int32_t* offsets, int64_t E, int64_t total_M, int64_t N,
                               int64_t K, void* y, bool out_bf16, bool b_shuffled,
                               hipStream_t stream) {
    if (b_shuffled || grouped_tiled_supported(E, total_M, N, K, a_scales, b_scales))
        return launch_grouped_gemm_tiled(a_codes, a_scales, b_codes, b_scales, offsets, E,
                                         total_M, N, K, y, out_bf16, b_shuffled, stream);
    constexpr int WM = 2, WN = 2, KSPLIT = 1;
    constexpr int TM = 16 * WM;
    constexpr int TN = 16 * WN * (4 / KSPLIT);
    const dim3 grid((unsigned)((N + TN - 1) / TN), (unsigned)((total_M + TM - 1) / TM + E));
    if (out_bf16)
        hipLaunchKernelGGL((grouped_gemm_kernel<WM, WN, KSPLIT, true>), grid, dim3(256), 0,
                           stream, a_codes, a_scales, b_codes, b_scales, offsets, E, total_M, N,
                           K, y);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<WM, WN, KSPLIT, false>), grid, dim3(256), 0,
                           stream, a_codes, a_scales, b_codes, b_scales, offsets, E, total_M, N,
                           K, y);
    return hipGetLastError();
}

}  // namespace mx
