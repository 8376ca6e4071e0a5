// gemm_skinny.hip -- weight-streaming MXFP4 GEMM for few activation rows
// (decode, M <= 64).  The time is the HBM read of the weights, so the kernel
// is organised around keeping enough weight bytes in flight and doing little
// else:
//
//  * one workgroup of NW = 4 or 8 wavefronts per CU, persistent over 16-row
//    weight tiles (tile t, t + grid, t + 2 grid, ...);
//  * the wavefronts split K in NW interleaved parts; each loads its share
//    of the activations (all M rows, padded to MT x 16) straight into
//    registers once, then issues its share of TPW weight tiles before the
//    first MFMA and refills a tile's registers as soon as they are consumed;
//  * the NW partial tiles are summed through LDS in a fixed order
//    (deterministic), one 16-row activation block per wavefront, from a
//    double-buffered reduction area (one barrier per tile).
// Eight wavefronts (two per SIMD) double the MFMA issue rate for the larger
// M, where one wavefront per SIMD cannot issue 16x16x128 MFMAs back to back;
// each then holds half the K share, so both fit in the register file.
//
// MFMA: v_mfma_scale_f32_16x16x128_f8f6f4, weight rows as the A operand, so
// lane l's accumulator holds output m = l%16 of its 16-row activation block
// and n = 4(l/16) + r.  Within a 512-K super-step (16 MX blocks), MFMA q
// covers blocks 4q..4q+3 with lane group g = l/16 on block 4q+g, so each
// 16-byte load instruction (weights and activations alike) reads 16 rows x
// 64 contiguous bytes: few, full memory requests.  A lane's scale byte for
// MFMA q is byte 4q+g of the row's 16 scale bytes of the super-step: loaded
// as 16 bytes, shifted right by 8g (the MFMA takes byte 0).
#include "mx_device.h"
#include "launch.h"

#include <type_traits>

namespace mx {
namespace skinny {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Reduction area: [2 buffers][NW waves][MT blocks][64 lanes] x 16 B.
template <int MT, int NW>
struct Smem {
    v4f red[2][NW][MT][64];
};

// One wavefront's share of a 16-row operand block: SPW super-steps x (4 x
// 16 B of codes + the row's 16 scale bytes).
template <int SPW>
struct Frag {
    v4u c[SPW][4];
    v4u s[SPW];
};

template <int S>
__device__ __forceinline__ v4f mfma_s(const v4u& a, const v4u& b, v4f acc, uint32_t sa,
                                      uint32_t sb) {
    const v8i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
    const v8i bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4, 4, S, (int)sa, S,
                                                            (int)sb);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, not for its global loads in flight (__syncthreads would drain
// those too and serialise the weight stream).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// This wave's share of one 16-row block (rows row0 + lane%16 of an operand
// with row stride K/2 code bytes and K/32 scale bytes): super-step
// ss = wave + NW j, load q brings blocks 4q..4q+3 (lane group g: block
// 4q+g).  Plain (cached) loads: non-temporal ones measured slower here.
// MASK: K covers only nss = K / 512 of the NW x SPW super-steps; this wave's
// super-steps past the last are neither loaded nor multiplied.
template <int SPW, int NW, bool MASK = false>
__device__ __forceinline__ void load_block(Frag<SPW>& f, const uint8_t* codes,
                                           const uint8_t* scales, int64_t row, int nkb) {
    const int lane = threadIdx.x & 63;
    const int wave = MASK ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
    const int g = lane >> 4;
    const uint8_t* crow = codes + row * (int64_t)nkb * 16;
    const uint8_t* srow = scales + row * (int64_t)nkb;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        if (MASK && (wave + NW * j) * 16 >= nkb) break;   // wave-uniform
        const int kb0 = (wave + NW * j) * 16;
        const v4u* p = reinterpret_cast<const v4u*>(crow + (int64_t)kb0 * 16 + 16 * g);
        const v4u* ps = reinterpret_cast<const v4u*>(srow + kb0);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            f.c[j][q] = p[4 * q];
        f.s[j] = *ps;
    }
}

// W4A8 activations: the same share of an MXFP8 row.  An E4M3 operand is 32
// bytes a lane, but in lane group g bytes 0..15 hold K 16g.. and bytes 16..31
// K 64+16g.. of the MFMA's 128 (measured), while the E2M1 weight operand and
// the scales go by 32-K blocks per lane group.  So MFMA q's block at K 32j..
// (super-step block 4q+j) is split over lane groups 2(j%2) and 2(j%2)+1:
// lane group g loads half g%2 of blocks 4q+g/2 (bytes 0..15) and 4q+2+g/2
// (bytes 16..31).  Scale bytes are loaded as for E2M1.  Rows are K bytes.
template <int SPW>
struct Frag8 {
    v4u c[SPW][4][2];
    v4u s[SPW];
};

template <int SPW, int NW>
__device__ __forceinline__ void load_block8(Frag8<SPW>& f, const uint8_t* codes,
                                            const uint8_t* scales, int64_t row, int nkb) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const uint8_t* crow = codes + row * (int64_t)nkb * 32 + 16 * (g & 1);
    const uint8_t* srow = scales + row * (int64_t)nkb;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        const int kb0 = (wave + NW * j) * 16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k0 = kb0 + 4 * q + (g >> 1);
            f.c[j][q][0] = *reinterpret_cast<const v4u*>(crow + (int64_t)k0 * 32);
            f.c[j][q][1] = *reinterpret_cast<const v4u*>(crow + (int64_t)(k0 + 2) * 32);
        }
        f.s[j] = *reinterpret_cast<const v4u*>(srow + kb0);
    }
}

// E2M1 weights (A, format code 4) times E4M3 activations (B, format code 0)
template <int S>
__device__ __forceinline__ v4f mfma_s8(const v4u& a, const v4u (&b)[2], v4f acc, uint32_t sa,
                                       uint32_t sb) {
    const v8i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
    const v8i bv = {(int)b[0][0], (int)b[0][1], (int)b[0][2], (int)b[0][3],
                    (int)b[1][0], (int)b[1][1], (int)b[1][2], (int)b[1][3]};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4, 0, S, (int)sa, S,
                                                            (int)sb);
}

// The same share of a 16-row block quantized from bf16 rows (row stride ldx
// elements) instead of loaded as MXFP4.  Each lane's operand is one whole
// 32-element MX block of one row, so the lane quantizes it alone, by the
// activation rule (quant_block32_bf16), into the layout load_block gives --
// except the scale word of MFMA q, which holds only this lane's byte, at bits
// 8g.  The codes and scales equal those of the act-quant kernel.  In two
// steps: load_raw issues the loads (before the weights', so that waiting for
// them does not wait for the weight stream: vmcnt counts in issue order),
// quant_raw does the arithmetic once they land.
template <int SPW>
struct RawX {
    v4u v[SPW][4][4];   // super-step j, MFMA q: the lane's 32 values, 4 x 16 B
};

template <int SPW, int NW>
__device__ __forceinline__ void load_raw(RawX<SPW>& r, const uint16_t* x, int64_t ldx,
                                         int64_t row) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const uint16_t* xrow = x + row * ldx;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        const int kb0 = (wave + NW * j) * 16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const v4u* p = reinterpret_cast<const v4u*>(xrow + (int64_t)(kb0 + 4 * q + g) * 32);
#pragma unroll
            for (int i = 0; i < 4; ++i) r.v[j][q][i] = p[i];
        }
    }
}

template <int SPW, bool UOS>
__device__ __forceinline__ void quant_raw(Frag<SPW>& f, const RawX<SPW>& r) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t v[16], c[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[4 * i] = r.v[j][q][i][0], v[4 * i + 1] = r.v[j][q][i][1],
                v[4 * i + 2] = r.v[j][q][i][2], v[4 * i + 3] = r.v[j][q][i][3];
            const uint32_t byte = quant_block32_bf16<UOS>(v, c);
            f.c[j][q] = v4u{c[0], c[1], c[2], c[3]};
            f.s[j][q] = byte << (8 * g);
        }
    }
}

// The W4A8 form of the two steps above: the lane's 32 E4M3 bytes are half g%2
// of two MX blocks (Frag8 layout), so it loads those two 16-value halves of
// bf16 and quantizes them by the MXFP8 rule.  Each block's other half sits in
// lane ^ 16, whose magnitude maximum completes the block's amax; lane group g
// then supplies MFMA q's scale for block 4q+g, which lane group 0 (g = 0: lo,
// g = 2: hi), 2 (g = 1: lo) or 3 (g = 3: hi) computed.  The codes and scales
// equal those of the MXFP8 act-quant kernel.
template <int SPW, int NW>
__device__ __forceinline__ void load_raw8(RawX<SPW>& r, const uint16_t* x, int64_t ldx,
                                          int64_t row) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const uint16_t* xrow = x + row * ldx + 16 * (g & 1);
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        const int kb0 = (wave + NW * j) * 16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int lo = kb0 + 4 * q + (g >> 1);
            const v4u* pl = reinterpret_cast<const v4u*>(xrow + (int64_t)lo * 32);
            const v4u* ph = reinterpret_cast<const v4u*>(xrow + (int64_t)(lo + 2) * 32);
            r.v[j][q][0] = pl[0];
            r.v[j][q][1] = pl[1];
            r.v[j][q][2] = ph[0];
            r.v[j][q][3] = ph[1];
        }
    }
}

template <int SPW>
__device__ __forceinline__ void quant_raw8(Frag8<SPW>& f, const RawX<SPW>& r) {
    typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, r16 = lane & 15;
    auto half_amax = [](const v4u& a, const v4u& b) {
        u16x2_t m = __builtin_bit_cast(u16x2_t, a[0] & 0x7FFF7FFFu);
#pragma unroll
        for (int i = 1; i < 4; ++i)
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, a[i] & 0x7FFF7FFFu));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, b[i] & 0x7FFF7FFFu));
        return max((uint32_t)m[0], (uint32_t)m[1]);
    };
    auto codes16 = [](const v4u& a, const v4u& b, uint32_t byte) {
        if (byte == 255u) return v4u{0u, 0u, 0u, 0u};
        const uint32_t wa[4] = {a[0], a[1], a[2], a[3]}, wb[4] = {b[0], b[1], b[2], b[3]};
        const uint2 ca = e4m3_codes8(wa, byte), cb = e4m3_codes8(wb, byte);
        return v4u{ca.x, ca.y, cb.x, cb.y};
    };
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        uint32_t sw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t alo = half_amax(r.v[j][q][0], r.v[j][q][1]);
            uint32_t ahi = half_amax(r.v[j][q][2], r.v[j][q][3]);
            alo = max(alo, (uint32_t)__shfl_xor((int)alo, 16));
            ahi = max(ahi, (uint32_t)__shfl_xor((int)ahi, 16));
            const uint32_t blo = mx8_scale_from_bf16_amax(alo);
            const uint32_t bhi = mx8_scale_from_bf16_amax(ahi);
            f.c[j][q][0] = codes16(r.v[j][q][0], r.v[j][q][1], blo);
            f.c[j][q][1] = codes16(r.v[j][q][2], r.v[j][q][3], bhi);
            const uint32_t from_lo = (uint32_t)__shfl((int)blo, r16 + 32 * (g & 1));
            const uint32_t from_hi = (uint32_t)__shfl((int)bhi, r16 + 48 * (g & 1));
            sw[q] = (g < 2 ? from_lo : from_hi) << (8 * g);
        }
        f.s[j] = v4u{sw[0], sw[1], sw[2], sw[3]};
    }
}

// BF16A: x is bf16 [M][ldx] (xs unused) and each wave quantizes its share of
// the activations itself while its weight loads stream (UOS: by the Qmax =
// 7.25 exponent rule).  A8: x is MXFP8 (the W4A8 activations).
template <int MT, int SPW, int NW, int TPW, bool OUT_BF16, bool BF16A, bool UOS = false,
          bool A8 = false, bool MASK = false>
__global__ __launch_bounds__(64 * NW, 1) void gemm_skinny_kernel(
    // no __restrict__ on the operands: with it the compiler may move their loads
    // across the points that order them (below the first MFMA, or the bf16
    // activation loads behind the weight loads), serialising the latencies
    const uint8_t* x, const uint8_t* xs, int64_t ldx, const uint8_t* w, const uint8_t* ws,
    int M, int N, int K, void* __restrict__ y, const uint16_t* __restrict__ bias) {
    __shared__ __attribute__((aligned(16))) Smem<MT, NW> sm;
    static_assert(!MASK || (!BF16A && !A8), "a partial super-step count for MXFP4 operands");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int nkb = K / 32;
    const int ntiles = (N + 15) / 16;
    const int stride = gridDim.x;
    // MASK: super-step j of this wave holds data only below nkb
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto live = [&](int j) { return !MASK || (wave_u + NW * j) * 16 < nkb; };

    auto tile_row = [&](int t) {
        const int tt = t < ntiles ? t : ntiles - 1;     // surplus loads: any valid row
        return (int64_t)min(tt * 16 + r16, N - 1);
    };

    // 1. this wave's share of the activations, rows m >= M repeating row M-1
    //    (their outputs are never stored); issued first so that the first
    //    MFMA (bf16: the quantization) waits for them and for the first
    //    weight tile only
    std::conditional_t<A8, Frag8<SPW>, Frag<SPW>> a[MT];
    RawX<SPW> xr[BF16A ? MT : 1];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t row = (int64_t)min(mt * 16 + r16, M - 1);
        if constexpr (BF16A && A8)
            load_raw8<SPW, NW>(xr[mt], reinterpret_cast<const uint16_t*>(x), ldx, row);
        else if constexpr (BF16A)
            load_raw<SPW, NW>(xr[mt], reinterpret_cast<const uint16_t*>(x), ldx, row);
        else if constexpr (A8)
            load_block8<SPW, NW>(a[mt], x, xs, row, nkb);
        else
            load_block<SPW, NW, MASK>(a[mt], x, xs, row, nkb);
    }
    // the activation loads stay ahead of the weight loads (a memory clobber
    // is a point no load moves across)
    if constexpr (BF16A) asm volatile("" ::: "memory");

    // The row bias (raw bf16 pairs) of this lane's 4 output columns of tile t
    // when all 4 are inside N; a tile that ends past N is the last of its
    // workgroup, and finish loads those values itself.  Loaded just before
    // the tile's weights: vmcnt counts in issue order, so a bias load issued
    // after them would make its first use wait for every weight load in flight.
    // The load is never predicated (merging a predicated load's result with
    // a default waits for it on the spot): the column is clamped, and without
    // a bias the first 2N bytes of the weight scales (N x K/32 bytes, 16-byte
    // aligned) stand in as the source, their values unused.  n is a multiple
    // of 4 and N >= 16, so the clamp keeps the 8-byte load aligned and inside
    // N, and leaves every tile whose 4 columns fit unchanged.
    const uint16_t* bias_src = bias ? bias : reinterpret_cast<const uint16_t*>(ws);
    auto load_bias = [&](int t) {
        const int n = min(t * 16 + 4 * g, (N & ~3) - 4);
        return *reinterpret_cast<const uint2*>(bias_src + n);
    };

    // 2. weights: TPW tiles in flight per wave
    Frag<SPW> slot[TPW];
    uint2 bslot[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        bslot[i] = load_bias(blockIdx.x + i * stride);
        load_block<SPW, NW, MASK>(slot[i], w, ws, tile_row(blockIdx.x + i * stride), nkb);
    }
    __builtin_amdgcn_sched_barrier(0);   // issue every load before the first use
    if constexpr (BF16A) {
        asm volatile("" ::: "memory");   // ... and every weight load before the quantization
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if constexpr (A8)
                quant_raw8<SPW>(a[mt], xr[mt]);
            else
                quant_raw<SPW, UOS>(a[mt], xr[mt]);
        }
    }

    const uint32_t sh = 8u * (uint32_t)g;
    auto compute = [&](const Frag<SPW>& f, v4f (&acc)[MT]) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            if (!live(j)) break;                  // wave-uniform
            // this lane's weight scale byte for MFMA q is byte 4q+g: word q >> 8g
            const uint32_t s0 = f.s[j][0] >> sh, s1 = f.s[j][1] >> sh;
            const uint32_t s2 = f.s[j][2] >> sh, s3 = f.s[j][3] >> sh;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const v4u& as = a[mt].s[j];
                if constexpr (A8) {
                    acc[mt] = mfma_s8<0>(f.c[j][0], a[mt].c[j][0], acc[mt], s0, as[0] >> sh);
                    acc[mt] = mfma_s8<0>(f.c[j][1], a[mt].c[j][1], acc[mt], s1, as[1] >> sh);
                    acc[mt] = mfma_s8<0>(f.c[j][2], a[mt].c[j][2], acc[mt], s2, as[2] >> sh);
                    acc[mt] = mfma_s8<0>(f.c[j][3], a[mt].c[j][3], acc[mt], s3, as[3] >> sh);
                } else {
                    acc[mt] = mfma_s<0>(f.c[j][0], a[mt].c[j][0], acc[mt], s0, as[0] >> sh);
                    acc[mt] = mfma_s<0>(f.c[j][1], a[mt].c[j][1], acc[mt], s1, as[1] >> sh);
                    acc[mt] = mfma_s<0>(f.c[j][2], a[mt].c[j][2], acc[mt], s2, as[2] >> sh);
                    acc[mt] = mfma_s<0>(f.c[j][3], a[mt].c[j][3], acc[mt], s3, as[3] >> sh);
                }
            }
        }
    };

    // 3. sum the waves' partial tiles (fixed order 0..NW-1) and store: wave
    //    w finishes activation blocks mt = w, w + NW, ... of the tile.  The
    //    buffer written here is next written two tiles on, after the next
    //    tile's barrier, by which point every wave has read it.
    auto finish = [&](int t, int buf, const v4f (&acc)[MT], const uint2 bv) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) sm.red[buf][wave][mt][lane] = acc[mt];
        lds_barrier();
        const int n = t * 16 + 4 * g;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (mt % NW != wave) continue;
            const int m = mt * 16 + r16;
            v4f v = sm.red[buf][0][mt][lane];
#pragma unroll
            for (int q = 1; q < NW; ++q) v += sm.red[buf][q][mt][lane];
            if (m >= M) continue;
            if (bias) {   // the row bias joins the fp32 sum before its one rounding
                if (n + 3 < N) {
                    v += v4f{__uint_as_float(bv.x << 16), __uint_as_float(bv.x & 0xFFFF0000u),
                             __uint_as_float(bv.y << 16), __uint_as_float(bv.y & 0xFFFF0000u)};
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N) v[r] += __uint_as_float((uint32_t)bias[n + r] << 16);
                }
            }
            if (OUT_BF16) {
                uint16_t* yr = reinterpret_cast<uint16_t*>(y) + (int64_t)m * N;
                if (n + 3 < N && (N % 4) == 0 && (reinterpret_cast<uintptr_t>(y) % 8) == 0) {
                    *reinterpret_cast<uint2*>(yr + n) =
                        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N) yr[n + r] = (uint16_t)f32_to_bf16_rne(v[r]);
                }
            } else {
                float* yr = reinterpret_cast<float*>(y) + (int64_t)m * N;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N) yr[n + r] = v[r];
            }
        }
    };

    // 4. tiles: slot i % TPW holds tile blockIdx.x + i*stride.  When every
    //    tile of the workgroup is already in flight (N <= 16 * TPW * grid),
    //    straight-line code: in the loop below the compiler copies the
    //    loop-carried slots, and each copy waits for its loads, so the first
    //    MFMA waited for all of them.
    if (ntiles <= TPW * stride) {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int t = blockIdx.x + i * stride;
            if (t >= ntiles) break;
            v4f acc[MT];
            compute(slot[i], acc);
            finish(t, i & 1, acc, bslot[i]);
        }
        return;
    }
    //    Otherwise a slot, once consumed, is refilled with the tile TPW
    //    further on.
    int k = 0;
    for (int base = blockIdx.x; base < ntiles; base += TPW * stride) {
#pragma unroll
        for (int i = 0; i < TPW; ++i, ++k) {
            const int t = base + i * stride;
            if (t >= ntiles) break;
            v4f acc[MT];
            compute(slot[i], acc);
            const uint2 bv = bslot[i];
            if (t + TPW * stride < ntiles) {
                bslot[i] = load_bias(t + TPW * stride);
                load_block<SPW, NW, MASK>(slot[i], w, ws, tile_row(t + TPW * stride), nkb);
            }
            finish(t, k & 1, acc, bv);
        }
    }
}

}  // namespace skinny

bool skinny_gemm_supported(int64_t M, int64_t N, int64_t K, const void* x, const void* x_scales,
                           const void* w_scales) {
    const bool aligned = (reinterpret_cast<uintptr_t>(x_scales) % 16) == 0 &&
                         (reinterpret_cast<uintptr_t>(w_scales) % 16) == 0 &&
                         (reinterpret_cast<uintptr_t>(x) % 16) == 0;
    return M >= 1 && M <= 64 && (K == 2048 || K == 4096) && N >= 16 && aligned;
}

// Other K (a multiple of 512 up to 16384): eight wavefronts, SPW = ceil(K /
// 4096) super-steps each, those past K masked off; the register file holds
// SPW x (MT activation blocks + TPW weight tiles) x 20 registers, which sets
// the largest M and the tiles in flight per SPW (any_k_config).
struct AnyK {
    int spw, mt_max;
};
static AnyK any_k_config(int64_t K) {
    const int nss = (int)(K / 512);
    const int spw = (nss + 7) / 8;
    static const int mt_max[5] = {0, 4, 4, 2, 1};
    return AnyK{spw, spw >= 1 && spw <= 4 ? mt_max[spw] : 0};
}

bool skinny_any_k_supported(int64_t M, int64_t N, int64_t K, const void* x, const void* x_scales,
                            const void* w_scales) {
    const bool aligned = (reinterpret_cast<uintptr_t>(x_scales) % 16) == 0 &&
                         (reinterpret_cast<uintptr_t>(w_scales) % 16) == 0 &&
                         (reinterpret_cast<uintptr_t>(x) % 16) == 0;
    // K <= 2048 keeps most of the eight waves idle (K = 1024, N = 4096, M = 16:
    // 4.2 us against the generic kernel's 3.8); K = 2048 and 4096 have kernels
    // of their own
    if (K % 512 != 0 || K < 2560 || K > 16384 || K == 4096 || N < 16 || M < 1 || !aligned)
        return false;
    return M <= 16 * any_k_config(K).mt_max;
}

// ldx > 0: `a` is bf16 activations [M][ldx] (as unused), quantized in the kernel.
// Shapes the act-quant + GEMM launch serves: those of the skinny GEMM with
// one 16-row activation block (the raw bf16 share of a wave, 64 registers a
// lane at one super-step, has to fit beside the weight tiles in flight),
// bf16 rows 16-byte aligned.
constexpr int64_t LINEAR_FUSED_MAX = 16;

bool linear_skinny_shape(int64_t M, int64_t N, int64_t K) {
    return M >= 1 && M <= LINEAR_FUSED_MAX && (K == 2048 || K == 4096) && N >= 16;
}

// Weight tiles in flight per wave: enough that 256 workgroups cover the
// tiles (one each up to 4096 rows, two up to 8192, else three).  Fewer
// workgroups, each with more tiles in flight, measured slower: 6.15 against
// 4.31 us at N = 4096, K = 4096, M = 1.
static int tiles_per_wave(int64_t N, int tpw_max) {
    const int64_t ntiles = (N + 15) / 16;
    const int tpw = ntiles <= 256 ? 1 : ntiles <= 512 ? 2 : 3;
    return tpw < tpw_max ? tpw : tpw_max;
}

template <int MT, int SPW, int NW, int TPW, bool A8>
static hipError_t launch_tpw(const uint8_t* a, const uint8_t* as, int64_t ldx, const uint8_t* b,
                             const uint8_t* bs, int64_t M, int64_t N, int64_t K, void* y,
                             const uint16_t* bias, bool out_bf16, hipStream_t stream,
                             bool uos) {
    const int ntiles = (int)((N + 15) / 16);
    int grid = (ntiles + TPW - 1) / TPW;
    if (grid > 256) grid = 256;
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(64 * NW), 0, stream, a, as, ldx, b, bs,
                           (int)M, (int)N, (int)K, y, bias);
        return hipGetLastError();
    };
    using namespace skinny;
    if (ldx > 0) {
        // the bf16 form exists for one block at one super-step per wave only
        if constexpr (MT == 1 && SPW == 1) {
            if constexpr (A8)
                return out_bf16 ? go(gemm_skinny_kernel<MT, SPW, NW, TPW, true, true, false, true>)
                                : go(gemm_skinny_kernel<MT, SPW, NW, TPW, false, true, false, true>);
            if (uos)
                return out_bf16 ? go(gemm_skinny_kernel<MT, SPW, NW, TPW, true, true, true>)
                                : go(gemm_skinny_kernel<MT, SPW, NW, TPW, false, true, true>);
            return out_bf16 ? go(gemm_skinny_kernel<MT, SPW, NW, TPW, true, true>)
                            : go(gemm_skinny_kernel<MT, SPW, NW, TPW, false, true>);
        }
        return hipErrorInvalidValue;
    }
    if constexpr (A8)
        return out_bf16 ? go(gemm_skinny_kernel<MT, SPW, NW, TPW, true, false, false, true>)
                        : go(gemm_skinny_kernel<MT, SPW, NW, TPW, false, false, false, true>);
    return out_bf16 ? go(gemm_skinny_kernel<MT, SPW, NW, TPW, true, false>)
                    : go(gemm_skinny_kernel<MT, SPW, NW, TPW, false, false>);
}

template <int MT, int SPW, int NW, bool A8 = false>
static hipError_t launch_mt(const uint8_t* a, const uint8_t* as, int64_t ldx, const uint8_t* b,
                            const uint8_t* bs, int64_t M, int64_t N, int64_t K, void* y,
                            const uint16_t* bias, bool out_bf16, hipStream_t stream,
                            bool uos = false) {
    switch (tiles_per_wave(N, 3)) {
        case 1: return launch_tpw<MT, SPW, NW, 1, A8>(a, as, ldx, b, bs, M, N, K, y, bias,
                                                       out_bf16, stream, uos);
        case 2: return launch_tpw<MT, SPW, NW, 2, A8>(a, as, ldx, b, bs, M, N, K, y, bias,
                                                       out_bf16, stream, uos);
        default: return launch_tpw<MT, SPW, NW, 3, A8>(a, as, ldx, b, bs, M, N, K, y, bias,
                                                        out_bf16, stream, uos);
    }
}

// K = 4096: NW super-steps of 512 K per wave pass (SPW = 8 / NW each);
// K = 2048: four waves, one super-step each.
template <int NW4096, bool A8 = false>
static hipError_t launch_k(const uint8_t* a, const uint8_t* as, int64_t ldx, const uint8_t* b,
                           const uint8_t* bs, int64_t M, int64_t N, int64_t K, void* y,
                           const uint16_t* bias, bool out_bf16, hipStream_t stream) {
    constexpr int SPW = 8 / NW4096;
    if (K == 2048) {
        if (M <= 16)
            return launch_mt<1, 1, 4, A8>(a, as, ldx, b, bs, M, N, K, y, bias, out_bf16,
                                             stream);
        if (M <= 32)
            return launch_mt<2, 1, 4, A8>(a, as, ldx, b, bs, M, N, K, y, bias, out_bf16,
                                             stream);
        if (M <= 48)
            return launch_mt<3, 1, 4, A8>(a, as, ldx, b, bs, M, N, K, y, bias, out_bf16,
                                             stream);
        return launch_mt<4, 1, 4, A8>(a, as, ldx, b, bs, M, N, K, y, bias, out_bf16, stream);
    }
    if (M <= 16)
        return launch_mt<1, SPW, NW4096, A8>(a, as, ldx, b, bs, M, N, K, y, bias, out_bf16,
                                                stream);
    if (M <= 32)
        return launch_mt<2, SPW, NW4096, A8>(a, as, ldx, b, bs, M, N, K, y, bias, out_bf16,
                                                stream);
    if (M <= 48)
        return launch_mt<3, SPW, NW4096, A8>(a, as, ldx, b, bs, M, N, K, y, bias, out_bf16,
                                                stream);
    // four activation blocks of E4M3 (twice the E2M1 registers) spill at two
    // wavefronts per SIMD: one wavefront per SIMD, two super-steps each
    if constexpr (A8)
        return launch_mt<4, 2, 4, true>(a, as, ldx, b, bs, M, N, K, y, bias, out_bf16, stream);
    else
        return launch_mt<4, SPW, NW4096>(a, as, ldx, b, bs, M, N, K, y, bias, out_bf16, stream);
}

template <int MT, int SPW, int TPW>
static hipError_t launch_masked_tpw(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                                    const uint8_t* bs, int64_t M, int64_t N, int64_t K, void* y,
                                    const uint16_t* bias, bool out_bf16, hipStream_t stream) {
    const int ntiles = (int)((N + 15) / 16);
    int grid = (ntiles + TPW - 1) / TPW;
    if (grid > 256) grid = 256;
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(512), 0, stream, a, as, (int64_t)0, b, bs,
                           (int)M, (int)N, (int)K, y, bias);
        return hipGetLastError();
    };
    using namespace skinny;
    return out_bf16 ? go(gemm_skinny_kernel<MT, SPW, 8, TPW, true, false, false, false, true>)
                    : go(gemm_skinny_kernel<MT, SPW, 8, TPW, false, false, false, false, true>);
}

// TPW_MAX: the most tiles in flight the register file holds at this MT, SPW
template <int MT, int SPW, int TPW_MAX>
static hipError_t launch_masked(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                                const uint8_t* bs, int64_t M, int64_t N, int64_t K, void* y,
                                const uint16_t* bias, bool out_bf16, hipStream_t stream) {
    const int tpw = tiles_per_wave(N, TPW_MAX);
    if constexpr (TPW_MAX >= 3)
        if (tpw == 3)
            return launch_masked_tpw<MT, SPW, 3>(a, as, b, bs, M, N, K, y, bias, out_bf16, stream);
    if constexpr (TPW_MAX >= 2)
        if (tpw == 2)
            return launch_masked_tpw<MT, SPW, 2>(a, as, b, bs, M, N, K, y, bias, out_bf16, stream);
    return launch_masked_tpw<MT, SPW, 1>(a, as, b, bs, M, N, K, y, bias, out_bf16, stream);
}

hipError_t launch_gemm_skinny_any_k(const uint8_t* a_codes, const uint8_t* a_scales,
                                    const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                    int64_t N, int64_t K, void* y, const uint16_t* bias,
                                    bool out_bf16, hipStream_t stream) {
    const int mt = (int)((M + 15) / 16);
    auto go = [&](auto launch) {
        return launch(a_codes, a_scales, b_codes, b_scales, M, N, K, y, bias, out_bf16, stream);
    };
    switch (any_k_config(K).spw * 8 + mt) {
        case 1 * 8 + 1: return go(launch_masked<1, 1, 3>);
        case 1 * 8 + 2: return go(launch_masked<2, 1, 3>);
        case 1 * 8 + 3: return go(launch_masked<3, 1, 3>);
        case 1 * 8 + 4: return go(launch_masked<4, 1, 3>);
        case 2 * 8 + 1: return go(launch_masked<1, 2, 3>);
        case 2 * 8 + 2: return go(launch_masked<2, 2, 3>);
        case 2 * 8 + 3: return go(launch_masked<3, 2, 2>);
        case 2 * 8 + 4: return go(launch_masked<4, 2, 1>);
        case 3 * 8 + 1: return go(launch_masked<1, 3, 2>);
        case 3 * 8 + 2: return go(launch_masked<2, 3, 1>);
        case 4 * 8 + 1: return go(launch_masked<1, 4, 1>);
        default: return hipErrorInvalidValue;
    }
}

// two wavefronts per SIMD (at K = 4096; measured 0.3-0.5 us less than one
// per SIMD at every M)
hipError_t launch_gemm_skinny(const uint8_t* a_codes, const uint8_t* a_scales,
                              const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                              int64_t N, int64_t K, void* y, const uint16_t* bias,
                              bool out_bf16, hipStream_t stream) {
    return launch_k<8>(a_codes, a_scales, 0, b_codes, b_scales, M, N, K, y, bias, out_bf16,
                       stream);
}

hipError_t launch_gemm_skinny_w4a8(const uint8_t* a_codes, const uint8_t* a_scales,
                                   const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                   int64_t N, int64_t K, void* y, const uint16_t* bias,
                                   bool out_bf16, hipStream_t stream) {
    return launch_k<8, true>(a_codes, a_scales, 0, b_codes, b_scales, M, N, K, y, bias, out_bf16,
                             stream);
}

hipError_t launch_linear_skinny_w4a8(const uint16_t* x, int64_t ldx, const uint8_t* b_codes,
                                     const uint8_t* b_scales, int64_t M, int64_t N, int64_t K,
                                     void* y, const uint16_t* bias, bool out_bf16,
                                     hipStream_t stream) {
    const uint8_t* a = reinterpret_cast<const uint8_t*>(x);
    if (K == 4096)
        return launch_mt<1, 1, 8, true>(a, nullptr, ldx, b_codes, b_scales, M, N, K, y, bias,
                                        out_bf16, stream);
    return launch_mt<1, 1, 4, true>(a, nullptr, ldx, b_codes, b_scales, M, N, K, y, bias,
                                    out_bf16, stream);
}

hipError_t launch_linear_skinny(const uint16_t* x, int64_t ldx, const uint8_t* b_codes,
                                const uint8_t* b_scales, int64_t M, int64_t N, int64_t K,
                                void* y, const uint16_t* bias, bool out_bf16, bool uos,
                                hipStream_t stream) {
    // M <= 16: one activation block; one super-step per wave (eight waves at
    // K = 4096, four at 2048)
    const uint8_t* a = reinterpret_cast<const uint8_t*>(x);
    if (K == 4096)
        return launch_mt<1, 1, 8>(a, nullptr, ldx, b_codes, b_scales, M, N, K, y, bias, out_bf16,
                                  stream, uos);
    return launch_mt<1, 1, 4>(a, nullptr, ldx, b_codes, b_scales, M, N, K, y, bias, out_bf16,
                              stream, uos);
}

}  // namespace mx
