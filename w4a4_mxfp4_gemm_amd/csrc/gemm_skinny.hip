// gemm_skinny.hip -- weight-streaming MXFP4 GEMM for few activation rows
// (decode, M <= 64).  The time is the HBM read of the weights, so the kernel
// is organised around keeping enough weight bytes in flight:
//
//  * one workgroup (4 wavefronts) per CU, persistent over 16-row weight tiles
//    (tile t, t + grid, t + 2 grid, ...);
//  * the 4 wavefronts split K in four interleaved parts; each issues its
//    whole share of a tile (SPW 512-K super-steps: 4 x 16 B of codes and 4
//    scale bytes per lane each) one tile ahead of its MFMAs;
//  * the activations (all M rows, padded to MT x 16, full K) are staged once
//    into LDS and read from there by every tile;
//  * partial tiles of the 4 wavefronts are summed through LDS in a fixed
//    order (deterministic), then stored.
//
// MFMA: v_mfma_scale_f32_16x16x128_f8f6f4, weight rows as the A operand, so
// lane l's accumulator holds output m = l%16 of its 16-row activation block
// and n = 4(l/16) + r.  Within a 512-K super-step (16 MX blocks), MFMA q
// covers blocks 4q..4q+3 with lane group g = l/16 on block 4q+g, so each
// 16-byte weight load instruction reads 16 rows x 64 contiguous bytes (few,
// full memory requests).  A lane's scale byte for MFMA q is byte 4q+g of the
// row's 16 scale bytes of the super-step: loaded as 16 bytes, shifted by 8g.
//
// LDS (activations): codes [MT*16 rows][K/2] with the 16-byte chunk c of row
// m stored at c ^ (m & 15) (conflict-free reads of 16 rows by 16 lanes);
// scales [MT*16][K/32]; reduction buffer 3 x MT x 1 KiB.  Each wave reads its
// activation fragments once and keeps them in registers for all its tiles.
#include "mx_device.h"
#include "launch.h"

namespace mx {
namespace skinny {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
#define AS_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int KMAX = 4096;

// Activation rows are packed densely (row stride K/2 and K/32 bytes).
template <int MT>
struct Smem {
    uint8_t codes[MT * 16 * (KMAX / 2)];     // swizzled 16-byte chunks
    uint8_t scales[MT * 16 * (KMAX / 32)];
    float red[3][MT][4][64];
};

// One wavefront's share of a weight tile: SPW super-steps x (4 x 16 B + 4
// scale bytes).
template <int SPW>
struct WFrag {
    v4u c[SPW][4];
    v4u s[SPW];          // the row's 16 scale bytes of each super-step
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

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Weight loads of one tile for this wave: super-step ss = wave + 4 j; load q
// of a super-step brings blocks 4q..4q+3 (lane group g: block 4q+g).
template <int SPW>
__device__ __forceinline__ void load_w(WFrag<SPW>& f, const uint8_t* w, const uint8_t* ws,
                                       int64_t row, int nkb) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const uint8_t* crow = w + row * (int64_t)nkb * 16;
    const uint8_t* srow = ws + row * (int64_t)nkb;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        const int kb0 = (wave + 4 * j) * 16;
        const v4u* p = reinterpret_cast<const v4u*>(crow + (int64_t)kb0 * 16 + 16 * g);
#pragma unroll
        for (int q = 0; q < 4; ++q) f.c[j][q] = __builtin_nontemporal_load(p + 4 * q);
        f.s[j] = *reinterpret_cast<const v4u*>(srow + kb0);
    }
}

template <int OFF>
__device__ __forceinline__ void ds_read_b128(v4u& r, uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_read_u8(uint32_t& r, uint32_t addr) {
    asm volatile("ds_read_u8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
}

// MT x 16 activation rows x 4 super-step quarters of this wave, from LDS.
template <int MT, int SPW>
struct AFrag {
    v4u c[SPW][MT][4];
    uint32_t s[SPW][MT][4];
};

// Lane-constant LDS addresses of the activation fragments: code chunk q of
// super-step j, row block 0 (row blocks are `mt_codes` / `mt_scales` apart).
struct AAddr {
    uint32_t c[4], s, mt_codes, mt_scales;
};

template <int J, int MT, int SPW>
__device__ __forceinline__ void read_a_step(AFrag<MT, SPW>& a, const AAddr& ad) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const uint32_t dc = (uint32_t)mt * ad.mt_codes;
        ds_read_b128<J * 1024>(a.c[J][mt][0], ad.c[0] + dc);
        ds_read_b128<J * 1024>(a.c[J][mt][1], ad.c[1] + dc);
        ds_read_b128<J * 1024>(a.c[J][mt][2], ad.c[2] + dc);
        ds_read_b128<J * 1024>(a.c[J][mt][3], ad.c[3] + dc);
        ds_read_u8<J * 64 + 0>(a.s[J][mt][0], ad.s + (uint32_t)mt * ad.mt_scales);
        ds_read_u8<J * 64 + 4>(a.s[J][mt][1], ad.s + (uint32_t)mt * ad.mt_scales);
        ds_read_u8<J * 64 + 8>(a.s[J][mt][2], ad.s + (uint32_t)mt * ad.mt_scales);
        ds_read_u8<J * 64 + 12>(a.s[J][mt][3], ad.s + (uint32_t)mt * ad.mt_scales);
    }
}

template <int MT, int SPW>
__device__ __forceinline__ void read_a(AFrag<MT, SPW>& a, const AAddr& ad) {
    read_a_step<0>(a, ad);
    if constexpr (SPW > 1) read_a_step<1>(a, ad);
    static_assert(SPW <= 2, "at most two super-steps per wave");
}

template <int MT, int SPW, int TPW, bool OUT_BF16>
__global__ __launch_bounds__(256, 1) void gemm_skinny_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ xs,
    // no __restrict__ on the weights: with it the compiler may sink the weight
    // loads below the activation wait, serialising the two memory latencies
    const uint8_t* w, const uint8_t* ws, int M, int N, int K, void* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) Smem<MT> sm;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int nkb = K / 32;
    const int ntiles = (N + 15) / 16;
    const int stride = gridDim.x;

    // 1. activations -> LDS with buffer loads that write LDS directly: codes in
    //    1 KiB slices (chunk c of row m goes to position c ^ (m & 15)), scales
    //    one dword per lane.  Rows m >= M repeat row M-1 (their outputs are
    //    never stored).  Issued before the weights so that waiting for them
    //    never waits for weight loads.
    {
        const auto rc = make_rsrc(x, (uint32_t)((int64_t)M * (K / 2)));
        const auto rs = make_rsrc(xs, (uint32_t)((int64_t)M * nkb));
        const int row_bytes = K / 2;
        constexpr int CODE_SLICES = MT * 16 * (KMAX / 2) / 1024;   // upper bound
#pragma unroll
        for (int i = 0; i < CODE_SLICES / 4; ++i) {
            const int o = (i * 4 + wave) * 1024 + lane * 16;     // LDS byte offset
            const int m = o / row_bytes;
            if (m < MT * 16) {
                const int p = (o - m * row_bytes) / 16;
                const int c = p ^ (m & 15);
                const uint32_t src = (uint32_t)(min(m, M - 1) * row_bytes + 16 * c);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rc, AS_LDS((lds_u8*)sm.codes + (i * 4 + wave) * 1024), 16, src, 0, 0, 0);
            }
        }
        constexpr int SCALE_SLICES = MT * 16 * (KMAX / 32) / 256;
#pragma unroll
        for (int i = 0; i < (SCALE_SLICES + 3) / 4; ++i) {
            const int sl = i * 4 + wave;
            const int o = sl * 256 + lane * 4;
            const int m = o / nkb;
            if (sl < SCALE_SLICES && m < MT * 16) {
                const uint32_t src = (uint32_t)(min(m, M - 1) * nkb + (o - m * nkb));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, AS_LDS((lds_u8*)sm.scales + sl * 256), 4, src, 0, 0, 0);
            }
        }
    }

    auto tile_row = [&](int t) {
        const int tt = t < ntiles ? t : ntiles - 1;     // surplus loads: any valid row
        return (int64_t)min(tt * 16 + r16, N - 1);
    };

    // 2. weights: TPW tiles in flight per wave
    WFrag<SPW> slot[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) load_w<SPW>(slot[i], w, ws, tile_row(blockIdx.x + i * stride), nkb);
    __builtin_amdgcn_sched_barrier(0);   // issue every weight load before waiting

    // 3. activations landed (only the weight loads may still be in flight)
    wait_vm<TPW * SPW * 5>();
    lds_barrier();

    // lane-constant LDS addresses of this wave's activation fragments: lane
    // (r16, g) reads row r16 of each 16-row block, code chunks (wave + 4j)*16 +
    // 4q + g at swizzled position ^ r16, and scale bytes (wave + 4j)*16 + 4q + g.
    AAddr ad;
    {
        const uint32_t cbase = (uint32_t)(uintptr_t)(lds_u8*)sm.codes;
        const uint32_t sbase = (uint32_t)(uintptr_t)(lds_u8*)sm.scales;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            ad.c[q] = cbase + (uint32_t)(r16 * (K / 2) + wave * 256 + 16 * ((4 * q + g) ^ r16));
        ad.s = sbase + (uint32_t)(r16 * nkb + wave * 16 + g);
        ad.mt_codes = (uint32_t)(16 * (K / 2));
        ad.mt_scales = (uint32_t)(16 * nkb);
    }
    AFrag<MT, SPW> a;
    read_a<MT, SPW>(a, ad);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // make every use of the fragments depend on the wait
#pragma unroll
    for (int j = 0; j < SPW; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            asm volatile("" : "+v"(a.c[j][mt][0]), "+v"(a.c[j][mt][1]), "+v"(a.c[j][mt][2]),
                              "+v"(a.c[j][mt][3]));
            asm volatile("" : "+v"(a.s[j][mt][0]), "+v"(a.s[j][mt][1]), "+v"(a.s[j][mt][2]),
                              "+v"(a.s[j][mt][3]));
        }

    auto finish = [&](int t, v4f (&acc)[MT]) {
        if (wave > 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) sm.red[wave - 1][mt][r][lane] = acc[mt][r];
        }
        lds_barrier();
        if (wave == 0) {
#pragma unroll
            for (int q = 0; q < 3; ++q)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[mt][r] += sm.red[q][mt][r][lane];
            const int n = t * 16 + 4 * g;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = mt * 16 + r16;
                if (m >= M) continue;
                const v4f v = acc[mt];
                if (OUT_BF16) {
                    uint16_t* yr = reinterpret_cast<uint16_t*>(y) + (int64_t)m * N;
                    if (n + 3 < N && (N % 4) == 0 &&
                        (reinterpret_cast<uintptr_t>(y) % 8) == 0) {
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
        }
        lds_barrier();
    };

    auto compute = [&](const WFrag<SPW>& f, v4f (&acc)[MT]) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            // this lane's weight scale byte for MFMA q is byte 4q+g: word q >> 8g
            const uint32_t sh = 8u * (uint32_t)g;
            const uint32_t s0 = f.s[j][0] >> sh, s1 = f.s[j][1] >> sh;
            const uint32_t s2 = f.s[j][2] >> sh, s3 = f.s[j][3] >> sh;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                acc[mt] = mfma_s<0>(f.c[j][0], a.c[j][mt][0], acc[mt], s0, a.s[j][mt][0]);
                acc[mt] = mfma_s<0>(f.c[j][1], a.c[j][mt][1], acc[mt], s1, a.s[j][mt][1]);
                acc[mt] = mfma_s<0>(f.c[j][2], a.c[j][mt][2], acc[mt], s2, a.s[j][mt][2]);
                acc[mt] = mfma_s<0>(f.c[j][3], a.c[j][mt][3], acc[mt], s3, a.s[j][mt][3]);
            }
        }
    };

    // 4. tiles: slot i % TPW holds tile blockIdx.x + i*stride; once consumed it
    //    is refilled with the tile TPW further on.
    for (int base = blockIdx.x; base < ntiles; base += TPW * stride) {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int t = base + i * stride;
            if (t >= ntiles) break;
            v4f acc[MT];
            compute(slot[i], acc);
            if (t + TPW * stride < ntiles)
                load_w<SPW>(slot[i], w, ws, tile_row(t + TPW * stride), nkb);
            finish(t, acc);
        }
    }
}

}  // namespace skinny

bool skinny_gemm_supported(int64_t M, int64_t N, int64_t K, const void* x, const void* x_scales,
                           const void* w_scales) {
    const bool aligned = (reinterpret_cast<uintptr_t>(x_scales) % 4) == 0 &&
                         (reinterpret_cast<uintptr_t>(w_scales) % 16) == 0 &&
                         (reinterpret_cast<uintptr_t>(x) % 16) == 0;
    return M >= 1 && M <= 64 && (K == 2048 || K == 4096) && N >= 16 && aligned;
}

template <int MT, int SPW>
static hipError_t launch_mt(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                            const uint8_t* bs, int64_t M, int64_t N, int64_t K, void* y,
                            bool out_bf16, hipStream_t stream) {
    // tiles in flight per wave: all of a workgroup's tiles when they fit
    constexpr int TPW = 3;
    const int ntiles = (int)((N + 15) / 16);
    int grid = (ntiles + TPW - 1) / TPW;
    if (grid > 256) grid = 256;
    if (out_bf16)
        hipLaunchKernelGGL((skinny::gemm_skinny_kernel<MT, SPW, TPW, true>), dim3(grid),
                           dim3(256), 0, stream, a, as, b, bs, (int)M, (int)N, (int)K, y);
    else
        hipLaunchKernelGGL((skinny::gemm_skinny_kernel<MT, SPW, TPW, false>), dim3(grid),
                           dim3(256), 0, stream, a, as, b, bs, (int)M, (int)N, (int)K, y);
    return hipGetLastError();
}

template <int SPW>
static hipError_t launch_spw(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                             const uint8_t* bs, int64_t M, int64_t N, int64_t K, void* y,
                             bool out_bf16, hipStream_t stream) {
    if (M <= 16) return launch_mt<1, SPW>(a, as, b, bs, M, N, K, y, out_bf16, stream);
    if (M <= 32) return launch_mt<2, SPW>(a, as, b, bs, M, N, K, y, out_bf16, stream);
    if (M <= 48) return launch_mt<3, SPW>(a, as, b, bs, M, N, K, y, out_bf16, stream);
    return launch_mt<4, SPW>(a, as, b, bs, M, N, K, y, out_bf16, stream);
}

hipError_t launch_gemm_skinny(const uint8_t* a_codes, const uint8_t* a_scales,
                              const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                              int64_t N, int64_t K, void* y, bool out_bf16, hipStream_t stream) {
    if (K == 2048)
        return launch_spw<1>(a_codes, a_scales, b_codes, b_scales, M, N, K, y, out_bf16, stream);
    return launch_spw<2>(a_codes, a_scales, b_codes, b_scales, M, N, K, y, out_bf16, stream);
}

}  // namespace mx
