// quant_kernels.hip -- NVFP4 -> MXFP4 requant and bf16 -> MXFP4 activation
// quantization for gfx950.
//
// Both are streaming kernels bound by HBM bandwidth: every byte is read once
// with 16-byte loads that are contiguous across a wavefront and written once
// with contiguous stores.  No LDS, no atomics.
#include "mx_device.h"
#include "launch.h"

namespace mx {

// ---------------------------------------------------------------------------
// Activation quantization.  One thread owns 8 consecutive bf16 values (one
// 16-byte load); the 4 lanes of an aligned quad own one 32-element MX block
// and share its amax through DPP.  Quads are laid out row-major over
// (row, block), so a wavefront reads 1 KiB of one row contiguously.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void act_quant_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const int32_t* __restrict__ row_index,
    int64_t M, int64_t K, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const int64_t quarters_per_row = K / 8;
    const int64_t total = M * quarters_per_row;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
        const int64_t m = t / quarters_per_row;
        const int64_t kq = t - m * quarters_per_row;          // which 8-element group
        const int64_t src = row_index ? (int64_t)row_index[m] : m;
        const uint4 raw = *reinterpret_cast<const uint4*>(x + src * ldx + kq * 8);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};

        // amax over the 8 values as bf16 magnitudes (monotone as integers);
        // NaN and Inf patterns sort above every finite value.
        uint32_t amax = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
            amax = max(amax, max(lo, hi));
        }
        amax = quad_max_u32(amax);
        const uint32_t byte = mx_scale_from_amax_bits(amax << 16);
        const int neg_exp = 127 - (int)byte;

        uint32_t packed = 0;
        if (byte != 255u) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t c0 = e2m1_encode(bf16_to_f32(w[i] & 0xFFFFu), neg_exp);
                uint32_t c1 = e2m1_encode(bf16_to_f32(w[i] >> 16), neg_exp);
                packed |= (c0 | (c1 << 4)) << (8 * i);
            }
        }
        *reinterpret_cast<uint32_t*>(codes + m * (K / 2) + kq * 4) = packed;
        if ((kq & 3) == 0) scales[m * (K / 32) + kq / 4] = (uint8_t)byte;
    }
}

// ---------------------------------------------------------------------------
// NVFP4 -> MXFP4 requant.  One thread owns one 32-element MX block: 16 code
// bytes (one 16-byte load), the two E4M3 scales of NVFP4 blocks 2j and 2j+1,
// and the tensor's fp32 global scale.  Values are materialised in registers
// only: v = fl32(fl32(e2m1 * e4m3) * g), optionally rounded to bf16.
// ---------------------------------------------------------------------------
template <bool BF16_INTERMEDIATE>
__global__ __launch_bounds__(256) void requant_kernel(
    const uint8_t* __restrict__ nv_codes, const uint8_t* __restrict__ nv_scales,
    const float* __restrict__ nv_global, int64_t T, int64_t N, int64_t K,
    uint8_t* __restrict__ mx_codes, uint8_t* __restrict__ mx_scales) {
    const int64_t blocks_per_tensor = N * (K / 32);
    const int64_t total = T * blocks_per_tensor;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < total; b += stride) {
        const int64_t t = b / blocks_per_tensor;
        const float g = nv_global[t];
        const uint4 raw = *reinterpret_cast<const uint4*>(nv_codes + b * 16);
        const uint32_t sc = *reinterpret_cast<const uint16_t*>(nv_scales + b * 2);
        const float s0 = e4m3_to_f32(sc & 0xFFu), s1 = e4m3_to_f32(sc >> 8);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};

        float v[32];
        uint32_t amax = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const uint32_t c = (w[i / 8] >> (4 * (i % 8))) & 15u;
            const float p = e2m1_to_f32(c) * (i < 16 ? s0 : s1);   // exact
            float x = p * g;                                         // one rounding
            if (BF16_INTERMEDIATE) x = bf16_to_f32(f32_to_bf16_rne(x));
            v[i] = x;
            amax = max(amax, __float_as_uint(x) & 0x7FFFFFFFu);
        }
        const uint32_t byte = mx_scale_from_amax_bits(amax);
        const int neg_exp = 127 - (int)byte;
        uint32_t out[4] = {0, 0, 0, 0};
        if (byte != 255u) {
#pragma unroll
            for (int i = 0; i < 32; ++i) out[i / 8] |= e2m1_encode(v[i], neg_exp) << (4 * (i % 8));
        }
        *reinterpret_cast<uint4*>(mx_codes + b * 16) = make_uint4(out[0], out[1], out[2], out[3]);
        mx_scales[b] = (uint8_t)byte;
    }
}

static int grid_for(int64_t threads_needed) {
    int64_t blocks = (threads_needed + 255) / 256;
    const int64_t cap = 256 * 64;     // enough waves to cover 256 CUs many times over
    if (blocks > cap) blocks = cap;
    return (int)(blocks < 1 ? 1 : blocks);
}

hipError_t launch_act_quant(const uint16_t* x, int64_t ldx, const int32_t* row_index,
                            int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                            hipStream_t stream) {
    const int64_t threads = M * (K / 8);
    hipLaunchKernelGGL(act_quant_kernel, dim3(grid_for(threads)), dim3(256), 0, stream,
                       x, ldx, row_index, M, K, codes, scales);
    return hipGetLastError();
}

hipError_t launch_requant(const uint8_t* nv_codes, const uint8_t* nv_scales,
                          const float* nv_global, int64_t T, int64_t N, int64_t K,
                          uint8_t* mx_codes, uint8_t* mx_scales, bool bf16_intermediate,
                          hipStream_t stream) {
    const int64_t threads = T * N * (K / 32);
    if (bf16_intermediate)
        hipLaunchKernelGGL(requant_kernel<true>, dim3(grid_for(threads)), dim3(256), 0, stream,
                           nv_codes, nv_scales, nv_global, T, N, K, mx_codes, mx_scales);
    else
        hipLaunchKernelGGL(requant_kernel<false>, dim3(grid_for(threads)), dim3(256), 0, stream,
                           nv_codes, nv_scales, nv_global, T, N, K, mx_codes, mx_scales);
    return hipGetLastError();
}

}  // namespace mx
