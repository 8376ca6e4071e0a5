// moe_epilogue.hip -- the top-k combine that closes an MoE layer on gfx950.
//
// After the down projection the expert outputs sit in expert-sorted rows;
// each token's output row is the weighted sum of its k routed rows.  A
// streaming gather-reduce bound by HBM: every sorted row is read once
// (non-temporal 16-byte loads, contiguous across a wavefront) and every
// output row written once.  No LDS, no atomics, so the result is the same
// on every run.
#include "mx_device.h"
#include "launch.h"

namespace mx {

namespace {

typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int COMBINE_BATCH = 8;   // routed rows loaded before any arithmetic

// One thread owns 8 consecutive columns of one token's output; blockIdx.y
// walks tokens.  Accumulation is fp32, one fma per routed row in the order
// the routing table lists them (error at most topk * 2^-24 * sum |w y|), then
// one rounding to the output type.  Row indices are clamped to [0, R), so a
// bad table gives wrong sums but never a read outside y.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void moe_combine_kernel(
    const uint16_t* __restrict__ y, int64_t ldy, int64_t R, const int32_t* __restrict__ rows,
    const float* __restrict__ weights, int64_t T, int topk, int64_t H,
    void* __restrict__ out) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= H / 8) return;
    for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < topk; j0 += COMBINE_BATCH) {
            v4u_t v[COMBINE_BATCH];
            float w[COMBINE_BATCH];
#pragma unroll
            for (int j = 0; j < COMBINE_BATCH; ++j) {
                if (j0 + j < topk) {
                    int64_t r = rows[t * topk + j0 + j];
                    r = r < 0 ? 0 : (r >= R ? R - 1 : r);
                    v[j] = __builtin_nontemporal_load(
                        reinterpret_cast<const v4u_t*>(y + r * ldy + c * 8));
                    w[j] = weights[t * topk + j0 + j];
                }
            }
#pragma unroll
            for (int j = 0; j < COMBINE_BATCH; ++j) {
                if (j0 + j < topk) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[2 * i] = __builtin_fmaf(w[j], __uint_as_float(v[j][i] << 16),
                                                    acc[2 * i]);
                        acc[2 * i + 1] = __builtin_fmaf(
                            w[j], __uint_as_float(v[j][i] & 0xFFFF0000u), acc[2 * i + 1]);
                    }
                }
            }
        }
        if constexpr (OUT_BF16) {
            typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
            typedef float f32x8_t __attribute__((ext_vector_type(8)));
            const f32x8_t a{acc[0], acc[1], acc[2], acc[3], acc[4], acc[5], acc[6], acc[7]};
            *reinterpret_cast<v4u_t*>(static_cast<uint16_t*>(out) + t * H + c * 8) =
                __builtin_bit_cast(v4u_t, __builtin_convertvector(a, bf16x8_t));
        } else {
            v4f_t* o = reinterpret_cast<v4f_t*>(static_cast<float*>(out) + t * H + c * 8);
            o[0] = v4f_t{acc[0], acc[1], acc[2], acc[3]};
            o[1] = v4f_t{acc[4], acc[5], acc[6], acc[7]};
        }
    }
}

}  // namespace

hipError_t launch_moe_combine(const uint16_t* y, int64_t ldy, int64_t R, const int32_t* rows,
                              const float* weights, int64_t T, int64_t topk, int64_t H,
                              void* out, bool out_bf16, hipStream_t stream) {
    const int64_t gx = (H / 8 + 255) / 256;
    const int64_t gy = T > 65535 ? 65535 : T;
    const dim3 grid((unsigned)gx, (unsigned)gy);
    if (out_bf16)
        hipLaunchKernelGGL(moe_combine_kernel<true>, grid, dim3(256), 0, stream, y, ldy, R, rows,
                           weights, T, (int)topk, H, out);
    else
        hipLaunchKernelGGL(moe_combine_kernel<false>, grid, dim3(256), 0, stream, y, ldy, R,
                           rows, weights, T, (int)topk, H, out);
    return hipGetLastError();
}

}  // namespace mx
