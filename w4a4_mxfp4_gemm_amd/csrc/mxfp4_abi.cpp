// mxfp4_abi.cpp -- the extern "C" entry points declared in include/mxfp4.h:
// argument validation, then one launch on the caller's stream.  Nothing here
// allocates, synchronises or keeps state.
#include "../../include/mxfp4.h"
#include "launch.h"

#include <stdint.h>

namespace {

constexpr int kVersion = 100;   // 0.1.0

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int from_hip(hipError_t e) { return e == hipSuccess ? MXFP4_OK : MXFP4_EHIP; }

int check_k(int64_t K) { return (K > 0 && K % 32 == 0) ? MXFP4_OK : MXFP4_EINVAL; }

// The linear call's workspace: codes [M][K/2], then scales [M][K/32] from the
// next 256-byte boundary.
size_t linear_codes_bytes(int64_t M, int64_t K) {
    return ((size_t)M * (size_t)(K / 2) + 255) / 256 * 256;
}

// MXFP8 codes: one byte per element
size_t fp8_codes_bytes(int64_t M, int64_t K) {
    return ((size_t)M * (size_t)K + 255) / 256 * 256;
}

int check_gemm_common(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                      const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* y,
                      int out_dtype, void* workspace, size_t workspace_bytes, uint32_t flags) {
    if (M < 0 || N <= 0 || check_k(K) != MXFP4_OK) return MXFP4_EINVAL;
    if (out_dtype != MXFP4_OUT_BF16 && out_dtype != MXFP4_OUT_FP32) return MXFP4_EINVAL;
    if (flags != 0) return MXFP4_EINVAL;
    if (workspace_bytes != 0 && workspace == nullptr) return MXFP4_EINVAL;
    if (M == 0) return MXFP4_OK;
    if (!a_codes || !a_scales || !b_codes || !b_scales || !y) return MXFP4_EINVAL;
    if (!aligned(a_codes, 16) || !aligned(b_codes, 16)) return MXFP4_EALIGN;
    if (!aligned(y, out_dtype == MXFP4_OUT_FP32 ? 4 : 2)) return MXFP4_EALIGN;
    return MXFP4_OK;
}

}  // namespace

namespace mx {

// The one-launch form (act-quant inside the skinny GEMM) is chosen by shape
// alone: the call requires every pointer alignment that form needs.
size_t linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || check_k(K) != MXFP4_OK) return 0;
    if (linear_skinny_shape(M, N, K)) return 0;
    return linear_codes_bytes(M, K) + (size_t)M * (size_t)(K / 32);
}

int check_linear_bf16(const void* x_bf16, int64_t ldx, int64_t M, int64_t N, int64_t K,
                      const uint8_t* b_codes, const uint8_t* b_scales, const void* bias_bf16,
                      void* y, int out_dtype, uint32_t flags) {
    if (M < 0 || N <= 0 || check_k(K) != MXFP4_OK || ldx < K) return MXFP4_EINVAL;
    if (out_dtype != MXFP4_OUT_BF16 && out_dtype != MXFP4_OUT_FP32) return MXFP4_EINVAL;
    if ((flags & ~(uint32_t)MXFP4_SCALE_UOS) != 0) return MXFP4_EINVAL;
    if (M == 0) return MXFP4_OK;
    if (!x_bf16 || !b_codes || !b_scales || !y) return MXFP4_EINVAL;
    if (!aligned(x_bf16, 16) || ldx % 8 != 0 || !aligned(b_codes, 16) || !aligned(b_scales, 16))
        return MXFP4_EALIGN;
    if (!aligned(y, out_dtype == MXFP4_OUT_FP32 ? 4 : 2)) return MXFP4_EALIGN;
    if (bias_bf16 && !aligned(bias_bf16, 16)) return MXFP4_EALIGN;
    return MXFP4_OK;
}

// Arguments checked by check_linear_bf16 (M > 0); workspace holds at least
// linear_workspace_bytes(M, N, K) bytes, 16-byte aligned.
int run_linear_bf16(const void* x_bf16, int64_t ldx, int64_t M, int64_t N, int64_t K,
                    const uint8_t* b_codes, const uint8_t* b_scales, const void* bias_bf16,
                    void* y, int out_dtype, uint8_t* workspace, uint32_t flags,
                    hipStream_t stream) {
    const bool out_bf16 = out_dtype == MXFP4_OUT_BF16;
    const bool uos = (flags & MXFP4_SCALE_UOS) != 0;
    const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
    const uint16_t* bias = static_cast<const uint16_t*>(bias_bf16);
    if (linear_skinny_shape(M, N, K))
        return from_hip(launch_linear_skinny(x, ldx, b_codes, b_scales, M, N, K, y, bias,
                                             out_bf16, uos, stream));
    // two launches through the workspace: the act-quant call, then the GEMM
    uint8_t* codes = workspace;
    uint8_t* scales = codes + linear_codes_bytes(M, K);
    const hipError_t e = launch_act_quant(x, ldx, nullptr, M, K, codes, scales, uos, stream);
    if (e != hipSuccess) return MXFP4_EHIP;
    return from_hip(launch_gemm(codes, scales, b_codes, b_scales, M, N, K, y, bias, out_bf16,
                                stream));
}

}  // namespace mx

extern "C" {

int mxfp4_requant_from_nvfp4(const uint8_t* nv_codes, const uint8_t* nv_scales,
                             const float* nv_global, int64_t T, int64_t N, int64_t K,
                             uint8_t* mx_codes, uint8_t* mx_scales, uint32_t flags,
                             hipStream_t stream) {
    if (T < 0 || N <= 0 || check_k(K) != MXFP4_OK) return MXFP4_EINVAL;
    if ((flags & ~(uint32_t)(MXFP4_REQ_INTERMEDIATE_BF16 | MXFP4_SCALE_UOS)) != 0)
        return MXFP4_EINVAL;
    if (T == 0) return MXFP4_OK;
    if (!nv_codes || !nv_scales || !nv_global || !mx_codes || !mx_scales) return MXFP4_EINVAL;
    if (!aligned(nv_codes, 16) || !aligned(mx_codes, 16) || !aligned(nv_scales, 2) ||
        !aligned(nv_global, 4))
        return MXFP4_EALIGN;
    return from_hip(mx::launch_requant(nv_codes, nv_scales, nv_global, T, N, K, nullptr, 0,
                                       mx_codes, mx_scales,
                                       (flags & MXFP4_REQ_INTERMEDIATE_BF16) != 0,
                                       (flags & MXFP4_SCALE_UOS) != 0, stream));
}

int mxfp4_requant_from_nvfp4_subset(const uint8_t* nv_codes, const uint8_t* nv_scales,
                                    const float* nv_global, int64_t T, int64_t N, int64_t K,
                                    const int32_t* tensors, int64_t n_tensors,
                                    uint8_t* mx_codes, uint8_t* mx_scales, uint32_t flags,
                                    hipStream_t stream) {
    if (T < 0 || N <= 0 || check_k(K) != MXFP4_OK || n_tensors < 0) return MXFP4_EINVAL;
    if ((flags & ~(uint32_t)(MXFP4_REQ_INTERMEDIATE_BF16 | MXFP4_SCALE_UOS)) != 0)
        return MXFP4_EINVAL;
    if (n_tensors == 0) return MXFP4_OK;
    if (!tensors) return MXFP4_EINVAL;
    for (int64_t i = 0; i < n_tensors; ++i)    // in range, strictly increasing
        if (tensors[i] < 0 || tensors[i] >= T || (i > 0 && tensors[i] <= tensors[i - 1]))
            return MXFP4_EINVAL;
    if (!nv_codes || !nv_scales || !nv_global || !mx_codes || !mx_scales) return MXFP4_EINVAL;
    if (!aligned(nv_codes, 16) || !aligned(mx_codes, 16) || !aligned(nv_scales, 2) ||
        !aligned(nv_global, 4))
        return MXFP4_EALIGN;
    return from_hip(mx::launch_requant(nv_codes, nv_scales, nv_global, T, N, K, tensors,
                                       n_tensors, mx_codes, mx_scales,
                                       (flags & MXFP4_REQ_INTERMEDIATE_BF16) != 0,
                                       (flags & MXFP4_SCALE_UOS) != 0, stream));
}

int mxfp4_quantize_act(const void* x_bf16, int64_t ldx, const int32_t* row_index, int64_t M,
                       int64_t K, uint8_t* codes, uint8_t* scales, uint32_t flags,
                       hipStream_t stream) {
    if (M < 0 || check_k(K) != MXFP4_OK || ldx < K) return MXFP4_EINVAL;
    if ((flags & ~(uint32_t)MXFP4_SCALE_UOS) != 0) return MXFP4_EINVAL;
    if (M == 0) return MXFP4_OK;
    if (!x_bf16 || !codes || !scales) return MXFP4_EINVAL;
    if (!aligned(x_bf16, 16) || ldx % 8 != 0 || !aligned(codes, 16)) return MXFP4_EALIGN;
    if (row_index && !aligned(row_index, 4)) return MXFP4_EALIGN;
    return from_hip(mx::launch_act_quant(static_cast<const uint16_t*>(x_bf16), ldx, row_index,
                                         M, K, codes, scales, (flags & MXFP4_SCALE_UOS) != 0,
                                         stream));
}

int mxfp4_quantize_act_scatter(const void* x_bf16, int64_t ldx, int64_t T, int64_t K,
                               const int32_t* dest_rows, int64_t fan, int64_t R, uint8_t* codes,
                               uint8_t* scales, uint32_t flags, hipStream_t stream) {
    if (T < 0 || check_k(K) != MXFP4_OK || ldx < K || fan < 1 || fan > (1 << 16) || R < 0)
        return MXFP4_EINVAL;
    if ((flags & ~(uint32_t)MXFP4_SCALE_UOS) != 0) return MXFP4_EINVAL;
    if (T == 0) return MXFP4_OK;
    if (R == 0 || !x_bf16 || !dest_rows || !codes || !scales) return MXFP4_EINVAL;
    if (!aligned(x_bf16, 16) || ldx % 8 != 0 || !aligned(codes, 16) || !aligned(dest_rows, 4))
        return MXFP4_EALIGN;
    return from_hip(mx::launch_act_quant_scatter(static_cast<const uint16_t*>(x_bf16), ldx, T,
                                                 K, dest_rows, fan, R, codes, scales,
                                                 (flags & MXFP4_SCALE_UOS) != 0, stream));
}

int mxfp4_quantize_act_smooth(const void* x_bf16, int64_t ldx, const int32_t* row_index,
                              const void* smooth_bf16, int64_t M, int64_t K, uint8_t* codes,
                              uint8_t* scales, uint32_t flags, hipStream_t stream) {
    if (M < 0 || check_k(K) != MXFP4_OK || ldx < K) return MXFP4_EINVAL;
    if ((flags & ~(uint32_t)MXFP4_SCALE_UOS) != 0) return MXFP4_EINVAL;
    if (M == 0) return MXFP4_OK;
    if (!x_bf16 || !smooth_bf16 || !codes || !scales) return MXFP4_EINVAL;
    if (!aligned(x_bf16, 16) || ldx % 8 != 0 || !aligned(codes, 16) || !aligned(smooth_bf16, 16))
        return MXFP4_EALIGN;
    if (row_index && !aligned(row_index, 4)) return MXFP4_EALIGN;
    return from_hip(mx::launch_act_quant(static_cast<const uint16_t*>(x_bf16), ldx, row_index,
                                         M, K, codes, scales, (flags & MXFP4_SCALE_UOS) != 0,
                                         stream, static_cast<const uint16_t*>(smooth_bf16)));
}

int mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
               const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* y,
               int out_dtype, void* workspace, size_t workspace_bytes, uint32_t flags,
               hipStream_t stream) {
    const int st = check_gemm_common(a_codes, a_scales, b_codes, b_scales, M, N, K, y, out_dtype,
                                     workspace, workspace_bytes, flags);
    if (st != MXFP4_OK || M == 0) return st;
    return from_hip(mx::launch_gemm(a_codes, a_scales, b_codes, b_scales, M, N, K, y, nullptr,
                                    out_dtype == MXFP4_OUT_BF16, stream));
}

size_t mxfp4_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
    return mx::linear_workspace_bytes(M, N, K);
}

int mxfp4_linear_bf16(const void* x_bf16, int64_t ldx, int64_t M, int64_t N, int64_t K,
                      const uint8_t* b_codes, const uint8_t* b_scales, const void* bias_bf16,
                      void* y, int out_dtype, void* workspace, size_t workspace_bytes,
                      uint32_t flags, hipStream_t stream) {
    if (workspace_bytes != 0 && workspace == nullptr) return MXFP4_EINVAL;
    const int st = mx::check_linear_bf16(x_bf16, ldx, M, N, K, b_codes, b_scales, bias_bf16, y,
                                         out_dtype, flags);
    if (st != MXFP4_OK || M == 0) return st;
    if (workspace_bytes < mx::linear_workspace_bytes(M, N, K)) return MXFP4_EINVAL;
    if (workspace && !aligned(workspace, 16)) return MXFP4_EALIGN;
    return mx::run_linear_bf16(x_bf16, ldx, M, N, K, b_codes, b_scales, bias_bf16, y, out_dtype,
                               static_cast<uint8_t*>(workspace), flags, stream);
}

int mxfp8_quantize_act(const void* x_bf16, int64_t ldx, const int32_t* row_index, int64_t M,
                       int64_t K, uint8_t* codes, uint8_t* scales, uint32_t flags,
                       hipStream_t stream) {
    if (M < 0 || check_k(K) != MXFP4_OK || ldx < K) return MXFP4_EINVAL;
    if (flags != 0) return MXFP4_EINVAL;
    if (M == 0) return MXFP4_OK;
    if (!x_bf16 || !codes || !scales) return MXFP4_EINVAL;
    if (!aligned(x_bf16, 16) || ldx % 8 != 0 || !aligned(codes, 16)) return MXFP4_EALIGN;
    if (row_index && !aligned(row_index, 4)) return MXFP4_EALIGN;
    return from_hip(mx::launch_act_quant_fp8(static_cast<const uint16_t*>(x_bf16), ldx,
                                             row_index, M, K, codes, scales, stream));
}

int mxfp8_quantize_act_smooth(const void* x_bf16, int64_t ldx, const int32_t* row_index,
                              const void* smooth_bf16, int64_t M, int64_t K, uint8_t* codes,
                              uint8_t* scales, uint32_t flags, hipStream_t stream) {
    if (M < 0 || check_k(K) != MXFP4_OK || ldx < K) return MXFP4_EINVAL;
    if (flags != 0) return MXFP4_EINVAL;
    if (M == 0) return MXFP4_OK;
    if (!x_bf16 || !smooth_bf16 || !codes || !scales) return MXFP4_EINVAL;
    if (!aligned(x_bf16, 16) || ldx % 8 != 0 || !aligned(codes, 16) || !aligned(smooth_bf16, 16))
        return MXFP4_EALIGN;
    if (row_index && !aligned(row_index, 4)) return MXFP4_EALIGN;
    return from_hip(mx::launch_act_quant_fp8(static_cast<const uint16_t*>(x_bf16), ldx,
                                             row_index, M, K, codes, scales, stream,
                                             static_cast<const uint16_t*>(smooth_bf16)));
}

int mxfp4_gemm_w4a8(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                    const uint8_t* b_scales, int64_t M, int64_t N, int64_t K,
                    const void* bias_bf16, void* y, int out_dtype, uint32_t flags,
                    hipStream_t stream) {
    const int st = check_gemm_common(a_codes, a_scales, b_codes, b_scales, M, N, K, y, out_dtype,
                                     nullptr, 0, flags);
    if (st != MXFP4_OK || M == 0) return st;
    if (bias_bf16 && !aligned(bias_bf16, 16)) return MXFP4_EALIGN;
    return from_hip(mx::launch_gemm_w4a8(a_codes, a_scales, b_codes, b_scales, M, N, K, y,
                                         static_cast<const uint16_t*>(bias_bf16),
                                         out_dtype == MXFP4_OUT_BF16, stream));
}

size_t mxfp4_linear_w4a8_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || check_k(K) != MXFP4_OK) return 0;
    if (mx::linear_skinny_shape(M, N, K)) return 0;
    return fp8_codes_bytes(M, K) + (size_t)M * (size_t)(K / 32);
}

int mxfp4_linear_w4a8_bf16(const void* x_bf16, int64_t ldx, int64_t M, int64_t N, int64_t K,
                           const uint8_t* b_codes, const uint8_t* b_scales,
                           const void* bias_bf16, void* y, int out_dtype, void* workspace,
                           size_t workspace_bytes, uint32_t flags, hipStream_t stream) {
    if (M < 0 || N <= 0 || check_k(K) != MXFP4_OK || ldx < K) return MXFP4_EINVAL;
    if (out_dtype != MXFP4_OUT_BF16 && out_dtype != MXFP4_OUT_FP32) return MXFP4_EINVAL;
    if (flags != 0) return MXFP4_EINVAL;
    if (workspace_bytes != 0 && workspace == nullptr) return MXFP4_EINVAL;
    if (M == 0) return MXFP4_OK;
    if (!x_bf16 || !b_codes || !b_scales || !y) return MXFP4_EINVAL;
    if (!aligned(x_bf16, 16) || ldx % 8 != 0 || !aligned(b_codes, 16) || !aligned(b_scales, 16))
        return MXFP4_EALIGN;
    if (!aligned(y, out_dtype == MXFP4_OUT_FP32 ? 4 : 2)) return MXFP4_EALIGN;
    if (bias_bf16 && !aligned(bias_bf16, 16)) return MXFP4_EALIGN;
    const uint16_t* bias = static_cast<const uint16_t*>(bias_bf16);
    if (mx::linear_skinny_shape(M, N, K))
        return from_hip(mx::launch_linear_skinny_w4a8(static_cast<const uint16_t*>(x_bf16), ldx,
                                                      b_codes, b_scales, M, N, K, y, bias,
                                                      out_dtype == MXFP4_OUT_BF16, stream));
    const size_t need = fp8_codes_bytes(M, K) + (size_t)M * (size_t)(K / 32);
    if (workspace_bytes < need) return MXFP4_EINVAL;
    if (!aligned(workspace, 16)) return MXFP4_EALIGN;
    uint8_t* codes = static_cast<uint8_t*>(workspace);
    uint8_t* scales = codes + fp8_codes_bytes(M, K);
    const hipError_t e = mx::launch_act_quant_fp8(static_cast<const uint16_t*>(x_bf16), ldx,
                                                  nullptr, M, K, codes, scales, stream);
    if (e != hipSuccess) return MXFP4_EHIP;
    return from_hip(mx::launch_gemm_w4a8(codes, scales, b_codes, b_scales, M, N, K, y,
                                         static_cast<const uint16_t*>(bias_bf16),
                                         out_dtype == MXFP4_OUT_BF16, stream));
}

int mxfp4_silu_mul_quantize(const void* gate_up_bf16, int64_t ldg, int64_t M, int64_t I,
                            uint8_t* codes, uint8_t* scales, uint32_t flags,
                            hipStream_t stream) {
    if (M < 0 || check_k(I) != MXFP4_OK || ldg < 2 * I) return MXFP4_EINVAL;
    if ((flags & ~(uint32_t)MXFP4_SCALE_UOS) != 0) return MXFP4_EINVAL;
    if (M == 0) return MXFP4_OK;
    if (!gate_up_bf16 || !codes || !scales) return MXFP4_EINVAL;
    if (!aligned(gate_up_bf16, 16) || ldg % 8 != 0 || !aligned(codes, 16)) return MXFP4_EALIGN;
    return from_hip(mx::launch_silu_mul_quantize(static_cast<const uint16_t*>(gate_up_bf16),
                                                 ldg, M, I, codes, scales,
                                                 (flags & MXFP4_SCALE_UOS) != 0, stream));
}

int mxfp4_grouped_gemm_silu_quantize(const uint8_t* a_codes, const uint8_t* a_scales,
                                     const uint8_t* b_codes, const uint8_t* b_scales,
                                     const int32_t* offsets, int64_t E, int64_t total_M,
                                     int64_t I, int64_t K, uint8_t* h_codes,
                                     uint8_t* h_scales, uint32_t flags, hipStream_t stream) {
    if (E <= 0 || total_M < 0 || check_k(I) != MXFP4_OK || check_k(K) != MXFP4_OK)
        return MXFP4_EINVAL;
    if ((flags & ~(uint32_t)(MXFP4_SCALE_UOS | MXFP4_B_PRESHUFFLED)) != 0) return MXFP4_EINVAL;
    const bool shuffled = (flags & MXFP4_B_PRESHUFFLED) != 0;
    if (total_M == 0) return MXFP4_OK;
    if (!a_codes || !a_scales || !b_codes || !b_scales || !offsets || !h_codes || !h_scales)
        return MXFP4_EINVAL;
    if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(h_codes, 16) ||
        !aligned(offsets, 4))
        return MXFP4_EALIGN;
    const int64_t N = 2 * I;
    if (!mx::grouped_glu_supported(E, total_M, N, K, a_scales, b_scales) ||
        (shuffled && !mx::grouped_stream_supported(E, total_M, N, K, a_scales, b_scales)))
        return MXFP4_EUNSUPPORTED;
    return from_hip(mx::launch_grouped_glu_quant(a_codes, a_scales, b_codes, b_scales, offsets,
                                                 E, total_M, N, K, h_codes, h_scales,
                                                 (flags & MXFP4_SCALE_UOS) != 0, shuffled,
                                                 stream));
}

int mxfp4_moe_combine(const void* y_bf16, int64_t ldy, int64_t R, const int32_t* rows,
                      const float* weights, int64_t T, int64_t topk, int64_t H, void* out,
                      int out_dtype, uint32_t flags, hipStream_t stream) {
    if (T < 0 || R <= 0 || topk < 1 || topk > MXFP4_COMBINE_MAX_TOPK || H <= 0 || H % 8 != 0 ||
        ldy < H)
        return MXFP4_EINVAL;
    if (out_dtype != MXFP4_OUT_BF16 && out_dtype != MXFP4_OUT_FP32) return MXFP4_EINVAL;
    if (flags != 0) return MXFP4_EINVAL;
    if (T == 0) return MXFP4_OK;
    if (!y_bf16 || !rows || !weights || !out) return MXFP4_EINVAL;
    if (!aligned(y_bf16, 16) || ldy % 8 != 0 || !aligned(out, 16) || !aligned(rows, 4) ||
        !aligned(weights, 4))
        return MXFP4_EALIGN;
    return from_hip(mx::launch_moe_combine(static_cast<const uint16_t*>(y_bf16), ldy, R, rows,
                                           weights, T, topk, H, out,
                                           out_dtype == MXFP4_OUT_BF16, stream));
}

int mxfp4_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                       const uint8_t* b_scales, const int32_t* offsets, int64_t E,
                       int64_t total_M, int64_t N, int64_t K, void* y, int out_dtype,
                       void* workspace, size_t workspace_bytes, uint32_t flags,
                       hipStream_t stream) {
    if (E <= 0) return MXFP4_EINVAL;
    const bool shuffled = (flags & MXFP4_B_PRESHUFFLED) != 0;
    const int st = check_gemm_common(a_codes, a_scales, b_codes, b_scales, total_M, N, K, y,
                                     out_dtype, workspace, workspace_bytes,
                                     flags & ~(uint32_t)MXFP4_B_PRESHUFFLED);
    if (st != MXFP4_OK || total_M == 0) return st;
    if (!offsets) return MXFP4_EINVAL;
    if (!aligned(offsets, 4)) return MXFP4_EALIGN;
    if (shuffled && !mx::grouped_stream_supported(E, total_M, N, K, a_scales, b_scales))
        return MXFP4_EUNSUPPORTED;
    return from_hip(mx::launch_grouped_gemm(a_codes, a_scales, b_codes, b_scales, offsets, E,
                                            total_M, N, K, y, out_dtype == MXFP4_OUT_BF16,
                                            shuffled, stream));
}

int mxfp4_preshuffle_weights(const uint8_t* codes, uint8_t* out, int64_t T, int64_t N,
                             int64_t K, hipStream_t stream) {
    if (T < 0 || N <= 0 || N % 32 != 0 || K <= 0 || K % 256 != 0) return MXFP4_EINVAL;
    if (T == 0) return MXFP4_OK;
    if (!codes || !out) return MXFP4_EINVAL;
    const uintptr_t a = reinterpret_cast<uintptr_t>(codes), b = reinterpret_cast<uintptr_t>(out);
    const uint64_t bytes = (uint64_t)T * (uint64_t)N * (uint64_t)(K / 2);
    if (a < b + bytes && b < a + bytes) return MXFP4_EINVAL;      // overlapping buffers
    if (!aligned(codes, 16) || !aligned(out, 16)) return MXFP4_EALIGN;
    return from_hip(mx::launch_preshuffle(codes, out, T, N, K, stream));
}

size_t mxfp4_gemm_workspace_size(int64_t, int64_t, int64_t) { return 0; }

const char* mxfp4_status_string(int status) {
    switch (status) {
        case MXFP4_OK: return "ok";
        case MXFP4_EINVAL: return "invalid argument (size, null pointer, flag or dtype)";
        case MXFP4_EALIGN: return "misaligned pointer or leading dimension";
        case MXFP4_EUNSUPPORTED: return "unsupported request";
        case MXFP4_EHIP: return "HIP runtime error at launch";
        case MXFP4_ESCRATCH:
            return "request needs more than the static scratch of the no-allocation call";
        default: return "unknown status";
    }
}

int mxfp4_version(void) { return kVersion; }

}  // extern "C"
