// launch.h -- host-side launchers shared between the kernel translation units
// and the C ABI.  Arguments reaching these functions are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// smooth: bf16 [K] per-channel pre-scale (values quantized: bf16(x * smooth)),
// or nullptr; 16-byte aligned.
hipError_t launch_act_quant(const uint16_t* x, int64_t ldx, const int32_t* row_index,
                            int64_t M, int64_t K, uint8_t* codes, uint8_t* scales, bool uos,
                            hipStream_t stream, const uint16_t* smooth = nullptr);

// tensors == nullptr: all T tensors; else the n_tensors listed (host memory,
// each in [0, T)).  uos: the Qmax = 7.25 shared-exponent rule, else OCP's.
// The same flag means the same for act-quant and the fused linear.
hipError_t launch_requant(const uint8_t* nv_codes, const uint8_t* nv_scales,
                          const float* nv_global, int64_t T, int64_t N, int64_t K,
                          const int32_t* tensors, int64_t n_tensors, uint8_t* mx_codes,
                          uint8_t* mx_scales, bool bf16_intermediate, bool uos,
                          hipStream_t stream);

// MoE expert activation + act-quant: gate_up bf16 [M][ldg] (gate = columns
// [0, I), up = [I, 2I)) -> MXFP4 of bf16(silu(gate) * up), [M][I/2] + [M][I/32].
// Act-quant of T rows, each written to rows dest[t * fan + j] (clamped to
// [0, R)) of the outputs.
hipError_t launch_act_quant_scatter(const uint16_t* x, int64_t ldx, int64_t T, int64_t K,
                                    const int32_t* dest, int64_t fan, int64_t R,
                                    uint8_t* codes, uint8_t* scales, bool uos,
                                    hipStream_t stream);

hipError_t launch_silu_mul_quantize(const uint16_t* gate_up, int64_t ldg, int64_t M, int64_t I,
                                   uint8_t* codes, uint8_t* scales, bool uos,
                                   hipStream_t stream);

// Top-k combine: out[t] = sum_j weights[t*topk+j] * y[rows[t*topk+j]] over
// bf16 y [R][ldy], H columns, bf16 or fp32 out [T][H].
hipError_t launch_moe_combine(const uint16_t* y, int64_t ldy, int64_t R, const int32_t* rows,
                              const float* weights, int64_t T, int64_t topk, int64_t H,
                              void* out, bool out_bf16, hipStream_t stream);

// Act-quant and weight-streaming GEMM in one launch: x bf16 [M][ldx], for
// the shapes linear_skinny_shape accepts, with x, ldx and the weight scales
// 16-byte aligned (the linear calls require that of every caller).
bool linear_skinny_shape(int64_t M, int64_t N, int64_t K);
hipError_t launch_linear_skinny(const uint16_t* x, int64_t ldx, const uint8_t* b_codes,
                                const uint8_t* b_scales, int64_t M, int64_t N, int64_t K,
                                void* y, const uint16_t* bias, bool out_bf16, bool uos,
                                hipStream_t stream);

// bias: bf16 [N] added to every row's fp32 sum before the output rounding, or
// nullptr (16-byte aligned when given).
// The W4A8 form: x quantized to MXFP8 in the kernel (same shapes).
hipError_t launch_linear_skinny_w4a8(const uint16_t* x, int64_t ldx, const uint8_t* b_codes,
                                     const uint8_t* b_scales, int64_t M, int64_t N, int64_t K,
                                     void* y, const uint16_t* bias, bool out_bf16,
                                     hipStream_t stream);

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                       const uint8_t* b_codes, const uint8_t* b_scales,
                       int64_t M, int64_t N, int64_t K, void* y, const uint16_t* bias,
                       bool out_bf16, hipStream_t stream);

hipError_t launch_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                               const uint8_t* b_codes, const uint8_t* b_scales,
                               const int32_t* offsets, int64_t E, int64_t total_M,
                               int64_t N, int64_t K, void* y, bool out_bf16, bool b_shuffled,
                               hipStream_t stream);

bool tiled_gemm_supported(int64_t M, int64_t N, int64_t K, const void* a_scales,
                          const void* b_scales);

hipError_t launch_gemm_tiled(const uint8_t* a_codes, const uint8_t* a_scales,
                             const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                             int64_t N, int64_t K, void* y, const uint16_t* bias,
                             bool out_bf16, hipStream_t stream);

bool grouped_tiled_supported(int64_t E, int64_t total_M, int64_t N, int64_t K,
                             const void* a_scales, const void* b_scales);

hipError_t launch_grouped_gemm_tiled(const uint8_t* a_codes, const uint8_t* a_scales,
                                     const uint8_t* b_codes, const uint8_t* b_scales,
                                     const int32_t* offsets, int64_t E, int64_t total_M,
                                     int64_t N, int64_t K, void* y, bool out_bf16,
                                     bool b_shuffled, hipStream_t stream);

// The grouped kernel with the weights streamed into registers (K % 1024 ==
// 0) on the tiled kernel's shapes, N % 32 == 0: the one that reads weights
// pre-shuffled by launch_preshuffle (T tensors [N][K/2], N % 32 == 0,
// K % 256 == 0).
bool grouped_stream_supported(int64_t E, int64_t total_M, int64_t N, int64_t K,
                              const void* a_scales, const void* b_scales);

hipError_t launch_preshuffle(const uint8_t* in, uint8_t* out, int64_t T, int64_t N, int64_t K,
                             hipStream_t stream);

// The grouped gate_up GEMM with the expert activation and its MXFP4
// quantization in the epilogue (gate/up weight rows interleaved by 32): the
// tiled kernel's shapes with N % 64 == 0.
bool grouped_glu_supported(int64_t E, int64_t total_M, int64_t N, int64_t K,
                           const void* a_scales, const void* b_scales);

hipError_t launch_grouped_glu_quant(const uint8_t* a_codes, const uint8_t* a_scales,
                                    const uint8_t* b_codes, const uint8_t* b_scales,
                                    const int32_t* offsets, int64_t E, int64_t total_M,
                                    int64_t N, int64_t K, uint8_t* h_codes, uint8_t* h_scales,
                                    bool uos, bool b_shuffled, hipStream_t stream);

bool skinny_gemm_supported(int64_t M, int64_t N, int64_t K, const void* x, const void* x_scales,
                           const void* w_scales);
// the weight-streaming kernel for other K (a multiple of 512 up to 16384) at
// the M its register file allows (W4A4 only)
bool skinny_any_k_supported(int64_t M, int64_t N, int64_t K, const void* x, const void* x_scales,
                            const void* w_scales);
hipError_t launch_gemm_skinny_any_k(const uint8_t* a_codes, const uint8_t* a_scales,
                                    const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                    int64_t N, int64_t K, void* y, const uint16_t* bias,
                                    bool out_bf16, hipStream_t stream);

// W4A8: A is MXFP8 (E4M3 codes [M][K], E8M0 [M][K/32]), B MXFP4.
hipError_t launch_act_quant_fp8(const uint16_t* x, int64_t ldx, const int32_t* row_index,
                                int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                                hipStream_t stream, const uint16_t* smooth = nullptr);
hipError_t launch_gemm_w4a8(const uint8_t* a_codes, const uint8_t* a_scales,
                            const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N,
                            int64_t K, void* y, const uint16_t* bias, bool out_bf16,
                            hipStream_t stream);
bool tiled_w4a8_supported(int64_t M, int64_t N, int64_t K, const void* a_scales,
                          const void* b_scales);
hipError_t launch_gemm_tiled_w4a8(const uint8_t* a_codes, const uint8_t* a_scales,
                                  const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                  int64_t N, int64_t K, void* y, const uint16_t* bias,
                                  bool out_bf16, hipStream_t stream);
hipError_t launch_gemm_skinny_w4a8(const uint8_t* a_codes, const uint8_t* a_scales,
                                   const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                   int64_t N, int64_t K, void* y, const uint16_t* bias,
                                   bool out_bf16, hipStream_t stream);

hipError_t launch_gemm_skinny(const uint8_t* a_codes, const uint8_t* a_scales,
                              const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                              int64_t N, int64_t K, void* y, const uint16_t* bias,
                              bool out_bf16, hipStream_t stream);

// Validation and dispatch of the bf16 linear call, shared by its entry
// points (mxfp4_abi.cpp): status codes of include/mxfp4.h.
size_t linear_workspace_bytes(int64_t M, int64_t N, int64_t K);
int check_linear_bf16(const void* x_bf16, int64_t ldx, int64_t M, int64_t N, int64_t K,
                      const uint8_t* b_codes, const uint8_t* b_scales, const void* bias_bf16,
                      void* y, int out_dtype, uint32_t flags);
int run_linear_bf16(const void* x_bf16, int64_t ldx, int64_t M, int64_t N, int64_t K,
                    const uint8_t* b_codes, const uint8_t* b_scales, const void* bias_bf16,
                    void* y, int out_dtype, uint8_t* workspace, uint32_t flags,
                    hipStream_t stream);

}  // namespace mx
