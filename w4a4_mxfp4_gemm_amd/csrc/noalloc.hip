// noalloc.hip -- mxfp4_linear_bf16_noalloc: the bf16 linear call for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  Where mxfp4_linear_bf16
// quantizes the activations into the caller's workspace (the two-launch form),
// this call uses `scratch`, a file-scope device array of a fixed size that
// each GPU holds from the library's load until the process ends.
//
// `scratch` is a device symbol: in host code its name is not a device
// address.  Its address on the current device comes from hipGetSymbolAddress,
// taken once per device on the first call made with that device current and
// kept in g_scratch; kernels receive that pointer, never the symbol.
#include "../../include/mxfp4.h"
#include "launch.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

namespace {

static __device__ __align__(256) uint8_t scratch[MXFP4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
uint8_t* g_scratch[kMaxDevices] = {};

// The current device's copy of `scratch`.
int scratch_on_current_device(uint8_t** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MXFP4_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return MXFP4_EUNSUPPORTED;
    std::lock_guard<std::mutex> hold(g_lock);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MXFP4_EHIP;
        g_scratch[dev] = static_cast<uint8_t*>(p);
    }
    *out = g_scratch[dev];
    return MXFP4_OK;
}

}  // namespace

extern "C" int mxfp4_linear_bf16_noalloc(const void* x_bf16, int64_t ldx, int64_t M, int64_t N,
                                         int64_t K, const uint8_t* b_codes,
                                         const uint8_t* b_scales, const void* bias_bf16,
                                         void* y, int out_dtype, uint32_t flags,
                                         hipStream_t stream) {
    const int st = mx::check_linear_bf16(x_bf16, ldx, M, N, K, b_codes, b_scales, bias_bf16, y,
                                         out_dtype, flags);
    if (st != MXFP4_OK || M == 0) return st;
    const size_t need = mx::linear_workspace_bytes(M, N, K);
    if (need > MXFP4_NOALLOC_SCRATCH_BYTES) return MXFP4_ESCRATCH;
    uint8_t* ws = nullptr;
    if (need > 0) {
        const int s = scratch_on_current_device(&ws);
        if (s != MXFP4_OK) return s;
    }
    return mx::run_linear_bf16(x_bf16, ldx, M, N, K, b_codes, b_scales, bias_bf16, y, out_dtype,
                               ws, flags, stream);
}
