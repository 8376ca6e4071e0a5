// calibrate.hip -- two kernels that measure this GPU's own ceilings, so that
// each roofline fraction can be stated against the chip as it runs as well as
// against its published peaks.  Built into libmxfp4_calibrate.so, apart from
// the product library: the benchmark loads it, nothing on the path does.
//
// mxfp4_calibrate_mfma: every SIMD runs one wavefront that issues
// back-to-back v_mfma_scale_f32_32x32x64_f8f6f4 on E2M1 operands (the GEMM's
// instruction and formats), 16 independent accumulators, operands changed
// every round so the multipliers see data that varies like real codes.  Each
// wave also reads the shader clock counter and the constant 100 MHz counter
// at its start and end, giving the clock the MFMAs actually ran at.
//
// mxfp4_calibrate_copy: a streaming copy with 16-byte loads and stores (HBM
// read + write bandwidth), in a few launch shapes, plain or non-temporal.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kAcc = 16;

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* sink,
                                                        unsigned long long* clocks) {
    uint32_t h = (blockIdx.x * 256u + threadIdx.x) * 2654435761u + 0x9E3779B9u;
    auto next = [&h]() {
        h ^= h << 13;
        h ^= h >> 17;
        h ^= h << 5;
        return (int)h;
    };
    v8i a = {next(), next(), next(), next(), 0, 0, 0, 0};
    v8i b = {next(), next(), next(), next(), 0, 0, 0, 0};
    v16f acc[kAcc];
#pragma unroll
    for (int j = 0; j < kAcc; ++j) acc[j] = v16f{};
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < kAcc; ++j)
            acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 4, 4, 0, 127,
                                                                     0, 127);
        // new operands for the next round (a few VALU ops beside 16 MFMAs)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            a[k] = a[k] * 1664525 + 1013904223;
            b[k] = b[k] * 22695477 + 1;
        }
    }
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kAcc; ++j)
#pragma unroll
        for (int k = 0; k < 16; ++k) s += acc[j][k];
    if (s == 1.2345f) sink[blockIdx.x * 256 + threadIdx.x] = s;   // keeps the MFMAs live
    if ((threadIdx.x & 63) == 0) {
        const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
        clocks[2 * w] = c1 - c0;
        clocks[2 * w + 1] = r1 - r0;
    }
}

// Each workgroup copies chunks of 256 * 16 * U bytes (U 16-byte vectors a
// thread, all loads issued before the stores), chunks walked with a grid
// stride; NT selects non-temporal loads and stores.
template <int U, bool NT>
__global__ __launch_bounds__(256) void copy_kernel(const v4u* __restrict__ src,
                                                   v4u* __restrict__ dst, size_t n) {
    const size_t chunk = (size_t)256 * U;
    for (size_t c = (size_t)blockIdx.x * chunk; c < n; c += (size_t)gridDim.x * chunk) {
        v4u x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = c + (size_t)u * 256 + threadIdx.x;
            if (i < n) x[u] = NT ? __builtin_nontemporal_load(src + i) : src[i];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = c + (size_t)u * 256 + threadIdx.x;
            if (i < n) {
                if (NT)
                    __builtin_nontemporal_store(x[u], dst + i);
                else
                    dst[i] = x[u];
            }
        }
    }
}

struct CopyConfig {
    int unroll, grid;
    bool nt;
};
constexpr CopyConfig kCopy[] = {{4, 4096, true},  {8, 2048, true},  {8, 4096, true},
                                {16, 2048, true}, {8, 8192, true},  {4, 4096, false},
                                {8, 2048, false}, {8, 4096, false}, {16, 2048, false}};

}  // namespace

extern "C" {

// Waves the MFMA loop runs: one per SIMD of 256 CUs.
int mxfp4_calibrate_mfma_waves(void) { return 1024; }

// FLOP per wave per round: kAcc MFMAs of 32 x 32 x 64 multiply-adds.
double mxfp4_calibrate_mfma_flop_per_round(void) { return 2.0 * 32 * 32 * 64 * kAcc; }

// clocks: device u64 [2 * 1024] (per wave: shader clock ticks, 100 MHz ticks);
// sink: device fp32 [256 * 256] (never written in practice).
int mxfp4_calibrate_mfma(int iters, unsigned long long* clocks, float* sink,
                         hipStream_t stream) {
    if (iters <= 0 || !clocks || !sink) return -1;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(256), dim3(256), 0, stream, iters, sink, clocks);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Copy configurations the benchmark sweeps (it keeps the fastest).
int mxfp4_calibrate_copy_configs(void) { return (int)(sizeof(kCopy) / sizeof(kCopy[0])); }

// dst = src with configuration `config`, bytes a multiple of 16, both 16-byte
// aligned device pointers.
int mxfp4_calibrate_copy(const void* src, void* dst, size_t bytes, int config,
                         hipStream_t stream) {
    if (!src || !dst || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) % 16) != 0 ||
        (reinterpret_cast<uintptr_t>(dst) % 16) != 0 || config < 0 ||
        config >= mxfp4_calibrate_copy_configs())
        return -1;
    const CopyConfig c = kCopy[config];
    const v4u* s = static_cast<const v4u*>(src);
    v4u* d = static_cast<v4u*>(dst);
    const size_t n = bytes / 16;
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(c.grid), dim3(256), 0, stream, s, d, n);
    };
    if (c.nt) {
        if (c.unroll == 4) go(copy_kernel<4, true>);
        else if (c.unroll == 8) go(copy_kernel<8, true>);
        else go(copy_kernel<16, true>);
    } else {
        if (c.unroll == 4) go(copy_kernel<4, false>);
        else if (c.unroll == 8) go(copy_kernel<8, false>);
        else go(copy_kernel<16, false>);
    }
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
