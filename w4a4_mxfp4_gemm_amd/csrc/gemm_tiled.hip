// gemm_tiled.hip -- compute-bound MXFP4 GEMM for large M (prefill, MoE expert
// groups): 256 x 256 output tile per workgroup of 4 wavefronts (128 x 128
// each), operands staged in LDS by gfx950's buffer loads with LDS destination,
// and v_mfma_scale_f32_32x32x64_f8f6f4.  (One wavefront per SIMD can keep the
// matrix core busy with back-to-back 32x32x64 scaled MFMAs, but not with
// 16x16x128 ones, which is why this tile uses the larger shape.)
//
// Roles.  The weight tile (rows n of B) is the MFMA's A operand and the
// activation tile (rows m of A) its B operand.  In a 32x32x64 MFMA lane l
// holds 32 E2M1 codes (one MX block, 16 bytes) of row l%32, K-half l/32, and
// that block's scale byte; its 16 accumulator registers r = 4b + i hold
// output m = l%32, n = 8b + 4(l/32) + i, so each register quad is four
// consecutive n: one 8-byte (bf16) or 16-byte (fp32) store.
//
// K stage = 256 elements = 8 MX blocks = 4 MFMA K-steps.  Lane half h takes
// blocks 4h..4h+3 of the stage (one per K-step t = 0..3), so its 4 scale
// bytes are contiguous: one 32-bit LDS read per row, the MFMA's op_sel picks
// byte t.  (Any assignment of blocks to K-steps is valid as long as both
// operands use the same one.)
//
// Memory traffic.  The load path is limited by the number of L1->L2
// requests, not by bytes, so every request should carry a whole 128-byte
// line: a stage reads 128 code bytes per operand row, and scale bytes are
// fetched 16 per row at a time (two stages' worth).  K must be a multiple of
// 512.
//
// LDS (144 KiB of 160):
//   codes  [2 stages][W, X][256 rows][128 B]        128 KiB
//   scales [3 chunks][W, X][256 rows][16 B]          24 KiB  (chunk = 2 stages)
// Inside a code row, 16-byte chunk c sits at position c ^ ((row >> 1) & 7),
// which spreads the 16 rows a 16-lane group reads over all 64 banks.  Each
// load instruction writes 1 KiB of consecutive LDS (8 rows), so the swizzle is
// applied to the global address each lane fetches.
//
// Pipeline, per stage kt (one barrier per stage):
//   read half 1 of stage kt;  MFMAs on half 0;  wait for the reads
//   wait for stage kt+1's loads; barrier; load stage kt+2 (+ one scale half-chunk)
//   read half 0 of stage kt+1;  MFMAs on half 1;  wait for the reads
// The compiler cannot tell which buffer an LDS read touches while loads into
// the other are in flight, and would drain every load before each read, so
// the operand reads are ds_read instructions in inline assembly with explicit
// lgkmcnt waits.
#include "mx_device.h"
#include "launch.h"

#include <type_traits>

namespace mx {
namespace tiled {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int BM = 256;                      // activation rows per tile
constexpr int BN = 256;                      // weight rows per tile
constexpr int BKB = 128;                     // code bytes per row per stage (256 K)
constexpr int CODE_OPERAND = 256 * BKB;      // 32 KiB
constexpr int CODE_STAGE = 2 * CODE_OPERAND; // W then X
constexpr int SCALE_OPERAND = 256 * 16;      // 4 KiB
constexpr int SCALE_CHUNK = 2 * SCALE_OPERAND;
constexpr int SCALE_BASE = 2 * CODE_STAGE;   // after the two code stages
constexpr int LDS_BYTES = SCALE_BASE + 3 * SCALE_CHUNK;
constexpr int LOADS_PER_STAGE = 8 + 8 + 1;   // vector memory ops per thread per stage

typedef __attribute__((address_space(3))) uint8_t lds_u8;
#define AS_LDS(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ uint32_t lds_addr(const lds_u8* p) { return (uint32_t)(uintptr_t)p; }

// Raw buffer descriptor over [base, base + bytes): loads past the end read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

struct Operands {
    __amdgpu_buffer_rsrc_t w, ws, x, xs;
};

// Per-lane byte offsets of this thread's loads (constant over K; the K
// position enters as the scalar offset).  Rows past an operand's end are
// clamped to its last row: those results are never stored.
struct LoadOffsets {
    uint32_t w[8], x[8], ws, xs;
};

__device__ __forceinline__ LoadOffsets load_offsets(int64_t n0, int64_t N, int64_t m0, int64_t M,
                                                    int64_t ldc, int64_t lds_) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    LoadOffsets o;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = (wave * 8 + i) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        o.w[i] = (uint32_t)(min(n0 + row, N - 1) * ldc + 16 * c);
        o.x[i] = (uint32_t)(min(m0 + row, M - 1) * ldc + 16 * c);
    }
    const int row = wave * 64 + lane;
    o.ws = (uint32_t)(min(n0 + row, N - 1) * lds_);
    o.xs = (uint32_t)(min(m0 + row, M - 1) * lds_);
    return o;
}

__device__ __forceinline__ void load_codes(lds_u8* lds, const Operands& op, const LoadOffsets& o,
                                           int buf, int kt) {
    const int wave = threadIdx.x >> 6;
    const uint32_t k = (uint32_t)kt * BKB;
    lds_u8* w = lds + buf * CODE_STAGE;
    lds_u8* x = w + CODE_OPERAND;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(op.w, AS_LDS(w + (wave * 8 + i) * 1024), 16,
                                                 o.w[i], k, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(op.x, AS_LDS(x + (wave * 8 + i) * 1024), 16,
                                                 o.x[i], k, 0, 0);
    }
}

// One operand's scales for chunk c (stages 2c, 2c+1): 16 bytes per row.
__device__ __forceinline__ void load_scales(lds_u8* lds, const Operands& op,
                                            const LoadOffsets& o, bool weights, int c) {
    const int wave = threadIdx.x >> 6;
    lds_u8* dst = lds + SCALE_BASE + (c % 3) * SCALE_CHUNK + (weights ? 0 : SCALE_OPERAND) +
                  wave * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(weights ? op.ws : op.xs, AS_LDS(dst), 16,
                                             weights ? o.ws : o.xs, (uint32_t)c * 16, 0, 0);
}

// vmcnt wait with the count packed into bits 3:0 and 15:14 (expcnt and
// lgkmcnt unconstrained).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int T>
__device__ __forceinline__ v16f mfma(const v4u& a, const v4u& b, v16f acc, uint32_t sa,
                                     uint32_t sb) {
    const v8i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
    const v8i bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 4, 4, T, (int)sa, T,
                                                           (int)sb);
}

// Half a stage of one wave's operands: 4 weight and 4 activation 32-row
// blocks, 2 K-steps each, 16 bytes per lane.
struct Half {
    v4u w[4][2], x[4][2];
};
// A stage's scale bytes: one 32-bit word (4 K-steps) per row block.
struct Scales {
    uint32_t w[4], x[4];
};

template <int OFF>
__device__ __forceinline__ void ds_read_b128(v4u& r, uint32_t addr) {
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_read_b32(uint32_t& r, uint32_t addr) {
    asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
}

// Lane-constant LDS offsets.  Row r32 of block i sits at
// (base_row + 32 i + r32); its swizzled chunk for K-step t depends on r32 and
// t only, so every block is the same address plus 4 KiB * i.
struct ReadOffsets {
    uint32_t w[4], x[4], ws, xs;
};

__device__ __forceinline__ ReadOffsets read_offsets(int wn, int wm) {
    const int lane = threadIdx.x & 63;
    const int r32 = lane & 31, h = lane >> 5;
    ReadOffsets r;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int pos = (4 * h + t) ^ ((r32 >> 1) & 7);
        r.w[t] = (uint32_t)((wn * 128 + r32) * BKB + 16 * pos);
        r.x[t] = (uint32_t)(CODE_OPERAND + (wm * 128 + r32) * BKB + 16 * pos);
    }
    r.ws = (uint32_t)((wn * 128 + r32) * 16 + 4 * h);
    r.xs = (uint32_t)(SCALE_OPERAND + (wm * 128 + r32) * 16 + 4 * h);
    return r;
}

// Issue the reads of K-steps 2H, 2H+1 of a stage at LDS byte address `codes`.
template <int H>
__device__ __forceinline__ void read_half(Half& f, uint32_t codes, const ReadOffsets& ro) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        ds_read_b128<0 * 32 * BKB>(f.w[0][s], codes + ro.w[2 * H + s]);
        ds_read_b128<1 * 32 * BKB>(f.w[1][s], codes + ro.w[2 * H + s]);
        ds_read_b128<2 * 32 * BKB>(f.w[2][s], codes + ro.w[2 * H + s]);
        ds_read_b128<3 * 32 * BKB>(f.w[3][s], codes + ro.w[2 * H + s]);
        ds_read_b128<0 * 32 * BKB>(f.x[0][s], codes + ro.x[2 * H + s]);
        ds_read_b128<1 * 32 * BKB>(f.x[1][s], codes + ro.x[2 * H + s]);
        ds_read_b128<2 * 32 * BKB>(f.x[2][s], codes + ro.x[2 * H + s]);
        ds_read_b128<3 * 32 * BKB>(f.x[3][s], codes + ro.x[2 * H + s]);
    }
}

// Scale words of a stage; `scales` is the LDS address of its chunk plus 8 for
// the chunk's second stage.
__device__ __forceinline__ void read_scales(Scales& sc, uint32_t scales, const ReadOffsets& ro) {
    ds_read_b32<0 * 32 * 16>(sc.w[0], scales + ro.ws);
    ds_read_b32<1 * 32 * 16>(sc.w[1], scales + ro.ws);
    ds_read_b32<2 * 32 * 16>(sc.w[2], scales + ro.ws);
    ds_read_b32<3 * 32 * 16>(sc.w[3], scales + ro.ws);
    ds_read_b32<0 * 32 * 16>(sc.x[0], scales + ro.xs);
    ds_read_b32<1 * 32 * 16>(sc.x[1], scales + ro.xs);
    ds_read_b32<2 * 32 * 16>(sc.x[2], scales + ro.xs);
    ds_read_b32<3 * 32 * 16>(sc.x[3], scales + ro.xs);
}

// Wait for this wave's LDS reads and make the fragment registers depend on
// the wait, so no use of them can be scheduled before it.
__device__ __forceinline__ void settle(Half& f) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.w[0][0]), "+v"(f.w[0][1]), "+v"(f.w[1][0]), "+v"(f.w[1][1]));
    asm volatile("" : "+v"(f.w[2][0]), "+v"(f.w[2][1]), "+v"(f.w[3][0]), "+v"(f.w[3][1]));
    asm volatile("" : "+v"(f.x[0][0]), "+v"(f.x[0][1]), "+v"(f.x[1][0]), "+v"(f.x[1][1]));
    asm volatile("" : "+v"(f.x[2][0]), "+v"(f.x[2][1]), "+v"(f.x[3][0]), "+v"(f.x[3][1]));
}
__device__ __forceinline__ void settle(Half& f, Scales& sc) {
    settle(f);
    asm volatile("" : "+v"(sc.w[0]), "+v"(sc.w[1]), "+v"(sc.w[2]), "+v"(sc.w[3]), "+v"(sc.x[0]),
                      "+v"(sc.x[1]), "+v"(sc.x[2]), "+v"(sc.x[3]));
}

// One operand load of a stage, selected by index: 0-7 weight codes, 8-15
// activation codes, 16 the stage's scale half-chunk.
template <int Q>
__device__ __forceinline__ void load_op(lds_u8* lds, const Operands& op, const LoadOffsets& o,
                                        int buf, int kt, bool scale_w, int chunk) {
    const int wave = threadIdx.x >> 6;
    if constexpr (Q < 8) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            op.w, AS_LDS(lds + buf * CODE_STAGE + (wave * 8 + Q) * 1024), 16, o.w[Q],
            (uint32_t)kt * BKB, 0, 0);
    } else if constexpr (Q < 16) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            op.x, AS_LDS(lds + buf * CODE_STAGE + CODE_OPERAND + (wave * 8 + Q - 8) * 1024), 16,
            o.x[Q - 8], (uint32_t)kt * BKB, 0, 0);
    } else {
        load_scales(lds, op, o, scale_w, chunk);
    }
}

// One LDS read of a half-stage (index 0-15: K-step s = Q / 8, operand
// Q % 8 / 4, block Q % 4), or for Q 16-23 one scale word.
template <int H, int Q>
__device__ __forceinline__ void read_op(Half& f, Scales& sc, uint32_t codes, uint32_t scales,
                                        const ReadOffsets& ro) {
    if constexpr (Q < 16) {
        constexpr int s = Q / 8, opnd = (Q % 8) / 4, blk = Q % 4;
        if constexpr (opnd == 0)
            ds_read_b128<blk * 32 * BKB>(f.w[blk][s], codes + ro.w[2 * H + s]);
        else
            ds_read_b128<blk * 32 * BKB>(f.x[blk][s], codes + ro.x[2 * H + s]);
    } else if constexpr (Q < 20) {
        ds_read_b32<(Q - 16) * 32 * 16>(sc.w[Q - 16], scales + ro.ws);
    } else {
        ds_read_b32<(Q - 20) * 32 * 16>(sc.x[Q - 20], scales + ro.xs);
    }
}

// The 32 MFMAs of K-steps 2H, 2H+1 (scale bytes 2H, 2H+1 of each word), with
// the other pipes' work threaded between them: after MFMA q, `step<q>()`
// issues that slot's loads / LDS reads, so the texture unit and LDS work
// while the matrix core is busy instead of in bursts.
template <int H, int Q = 0, typename Step>
__device__ __forceinline__ void mfma_half(const Half& f, const Scales& sc, v16f (&acc)[4][4],
                                          Step&& step) {
    if constexpr (Q < 32) {
        constexpr int t = Q / 16, i = (Q / 4) % 4, j = Q % 4;
        acc[i][j] = mfma<2 * H + t>(f.w[i][t], f.x[j][t], acc[i][j], sc.w[i], sc.x[j]);
        step(std::integral_constant<int, Q>{});
        __builtin_amdgcn_sched_barrier(0);   // keep this slot's order
        mfma_half<H, Q + 1>(f, sc, acc, step);
    }
}

// XCD-aware tile order: workgroup ids are dealt to the 8 XCDs round-robin, so
// id -> (xcd, local) is remapped to a linear tile index that gives each XCD a
// contiguous run, walked in groups of `gm` tile-rows so the run covers a
// compact block of the output (shared operand rows stay in that XCD's L2).
__device__ __forceinline__ bool tile_coords(int tiles_m, int tiles_n, int gm, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    const int per_xcd = (int)gridDim.x / 8;
    const int id = (int)blockIdx.x;
    const int t = (id % 8) * per_xcd + id / 8;
    if (t >= total) return false;
    const int group_size = gm * tiles_n;
    const int group = t / group_size;
    const int first_m = group * gm;
    const int rows = min(gm, tiles_m - first_m);
    const int in_group = t - group * group_size;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
    return true;
}

template <bool OUT_BF16>
__device__ __forceinline__ void store_tile(const v16f (&acc)[4][4], void* __restrict__ y,
                                           int64_t m0, int64_t m_end, int64_t n0, int64_t N,
                                           int wn, int wm) {
    const int lane = threadIdx.x & 63;
    const int r32 = lane & 31, h = lane >> 5;
    const bool vec_ok = (N % 4) == 0 && (reinterpret_cast<uintptr_t>(y) % 16) == 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t m = m0 + wm * 128 + 32 * j + r32;
        if (m >= m_end) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int64_t n = n0 + wn * 128 + 32 * i + 8 * b + 4 * h;
                if (n >= N) continue;
                const float v0 = acc[i][j][4 * b], v1 = acc[i][j][4 * b + 1];
                const float v2 = acc[i][j][4 * b + 2], v3 = acc[i][j][4 * b + 3];
                if (vec_ok && n + 3 < N) {
                    if (OUT_BF16)
                        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + m * N + n) =
                            make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
                    else
                        *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + m * N + n) =
                            make_float4(v0, v1, v2, v3);
                } else {
                    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (n + r >= N) break;
                        if (OUT_BF16)
                            reinterpret_cast<uint16_t*>(y)[m * N + n + r] =
                                (uint16_t)f32_to_bf16_rne(v[r]);
                        else
                            reinterpret_cast<float*>(y)[m * N + n + r] = v[r];
                    }
                }
            }
        }
    }
}

// The pipelined main loop for one output tile: x rows [m0, m_end) of the
// activations, w rows [n0, n0+256) of the weights.
template <bool OUT_BF16>
__device__ __forceinline__ void tile_gemm(lds_u8* lds, const uint8_t* __restrict__ x,
                                          const uint8_t* __restrict__ xs,
                                          const uint8_t* __restrict__ w,
                                          const uint8_t* __restrict__ ws, int64_t m0,
                                          int64_t m_end, int64_t n0, int64_t N, int64_t K,
                                          void* __restrict__ y) {
    const int wave = threadIdx.x >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int64_t ldc = K / 2, lds_ = K / 32;
    const int nkt = (int)(K / 256);           // even: K % 512 == 0
    const int last_chunk = nkt / 2 - 1;

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

    const Operands op{make_rsrc(w, (uint32_t)(N * ldc)), make_rsrc(ws, (uint32_t)(N * lds_)),
                      make_rsrc(x, (uint32_t)(m_end * ldc)),
                      make_rsrc(xs, (uint32_t)(m_end * lds_))};
    const LoadOffsets o = load_offsets(n0, N, m0, m_end, ldc, lds_);
    const ReadOffsets ro = read_offsets(wn, wm);
    const uint32_t lds0 = lds_addr(lds);

    // Loads of stage s >= 2 also bring half of scale chunk s/2 + 1 (weights
    // for even s, activations for odd s); chunk c is complete once stage
    // 2c-1's loads land and is first used by stage 2c.  Loads past the last
    // stage or chunk are clamped to it (they land in buffers nobody reads
    // again), so every stage issues the same number of loads.
    auto issue = [&](int s) {
        load_codes(lds, op, o, s & 1, s < nkt ? s : nkt - 1);
        const int c = s / 2 + 1;
        load_scales(lds, op, o, (s & 1) == 0, c <= last_chunk ? c : last_chunk);
    };
    auto code_addr = [&](int s) { return lds0 + (uint32_t)((s & 1) * CODE_STAGE); };
    auto scale_addr = [&](int s) {
        return lds0 + (uint32_t)(SCALE_BASE + ((s / 2) % 3) * SCALE_CHUNK + (s & 1) * 8);
    };

    // Prologue: stage 0 with chunks 0 and 1, stage 1; then stage 0's first half.
    load_codes(lds, op, o, 0, 0);
    load_scales(lds, op, o, true, 0);
    load_scales(lds, op, o, false, 0);
    load_scales(lds, op, o, true, last_chunk >= 1 ? 1 : 0);
    load_scales(lds, op, o, false, last_chunk >= 1 ? 1 : 0);
    load_codes(lds, op, o, 1, nkt > 1 ? 1 : 0);
    wait_vm<16>();
    __builtin_amdgcn_s_barrier();

    Half h0, h1;
    Scales sc_cur, sc_nxt;
    read_half<0>(h0, code_addr(0), ro);
    read_scales(sc_cur, scale_addr(0), ro);
    settle(h0, sc_cur);

    for (int kt = 0; kt < nkt; ++kt) {
        // first half: MFMAs on stage kt's K-steps 0-1, reads of its K-steps 2-3
        {
            const uint32_t codes = code_addr(kt);
            Scales unused;
            mfma_half<0>(h0, sc_cur, acc, [&](auto q) {
                constexpr int Q = decltype(q)::value;
                if constexpr (Q < 16) read_op<1, Q>(h1, unused, codes, 0, ro);
            });
            settle(h1);
        }
        // stage kt+1 landed for every wave; every wave is done reading stage kt
        wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        // second half: MFMAs on K-steps 2-3, loads of stage kt+2 into stage
        // kt's buffer, reads of stage kt+1's K-steps 0-1 and scales
        {
            const int s2 = kt + 2;
            const int ks = s2 < nkt ? s2 : nkt - 1;
            const int c = s2 / 2 + 1;
            const int chunk = c <= last_chunk ? c : last_chunk;
            const bool scale_w = (s2 & 1) == 0;
            const uint32_t codes = code_addr(kt + 1), scales = scale_addr(kt + 1);
            mfma_half<1>(h1, sc_cur, acc, [&](auto q) {
                constexpr int Q = decltype(q)::value;
                if constexpr (Q < 17) load_op<Q>(lds, op, o, s2 & 1, ks, scale_w, chunk);
                if constexpr (Q >= 4 && Q < 28) read_op<0, Q - 4>(h0, sc_nxt, codes, scales, ro);
            });
            settle(h0, sc_nxt);
            sc_cur = sc_nxt;
        }
    }
    // drain the surplus loads before the workgroup's LDS can be reused
    wait_vm<0>();

    store_tile<OUT_BF16>(acc, y, m0, m_end, n0, N, wn, wm);
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256, 1) void gemm_tiled_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ xs,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws, int64_t M, int64_t N,
    int64_t K, void* __restrict__ y, int gm) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    int tm, tn;
    if (!tile_coords(tiles_m, tiles_n, gm, tm, tn)) return;
    tile_gemm<OUT_BF16>((lds_u8*)smem, x, xs, w, ws, (int64_t)tm * BM, M, (int64_t)tn * BN, N,
                        K, y);
}

}  // namespace tiled

bool tiled_gemm_supported(int64_t M, int64_t N, int64_t K, const void* a_scales,
                          const void* b_scales) {
    // buffer offsets are 32-bit: every operand must span less than 2 GiB
    const int64_t lim = (int64_t)1 << 31;
    return M >= 128 && K % 512 == 0 && M * (K / 2) < lim && N * (K / 2) < lim &&
           (reinterpret_cast<uintptr_t>(a_scales) % 4) == 0 &&
           (reinterpret_cast<uintptr_t>(b_scales) % 4) == 0;
}

static int group_rows(int tiles_m, int per_xcd) {
    int gm = 1;
    while (gm * 2 <= tiles_m && (gm * 2) * (gm * 2) <= 2 * per_xcd) gm *= 2;
    return gm;
}

hipError_t launch_gemm_tiled(const uint8_t* a_codes, const uint8_t* a_scales,
                             const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                             int64_t N, int64_t K, void* y, bool out_bf16, hipStream_t stream) {
    using namespace tiled;
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const int total = tiles_m * tiles_n;
    const int per_xcd = (total + 7) / 8;
    const int gm = group_rows(tiles_m, per_xcd);
    const dim3 grid((unsigned)(per_xcd * 8));
    if (out_bf16)
        hipLaunchKernelGGL(gemm_tiled_kernel<true>, grid, dim3(256), 0, stream, a_codes, a_scales,
                           b_codes, b_scales, M, N, K, y, gm);
    else
        hipLaunchKernelGGL(gemm_tiled_kernel<false>, grid, dim3(256), 0, stream, a_codes,
                           a_scales, b_codes, b_scales, M, N, K, y, gm);
    return hipGetLastError();
}

}  // namespace mx
