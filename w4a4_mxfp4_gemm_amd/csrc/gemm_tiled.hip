// gemm_tiled.hip -- MFMA-bound MXFP4 GEMM for many activation rows (prefill)
// and its grouped form for MoE experts.  A workgroup of 4 wavefronts owns one
// output tile; operands are staged in LDS by gfx950's buffer loads with LDS
// destination and multiplied with v_mfma_scale_f32_32x32x64_f8f6f4.  (One
// wavefront per SIMD keeps the matrix core busy with back-to-back 32x32x64
// scaled MFMAs, but not with 16x16x128 ones, which is why the tiles use the
// larger shape.)
//
// Tile shapes (Shape<MB, NB, WGM, WGN>: each wave owns MB x NB blocks of
// 32 x 32 outputs, the 4 waves form a WGM x WGN grid):
//   dense    256 activation rows x 256 weight rows, waves 2 x 2, 128 x 128 each
//   grouped  128 activation rows x 256 weight rows, waves 1 x 4, 128 x 64 each
// The grouped tile matches MoE expert groups of ~128 tokens: all four waves
// stay busy, and 32-row blocks past the expert's last row skip their MFMAs.
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
// LDS:
//   codes  [2 stages][W: BN rows, X: BM rows][128 B]    (128 / 96 KiB)
//   scales [3 chunks][W, X][256 rows][16 B]              24 KiB (chunk = 2 stages)
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

constexpr int BKB = 128;                     // code bytes per row per stage (256 K)
constexpr int SCALE_OPERAND = 256 * 16;      // 4 KiB: 256 rows x 16 B
constexpr int SCALE_CHUNK = 2 * SCALE_OPERAND;

template <int MB_, int NB_, int WGM_, int WGN_>
struct Shape {
    static_assert(WGM_ * WGN_ == 4, "four wavefronts per workgroup");
    static constexpr int MB = MB_, NB = NB_, WGM = WGM_, WGN = WGN_;
    static constexpr int BM = 32 * MB * WGM;              // activation rows per tile
    static constexpr int BN = 32 * NB * WGN;              // weight rows per tile
    static_assert(BM <= 256 && BN == 256, "scale staging holds 256 rows per operand");
    static constexpr int WLOADS = BN / 32;                // 1 KiB code loads per thread per stage
    static constexpr int XLOADS = BM / 32;
    static constexpr int W_OPERAND = BN * BKB;
    static constexpr int CODE_STAGE = (BN + BM) * BKB;    // W then X
    static constexpr int SCALE_BASE = 2 * CODE_STAGE;     // after the two code stages
    static constexpr int LDS_BYTES = SCALE_BASE + 3 * SCALE_CHUNK;
    static constexpr int LOADS_PER_STAGE = WLOADS + XLOADS + 1;
    static constexpr int SLOTS = 2 * MB * NB;             // MFMAs per half stage
    static constexpr int CODE_READS = 2 * (MB + NB);      // ds_read_b128 per half stage
    static constexpr int SCALE_READS = MB + NB;           // ds_read_b32 per stage
    static_assert(LOADS_PER_STAGE <= SLOTS && CODE_READS <= SLOTS, "slot budget");
};

using DenseShape = Shape<4, 4, 2, 2>;
using GroupShape = Shape<4, 2, 1, 4>;

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

// One 16-byte-per-lane buffer load into LDS: the wavefront's 64 lanes fill
// 1 KiB of LDS starting at `dst` (lane order), each from its own voffset.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_u8* dst, uint32_t voff,
                                      uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, AS_LDS(dst), 16, voff, soff, 0, 0);
}

// Per-lane byte offsets of this thread's loads (constant over K; the K
// position enters as the scalar offset).  Rows past an operand's end are
// clamped to its last row: those results are never stored.
template <class S>
struct LoadOffsets {
    uint32_t w[S::WLOADS], x[S::XLOADS], ws, xs;
};

template <class S>
__device__ __forceinline__ LoadOffsets<S> load_offsets(int64_t n0, int64_t N, int64_t m0,
                                                       int64_t M, int64_t ldc, int64_t lds_) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    LoadOffsets<S> o;
#pragma unroll
    for (int i = 0; i < S::WLOADS; ++i) {
        const int row = (wave * S::WLOADS + i) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        o.w[i] = (uint32_t)(min(n0 + row, N - 1) * ldc + 16 * c);
    }
#pragma unroll
    for (int i = 0; i < S::XLOADS; ++i) {
        const int row = (wave * S::XLOADS + i) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        o.x[i] = (uint32_t)(min(m0 + row, M - 1) * ldc + 16 * c);
    }
    const int row = wave * 64 + lane;
    o.ws = (uint32_t)(min(n0 + row, N - 1) * lds_);
    o.xs = (uint32_t)(min(m0 + row, M - 1) * lds_);
    return o;
}

template <class S>
__device__ __forceinline__ void load_codes(lds_u8* lds, const Operands& op,
                                           const LoadOffsets<S>& o, int buf, int kt) {
    const int wave = threadIdx.x >> 6;
    const uint32_t k = (uint32_t)kt * BKB;
    lds_u8* w = lds + buf * S::CODE_STAGE;
    lds_u8* x = w + S::W_OPERAND;
#pragma unroll
    for (int i = 0; i < S::WLOADS; ++i)
        dma16(op.w, w + (wave * S::WLOADS + i) * 1024, o.w[i], k);
#pragma unroll
    for (int i = 0; i < S::XLOADS; ++i)
        dma16(op.x, x + (wave * S::XLOADS + i) * 1024, o.x[i], k);
}

// One operand's scales for chunk c (stages 2c, 2c+1): 16 bytes per row, 256
// rows (an activation tile of fewer rows repeats its last row).
template <class S>
__device__ __forceinline__ void load_scales(lds_u8* lds, const Operands& op,
                                            const LoadOffsets<S>& o, bool weights, int c) {
    const int wave = threadIdx.x >> 6;
    lds_u8* dst = lds + S::SCALE_BASE + (c % 3) * SCALE_CHUNK + (weights ? 0 : SCALE_OPERAND) +
                  wave * 1024;
    dma16(weights ? op.ws : op.xs, dst, weights ? o.ws : o.xs, (uint32_t)c * 16);
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

// Half a stage of one wave's operands: NB weight and MB activation 32-row
// blocks, 2 K-steps each, 16 bytes per lane.
template <class S>
struct Half {
    v4u w[S::NB][2], x[S::MB][2];
};
// A stage's scale bytes: one 32-bit word (4 K-steps) per row block.
template <class S>
struct Scales {
    uint32_t w[S::NB], x[S::MB];
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

template <class S>
__device__ __forceinline__ ReadOffsets read_offsets(int wn, int wm) {
    const int lane = threadIdx.x & 63;
    const int r32 = lane & 31, h = lane >> 5;
    ReadOffsets r;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int pos = (4 * h + t) ^ ((r32 >> 1) & 7);
        r.w[t] = (uint32_t)((wn * 32 * S::NB + r32) * BKB + 16 * pos);
        r.x[t] = (uint32_t)(S::W_OPERAND + (wm * 32 * S::MB + r32) * BKB + 16 * pos);
    }
    r.ws = (uint32_t)((wn * 32 * S::NB + r32) * 16 + 4 * h);
    r.xs = (uint32_t)(SCALE_OPERAND + (wm * 32 * S::MB + r32) * 16 + 4 * h);
    return r;
}

// Wait for this wave's LDS reads and make the fragment registers depend on
// the wait, so no use of them can be scheduled before it.
template <class S>
__device__ __forceinline__ void settle(Half<S>& f) {
    static_assert(S::NB >= 2, "the wait is tied to the first two weight blocks");
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.w[0][0]), "+v"(f.w[0][1]), "+v"(f.w[1][0]), "+v"(f.w[1][1]));
#pragma unroll
    for (int i = 2; i < S::NB; ++i) asm volatile("" : "+v"(f.w[i][0]), "+v"(f.w[i][1]));
#pragma unroll
    for (int j = 0; j < S::MB; ++j) asm volatile("" : "+v"(f.x[j][0]), "+v"(f.x[j][1]));
}
template <class S>
__device__ __forceinline__ void settle(Half<S>& f, Scales<S>& sc) {
    settle(f);
#pragma unroll
    for (int i = 0; i < S::NB; ++i) asm volatile("" : "+v"(sc.w[i]));
#pragma unroll
    for (int j = 0; j < S::MB; ++j) asm volatile("" : "+v"(sc.x[j]));
}

// One operand load of a stage, selected by index: weight codes, then
// activation codes, then the stage's scale half-chunk.
template <class S, int Q>
__device__ __forceinline__ void load_op(lds_u8* lds, const Operands& op, const LoadOffsets<S>& o,
                                        int buf, int kt, bool scale_w, int chunk) {
    const int wave = threadIdx.x >> 6;
    if constexpr (Q < S::WLOADS) {
        dma16(op.w, lds + buf * S::CODE_STAGE + (wave * S::WLOADS + Q) * 1024, o.w[Q],
              (uint32_t)kt * BKB);
    } else if constexpr (Q < S::WLOADS + S::XLOADS) {
        constexpr int i = Q - S::WLOADS;
        dma16(op.x, lds + buf * S::CODE_STAGE + S::W_OPERAND + (wave * S::XLOADS + i) * 1024,
              o.x[i], (uint32_t)kt * BKB);
    } else {
        load_scales<S>(lds, op, o, scale_w, chunk);
    }
}

// One LDS read of a half-stage: for Q < CODE_READS, K-step s = Q / (NB+MB),
// then NB weight blocks and MB activation blocks; after that one scale word
// per row block (weights first).
template <class S, int H, int Q>
__device__ __forceinline__ void read_op(Half<S>& f, Scales<S>& sc, uint32_t codes,
                                        uint32_t scales, const ReadOffsets& ro) {
    constexpr int P = S::NB + S::MB;
    if constexpr (Q < S::CODE_READS) {
        constexpr int s = Q / P, r = Q % P;
        if constexpr (r < S::NB)
            ds_read_b128<r * 32 * BKB>(f.w[r][s], codes + ro.w[2 * H + s]);
        else
            ds_read_b128<(r - S::NB) * 32 * BKB>(f.x[r - S::NB][s], codes + ro.x[2 * H + s]);
    } else if constexpr (Q < S::CODE_READS + S::NB) {
        constexpr int i = Q - S::CODE_READS;
        ds_read_b32<i * 32 * 16>(sc.w[i], scales + ro.ws);
    } else {
        constexpr int j = Q - S::CODE_READS - S::NB;
        ds_read_b32<j * 32 * 16>(sc.x[j], scales + ro.xs);
    }
}

// Issue reads [R0, R1) of a half-stage.
template <class S, int H, int R0, int R1>
__device__ __forceinline__ void read_range(Half<S>& f, Scales<S>& sc, uint32_t codes,
                                           uint32_t scales, const ReadOffsets& ro) {
    if constexpr (R0 < R1) {
        read_op<S, H, R0>(f, sc, codes, scales, ro);
        read_range<S, H, R0 + 1, R1>(f, sc, codes, scales, ro);
    }
}

// The MFMAs of K-steps 2H, 2H+1 (scale bytes 2H, 2H+1 of each word), with
// the other pipes' work threaded between them: after MFMA q, `step<q>()`
// issues that slot's loads / LDS reads, so the texture unit and LDS work
// while the matrix core is busy instead of in bursts.  Activation blocks
// j >= JL (past the last row of the tile) are not multiplied.
template <class S, int JL, int H, int Q = 0, typename Step>
__device__ __forceinline__ void mfma_half(const Half<S>& f, const Scales<S>& sc,
                                          v16f (&acc)[S::NB][S::MB], Step&& step) {
    if constexpr (Q < S::SLOTS) {
        constexpr int t = Q / (S::NB * S::MB), i = (Q / S::MB) % S::NB, j = Q % S::MB;
        if constexpr (j < JL)
            acc[i][j] = mfma<2 * H + t>(f.w[i][t], f.x[j][t], acc[i][j], sc.w[i], sc.x[j]);
        step(std::integral_constant<int, Q>{});
        __builtin_amdgcn_sched_barrier(0);   // keep this slot's order
        mfma_half<S, JL, H, Q + 1>(f, sc, acc, step);
    }
}

template <class S, bool OUT_BF16>
__device__ __forceinline__ void store_tile(const v16f (&acc)[S::NB][S::MB], void* __restrict__ y,
                                           int64_t m0, int64_t m_end, int64_t n0, int64_t N,
                                           int wn, int wm) {
    const int lane = threadIdx.x & 63;
    const int r32 = lane & 31, h = lane >> 5;
    const bool vec_ok = (N % 4) == 0 && (reinterpret_cast<uintptr_t>(y) % 16) == 0;
#pragma unroll
    for (int j = 0; j < S::MB; ++j) {
        const int64_t m = m0 + wm * 32 * S::MB + 32 * j + r32;
        if (m >= m_end) continue;
#pragma unroll
        for (int i = 0; i < S::NB; ++i) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int64_t n = n0 + wn * 32 * S::NB + 32 * i + 8 * b + 4 * h;
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

// Reads of the next stage in the second half-stage: R reads spread evenly
// over the slots [SLOTS/8, SLOTS - SLOTS/8); first read index of slot q.
template <class S>
constexpr int second_half_read(int q) {
    constexpr int R = S::CODE_READS + S::SCALE_READS;
    constexpr int off = S::SLOTS / 8, win = S::SLOTS - 2 * (S::SLOTS / 8);
    const int v = (q - off) * R / win;
    return v < 0 ? 0 : (v > R ? R : v);
}

// The pipelined main loop for one output tile: x rows [m0, min(m0+BM, m_end))
// of the activations (row m_end - 1 is the last one the operand may touch),
// w rows [n0, n0+BN) of the weights.  Only the first JL 32-row activation
// blocks of each wave are multiplied (the caller guarantees the rest are
// past m_end).
template <class S, int JL, bool OUT_BF16>
__device__ __forceinline__ void tile_gemm(lds_u8* lds, const uint8_t* __restrict__ x,
                                          const uint8_t* __restrict__ xs,
                                          const uint8_t* __restrict__ w,
                                          const uint8_t* __restrict__ ws, int64_t m0,
                                          int64_t m_end, int64_t n0, int64_t N, int64_t K,
                                          void* __restrict__ y) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % S::WGN, wm = wave / S::WGN;
    const int64_t ldc = K / 2, lds_ = K / 32;
    const int nkt = (int)(K / 256);           // even: K % 512 == 0
    const int last_chunk = nkt / 2 - 1;

    v16f acc[S::NB][S::MB];
#pragma unroll
    for (int i = 0; i < S::NB; ++i)
#pragma unroll
        for (int j = 0; j < S::MB; ++j) acc[i][j] = v16f{};

    const Operands op{make_rsrc(w, (uint32_t)(N * ldc)), make_rsrc(ws, (uint32_t)(N * lds_)),
                      make_rsrc(x, (uint32_t)(m_end * ldc)),
                      make_rsrc(xs, (uint32_t)(m_end * lds_))};
    const LoadOffsets<S> o = load_offsets<S>(n0, N, m0, m_end, ldc, lds_);
    const ReadOffsets ro = read_offsets<S>(wn, wm);
    const uint32_t lds0 = lds_addr(lds);

    // Loads of stage s >= 2 also bring half of scale chunk s/2 + 1 (weights
    // for even s, activations for odd s); chunk c is complete once stage
    // 2c-1's loads land and is first used by stage 2c.  Loads past the last
    // stage or chunk are clamped to it (they land in buffers nobody reads
    // again), so every stage issues the same number of loads.
    auto code_addr = [&](int s) { return lds0 + (uint32_t)((s & 1) * S::CODE_STAGE); };
    auto scale_addr = [&](int s) {
        return lds0 + (uint32_t)(S::SCALE_BASE + ((s / 2) % 3) * SCALE_CHUNK + (s & 1) * 8);
    };

    // Prologue: stage 0 with chunks 0 and 1, stage 1; then stage 0's first half.
    load_codes<S>(lds, op, o, 0, 0);
    load_scales<S>(lds, op, o, true, 0);
    load_scales<S>(lds, op, o, false, 0);
    load_scales<S>(lds, op, o, true, last_chunk >= 1 ? 1 : 0);
    load_scales<S>(lds, op, o, false, last_chunk >= 1 ? 1 : 0);
    load_codes<S>(lds, op, o, 1, nkt > 1 ? 1 : 0);
    wait_vm<S::WLOADS + S::XLOADS>();
    __builtin_amdgcn_s_barrier();

    Half<S> h0, h1;
    Scales<S> sc_cur, sc_nxt;
    read_range<S, 0, 0, S::CODE_READS + S::SCALE_READS>(h0, sc_cur, code_addr(0),
                                                        scale_addr(0), ro);
    settle(h0, sc_cur);

    for (int kt = 0; kt < nkt; ++kt) {
        // first half: MFMAs on stage kt's K-steps 0-1, reads of its K-steps 2-3
        {
            const uint32_t codes = code_addr(kt);
            Scales<S> unused;
            mfma_half<S, JL, 0>(h0, sc_cur, acc, [&](auto q) {
                constexpr int Q = decltype(q)::value;
                if constexpr (Q < S::CODE_READS) read_op<S, 1, Q>(h1, unused, codes, 0, ro);
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
            mfma_half<S, JL, 1>(h1, sc_cur, acc, [&](auto q) {
                constexpr int Q = decltype(q)::value;
                if constexpr (Q < S::LOADS_PER_STAGE)
                    load_op<S, Q>(lds, op, o, s2 & 1, ks, scale_w, chunk);
                read_range<S, 0, second_half_read<S>(Q), second_half_read<S>(Q + 1)>(
                    h0, sc_nxt, codes, scales, ro);
            });
            settle(h0, sc_nxt);
            sc_cur = sc_nxt;
        }
    }
    // drain the surplus loads before the workgroup's LDS can be reused
    wait_vm<0>();

    store_tile<S, OUT_BF16>(acc, y, m0, m_end, n0, N, wn, wm);
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
__global__ __launch_bounds__(256, 1) void gemm_tiled_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ xs,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws, int64_t M, int64_t N,
    int64_t K, void* __restrict__ y, int gm) {
    using S = DenseShape;
    __shared__ __attribute__((aligned(16))) uint8_t smem[S::LDS_BYTES];
    const int tiles_m = (int)((M + S::BM - 1) / S::BM);
    const int tiles_n = (int)((N + S::BN - 1) / S::BN);
    int tm, tn;
    if (!tile_coords(tiles_m, tiles_n, gm, tm, tn)) return;
    tile_gemm<S, S::MB, OUT_BF16>((lds_u8*)smem, x, xs, w, ws, (int64_t)tm * S::BM, M,
                                  (int64_t)tn * S::BN, N, K, y);
}

// ---------------------------------------------------------------------------
// Grouped (MoE) GEMM.  Work items are (expert e, weight tile tn, activation
// tile mt) with mt < ceil(rows_e / BM), ordered by e, then tn, then mt, and
// numbered 0..total-1.  Every workgroup derives the numbering from the
// offset table itself (one wavefront scans it), then takes item
//   t = xcd * ceil(total / 8) + local      (xcd = id % 8, local = id / 8),
// so each XCD walks a contiguous run: the activation tiles of one weight tile
// run back to back on one XCD (the weight rows are fetched from HBM once and
// re-read from its L2), and an expert's rows stay in that L2 across its
// weight tiles.  The grid is sized for the worst case; surplus workgroups
// exit at once.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d *= 2) {
        const int u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    return v;
}

struct GroupItem {
    int e, tn;
    int m0, m_end;
};

// Row range of expert e, clamped into [0, total_M) and non-decreasing.
__device__ __forceinline__ void expert_rows(const int32_t* __restrict__ offsets, int e,
                                            int total_M, int& a0, int& a1) {
    a0 = offsets[e];
    a1 = offsets[e + 1];
    a0 = a0 < 0 ? 0 : (a0 > total_M ? total_M : a0);
    a1 = a1 < a0 ? a0 : (a1 > total_M ? total_M : a1);
}

template <int BM>
__device__ GroupItem find_item(const int32_t* __restrict__ offsets, int E, int total_M,
                               int tiles_n) {
    const int lane = threadIdx.x & 63;
    GroupItem it{-1, 0, 0, 0};
    int total = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
        int cnt = 0;
        if (e0 + lane < E) {
            int a0, a1;
            expert_rows(offsets, e0 + lane, total_M, a0, a1);
            cnt = (a1 - a0 + BM - 1) / BM * tiles_n;
        }
        total += __shfl(wave_inclusive_scan(cnt), 63, 64);
    }
    const int per_xcd = (total + 7) / 8;
    const int id = (int)blockIdx.x;
    const int local = id / 8;
    const int t = (id % 8) * per_xcd + local;
    if (local >= per_xcd || t >= total) return it;
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
        int cnt = 0, a0 = 0, a1 = 0;
        if (e0 + lane < E) {
            expert_rows(offsets, e0 + lane, total_M, a0, a1);
            cnt = (a1 - a0 + BM - 1) / BM * tiles_n;
        }
        const int incl = wave_inclusive_scan(cnt);
        const int lo = base + incl - cnt;
        const uint64_t hit = __ballot(cnt > 0 && t >= lo && t < lo + cnt);
        if (hit) {
            const int src = __ffsll((unsigned long long)hit) - 1;
            const int r = __shfl(t - lo, src, 64);
            const int mts = __shfl(cnt / tiles_n, src, 64);
            it.e = e0 + src;
            it.tn = r / mts;
            it.m0 = __shfl(a0, src, 64) + (r % mts) * BM;
            it.m_end = __shfl(a1, src, 64);
            return it;
        }
        base += __shfl(incl, 63, 64);
    }
    return it;
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256, 1) void grouped_tiled_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ xs,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws,
    const int32_t* __restrict__ offsets, int E, int total_M, int64_t N, int64_t K,
    void* __restrict__ y) {
    using S = GroupShape;
    __shared__ __attribute__((aligned(16))) uint8_t smem[S::LDS_BYTES];
    const int tiles_n = (int)((N + S::BN - 1) / S::BN);
    GroupItem* shared_item = reinterpret_cast<GroupItem*>(smem);
    if (threadIdx.x < 64) {
        const GroupItem it = find_item<S::BM>(offsets, E, total_M, tiles_n);
        if (threadIdx.x == 0) *shared_item = it;
    }
    __syncthreads();
    const GroupItem it = *shared_item;
    __syncthreads();                           // the pipeline reuses this LDS
    const int e = __builtin_amdgcn_readfirstlane(it.e);
    if (e < 0) return;
    const int tn = __builtin_amdgcn_readfirstlane(it.tn);
    const int m0 = __builtin_amdgcn_readfirstlane(it.m0);
    const int m_end = __builtin_amdgcn_readfirstlane(it.m_end);
    const int64_t nkb = K / 32;
    const uint8_t* we = w + (int64_t)e * N * nkb * 16;
    const uint8_t* wse = ws + (int64_t)e * N * nkb;
    const int64_t n0 = (int64_t)tn * S::BN;
    static_assert(S::WGM == 1 && S::MB == 4, "one wave row of four 32-row blocks");
    // 32-row blocks of the tile that hold rows of this expert (1..4)
    const int blocks = (min(m_end - m0, S::BM) + 31) / 32;
    if (blocks >= 4)
        tile_gemm<S, 4, OUT_BF16>((lds_u8*)smem, x, xs, we, wse, m0, m_end, n0, N, K, y);
    else if (blocks == 3)
        tile_gemm<S, 3, OUT_BF16>((lds_u8*)smem, x, xs, we, wse, m0, m_end, n0, N, K, y);
    else if (blocks == 2)
        tile_gemm<S, 2, OUT_BF16>((lds_u8*)smem, x, xs, we, wse, m0, m_end, n0, N, K, y);
    else
        tile_gemm<S, 1, OUT_BF16>((lds_u8*)smem, x, xs, we, wse, m0, m_end, n0, N, K, y);
}

}  // namespace tiled

// Buffer offsets are 32-bit: every operand must span less than 2 GiB.
static bool fits_buffer(int64_t rows, int64_t K) {
    return rows * (K / 2) < ((int64_t)1 << 31);
}

bool tiled_gemm_supported(int64_t M, int64_t N, int64_t K, const void* a_scales,
                          const void* b_scales) {
    return M >= 128 && K % 512 == 0 && fits_buffer(M, K) && fits_buffer(N, K) &&
           (reinterpret_cast<uintptr_t>(a_scales) % 4) == 0 &&
           (reinterpret_cast<uintptr_t>(b_scales) % 4) == 0;
}

bool grouped_tiled_supported(int64_t E, int64_t total_M, int64_t N, int64_t K,
                             const void* a_scales, const void* b_scales) {
    using S = tiled::GroupShape;
    const int64_t bound = ((total_M + S::BM - 1) / S::BM + E) * ((N + S::BN - 1) / S::BN);
    return K % 512 == 0 && fits_buffer(total_M, K) && fits_buffer(N, K) &&
           total_M < ((int64_t)1 << 30) && E < ((int64_t)1 << 30) &&
           bound + 8 < ((int64_t)1 << 31) &&
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
    using S = tiled::DenseShape;
    const int tiles_m = (int)((M + S::BM - 1) / S::BM);
    const int tiles_n = (int)((N + S::BN - 1) / S::BN);
    const int total = tiles_m * tiles_n;
    const int per_xcd = (total + 7) / 8;
    const int gm = group_rows(tiles_m, per_xcd);
    const dim3 grid((unsigned)(per_xcd * 8));
    if (out_bf16)
        hipLaunchKernelGGL(tiled::gemm_tiled_kernel<true>, grid, dim3(256), 0, stream, a_codes,
                           a_scales, b_codes, b_scales, M, N, K, y, gm);
    else
        hipLaunchKernelGGL(tiled::gemm_tiled_kernel<false>, grid, dim3(256), 0, stream, a_codes,
                           a_scales, b_codes, b_scales, M, N, K, y, gm);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm_tiled(const uint8_t* a_codes, const uint8_t* a_scales,
                                     const uint8_t* b_codes, const uint8_t* b_scales,
                                     const int32_t* offsets, int64_t E, int64_t total_M,
                                     int64_t N, int64_t K, void* y, bool out_bf16,
                                     hipStream_t stream) {
    using S = tiled::GroupShape;
    const int64_t bound = ((total_M + S::BM - 1) / S::BM + E) * ((N + S::BN - 1) / S::BN);
    const dim3 grid((unsigned)((bound + 7) / 8 * 8));
    if (out_bf16)
        hipLaunchKernelGGL(tiled::grouped_tiled_kernel<true>, grid, dim3(256), 0, stream,
                           a_codes, a_scales, b_codes, b_scales, offsets, (int)E, (int)total_M, N,
                           K, y);
    else
        hipLaunchKernelGGL(tiled::grouped_tiled_kernel<false>, grid, dim3(256), 0, stream,
                           a_codes, a_scales, b_codes, b_scales, offsets, (int)E, (int)total_M, N,
                           K, y);
    return hipGetLastError();
}

}  // namespace mx
