// gemm_tiled.hip -- MFMA-bound MXFP4 GEMM for many activation rows (prefill)
// and its grouped form for MoE experts.  A workgroup of 4 or 8 wavefronts
// owns one output tile; operands are staged in LDS by gfx950's buffer loads
// with LDS destination and multiplied with v_mfma_scale_f32_32x32x64_f8f6f4.
// (One wavefront per SIMD keeps the matrix core busy with back-to-back
// 32x32x64 scaled MFMAs, but not with 16x16x128 ones, which is why the tiles
// use the larger shape.)
//
// Tile shapes (Shape<MB, NB, WGM, WGN>: each wave owns MB x NB blocks of
// 32 x 32 outputs, the waves form a WGM x WGN grid):
//   dense    256 activation rows x 256 weight rows, 8 waves 2 x 4, 128 x 64 each
//            (two per SIMD; its own K-step pipeline, gemm_dense_kernel)
//   W4A8     128 activation rows x 256 weight rows, 4 waves 2 x 2, 64 x 128 each
//   grouped  128 activation rows x 256 weight rows, 4 waves 1 x 4, 128 x 64 each
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
// Pipeline of the 4-wave tiles, per stage kt (one barrier per stage):
//   read half 1 of stage kt;  MFMAs on half 0;  wait for the reads
//   wait for stage kt+1's loads; barrier; load stage kt+2 (+ one scale half-chunk)
//   read half 0 of stage kt+1;  MFMAs on half 1;  wait for the reads
// The compiler cannot tell which buffer an LDS read touches while loads into
// the other are in flight, and would drain every load before each read, so
// the LDS-DMA loads are issued from inline assembly (invisible to its wait
// insertion) and ordered by the kernel's own vmcnt waits and barriers; the
// LDS reads are ordinary loads whose lgkmcnt waits the compiler places.
#include "mx_device.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>
#include <utility>

namespace mx {
namespace tiled {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BKB = 128;                     // code bytes per row per stage (256 K)
constexpr int SCALE_OPERAND = 256 * 16;      // 4 KiB: 256 rows x 16 B
constexpr int SCALE_CHUNK = 2 * SCALE_OPERAND;

// A8: the activations are MXFP8 (E4M3, one byte per element; W4A8), so an
// activation row carries 256 code bytes per 256-K stage and each activation
// fragment is two 16-byte reads (see read_offsets).
template <int MB_, int NB_, int WGM_, int WGN_, bool A8_ = false>
struct Shape {
    static constexpr int NW = WGM_ * WGN_;                // wavefronts per workgroup
    static_assert(NW == 4 || NW == 8, "four or eight wavefronts per workgroup");
    static constexpr int MB = MB_, NB = NB_, WGM = WGM_, WGN = WGN_;
    static constexpr bool A8 = A8_;
    static constexpr int BM = 32 * MB * WGM;              // activation rows per tile
    static constexpr int BN = 32 * NB * WGN;              // weight rows per tile
    static_assert(BM <= 256 && BN == 256, "scale staging holds 256 rows per operand");
    static constexpr int XBKB = A8 ? 2 * BKB : BKB;       // activation code bytes per row, stage
    static constexpr int XPARTS = A8 ? 2 : 1;             // 16-byte reads per activation fragment
    static constexpr int WLOADS = BN * BKB / 1024 / NW;   // 1 KiB code loads per thread per stage
    static constexpr int XLOADS = BM * XBKB / 1024 / NW;
    static constexpr int W_OPERAND = BN * BKB;
    static constexpr int CODE_STAGE = BN * BKB + BM * XBKB;   // W then X
    static constexpr int SCALE_BASE = 2 * CODE_STAGE;     // after the two code stages
    static constexpr int LDS_BYTES = SCALE_BASE + 3 * SCALE_CHUNK;
    static constexpr int LOADS_PER_STAGE = WLOADS + XLOADS + 1;
    static constexpr int SLOTS = 2 * MB * NB;             // MFMAs per half stage
    static constexpr int CODE_READS = 2 * (NB + MB * XPARTS);   // ds_read_b128 per half stage
    static constexpr int SCALE_READS = MB + NB;           // ds_read_b32 per stage
    // a stage's loads take one or two per MFMA slot
    static_assert(LOADS_PER_STAGE <= 2 * SLOTS && CODE_READS <= SLOTS, "slot budget");
};

using DenseShape = Shape<4, 2, 2, 4>;
// 128 activation rows x 256 weight rows, 8 waves of 64 x 64: for shapes with
// too few 256 x 256 tiles to fill the chip
using DenseHalfShape = Shape<2, 2, 2, 4>;
using GroupShape = Shape<4, 2, 1, 4>;
// W4A8: 128 activation rows, so that two stages of 256-byte rows fit the LDS
using W4A8Shape = Shape<2, 4, 2, 2, true>;

typedef __attribute__((address_space(3))) uint8_t lds_u8;
#define AS_LDS(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ uint32_t lds_addr(const lds_u8* p) { return (uint32_t)(uintptr_t)p; }

typedef int v4i __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over [base, base + bytes) (stride 0; loads past the
// end read 0): base address, num_records, and the gfx950 format word.
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return v4i{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}

struct Operands {
    v4i w, ws, x, xs;
};

// One 16-byte-per-lane buffer load into LDS: the wavefront's 64 lanes fill
// 1 KiB of LDS starting at `dst` (lane order, M0 = dst), each lane from its
// own voffset.  Written as inline assembly on purpose: the compiler then
// does not see these LDS writes, so it does not drain them before every LDS
// read (it cannot tell the buffers apart); the kernel orders them itself
// with explicit vmcnt waits and barriers.
__device__ __forceinline__ void dma16(v4i r, lds_u8* dst, uint32_t voff, uint32_t soff) {
    const v4i rs = {__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
                    __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_addr(dst))), "v"(voff), "s"(rs),
                   "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory", "m0");
}

// The wavefront's index in the workgroup as a scalar (uniform) value, so the
// LDS destinations of the DMA loads are computed in scalar registers.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Per-lane byte offsets of this thread's loads from a tile's first row: the
// same for every tile (the tile's first row is the buffer descriptors' base)
// and over K (the K position enters as the scalar offset).  A row past an
// operand's end has an offset past its descriptor's range, so its loads
// return zeros without touching memory; those rows' results are never
// stored.
template <class S>
struct LoadOffsets {
    uint32_t w[S::WLOADS], x[S::XLOADS], ws, xs;
};

// E2M1 rows are 8 chunks of 16 bytes per stage, swizzled by (row >> 1) & 7;
// E4M3 activation rows are 16 chunks, swizzled by row & 15 (16 rows of a
// 16-lane read group then cover all 64 banks).
template <class S>
__device__ __forceinline__ LoadOffsets<S> load_offsets(int64_t ldc, int64_t ldx, int64_t lds_) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    LoadOffsets<S> o;
#pragma unroll
    for (int i = 0; i < S::WLOADS; ++i) {
        const int row = (wave * S::WLOADS + i) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        o.w[i] = (uint32_t)(row * ldc + 16 * c);
    }
    constexpr int XCH = S::XBKB / 16;          // chunks per row and stage
#pragma unroll
    for (int i = 0; i < S::XLOADS; ++i) {
        const int row = (wave * S::XLOADS + i) * (1024 / S::XBKB) + lane / XCH;
        const int slot = lane % XCH;
        const int c = S::A8 ? (slot ^ (row & 15)) : (slot ^ ((row >> 1) & 7));
        o.x[i] = (uint32_t)(row * ldx + 16 * c);
    }
    const int row = wave * 64 + lane;
    o.ws = (uint32_t)(row * lds_);
    o.xs = (uint32_t)(row * lds_);
    return o;
}

template <class S>
__device__ __forceinline__ void load_codes(lds_u8* lds, const Operands& op,
                                           const LoadOffsets<S>& o, int buf, int kt) {
    const int wave = wave_id();
    const uint32_t k = (uint32_t)kt * BKB;
    const uint32_t kx = S::A8 ? (uint32_t)kt * S::XBKB : k;
    lds_u8* w = lds + buf * S::CODE_STAGE;
    lds_u8* x = w + S::W_OPERAND;
#pragma unroll
    for (int i = 0; i < S::WLOADS; ++i)
        dma16(op.w, w + (wave * S::WLOADS + i) * 1024, o.w[i], k);
#pragma unroll
    for (int i = 0; i < S::XLOADS; ++i)
        dma16(op.x, x + (wave * S::XLOADS + i) * 1024, o.x[i], kx);
}

// One operand's scales for chunk c (stages 2c, 2c+1) into ring slot `slot`:
// 16 bytes per row, 256 rows (an activation tile of fewer rows repeats its
// last row), one load by each of the first four wavefronts.
template <class S>
__device__ __forceinline__ void load_scales(lds_u8* lds, const Operands& op,
                                            const LoadOffsets<S>& o, bool weights, int c,
                                            int slot) {
    const int wave = wave_id();
    if (S::NW > 4 && wave >= 4) return;       // wave-uniform
    lds_u8* dst = lds + S::SCALE_BASE + slot * SCALE_CHUNK + (weights ? 0 : SCALE_OPERAND) +
                  wave * 1024;
    dma16(weights ? op.ws : op.xs, dst, weights ? o.ws : o.xs, (uint32_t)c * 16);
}

// Where one output tile's operands come from: the four buffer descriptors,
// each starting at the tile's first row and ending at its operand's end.
template <class S>
struct TileSrc {
    Operands op;
};

template <class S>
__device__ __forceinline__ TileSrc<S> tile_src(const uint8_t* x, const uint8_t* xs,
                                               const uint8_t* w, const uint8_t* ws, int64_t m0,
                                               int64_t m_end, int64_t n0, int64_t N, int64_t K) {
    const int64_t ldc = K / 2, ldx = S::A8 ? K : K / 2, lds_ = K / 32;
    const int64_t rows_w = N > n0 ? N - n0 : 0, rows_x = m_end > m0 ? m_end - m0 : 0;
    TileSrc<S> t;
    t.op = Operands{make_rsrc(w + n0 * ldc, (uint32_t)(rows_w * ldc)),
                    make_rsrc(ws + n0 * lds_, (uint32_t)(rows_w * lds_)),
                    make_rsrc(x + m0 * ldx, (uint32_t)(rows_x * ldx)),
                    make_rsrc(xs + m0 * lds_, (uint32_t)(rows_x * lds_))};
    return t;
}

// Field-wise uniform select between two tiles' sources.
template <class S>
__device__ __forceinline__ TileSrc<S> pick(bool p, const TileSrc<S>& a, const TileSrc<S>& b) {
    TileSrc<S> t;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        t.op.w[k] = p ? a.op.w[k] : b.op.w[k];
        t.op.ws[k] = p ? a.op.ws[k] : b.op.ws[k];
        t.op.x[k] = p ? a.op.x[k] : b.op.x[k];
        t.op.xs[k] = p ? a.op.xs[k] : b.op.xs[k];
    }
    return t;
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

// E2M1 weights (format code 4) times E4M3 activations (format code 0): the
// activation operand is 32 bytes a lane, bytes 0..15 and 16..31 as read_offsets
// places them.
template <int T>
__device__ __forceinline__ v16f mfma8(const v4u& a, const v4u& b0, const v4u& b1, v16f acc,
                                      uint32_t sa, uint32_t sb) {
    const v8i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
    const v8i bv = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                    (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 4, 0, T, (int)sa, T,
                                                           (int)sb);
}

template <class S>
constexpr int XP1 = S::XPARTS - 1;

// Half a stage of one wave's operands: NB weight and MB activation 32-row
// blocks, 2 K-steps each, 16 bytes per lane (activations: XPARTS x 16 bytes).
template <class S>
struct Half {
    v4u w[S::NB][2], x[S::MB][2][S::XPARTS];
};
// A stage's scale bytes: one 32-bit word (4 K-steps) per row block.
template <class S>
struct Scales {
    uint32_t w[S::NB], x[S::MB];
};

// Plain LDS reads: the compiler tracks their lgkmcnt itself.
typedef __attribute__((address_space(3))) const v4u lds_v4u;
typedef __attribute__((address_space(3))) const uint32_t lds_u32;
template <int OFF>
__device__ __forceinline__ void ds_read_b128(v4u& r, uint32_t addr) {
    r = *reinterpret_cast<lds_v4u*>((uintptr_t)(addr + OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_read_b32(uint32_t& r, uint32_t addr) {
    r = *reinterpret_cast<lds_u32*>((uintptr_t)(addr + OFF));
}

// Lane-constant LDS offsets.  Row r32 of block i sits at
// (base_row + 32 i + r32); its swizzled chunk for K-step t depends on r32 and
// t only, so every block is the same address plus 4 KiB * i.
struct ReadOffsetsE2M1 {
    uint32_t w[4], x[4], ws, xs;
};
struct ReadOffsetsE4M3 {
    uint32_t w[4], x[4], xh[4], ws, xs;   // xh: bytes 16..31 of an activation fragment
};
template <class S>
using ReadOffsets = std::conditional_t<S::A8, ReadOffsetsE4M3, ReadOffsetsE2M1>;

template <class S>
__device__ __forceinline__ ReadOffsets<S> read_offsets(int wn, int wm) {
    const int lane = threadIdx.x & 63;
    const int r32 = lane & 31, h = lane >> 5;
    ReadOffsets<S> r;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int pos = (4 * h + t) ^ ((r32 >> 1) & 7);
        r.w[t] = (uint32_t)((wn * 32 * S::NB + r32) * BKB + 16 * pos);
        if constexpr (S::A8) {
            const uint32_t xrow = (uint32_t)(S::W_OPERAND + (wm * 32 * S::MB + r32) * S::XBKB);
            // the E4M3 operand of the 32x32x64 MFMA (measured): lane half h
            // holds, in bytes 0..15, half h of the 32-K block whose scale lane
            // half 0 supplies and, in bytes 16..31, half h of lane half 1's.
            // In K-step t those are blocks t and 4+t of the stage (as for
            // E2M1), i.e. 16-byte chunks 2t+h and 8+2t+h of the row.
            r.x[t] = xrow + 16 * ((2 * t + h) ^ (r32 & 15));
            r.xh[t] = xrow + 16 * ((8 + 2 * t + h) ^ (r32 & 15));
        } else {
            r.x[t] = (uint32_t)(S::W_OPERAND + (wm * 32 * S::MB + r32) * BKB + 16 * pos);
        }
    }
    r.ws = (uint32_t)((wn * 32 * S::NB + r32) * 16 + 4 * h);
    r.xs = (uint32_t)(SCALE_OPERAND + (wm * 32 * S::MB + r32) * 16 + 4 * h);
    return r;
}

// End of a half-stage's reads.  The reads are ordinary loads, so the
// compiler places the lgkmcnt waits before the first use of each fragment.
template <class S>
__device__ __forceinline__ void settle(Half<S>&) {}
template <class S>
__device__ __forceinline__ void settle(Half<S>&, Scales<S>&) {}

// One operand load of a stage, selected by index: weight codes, then
// activation codes (both from `cs`), then the stage's scale half-chunk
// (from `ss`: chunk `chunk` of that tile into ring slot `slot`).
template <class S, int Q>
__device__ __forceinline__ void load_op(lds_u8* lds, const TileSrc<S>& cs, const TileSrc<S>& ss,
                                        const LoadOffsets<S>& lo, int buf, int kt, bool scale_w,
                                        int chunk, int slot) {
    const int wave = wave_id();
    if constexpr (Q < S::WLOADS) {
        dma16(cs.op.w, lds + buf * S::CODE_STAGE + (wave * S::WLOADS + Q) * 1024, lo.w[Q],
              (uint32_t)kt * BKB);
    } else if constexpr (Q < S::WLOADS + S::XLOADS) {
        constexpr int i = Q - S::WLOADS;
        dma16(cs.op.x, lds + buf * S::CODE_STAGE + S::W_OPERAND + (wave * S::XLOADS + i) * 1024,
              lo.x[i], (uint32_t)kt * S::XBKB);
    } else {
        load_scales<S>(lds, ss.op, lo, scale_w, chunk, slot);
    }
}

// One LDS read of a half-stage: for Q < CODE_READS, K-step s = Q / (NB+MB),
// then NB weight blocks and MB activation blocks; after that one scale word
// per row block (weights first).
template <class S, int H, int Q>
__device__ __forceinline__ void read_op(Half<S>& f, Scales<S>& sc, uint32_t codes,
                                        uint32_t scales, const ReadOffsets<S>& ro) {
    constexpr int P = S::NB + S::MB * S::XPARTS;
    if constexpr (Q < S::CODE_READS) {
        constexpr int s = Q / P, r = Q % P;
        if constexpr (r < S::NB) {
            ds_read_b128<r * 32 * BKB>(f.w[r][s], codes + ro.w[2 * H + s]);
        } else {
            constexpr int j = (r - S::NB) / S::XPARTS, part = (r - S::NB) % S::XPARTS;
            if constexpr (part == 0)
                ds_read_b128<j * 32 * S::XBKB>(f.x[j][s][0], codes + ro.x[2 * H + s]);
            else
                ds_read_b128<j * 32 * S::XBKB>(f.x[j][s][part], codes + ro.xh[2 * H + s]);
        }
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
                                           uint32_t scales, const ReadOffsets<S>& ro) {
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
        if constexpr (j < JL) {
            if constexpr (S::A8)
                acc[i][j] = mfma8<2 * H + t>(f.w[i][t], f.x[j][t][0], f.x[j][t][XP1<S>], acc[i][j],
                                             sc.w[i], sc.x[j]);
            else
                acc[i][j] = mfma<2 * H + t>(f.w[i][t], f.x[j][t][0], acc[i][j], sc.w[i], sc.x[j]);
        }
        step(std::integral_constant<int, Q>{});
        __builtin_amdgcn_sched_barrier(0);   // keep this slot's order
        mfma_half<S, JL, H, Q + 1>(f, sc, acc, step);
    }
}

// Epilogue.  The MFMA result layout gives each lane one output row and runs
// of 4 columns, so storing straight from the accumulators writes 8-16 bytes
// into each of 32 rows per instruction, and the write path then runs at a
// fraction of HBM speed.  Instead each wave parks ROWS rows of its tile in a
// private LDS region and writes them back as row segments: 16 bytes a lane,
// consecutive lanes along a row, so one instruction covers whole lines.  The
// region's row pitch is padded by 16 bytes, which puts the rows that one
// parking instruction writes on different banks and keeps every parking
// address a lane base plus an immediate.
template <class S, bool OUT_BF16>
struct Stage {
    static constexpr int ESIZE = OUT_BF16 ? 2 : 4;
    static constexpr int ROW_BYTES = 32 * S::NB * ESIZE;  // one wave's columns
    static constexpr int PITCH = ROW_BYTES + 16;
    static constexpr int CHUNKS = ROW_BYTES / 16;         // 16-byte pieces a row
    static constexpr int EPC = 16 / ESIZE;                // elements a piece
    // most rows per pass (32 .. 2, a whole number of 64-lane write-backs)
    // that fit a per-wave region of `budget` bytes
    static constexpr int rows_for(int budget) {
        int rows = 32;
        while (rows > 2 && (rows * PITCH > budget || (rows * CHUNKS) % 64 != 0)) rows /= 2;
        return rows;
    }
    static constexpr int bytes(int rows) { return rows * PITCH; }
};

// Store this wave's accumulators (rows [m0 + wm*32*MB, +32*MB) clipped to
// m_end, columns [n0 + wn*32*NB, +32*NB) clipped to N) through `stage`, this
// wave's own Stage::bytes(ROWS) bytes of LDS.  No other wave touches the
// region, and one wave's LDS instructions take effect in issue order, so the
// passes need only compiler fences: a read after the parking writes sees
// them, and the next pass's writes cannot overtake this pass's reads.
// bf16 bias[col .. col+3] as fp32 (0 past N); col is a multiple of 4, so the
// four values are one aligned 8-byte load when all are inside.
__device__ __forceinline__ v4f bias4(const uint16_t* __restrict__ bias, int64_t col, int64_t N) {
    if (col + 3 < N) {
        const v2u b = *reinterpret_cast<const v2u*>(bias + col);
        return v4f{__uint_as_float(b[0] << 16), __uint_as_float(b[0] & 0xFFFF0000u),
                   __uint_as_float(b[1] << 16), __uint_as_float(b[1] & 0xFFFF0000u)};
    }
    v4f r;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        r[e] = col + e < N ? __uint_as_float((uint32_t)bias[col + e] << 16) : 0.f;
    return r;
}

// BIAS: bias[n] (bf16) joins each fp32 sum before its one rounding.  BUF:
// whole pieces through a buffer descriptor (below).
template <class S, bool OUT_BF16, int ROWS, bool BIAS = false, bool BUF = false>
__device__ __forceinline__ void store_tile(const v16f (&acc)[S::NB][S::MB], lds_u8* stage,
                                           void* __restrict__ y, int64_t m0, int64_t m_end,
                                           int64_t n0, int64_t N, int wn, int wm,
                                           const uint16_t* __restrict__ bias = nullptr) {
    using T = Stage<S, OUT_BF16>;
    static_assert(ROWS >= 2 && ROWS <= 32 && (ROWS & (ROWS - 1)) == 0, "a 32-row block in passes");
    static_assert((ROWS * T::CHUNKS) % 64 == 0, "whole instructions per pass");
    // an opaque lane index keeps the per-lane addresses below inside the
    // epilogue: hoisted out of a persistent walk's tile loop they are held
    // across the main loop, which spills them
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int r32 = lane & 31, h = lane >> 5;
    const bool vec_ok = (N % T::EPC) == 0 && (reinterpret_cast<uintptr_t>(y) % 16) == 0;
    const int64_t col0 = n0 + wn * 32 * S::NB;
    // BUF: whole 16-byte pieces go through a buffer descriptor over the
    // pass's rows: its range drops the rows past m_end, and a piece past N
    // gets an offset beyond any range.  Each store is then one 32-bit offset,
    // not a 64-bit address, two 64-bit compares and a branch.  The wave's
    // rows must span under 2 GiB of y.  Measured 1-2% faster for the grouped
    // GEMMs, whose epilogues nothing overlaps; no gain for the dense tiles.
    const int64_t pitch = N * T::ESIZE;
    const bool fast =
        BUF && vec_ok && col0 < N && pitch * (32 * S::MB) < ((int64_t)1 << 31);
    const int cols_left = (int)min(N - col0, (int64_t)(32 * S::NB));
#pragma unroll
    for (int j = 0; j < S::MB; ++j) {
#pragma unroll
        for (int p = 0; p < 32 / ROWS; ++p) {
            const int64_t row0 = m0 + wm * 32 * S::MB + 32 * j + p * ROWS;
            if (row0 >= m_end) return;            // wave-uniform
            // park: lane (r32, h) holds row r32, columns 32i + 8b + 4h + 0..3
            const int r = r32 - p * ROWS;
            if (ROWS == 32 || (r >= 0 && r < ROWS)) {
#pragma unroll
                for (int i = 0; i < S::NB; ++i) {
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        lds_u8* dst = stage + r * T::PITCH + (32 * i + 8 * b + 4 * h) * T::ESIZE;
                        float v0 = acc[i][j][4 * b], v1 = acc[i][j][4 * b + 1];
                        float v2 = acc[i][j][4 * b + 2], v3 = acc[i][j][4 * b + 3];
                        if constexpr (BIAS) {
                            const v4f bv = bias4(bias, col0 + 32 * i + 8 * b + 4 * h, N);
                            v0 += bv[0], v1 += bv[1], v2 += bv[2], v3 += bv[3];
                        }
                        if (OUT_BF16)
                            *reinterpret_cast<__attribute__((address_space(3))) v2u*>(dst) =
                                v2u{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
                        else
                            *reinterpret_cast<__attribute__((address_space(3))) v4u*>(dst) =
                                v4u{__float_as_uint(v0), __float_as_uint(v1), __float_as_uint(v2),
                                    __float_as_uint(v3)};
                    }
                }
            }
            asm volatile("" ::: "memory");         // reads after the writes
            if (fast) {
                const int64_t rows_left = m_end - row0;   // > 0
                const int ipitch = (int)pitch;
                const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(
                    reinterpret_cast<uint8_t*>(y) + row0 * pitch + col0 * T::ESIZE, (short)0,
                    (int)(min(rows_left, (int64_t)ROWS) * pitch - col0 * T::ESIZE), 0x00020000);
#pragma unroll
                for (int q = 0; q < ROWS * T::CHUNKS / 64; ++q) {
                    const int c = q * 64 + lane;
                    const int rr = c / T::CHUNKS, cc = c % T::CHUNKS;
                    const v4u v = *reinterpret_cast<const __attribute__((address_space(3))) v4u*>(
                        stage + rr * T::PITCH + cc * 16);
                    const int off = cc * T::EPC < cols_left ? rr * ipitch + cc * 16 : 0x7FFFFFF0;
                    // non-temporal, as below
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v), out, off,
                                                           0, 2);
                }
                asm volatile("" ::: "memory");     // next writes after the reads
                continue;
            }
#pragma unroll
            for (int q = 0; q < ROWS * T::CHUNKS / 64; ++q) {
                const int c = q * 64 + lane;
                const int rr = c / T::CHUNKS, cc = c % T::CHUNKS;
                const v4u v = *reinterpret_cast<const __attribute__((address_space(3))) v4u*>(
                    stage + rr * T::PITCH + cc * 16);
                const int64_t m = row0 + rr;
                const int64_t n = col0 + (int64_t)cc * T::EPC;
                if (m >= m_end || n >= N) continue;
                if (vec_ok && n + T::EPC <= N) {
                    // non-temporal: Y is written once and not read back here,
                    // and streaming it past the Infinity Cache keeps the
                    // operands of the next launches there (measured: the
                    // prefill step 5% faster)
                    __builtin_nontemporal_store(
                        v, reinterpret_cast<v4u*>(reinterpret_cast<uint8_t*>(y) +
                                                  (m * N + n) * T::ESIZE));
                } else {
#pragma unroll
                    for (int e = 0; e < T::EPC; ++e) {
                        if (n + e >= N) break;
                        if (OUT_BF16)
                            reinterpret_cast<uint16_t*>(y)[m * N + n + e] =
                                (uint16_t)(v[e / 2] >> (16 * (e % 2)));
                        else
                            reinterpret_cast<uint32_t*>(y)[m * N + n + e] = v[e];
                    }
                }
            }
            asm volatile("" ::: "memory");         // next writes after the reads
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

// Pipeline registers of one wavefront: two half-stages of fragments and the
// scale words of the current and the next stage.
template <class S>
struct Pipe {
    Half<S> h0, h1;
    Scales<S> sc_cur, sc_nxt;
};

__device__ __forceinline__ uint32_t code_addr(uint32_t lds0, int s, int code_stage) {
    return lds0 + (uint32_t)((s & 1) * code_stage);
}
// Scale words of stage s of a tile whose chunk 0 sits in ring slot cbase % 3.
template <class S>
__device__ __forceinline__ uint32_t scale_addr(uint32_t lds0, int cbase, int s) {
    return lds0 + (uint32_t)(S::SCALE_BASE + ((cbase + s / 2) % 3) * SCALE_CHUNK + (s & 1) * 8);
}

// Stage loads and their scale halves.  Stage s of a tile (nkt stages, chunks
// 0..nkt/2-1, chunk 0 in ring slot cbase % 3) brings half s&1 (weights, then
// activations) of chunk s/2 + 1; chunk 0 is loaded on its own before stage 0.
// When that chunk does not exist (the last two stages), the slot carries
// chunk 0 of the next tile if one is being prefetched, else it reloads the
// tile's last chunk (the same bytes, harmless).
//
// Prologue: chunk 0, stage 0, stage 1; wait for stage 0; read its first half.
template <class S>
__device__ __forceinline__ void prologue(lds_u8* lds, const TileSrc<S>& src,
                                         const LoadOffsets<S>& lo, int nkt, int cbase, Pipe<S>& pp,
                                         const ReadOffsets<S>& ro) {
    const int last_chunk = nkt / 2 - 1;
    const int c1 = last_chunk >= 1 ? 1 : 0;
    load_codes<S>(lds, src.op, lo, 0, 0);
    load_scales<S>(lds, src.op, lo, true, 0, cbase % 3);
    load_scales<S>(lds, src.op, lo, false, 0, cbase % 3);
    load_scales<S>(lds, src.op, lo, true, c1, (cbase + c1) % 3);
    load_scales<S>(lds, src.op, lo, false, c1, (cbase + c1) % 3);
    load_codes<S>(lds, src.op, lo, 1, nkt > 1 ? 1 : 0);
    wait_vm<S::WLOADS + S::XLOADS>();
    __builtin_amdgcn_s_barrier();
    const uint32_t lds0 = lds_addr(lds);
    read_range<S, 0, 0, S::CODE_READS + S::SCALE_READS>(
        pp.h0, pp.sc_cur, code_addr(lds0, 0, S::CODE_STAGE), scale_addr<S>(lds0, cbase, 0), ro);
    settle(pp.h0, pp.sc_cur);
}

// The pipelined main loop of one output tile (its stages 0 and 1 are loaded
// and stage 0's first half is in pp.h0 / pp.sc_cur).  Only the first JL
// 32-row activation blocks of each wave are multiplied.  With PREFETCH, the
// loads of stages nkt and nkt+1 are the next tile's stages 0 and 1 (and its
// scale chunks 0 and 1), and the loop ends with the next tile's stage 0
// first half in pp.h0 / pp.sc_cur: the next tile needs no prologue.
// PREFETCH needs nkt >= 4.  With DEFER as well, the next tile's stage 1 code
// loads are left out, so the stage-1 buffer is free once the loop ends (the
// last stage's barrier is past every wave's reads of it); the caller issues
// them (load_codes into buffer 1) after using the buffer.
// Per stage kt (one barrier per stage):
//   read half 1 of stage kt;  MFMAs on half 0;  wait for the reads
//   wait for stage kt+1's loads; barrier; load stage kt+2 (+ one scale half-chunk)
//   read half 0 of stage kt+1;  MFMAs on half 1;  wait for the reads
template <class S, int JL, bool PREFETCH, bool DEFER = false>
__device__ __forceinline__ void main_loop(lds_u8* lds, const TileSrc<S>& cur,
                                          const TileSrc<S>& nxt, const LoadOffsets<S>& lo,
                                          int nkt, int cbase, Pipe<S>& pp,
                                          v16f (&acc)[S::NB][S::MB], const ReadOffsets<S>& ro) {
    const int last_chunk = nkt / 2 - 1;
    const uint32_t lds0 = lds_addr(lds);
    for (int kt = 0; kt < nkt; ++kt) {
        // first half: MFMAs on stage kt's K-steps 0-1, reads of its K-steps 2-3
        {
            const uint32_t codes = code_addr(lds0, kt, S::CODE_STAGE);
            Scales<S> unused;
            mfma_half<S, JL, 0>(pp.h0, pp.sc_cur, acc, [&](auto q) {
                constexpr int Q = decltype(q)::value;
                if constexpr (Q < S::CODE_READS) read_op<S, 1, Q>(pp.h1, unused, codes, 0, ro);
            });
            settle(pp.h1);
        }
        // stage kt+1 landed for every wave; every wave is done reading stage kt
        wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        // second half: MFMAs on K-steps 2-3, loads of stage kt+2 into stage
        // kt's buffer, reads of stage kt+1's K-steps 0-1 and scales
        {
            const int s2 = kt + 2;
            const bool code_next = PREFETCH && s2 >= nkt;
            const int ks = s2 < nkt ? s2 : (PREFETCH ? s2 - nkt : nkt - 1);
            const int c = s2 / 2 + 1;
            bool scale_next = false;
            int chunk = c, slot = (cbase + c) % 3;
            if (c > last_chunk) {
                if (PREFETCH) {
                    scale_next = true;
                    chunk = s2 < nkt ? 0 : 1;
                    slot = (cbase + last_chunk + 1 + chunk) % 3;
                } else {
                    chunk = last_chunk;
                    slot = (cbase + last_chunk) % 3;
                }
            }
            const bool scale_w = (s2 & 1) == 0;
            const uint32_t codes = code_addr(lds0, kt + 1, S::CODE_STAGE);
            const uint32_t scales = scale_addr<S>(lds0, cbase, kt + 1);
            const TileSrc<S> cs = PREFETCH ? pick(code_next, nxt, cur) : cur;
            const TileSrc<S> ss = PREFETCH ? pick(scale_next, nxt, cur) : cur;
            const bool codes_deferred = PREFETCH && DEFER && kt == nkt - 1;
            mfma_half<S, JL, 1>(pp.h1, pp.sc_cur, acc, [&](auto q) {
                constexpr int Q = decltype(q)::value;
                if constexpr (Q < S::WLOADS + S::XLOADS) {
                    if (!codes_deferred)
                        load_op<S, Q>(lds, cs, ss, lo, s2 & 1, ks, scale_w, chunk, slot);
                } else if constexpr (Q < S::LOADS_PER_STAGE) {
                    load_op<S, Q>(lds, cs, ss, lo, s2 & 1, ks, scale_w, chunk, slot);
                }
                // a stage with more loads than slots (W4A8): the rest, scale
                // loads only, ride along from slot 0
                if constexpr (Q + S::SLOTS < S::LOADS_PER_STAGE) {
                    static_assert(Q + S::SLOTS >= S::WLOADS + S::XLOADS, "only scale loads");
                    load_op<S, Q + S::SLOTS>(lds, cs, ss, lo, s2 & 1, ks, scale_w, chunk, slot);
                }
                read_range<S, 0, second_half_read<S>(Q), second_half_read<S>(Q + 1)>(
                    pp.h0, pp.sc_nxt, codes, scales, ro);
            });
            settle(pp.h0, pp.sc_nxt);
            pp.sc_cur = pp.sc_nxt;
        }
    }
}

template <class S>
__device__ __forceinline__ void zero_acc(v16f (&acc)[S::NB][S::MB]) {
#pragma unroll
    for (int i = 0; i < S::NB; ++i)
#pragma unroll
        for (int j = 0; j < S::MB; ++j) acc[i][j] = v16f{};
}

// Linear tile index -> (tile row, tile column), walked in groups of `gm`
// tile-rows so that a run of consecutive indices covers a compact block of
// the output (the operand rows it shares stay in one XCD's L2).
__device__ __forceinline__ void tile_of(int t, int tiles_m, int tiles_n, int gm, int& tm, int& tn) {
    const int group_size = gm * tiles_n;
    const int group = t / group_size;
    const int first_m = group * gm;
    const int rows = min(gm, tiles_m - first_m);
    const int in_group = t - group * group_size;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
}

// Zero the accumulators for the next tile of a persistent walk, after the
// epilogue.  With a plain zero_acc the compiler zeroes the next tile's AGPRs
// before the epilogue and first moves all results into VGPRs, which spills;
// zeros that come out of a volatile asm cannot move above the epilogue's
// LDS writes.
template <class S>
__device__ __forceinline__ void rezero_acc(v16f (&acc)[S::NB][S::MB]) {
    v16f z = v16f{};
    asm volatile("" : "+v"(z));
#pragma unroll
    for (int i = 0; i < S::NB; ++i)
#pragma unroll
        for (int j = 0; j < S::MB; ++j) acc[i][j] = z;
}

// XCD-aware tile order: workgroup ids are dealt to the 8 XCDs round-robin, so
// id -> (xcd, local) is remapped to a linear tile index that gives each XCD a
// contiguous run.
__device__ __forceinline__ bool tile_coords(int tiles_m, int tiles_n, int gm, int& tm, int& tn) {
    const int per_xcd = (int)gridDim.x / 8;
    const int id = (int)blockIdx.x;
    const int t = (id % 8) * per_xcd + id / 8;
    if (t >= tiles_m * tiles_n) return false;
    tile_of(t, tiles_m, tiles_n, gm, tm, tn);
    return true;
}

// The epilogue of an MoE gate_up GEMM fused with the expert activation and
// its MXFP4 quantization.  The gate_up weight rows are interleaved in groups
// of 64: 32 gate rows, then the 32 up rows of the same columns of h, so a
// wave's 64 output columns are the gate and up halves of one 32-column MX
// block of h.  The accumulators are parked as bf16 (RNE, what the plain
// GEMM would store); then the 64 lanes split a pass's ROWS rows, 64 / ROWS
// lanes a row, each taking a run of the block's gate and up values:
// h = bf16(silu(g) * u) in the act-quant kernel's GLU arithmetic, the block
// amax across the row's lanes, and the codes and scale byte by the act-quant
// rule.  So the result equals the plain GEMM followed by the act-quant
// kernel's GLU mode, bit for bit.  h codes are [rows][N/4] bytes, scales
// [rows][N/64].
template <class S, int ROWS, bool UOS>
__device__ __forceinline__ void store_tile_glu(const v16f (&acc)[S::NB][S::MB], lds_u8* stage,
                                               uint8_t* __restrict__ hc,
                                               uint8_t* __restrict__ hs, int64_t m0,
                                               int64_t m_end, int64_t n0, int64_t N, int wn,
                                               int wm) {
    static_assert(S::NB == 2, "one gate block and one up block per wave");
    static_assert(ROWS == 16 || ROWS == 32, "4 or 2 lanes a row");
    using T = Stage<S, true>;
    constexpr int LPR = 64 / ROWS;            // lanes a row
    constexpr int WPL = 16 / LPR;             // packed bf16 pairs a lane (4 or 8)
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int r32 = lane & 31, h = lane >> 5;
    const int rr = lane % ROWS, part = lane / ROWS;
    const int64_t col0 = n0 + wn * 64;
    if (col0 >= N) return;                    // wave-uniform; N % 64 == 0
    const int64_t blk = col0 / 64;            // this wave's MX block of h
    const int64_t hrow = N / 4, srow = N / 64;
#pragma unroll
    for (int j = 0; j < S::MB; ++j) {
#pragma unroll
        for (int p = 0; p < 32 / ROWS; ++p) {
            const int64_t row0 = m0 + wm * 32 * S::MB + 32 * j + p * ROWS;
            if (row0 >= m_end) return;            // wave-uniform
            const int r = r32 - p * ROWS;
            if (ROWS == 32 || (r >= 0 && r < ROWS)) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        lds_u8* dst = stage + r * T::PITCH + (32 * i + 8 * b + 4 * h) * 2;
                        *reinterpret_cast<__attribute__((address_space(3))) v2u*>(dst) =
                            v2u{pack_bf16x2(acc[i][j][4 * b], acc[i][j][4 * b + 1]),
                                pack_bf16x2(acc[i][j][4 * b + 2], acc[i][j][4 * b + 3])};
                    }
                }
            }
            asm volatile("" ::: "memory");         // reads after the writes
            // lane: row rr, columns [2 WPL part, 2 WPL (part + 1)) of the block
            const lds_u8* src = stage + rr * T::PITCH + part * 4 * WPL;
            uint32_t w[WPL];
#pragma unroll
            for (int c = 0; c < WPL / 4; ++c) {
                const v4u gv =
                    *reinterpret_cast<const __attribute__((address_space(3))) v4u*>(src + 16 * c);
                const v4u uv = *reinterpret_cast<const __attribute__((address_space(3))) v4u*>(
                    src + 64 + 16 * c);
#pragma unroll
                for (int e = 0; e < 4; ++e) w[4 * c + e] = glu_pair(gv[e], uv[e]);
            }
            asm volatile("" ::: "memory");         // the next pass's writes after these reads
            // the act-quant rule on the block: amax of the bf16 magnitudes
            // (as integers) over the row's lanes, then one scale for all
            uint32_t amax = 0;
#pragma unroll
            for (int i = 0; i < WPL; ++i) {
                const uint32_t a = w[i] & 0x7FFF7FFFu;
                amax = max(amax, max(a & 0xFFFFu, a >> 16));
            }
#pragma unroll
            for (int o = ROWS; o < 64; o *= 2) amax = max(amax, (uint32_t)__shfl_xor((int)amax, o));
            const uint32_t byte = mx_scale_byte<UOS>(amax << 16);
            const float scale = e8m0_to_f32(byte);
            const int64_t m = row0 + rr;
            if (m < m_end) {
                uint32_t c[WPL / 4];
#pragma unroll
                for (int d = 0; d < WPL / 4; ++d) {
                    uint32_t v = cvt_fp4x2_bf16<0>(0u, w[4 * d], scale);
                    v = cvt_fp4x2_bf16<1>(v, w[4 * d + 1], scale);
                    v = cvt_fp4x2_bf16<2>(v, w[4 * d + 2], scale);
                    v = cvt_fp4x2_bf16<3>(v, w[4 * d + 3], scale);
                    c[d] = byte == 255u ? 0u : v;
                }
                uint8_t* dst = hc + m * hrow + blk * 16 + part * WPL;   // WPL code bytes a lane
                if constexpr (WPL == 4)
                    *reinterpret_cast<uint32_t*>(dst) = c[0];
                else
                    *reinterpret_cast<uint2*>(dst) = make_uint2(c[0], c[1]);
                if (part == 0) hs[m * srow + blk] = (uint8_t)byte;
            }
        }
    }
}

template <bool OUT_BF16, bool BIAS, class S>
__global__ __launch_bounds__(256, 1) void gemm_tiled_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ xs,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws, int64_t M, int64_t N,
    int64_t K, void* __restrict__ y, int gm, const uint16_t* __restrict__ bias) {
    static_assert(S::NW == 4, "the half-stage pipeline of four wavefronts");
    __shared__ __attribute__((aligned(16))) uint8_t smem[S::LDS_BYTES];
    const int tiles_m = (int)((M + S::BM - 1) / S::BM);
    const int tiles_n = (int)((N + S::BN - 1) / S::BN);
    int tm, tn;
    if (!tile_coords(tiles_m, tiles_n, gm, tm, tn)) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % S::WGN, wm = wave / S::WGN;
    const int64_t m0 = (int64_t)tm * S::BM, n0 = (int64_t)tn * S::BN;
    const int nkt = (int)(K / 256);           // even: K % 512 == 0
    lds_u8* lds = (lds_u8*)smem;
    const TileSrc<S> src = tile_src<S>(x, xs, w, ws, m0, M, n0, N, K);
    const ReadOffsets<S> ro = read_offsets<S>(wn, wm);
    const LoadOffsets<S> lo = load_offsets<S>(K / 2, S::A8 ? K : K / 2, K / 32);
    v16f acc[S::NB][S::MB];
    zero_acc<S>(acc);
    Pipe<S> pp;
    prologue<S>(lds, src, lo, nkt, 0, pp, ro);
    main_loop<S, S::MB, false>(lds, src, src, lo, nkt, 0, pp, acc, ro);
    wait_vm<0>();                             // drain the surplus loads
    // every wave is past its last read of the stage buffers, which now hold
    // the four waves' epilogue regions
    __syncthreads();
    using T = Stage<S, OUT_BF16>;
    constexpr int ROWS = T::rows_for(S::SCALE_BASE / 4);   // both code stages
    store_tile<S, OUT_BF16, ROWS, BIAS>(acc, lds + wave * T::bytes(ROWS), y, m0, M, n0, N, wn,
                                        wm, bias);
}

// ---------------------------------------------------------------------------
// Dense GEMM of a 4-wave shape (the W4A8 tile), persistent, for more than one
// round of tiles and K >= 1024: one workgroup per CU walks the tiles
//   t = xcd * ceil(total / 8) + local + k * (grid / 8)   (xcd = id % 8, local = id / 8)
// (the XCD-contiguous runs above, now visited by the XCD's workgroups side by
// side).  While a tile's last two stages run, the next tile's first stage
// and its first two scale chunks load into the freed buffers, so only a
// workgroup's first tile pays the prologue.  The epilogue parks each wave's
// rows in the part of the stage-1 buffer that the wave's own loads of the
// next tile's stage 1 fill, and issues those loads right after: Y's stores
// then drain while the next tile runs.
// ---------------------------------------------------------------------------
constexpr int LDS_LIMIT = 160 * 1024;           // LDS a workgroup may hold

template <bool OUT_BF16, bool BIAS, class S>
__global__ __launch_bounds__(256, 1) void gemm_persistent_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ xs,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws, int64_t M, int64_t N,
    int64_t K, void* __restrict__ y, int gm, const uint16_t* __restrict__ bias) {
    static_assert(S::NW == 4, "the half-stage pipeline of four wavefronts");
    using T = Stage<S, OUT_BF16>;
    constexpr int ROWS = T::rows_for(S::WLOADS * 1024);   // a wave's weight rows of a stage
    __shared__ __attribute__((aligned(16))) uint8_t smem[S::LDS_BYTES];
    const int tiles_m = (int)((M + S::BM - 1) / S::BM);
    const int tiles_n = (int)((N + S::BN - 1) / S::BN);
    const int total = tiles_m * tiles_n;
    const int per_xcd = (total + 7) / 8;
    const int stride = (int)gridDim.x / 8;
    const int xcd = (int)blockIdx.x % 8;
    const int t_end = min(xcd * per_xcd + per_xcd, total);
    int t = xcd * per_xcd + (int)blockIdx.x / 8;
    if (t >= t_end) return;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % S::WGN, wm = wave / S::WGN;
    const int nkt = (int)(K / 256);           // even, >= 4: K % 512 == 0, K >= 1024
    lds_u8* lds = (lds_u8*)smem;
    // where load_codes puts this wave's weight rows of stage 1
    lds_u8* stage = lds + S::CODE_STAGE + wave * S::WLOADS * 1024;
    const ReadOffsets<S> ro = read_offsets<S>(wn, wm);
    const LoadOffsets<S> lo = load_offsets<S>(K / 2, S::A8 ? K : K / 2, K / 32);
    int tm, tn;
    tile_of(t, tiles_m, tiles_n, gm, tm, tn);
    TileSrc<S> cur =
        tile_src<S>(x, xs, w, ws, (int64_t)tm * S::BM, M, (int64_t)tn * S::BN, N, K);
    v16f acc[S::NB][S::MB];
    zero_acc<S>(acc);
    Pipe<S> pp;
    int cbase = 0;
    prologue<S>(lds, cur, lo, nkt, cbase, pp, ro);
    for (;;) {
        const int t_next = t + stride;
        const bool have_next = t_next < t_end;
        int tm_next = tm, tn_next = tn;
        if (have_next) tile_of(t_next, tiles_m, tiles_n, gm, tm_next, tn_next);
        // the last tile streams its own first stages again: surplus loads,
        // drained before the workgroup ends, that keep one loop body
        const TileSrc<S> nxt = tile_src<S>(x, xs, w, ws, (int64_t)tm_next * S::BM, M,
                                           (int64_t)tn_next * S::BN, N, K);
        main_loop<S, S::MB, true, true>(lds, cur, nxt, lo, nkt, cbase, pp, acc, ro);
        store_tile<S, OUT_BF16, ROWS, BIAS>(acc, stage, y, (int64_t)tm * S::BM, M,
                                            (int64_t)tn * S::BN, N, wn, wm, bias);
        if (!have_next) break;
        load_codes<S>(lds, nxt.op, lo, 1, 1);     // after this wave's epilogue reads
        rezero_acc<S>(acc);
        cbase += nkt / 2;
        cur = nxt;
        t = t_next;
        tm = tm_next;
        tn = tn_next;
    }
    wait_vm<0>();
}

// ---------------------------------------------------------------------------
// Dense GEMM, 8 wavefronts, two on every SIMD: the 256 x 256 tile of
// DenseShape (each wave 128 activation rows x 64 weight rows) or the 128 x
// 256 tile of DenseHalfShape (64 x 64 a wave).  Whenever one of a SIMD's
// waves stalls issuing a load or waiting on LDS, the other can issue its
// MFMAs.  Its accumulators (128 registers at DenseShape) leave room for only
// one K-step's fragments ahead, so the register pipeline runs at K-step
// granularity; the LDS layout and the operand order are those of the 4-wave
// tiles, and the outputs are bit-identical to theirs.
//
// Per stage kt (4 K-steps, one barrier):
//   K-step 0: MFMAs on f0;  read K-step 1 into f1;  DMA group B of stage kt+1
//   K-step 1: MFMAs on f1;  read K-step 2 into f0
//   K-step 2: MFMAs on f0;  read K-step 3 into f1
//   wait for this wave's loads (stage kt+1 landed); barrier
//   K-step 3: MFMAs on f1;  read stage kt+1's K-step 0 into f0 and its scale
//             words;  DMA group A of stage kt+2 (into stage kt's buffer,
//             which no wave reads after the barrier) and its scale half-chunk
// A stage's code loads a wave (8, or 6 at DenseHalfShape) are split into two
// halves: group A waits behind the barrier, group B rides on the next
// stage's first K-step.  Past the last stage the loads repeat the last stage
// (into a buffer nothing reads again) and the reads fetch unused values, so
// every stage issues the same instructions; the surplus loads drain at the
// end.
// ---------------------------------------------------------------------------
namespace d8 {

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// One K-step of one wave's operands: NB weight and MB activation fragments.
template <class S>
struct KFrag {
    v4u w[S::NB], x[S::MB];
};

// Read R of K-step T of the stage at `codes`: weight fragments first.
template <class S, int T, int R>
__device__ __forceinline__ void kread(KFrag<S>& f, uint32_t codes, const ReadOffsets<S>& ro) {
    if constexpr (R < S::NB)
        ds_read_b128<R * 32 * BKB>(f.w[R], codes + ro.w[T]);
    else
        ds_read_b128<(R - S::NB) * 32 * BKB>(f.x[R - S::NB], codes + ro.x[T]);
}
template <class S, int R>
__device__ __forceinline__ void sread(Scales<S>& sc, uint32_t scales, const ReadOffsets<S>& ro) {
    if constexpr (R < S::NB)
        ds_read_b32<R * 32 * 16>(sc.w[R], scales + ro.ws);
    else
        ds_read_b32<(R - S::NB) * 32 * 16>(sc.x[R - S::NB], scales + ro.xs);
}

// The MFMAs of K-step T; after MFMA q, step(q) issues that slot's reads and
// loads.  Each MFMA is pinned in program order: left free, the compiler sank
// them below the reads threaded between them, which kept several K-steps'
// fragments alive at once and spilled.  MF = false: a wave with no rows to
// multiply (half tiles) keeps the slots' loads and drops its MFMAs.
template <class S, int T, bool MF, int Q = 0, typename Step>
__device__ __forceinline__ void kmfma(const KFrag<S>& f, const Scales<S>& sc,
                                      v16f (&acc)[S::NB][S::MB], Step&& step) {
    if constexpr (Q < S::NB * S::MB) {
        constexpr int i = Q / S::MB, j = Q % S::MB;
        if constexpr (MF) {
            acc[i][j] = mfma<T>(f.w[i], f.x[j], acc[i][j], sc.w[i], sc.x[j]);
            asm volatile("" ::"v"(acc[i][j]));
        }
        step(std::integral_constant<int, Q>{});
        __builtin_amdgcn_sched_barrier(0);
        kmfma<S, T, MF, Q + 1>(f, sc, acc, step);
    }
}

// Code load l of a stage (0 .. WLOADS + XLOADS - 1) in group [L0, L1),
// spread over the K-step's MFMA slots: the load slot q issues, or -1.
template <int L0, int L1, int SLOTS>
constexpr int slot_load(int q) {
    const int n = L1 - L0;
    for (int k = 0; k < n; ++k)
        if (q == k * SLOTS / n) return L0 + k;
    return -1;
}

template <class S>
struct Groups {
    static constexpr int NL = S::WLOADS + S::XLOADS;   // code loads a wave, a stage
    static constexpr int A = NL / 2;                   // [0, A) behind the barrier
    static constexpr int B1 = NL;                      // [A, B1) in the next K-step 0
    static_assert(A + 1 <= S::NB * S::MB, "group A and the scale load fit the slots");
};

// Stage 0, the scale chunks of stages 0-3 and stage 1's group A; then stage
// 0's K-step 0 fragments and scale words (MF: the wave multiplies).
template <class S, bool MF>
__device__ __forceinline__ void prologue(lds_u8* lds, const TileSrc<S>& src,
                                         const LoadOffsets<S>& lo, int nkt, KFrag<S>& f0,
                                         Scales<S>& sc, const ReadOffsets<S>& ro) {
    using G = Groups<S>;
    const int c1 = nkt / 2 - 1 >= 1 ? 1 : 0;
    load_codes<S>(lds, src.op, lo, 0, 0);
    load_scales<S>(lds, src.op, lo, true, 0, 0);
    load_scales<S>(lds, src.op, lo, false, 0, 0);
    load_scales<S>(lds, src.op, lo, true, c1, c1);
    load_scales<S>(lds, src.op, lo, false, c1, c1);
    static_for<G::A>([&](auto l) {
        load_op<S, decltype(l)::value>(lds, src, src, lo, 1, 1, true, 0, 0);
    });
    wait_vm<G::A>();                          // all but stage 1's group A
    __builtin_amdgcn_s_barrier();
    const uint32_t lds0 = lds_addr(lds);
    if constexpr (MF)
        static_for<S::NB + S::MB>([&](auto r) {
            kread<S, 0, decltype(r)::value>(f0, code_addr(lds0, 0, S::CODE_STAGE), ro);
            sread<S, decltype(r)::value>(sc, scale_addr<S>(lds0, 0, 0), ro);
        });
}

template <class S, bool MF>
__device__ __forceinline__ void main_loop(lds_u8* lds, const TileSrc<S>& src,
                                          const LoadOffsets<S>& lo, int nkt, KFrag<S>& f0,
                                          KFrag<S>& f1, Scales<S>& sc,
                                          v16f (&acc)[S::NB][S::MB], const ReadOffsets<S>& ro) {
    using G = Groups<S>;
    constexpr int SL = S::NB * S::MB;        // MFMA slots of a K-step
    constexpr int NR = S::NB + S::MB;        // fragment reads of a K-step
    static_assert(NR <= SL, "one fragment read and one scale read a slot");
    const int last_chunk = nkt / 2 - 1;
    const uint32_t lds0 = lds_addr(lds);
    for (int kt = 0; kt < nkt; ++kt) {
        const uint32_t codes = code_addr(lds0, kt, S::CODE_STAGE);
        const int k1 = kt + 1;
        const int ks1 = k1 < nkt ? k1 : nkt - 1;
        kmfma<S, 0, MF>(f0, sc, acc, [&](auto q) {
            constexpr int Q = decltype(q)::value;
            if constexpr (MF && Q < NR) kread<S, 1, Q>(f1, codes, ro);
            constexpr int L = slot_load<G::A, G::B1, SL>(Q);
            if constexpr (L >= 0) load_op<S, L>(lds, src, src, lo, k1 & 1, ks1, true, 0, 0);
        });
        kmfma<S, 1, MF>(f1, sc, acc, [&](auto q) {
            constexpr int Q = decltype(q)::value;
            if constexpr (MF && Q < NR) kread<S, 2, Q>(f0, codes, ro);
        });
        kmfma<S, 2, MF>(f0, sc, acc, [&](auto q) {
            constexpr int Q = decltype(q)::value;
            if constexpr (MF && Q < NR) kread<S, 3, Q>(f1, codes, ro);
        });
        // stage kt+1 landed for every wave; every wave has issued its reads
        // of stage kt (LDS reads finish long before a DMA's data arrives)
        wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        const int s2 = kt + 2;
        const int ks2 = s2 < nkt ? s2 : nkt - 1;
        const int c = min(s2 / 2 + 1, last_chunk);   // past the last: that chunk again
        const bool scale_w = (s2 & 1) == 0;
        const uint32_t ncodes = code_addr(lds0, k1, S::CODE_STAGE);
        const uint32_t nscales = scale_addr<S>(lds0, 0, k1);
        Scales<S> sn;
        kmfma<S, 3, MF>(f1, sc, acc, [&](auto q) {
            constexpr int Q = decltype(q)::value;
            if constexpr (MF && Q < NR) {
                kread<S, 0, Q>(f0, ncodes, ro);
                sread<S, Q>(sn, nscales, ro);
            }
            constexpr int L = slot_load<0, G::A + 1, SL>(Q);   // group A, then the scales
            if constexpr (L >= 0 && L < G::A)
                load_op<S, L>(lds, src, src, lo, s2 & 1, ks2, true, 0, 0);
            else if constexpr (L == G::A)
                load_op<S, G::NL>(lds, src, src, lo, 0, 0, scale_w, c, c % 3);
        });
        sc = sn;
    }
}

}  // namespace d8

//
// HALVES: the last round of tiles is at most half full, so the workgroups of
// each XCD are laid out as `halves` top halves of its first tiles, then its
// whole tiles, then the bottom halves of those first tiles.  The CUs that
// start on a half tile run half a tile out of phase with the others, and the
// bottom halves fill the last round; every tile is still summed the same way
// (bit-identical output).  A half tile (128 rows, rows past it outside the
// activation descriptor) is multiplied by the four waves of its rows; the
// other four only load and wait.
template <bool OUT_BF16, bool BIAS, class S = DenseShape, bool HALVES = false>
__global__ __launch_bounds__(512, 1) void gemm_dense_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ xs,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws, int64_t M, int64_t N,
    int64_t K, void* __restrict__ y, int gm, const uint16_t* __restrict__ bias, int halves) {
    static_assert(S::NW == 8, "two wavefronts a SIMD");
    static_assert(!HALVES || S::MB * S::WGM == 8, "half tiles split the 256-row tile");
    __shared__ __attribute__((aligned(16))) uint8_t smem[S::LDS_BYTES];
    const int tiles_m = (int)((M + S::BM - 1) / S::BM);
    const int tiles_n = (int)((N + S::BN - 1) / S::BN);
    int tm, tn, part = 0;                     // part: 0 whole tile, 1 top half, 2 bottom half
    if constexpr (HALVES) {
        const int per_xcd = (int)gridDim.x / 8 - halves;
        const int id = (int)blockIdx.x, j = id / 8;
        part = j < halves ? 1 : (j < per_xcd ? 0 : 2);
        const int t = (id % 8) * per_xcd + (part == 2 ? j - per_xcd : j);
        if (t >= tiles_m * tiles_n) return;
        tile_of(t, tiles_m, tiles_n, gm, tm, tn);
    } else {
        if (!tile_coords(tiles_m, tiles_n, gm, tm, tn)) return;
    }
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % S::WGN, wm = wave / S::WGN;
    const int64_t m0 = (int64_t)tm * S::BM + (part == 2 ? S::BM / 2 : 0);
    const int64_t n0 = (int64_t)tn * S::BN;
    if (m0 >= M) return;                      // a bottom half past the last row
    const int64_t m_end = part != 0 ? min(M, m0 + S::BM / 2) : M;
    const int nkt = (int)(K / 256);           // even: K % 512 == 0
    lds_u8* lds = (lds_u8*)smem;
    const TileSrc<S> src = tile_src<S>(x, xs, w, ws, m0, m_end, n0, N, K);
    const ReadOffsets<S> ro = read_offsets<S>(wn, wm);
    const LoadOffsets<S> lo = load_offsets<S>(K / 2, K / 2, K / 32);
    v16f acc[S::NB][S::MB];
    zero_acc<S>(acc);
    d8::KFrag<S> f0, f1;
    Scales<S> sc;
    if (HALVES && part != 0 && wm == 1) {     // no rows of this half tile
        d8::prologue<S, false>(lds, src, lo, nkt, f0, sc, ro);
        d8::main_loop<S, false>(lds, src, lo, nkt, f0, f1, sc, acc, ro);
    } else {
        d8::prologue<S, true>(lds, src, lo, nkt, f0, sc, ro);
        d8::main_loop<S, true>(lds, src, lo, nkt, f0, f1, sc, acc, ro);
    }
    wait_vm<0>();                             // drain the surplus loads
    // every wave is past its last read of the stage buffers, which now hold
    // the eight waves' epilogue regions
    __syncthreads();
    using T = Stage<S, OUT_BF16>;
    constexpr int ROWS = T::rows_for(S::SCALE_BASE / S::NW);
    store_tile<S, OUT_BF16, ROWS, BIAS>(acc, lds + wave * T::bytes(ROWS), y, m0, m_end, n0, N, wn,
                                        wm, bias);
}

// ---------------------------------------------------------------------------
// Grouped (MoE) GEMM, persistent.  Work items are (expert e, weight tile tn,
// activation tile mt) with mt < ceil(rows_e / BM), ordered by e, then tn, then
// mt, and numbered 0..total-1.  Each workgroup first builds, in LDS, the
// table of the first item of every expert (one wavefront scans the clamped
// offset table), then walks the items
//   t = xcd * ceil(total / 8) + local + k * (grid / 8)   (xcd = id % 8, local = id / 8)
// so each XCD's workgroups run a contiguous range together: the activation
// tiles of one weight tile run side by side on one XCD (the weight rows come
// from HBM once and from its L2 after), and an expert's rows stay in that L2
// across its weight tiles.  While a tile's last stages run, the next tile's
// first two stages are already loading into the freed buffers.
// ---------------------------------------------------------------------------
constexpr int GROUP_MAX_E = 2048;
constexpr int GROUP_TABLE_BYTES = (3 * GROUP_MAX_E + 1) * 4;

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
    int e, tn, m0, m_end, jl;   // jl: 32-row blocks of the tile holding rows (1..4)
};

// first[e] = number of the expert's first item (first[E] = total),
// row0[e], row1[e] = its clamped row range [row0, row1).
struct GroupTable {
    int* first;
    int* row0;
    int* row1;
};

__device__ __forceinline__ int wave_inclusive_max(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d *= 2) {
        const int u = __shfl_up(v, d, 64);
        if (lane >= d) v = max(v, u);
    }
    return v;
}

// The offset table is read as row ends clamped to [0, total_M] and made
// non-decreasing by a running maximum: expert e gets rows [end(e-1), end(e))
// with end(-1) = clamp(offsets[0]).  A well-formed table is unchanged; a
// malformed one still gives disjoint ranges inside [0, total_M), so the item
// count stays below (ceil(total_M / BM) + E) * tiles_n, the bound the host
// checks, and no sum can wrap.
template <int BM>
__device__ void build_table(const int32_t* __restrict__ offsets, int E, int total_M, int tiles_n,
                            GroupTable tb) {
    const int lane = threadIdx.x & 63;
    int base = 0;
    int prev_end = min(max((int)offsets[0], 0), total_M);
    for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        const int v = e < E ? min(max((int)offsets[e + 1], 0), total_M) : 0;
        const int a1 = max(wave_inclusive_max(v), prev_end);
        int a0 = __shfl_up(a1, 1, 64);
        if (lane == 0) a0 = prev_end;
        prev_end = __shfl(a1, 63, 64);
        const int cnt = e < E ? (a1 - a0 + BM - 1) / BM * tiles_n : 0;
        const int incl = wave_inclusive_scan(cnt);
        if (e < E) {
            tb.first[e] = base + incl - cnt;
            tb.row0[e] = a0;
            tb.row1[e] = a1;
        }
        base += __shfl(incl, 63, 64);
    }
    if (lane == 0) tb.first[E] = base;
}

// Item t (< total), searching experts from `from` on (items only grow).
// it.e < 0 if no expert holds item t (the table guarantees one does; the
// caller then ends its walk rather than index the table with it).
template <int BM>
__device__ __forceinline__ GroupItem decode_item(GroupTable tb, int E, int tiles_n, int t,
                                                 int from) {
    const int lane = threadIdx.x & 63;
    int e = -1;
    for (int e0 = from; e0 < E; e0 += 64) {
        const int c = e0 + lane;
        const bool hit = c < E && tb.first[c] <= t && t < tb.first[c + 1];
        const uint64_t m = __ballot(hit);
        if (m) {
            e = e0 + __ffsll((unsigned long long)m) - 1;
            break;
        }
    }
    GroupItem it;
    it.e = __builtin_amdgcn_readfirstlane(e);
    if (it.e < 0) {
        it.tn = it.m0 = it.m_end = 0;
        it.jl = 1;
        return it;
    }
    const int a0 = __builtin_amdgcn_readfirstlane(tb.row0[it.e]);
    const int a1 = __builtin_amdgcn_readfirstlane(tb.row1[it.e]);
    const int r = t - __builtin_amdgcn_readfirstlane(tb.first[it.e]);
    const int mts = (a1 - a0 + BM - 1) / BM;
    it.tn = r / mts;
    it.m0 = a0 + (r - it.tn * mts) * BM;
    it.m_end = a1;
    const int rows = min(a1 - it.m0, BM);
    it.jl = (rows + 31) / 32;
    return it;
}

template <class S>
__device__ __forceinline__ TileSrc<S> item_src(const GroupItem& it, const uint8_t* x,
                                               const uint8_t* xs, const uint8_t* w,
                                               const uint8_t* ws, int64_t N, int64_t K) {
    const int64_t nkb = K / 32;
    return tile_src<S>(x, xs, w + (int64_t)it.e * N * nkb * 16, ws + (int64_t)it.e * N * nkb,
                       it.m0, it.m_end, (int64_t)it.tn * S::BN, N, K);
}

template <class S, bool PREFETCH>
__device__ __forceinline__ void main_loop_jl(int jl, lds_u8* lds, const TileSrc<S>& cur,
                                             const TileSrc<S>& nxt, const LoadOffsets<S>& lo,
                                             int nkt, int cbase,
                                             Pipe<S>& pp, v16f (&acc)[S::NB][S::MB],
                                             const ReadOffsets<S>& ro) {
    static_assert(S::WGM == 1 && S::MB == 4, "one wave row of four 32-row blocks");
    if (jl >= 4)
        main_loop<S, 4, PREFETCH>(lds, cur, nxt, lo, nkt, cbase, pp, acc, ro);
    else if (jl == 3)
        main_loop<S, 3, PREFETCH>(lds, cur, nxt, lo, nkt, cbase, pp, acc, ro);
    else if (jl == 2)
        main_loop<S, 2, PREFETCH>(lds, cur, nxt, lo, nkt, cbase, pp, acc, ro);
    else
        main_loop<S, 1, PREFETCH>(lds, cur, nxt, lo, nkt, cbase, pp, acc, ro);
}

// GLU: y is the MXFP4 codes of h = bf16(silu(gate) * up) and hs its scales
// (store_tile_glu); otherwise hs is unused.
template <bool OUT_BF16, bool GLU = false, bool UOS = false>
__global__ __launch_bounds__(256, 1) void grouped_tiled_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ xs,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws,
    const int32_t* __restrict__ offsets, int E, int total_M, int64_t N, int64_t K,
    void* __restrict__ y, uint8_t* __restrict__ hs) {
    static_assert(!GLU || OUT_BF16, "the GLU epilogue parks bf16");
    using S = GroupShape;
    // pipeline, expert table, then the four waves' epilogue regions (the
    // pipeline buffers already hold the next tile's first stages when a tile
    // is stored)
    using T = Stage<S, OUT_BF16>;
    constexpr int STAGE_BASE = (S::LDS_BYTES + GROUP_TABLE_BYTES + 15) / 16 * 16;
    constexpr int ROWS = T::rows_for((LDS_LIMIT - STAGE_BASE) / 4);
    static_assert(STAGE_BASE + 4 * T::bytes(ROWS) <= LDS_LIMIT, "LDS budget");
    __shared__ __attribute__((aligned(16))) uint8_t smem[STAGE_BASE + 4 * T::bytes(ROWS)];
    lds_u8* lds = (lds_u8*)smem;
    int* table = reinterpret_cast<int*>(smem + S::LDS_BYTES);
    const GroupTable tb{table, table + GROUP_MAX_E + 1, table + 2 * GROUP_MAX_E + 1};
    const int tiles_n = (int)((N + S::BN - 1) / S::BN);
    if (threadIdx.x < 64) build_table<S::BM>(offsets, E, total_M, tiles_n, tb);
    __syncthreads();

    const int total = __builtin_amdgcn_readfirstlane(tb.first[E]);
    const int per_xcd = (total + 7) / 8;
    const int stride = (int)gridDim.x / 8;
    const int t_end = min((int)(blockIdx.x % 8) * per_xcd + per_xcd, total);
    int t = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (t >= t_end) return;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % S::WGN, wm = wave / S::WGN;
    const int nkt = (int)(K / 256);           // even: K % 512 == 0
    const ReadOffsets<S> ro = read_offsets<S>(wn, wm);
    const LoadOffsets<S> lo = load_offsets<S>(K / 2, S::A8 ? K : K / 2, K / 32);

    GroupItem it = decode_item<S::BM>(tb, E, tiles_n, t, 0);
    if (it.e < 0) return;
    TileSrc<S> cur = item_src<S>(it, x, xs, w, ws, N, K);
    v16f acc[S::NB][S::MB];
    zero_acc<S>(acc);
    Pipe<S> pp;
    int cbase = 0;
    prologue<S>(lds, cur, lo, nkt, cbase, pp, ro);
    for (;;) {
        const int tn = t + stride;
        GroupItem nx = it;
        bool have_next = tn < t_end;
        if (have_next) {
            nx = decode_item<S::BM>(tb, E, tiles_n, tn, it.e);
            have_next = nx.e >= 0;
            if (!have_next) nx = it;
        }
        const TileSrc<S> nxt = item_src<S>(nx, x, xs, w, ws, N, K);
        const bool prefetch = have_next && nkt >= 4;
        if (prefetch)
            main_loop_jl<S, true>(it.jl, lds, cur, nxt, lo, nkt, cbase, pp, acc, ro);
        else
            main_loop_jl<S, false>(it.jl, lds, cur, cur, lo, nkt, cbase, pp, acc, ro);
        if (!prefetch) wait_vm<0>();          // drain the surplus loads
        if constexpr (GLU)
            store_tile_glu<S, ROWS, UOS>(acc, lds + STAGE_BASE + wave * T::bytes(ROWS),
                                         static_cast<uint8_t*>(y), hs, it.m0, it.m_end,
                                         (int64_t)it.tn * S::BN, N, wn, wm);
        else
            store_tile<S, OUT_BF16, ROWS>(acc, lds + STAGE_BASE + wave * T::bytes(ROWS), y,
                                          it.m0, it.m_end, (int64_t)it.tn * S::BN, N, wn, wm);
        if (!have_next) break;
        zero_acc<S>(acc);
        if (prefetch) {
            cbase += nkt / 2;
        } else {
            // every wave is past its last LDS read of this tile
            __builtin_amdgcn_s_barrier();
            cbase = 0;
            prologue<S>(lds, nxt, lo, nkt, cbase, pp, ro);
        }
        it = nx;
        cur = nxt;
        t = tn;
    }
    wait_vm<0>();
}

// ---------------------------------------------------------------------------
// Grouped (MoE) GEMM with the weights streamed into registers.  At ~128 rows
// an expert the grouped GEMM is bound by the weight stream, and staging the
// weights through LDS caps it: the LDS holds only two stages, so too few
// bytes are in flight.  In the 128 x 256 grouped tile every weight row is
// used by one wavefront only (waves 1 x 4, each 128 activation rows x 64
// weight rows), so it needs no sharing: here each wave loads its own 64
// weight rows straight into registers in the MFMA's operand layout, four
// stages ahead, and only the activation tile, which all four waves read,
// goes through LDS (LDS-DMA, a ring of four stage buffers).
//
// Stage g of a wave's walk (K stage = 256 elements; stages are numbered
// across the wave's items, and an item has a multiple of 4, so g % 4 is
// static in the unrolled loop and names the stage's weight set and LDS
// buffer).  Entering it, the wave holds K-step 0's activation fragments.
//   K-step 0: read K-step 1's fragments; its MFMAs
//   K-step 1: read K-step 2's; MFMAs
//   wait until stage g+1's activations landed; barrier; DMA stage g+3's
//             activation codes and scales into the buffer of stage g-1
//   K-step 2: read K-step 3's; MFMAs
//   K-step 3: read stage g+1's K-step 0 fragments and scale words; MFMAs
//   load weight set g % 4 with stage g+4 (codes, then scale words)
// Each stage issues 10 weight loads (ordinary buffer loads: the compiler
// places their waits) and 5 activation DMA loads (inline assembly, waited
// for explicitly).  Vector memory loads complete in issue order, so at the
// wait in stage g, "stage g+1's activations (issued in stage g-2) landed" is
// "at most 10 + 15 = 25 loads outstanding": the weight loads that followed
// them in stage g-2 and the 15 loads of stage g-1.
// The next item's first stages are loaded during the current item's last
// ones; the last item loads its own first stages again (surplus, drained at
// the end) so that every stage issues the same loads.
// ---------------------------------------------------------------------------
namespace rs {

// The geometry of an item: MB 32-row activation blocks (BM = 32 MB rows)
// against the 256 weight rows of a tile, and what follows from MB; SHUF: the
// weight codes are pre-shuffled (mxfp4_preshuffle_weights' order).
template <int MB_, bool SHUF_>
struct Geo {
    static constexpr int MB = MB_;
    static constexpr bool SHUF = SHUF_;
    static constexpr int BM = 32 * MB;
    using Shape = tiled::Shape<MB, 2, 1, 4>;      // the accumulator and epilogue layout
    // The activation ring: four stage buffers, each a __shared__ array of its
    // own, always named statically (the stage's position in its group of
    // four), so the compiler can tell which buffer a DMA writes and which one
    // an LDS read reads, and counts the DMA loads in the waits it places for
    // the weight registers instead of draining them before every read.
    static constexpr int XBUF = BM * BKB;         // a stage's activation codes
    static constexpr int XL = MB;                 // their DMA loads a wave (8 rows each)
    // The scale bytes of a group of four stages, 32 a row (8 a stage): the
    // 256 weight rows, then 128 XSL activation rows.  Two groups' buffers, at
    // the start of the kernel's other LDS array.
    static constexpr int XSL = (MB + 3) / 4;      // activation scale DMA loads a wave (32 rows)
    static constexpr int SL = 2 + XSL;            // all scale DMA loads of a wave, a group
    static constexpr int SCW = 256 * 32;
    static constexpr int SC = SCW + 128 * XSL * 32;
    static constexpr int LDS_END = 2 * SC;
    // The wait in stage U of a group for stage g+1's activations (loaded in
    // stage g-2): the 8 weight loads of stage g-2 and the XL + 8 of stage g-1
    // were issued after them, and the SL scale loads of the group's first
    // stage when it is one of those two (they follow its activation loads).
    template <int U>
    static constexpr int wait_x() {
        return 16 + XL + (U == 1 || U == 2 ? SL : 0);
    }
};

struct Ring {
    lds_u8* b[4];
};

// One stage of one wave's weight codes: blocks i (32 rows), K-steps t.
struct WSet {
    v4u c[2][4];
};

// Per-lane offsets, the same for every item and stage.  As in the LDS-staged
// kernels, lane half h takes MX blocks 4h..4h+3 of a stage, one per K-step,
// so its 4 scale bytes of a stage are one 32-bit word.  The weight codes are
// read row-major ([N][K/2]: a load brings 16 bytes from each of 32 rows) or,
// pre-shuffled, in the MFMA's operand order (each load 1 KiB contiguous:
// a quarter of the vector L1's tag lookups); the layout only changes where a
// lane's 16 bytes are, through the two strides.
template <class G>
struct Offs {
    uint32_t w[2];              // weight code loads of blocks i, K-step 0 of stage 0
    uint32_t wt, wk;            // + wt per K-step, + wk per stage
    uint32_t x[G::XL];          // activation code DMA
    uint32_t sw[2], sx[G::XSL]; // scale DMA: the wave's weight rows (two loads), activation rows
    uint32_t rx[4];             // LDS reads: code chunk of K-step t
    uint32_t rsw, rsx;          // LDS reads: scale words of weight / activation block 0
};

template <class G>
__device__ __forceinline__ Offs<G> offsets(int64_t K, int wave) {
    const int lane = threadIdx.x & 63;
    const int r32 = lane & 31, h = lane >> 5;
    const uint32_t ldc = (uint32_t)(K / 2), lds_ = (uint32_t)(K / 32);
    Offs<G> o;
    if constexpr (G::SHUF) {
        // 32-row block b of the tile, stage kt, K-step t: 1 KiB at
        // ((b * K/256 + kt) * 4 + t) * 1024, lane l at 16 l
#pragma unroll
        for (int i = 0; i < 2; ++i)
            o.w[i] = (uint32_t)(2 * wave + i) * (uint32_t)(K / 256) * 4096u + 16u * (uint32_t)lane;
        o.wt = 1024;
        o.wk = 4096;
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) o.w[i] = (uint32_t)(64 * wave + 32 * i + r32) * ldc + 64 * h;
        o.wt = 16;
        o.wk = BKB;
    }
#pragma unroll
    for (int q = 0; q < G::XL; ++q) {
        const int row = (wave * G::XL + q) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        o.x[q] = (uint32_t)row * ldc + 16 * c;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
        o.sw[q] = (uint32_t)(64 * wave + 32 * q + (lane >> 1)) * lds_ + 16 * (lane & 1);
#pragma unroll
    for (int q = 0; q < G::XSL; ++q)
        o.sx[q] = (uint32_t)((wave * G::XSL + q) * 32 + (lane >> 1)) * lds_ + 16 * (lane & 1);
#pragma unroll
    for (int t = 0; t < 4; ++t)
        o.rx[t] = (uint32_t)(r32 * BKB + 16 * ((4 * h + t) ^ ((r32 >> 1) & 7)));
    o.rsw = (uint32_t)((64 * wave + r32) * 32 + 4 * h);
    o.rsx = (uint32_t)(G::SCW + r32 * 32 + 4 * h);
    return o;
}

// Where an item's operands come from, each starting at the item's first row
// (rows past N, or past the expert's last row, read 0): the weight codes as
// a buffer resource for ordinary loads, the rest for the DMA.
struct Src {
    __amdgpu_buffer_rsrc_t w, x;
    v4i ws, xs;
};

__device__ __forceinline__ Src item_src(const GroupItem& it, const uint8_t* x, const uint8_t* xs,
                                        const uint8_t* w, const uint8_t* ws, int64_t N,
                                        int64_t K) {
    const int64_t ldc = K / 2, lds_ = K / 32;
    const int64_t n0 = (int64_t)it.tn * 256;
    const int64_t rows_w = N > n0 ? N - n0 : 0;
    const int64_t rows_x = it.m_end > it.m0 ? it.m_end - it.m0 : 0;
    const int64_t wrow = (int64_t)it.e * N + n0;
    Src s;
    s.w = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w + wrow * ldc), (short)0,
                                            (int)(rows_w * ldc), 0x00020000);
    s.ws = make_rsrc(ws + wrow * lds_, (uint32_t)(rows_w * lds_));
    s.x = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(x + (int64_t)it.m0 * ldc),
                                            (short)0, (int)(rows_x * ldc), 0x00020000);
    s.xs = make_rsrc(xs + (int64_t)it.m0 * lds_, (uint32_t)(rows_x * lds_));
    return s;
}

// Stage kt's activation codes of the item `s` into ring buffer B.
template <class G, int B>
__device__ __forceinline__ void load_x(const Ring& ring, const Src& s, const Offs<G>& o, int wave,
                                       int kt) {
#pragma unroll
    for (int q = 0; q < G::XL; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            s.x, (__attribute__((address_space(3))) void*)(ring.b[B] + (wave * G::XL + q) * 1024),
            16, (int)o.x[q], kt * BKB, 0, 0);
}

// The scales of stages 4 grp .. 4 grp + 3 into scale buffer `par`: each wave
// its own 64 weight rows and 32 XSL of the activation rows, two lanes a row.
template <class G>
__device__ __forceinline__ void load_sc(lds_u8* lds, int par, const Src& s, const Offs<G>& o,
                                        int wave, int grp) {
    lds_u8* b = lds + par * G::SC;
    const uint32_t k = (uint32_t)grp * 32;
    dma16(s.ws, b + (2 * wave) * 1024, o.sw[0], k);
    dma16(s.ws, b + (2 * wave + 1) * 1024, o.sw[1], k);
#pragma unroll
    for (int q = 0; q < G::XSL; ++q)
        dma16(s.xs, b + G::SCW + (wave * G::XSL + q) * 1024, o.sx[q], k);
}

// Stage kt's weight codes into a set: each 32-row block's four K-step
// registers back to back, so each row's 128-byte line is still in L1 for
// the three loads after the first.
template <class G>
__device__ __forceinline__ void load_w(WSet& w, const Src& s, const Offs<G>& o, int kt) {
    // Pre-shuffled, a load fills 8 whole 128-byte lines that nothing reads
    // again: the non-temporal hint keeps them from pushing the activation
    // rows, which the expert's other weight tiles read, out of L2 (measured
    // 5% faster).  Row-major, a load takes 32 bytes of each of 32 lines and
    // the next K-steps take the rest: there the hint made every GEMM ~40%
    // slower, so row-major loads stay plain.
    constexpr int CPOL = G::SHUF ? 2 : 0;   // nt
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t)
            w.c[i][t] = __builtin_bit_cast(
                v4u,
                __builtin_amdgcn_raw_buffer_load_b128(s.w, (int)(o.w[i] + o.wt * t),
                                                      kt * (int)o.wk, CPOL));
}

// K-step T's activation fragments of the stage in ring buffer B (all MB
// 32-row blocks).
template <class G>
struct XFrag {
    v4u x[G::MB];
};
template <class G, int B, int T>
__device__ __forceinline__ void read_x(XFrag<G>& f, const Ring& ring, const Offs<G>& o) {
#pragma unroll
    for (int j = 0; j < G::MB; ++j)
        f.x[j] = *reinterpret_cast<lds_v4u*>(ring.b[B] + o.rx[T] + j * 32 * BKB);
}
// Stage S (of its group, in scale buffer `sb`): the scale words of the
// wave's two weight blocks and of the MB activation blocks.
template <class G, int S>
__device__ __forceinline__ void read_scales(uint32_t (&wsc)[2], uint32_t (&sc)[G::MB],
                                            const lds_u8* sb, const Offs<G>& o) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
        wsc[i] = *reinterpret_cast<lds_u32*>(sb + o.rsw + i * 32 * 32 + 8 * S);
#pragma unroll
    for (int j = 0; j < G::MB; ++j)
        sc[j] = *reinterpret_cast<lds_u32*>(sb + o.rsx + j * 32 * 32 + 8 * S);
}

// The MFMAs of K-step T on the activation blocks that hold rows (j < jl,
// uniform: the blocks past an expert's last row are skipped).
template <class G, int T>
__device__ __forceinline__ void mfma_k(v16f (&acc)[2][G::MB], const WSet& w, const XFrag<G>& f,
                                       const uint32_t (&wsc)[2], const uint32_t (&sc)[G::MB],
                                       int jl) {
#pragma unroll
    for (int j = 0; j < G::MB; ++j) {
        if (j == 0 || jl > j) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                acc[i][j] = mfma<T>(w.c[i][T], f.x[j], acc[i][j], wsc[i], sc[j]);
        }
    }
}

// Pipeline registers of a wave: the four weight sets, two K-steps of
// activation fragments, the scale words of the stage the MFMAs use.
template <class G>
struct Pipe {
    WSet w[4];
    XFrag<G> f[2];
    uint32_t wsc[2], sc[G::MB];
};

// Stage kt = 4q + U of item `cur`, in the group whose scales are in buffer
// `par`.  It loads stage kt+3's activations and stage kt+4's weights (and,
// in a group's first stage, the next group's scales); in an item's last
// four stages (LAST) those belong to the next item.  On entry f[0] holds
// K-step 0's fragments; each K-step reads the next one's into the other
// slot (K-step 3: stage kt+1's K-step 0, and its scale words).
template <class G, int U, bool LAST>
__device__ __forceinline__ void stage(lds_u8* lds, const Ring& ring, const Src& cur, const Src& nxt,
                                      const Offs<G>& o, int wave, int kt, int jl, int par,
                                      Pipe<G>& p, v16f (&acc)[2][G::MB]) {
    constexpr bool X_NEXT = LAST && U >= 1;
    const Src& sw = LAST ? nxt : cur;
    const Src& sx = X_NEXT ? nxt : cur;
    const int kw = LAST ? U : kt + 4;
    const int kx = X_NEXT ? U - 1 : kt + 3;
    WSet& w = p.w[U];
    // jl is the same for the whole item; made opaque here so that the
    // compiler neither versions the loop on it nor moves one block's MFMAs
    // out of their stage (either keeps every weight set alive far longer)
    asm volatile("" : "+s"(jl));
    read_x<G, U, 1>(p.f[1], ring, o);
    __builtin_amdgcn_sched_barrier(0);
    mfma_k<G, 0>(acc, w, p.f[0], p.wsc, p.sc, jl);
    read_x<G, U, 2>(p.f[0], ring, o);
    __builtin_amdgcn_sched_barrier(0);
    mfma_k<G, 1>(acc, w, p.f[1], p.wsc, p.sc, jl);
    // stage kt+1's activations (and, in the group's last stage, the next
    // group's scales) landed in every wave; every wave is done with the
    // buffers about to be reloaded
    wait_vm<G::template wait_x<U>()>();
    __builtin_amdgcn_s_barrier();
    load_x<G, (U + 3) % 4>(ring, sx, o, wave, kx);
    if constexpr (U == 0) load_sc<G>(lds, par ^ 1, sw, o, wave, LAST ? 0 : kt / 4 + 1);
    read_x<G, U, 3>(p.f[1], ring, o);
    __builtin_amdgcn_sched_barrier(0);
    mfma_k<G, 2>(acc, w, p.f[0], p.wsc, p.sc, jl);
    uint32_t wsc_next[2], sc_next[G::MB];
    read_x<G, (U + 1) % 4, 0>(p.f[0], ring, o);
    read_scales<G, (U + 1) % 4>(wsc_next, sc_next, lds + (U == 3 ? par ^ 1 : par) * G::SC, o);
    __builtin_amdgcn_sched_barrier(0);
    mfma_k<G, 3>(acc, w, p.f[1], p.wsc, p.sc, jl);
    __builtin_amdgcn_sched_barrier(0);
    load_w<G>(w, sw, o, kw);                  // the set's registers are free
#pragma unroll
    for (int i = 0; i < 2; ++i) p.wsc[i] = wsc_next[i];
#pragma unroll
    for (int j = 0; j < G::MB; ++j) p.sc[j] = sc_next[j];
    // this stage's MFMAs complete their chains here
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < G::MB; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// All stages of item `cur`; par: the scale buffer of its first group
// (toggled per group).
template <class G>
__device__ __forceinline__ void item_stages(lds_u8* lds, const Ring& ring, const Src& cur,
                                            const Src& nxt, const Offs<G>& o, int wave, int nkt,
                                            int jl, int& par, Pipe<G>& p,
                                            v16f (&acc)[2][G::MB]) {
    int kt = 0;
    for (; kt < nkt - 4; kt += 4) {
        stage<G, 0, false>(lds, ring, cur, nxt, o, wave, kt, jl, par, p, acc);
        stage<G, 1, false>(lds, ring, cur, nxt, o, wave, kt + 1, jl, par, p, acc);
        stage<G, 2, false>(lds, ring, cur, nxt, o, wave, kt + 2, jl, par, p, acc);
        stage<G, 3, false>(lds, ring, cur, nxt, o, wave, kt + 3, jl, par, p, acc);
        par ^= 1;
    }
    stage<G, 0, true>(lds, ring, cur, nxt, o, wave, kt, jl, par, p, acc);
    stage<G, 1, true>(lds, ring, cur, nxt, o, wave, kt + 1, jl, par, p, acc);
    stage<G, 2, true>(lds, ring, cur, nxt, o, wave, kt + 2, jl, par, p, acc);
    stage<G, 3, true>(lds, ring, cur, nxt, o, wave, kt + 3, jl, par, p, acc);
    par ^= 1;
}

// The first item's loads in the order the stages issue them (as if stages
// -4..-1 had run, the first group's scales ahead of them), then its stage
// 0's first fragments and scale words.
template <class G>
__device__ __forceinline__ void prologue(lds_u8* lds, const Ring& ring, const Src& s,
                                         const Offs<G>& o, int wave, Pipe<G>& p) {
    load_sc<G>(lds, 0, s, o, wave, 0);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        if (g == 1) load_x<G, 0>(ring, s, o, wave, 0);
        if (g == 2) load_x<G, 1>(ring, s, o, wave, 1);
        if (g == 3) load_x<G, 2>(ring, s, o, wave, 2);
        load_w<G>(p.w[g], s, o, g);
    }
    // stage 0's activations: 8 + 2 (XL + 8) loads were issued after them
    wait_vm<24 + 2 * G::XL>();
    __builtin_amdgcn_s_barrier();
    read_x<G, 0, 0>(p.f[0], ring, o);
    read_scales<G, 0>(p.wsc, p.sc, lds, o);
}

}  // namespace rs

// K % 1024 == 0 (stages of an item a multiple of 4).  MB 32-row activation
// blocks a tile (4 or 5).  SHUF: the weight codes are in the order
// mxfp4_preshuffle_weights writes (N % 32 == 0).
template <int MB, bool OUT_BF16, bool GLU, bool UOS, bool SHUF>
__global__ __launch_bounds__(256, 1) void grouped_stream_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ xs,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws,
    const int32_t* __restrict__ offsets, int E, int total_M, int64_t N, int64_t K,
    void* __restrict__ y, uint8_t* __restrict__ hs) {
    static_assert(!GLU || OUT_BF16, "the GLU epilogue parks bf16");
    using G = rs::Geo<MB, SHUF>;
    using S = typename G::Shape;
    using T = Stage<S, OUT_BF16>;
    constexpr int TABLE = G::LDS_END;
    constexpr int STAGE_BASE = (TABLE + GROUP_TABLE_BYTES + 15) / 16 * 16;
    constexpr int ROWS = T::rows_for((LDS_LIMIT - 4 * G::XBUF - STAGE_BASE) / 4);
    static_assert(4 * G::XBUF + STAGE_BASE + 4 * T::bytes(ROWS) <= LDS_LIMIT, "LDS budget");
    __shared__ __attribute__((aligned(16))) uint8_t smem[STAGE_BASE + 4 * T::bytes(ROWS)];
    __shared__ __attribute__((aligned(16))) uint8_t xr0[G::XBUF], xr1[G::XBUF], xr2[G::XBUF],
        xr3[G::XBUF];
    lds_u8* lds = (lds_u8*)smem;
    const rs::Ring ring{{(lds_u8*)xr0, (lds_u8*)xr1, (lds_u8*)xr2, (lds_u8*)xr3}};
    int* table = reinterpret_cast<int*>(smem + TABLE);
    const GroupTable tb{table, table + GROUP_MAX_E + 1, table + 2 * GROUP_MAX_E + 1};
    const int tiles_n = (int)((N + S::BN - 1) / S::BN);
    if (threadIdx.x < 64) build_table<S::BM>(offsets, E, total_M, tiles_n, tb);
    __syncthreads();

    const int total = __builtin_amdgcn_readfirstlane(tb.first[E]);
    const int per_xcd = (total + 7) / 8;
    const int stride = (int)gridDim.x / 8;
    const int t_end = min((int)(blockIdx.x % 8) * per_xcd + per_xcd, total);
    int t = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (t >= t_end) return;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nkt = (int)(K / 256);             // a multiple of 4
    const rs::Offs<G> o = rs::offsets<G>(K, wave);
    GroupItem it = decode_item<S::BM>(tb, E, tiles_n, t, 0);
    if (it.e < 0) return;
    rs::Src cur = rs::item_src(it, x, xs, w, ws, N, K);
    v16f acc[2][MB];
    zero_acc<S>(acc);
    rs::Pipe<G> p;
    rs::prologue<G>(lds, ring, cur, o, wave, p);
    int par = 0;
    for (;;) {
        const int tn = t + stride;
        GroupItem nx = it;
        bool have_next = tn < t_end;
        if (have_next) {
            nx = decode_item<S::BM>(tb, E, tiles_n, tn, it.e);
            have_next = nx.e >= 0;
            if (!have_next) nx = it;
        }
        const rs::Src nxt = rs::item_src(nx, x, xs, w, ws, N, K);
        rs::item_stages<G>(lds, ring, cur, nxt, o, wave, nkt, it.jl, par, p, acc);
        // keep the loads in flight plus the epilogue's stores within the
        // 6-bit load counter
        wait_vm<24>();
        if constexpr (GLU)
            store_tile_glu<S, ROWS, UOS>(acc, lds + STAGE_BASE + wave * T::bytes(ROWS),
                                         static_cast<uint8_t*>(y), hs, it.m0, it.m_end,
                                         (int64_t)it.tn * S::BN, N, wave, 0);
        else
            store_tile<S, OUT_BF16, ROWS, false, true>(acc, lds + STAGE_BASE + wave * T::bytes(ROWS),
                                                       y, it.m0, it.m_end, (int64_t)it.tn * S::BN,
                                                       N, wave, 0);
        if (!have_next) break;
        rezero_acc<S>(acc);
        it = nx;
        cur = nxt;
        t = tn;
    }
    wait_vm<0>();                               // the surplus loads, before the LDS is released
}

// The pre-shuffled weight layout: for T tensors [N][K/2] of E2M1 codes, piece
// p (16 bytes) of a tensor is the A operand of lane l = p % 64 in K-step
// t = (p / 64) % 4 of stage s = (p / 256) % (K/256) of 32-row block
// b = p / (64 K): row 32 b + l % 32, bytes 128 s + 16 (4 (l / 32) + t).
// One thread a piece: the writes are coalesced, the reads 32 bytes a row.
__global__ __launch_bounds__(256) void preshuffle_kernel(const uint8_t* __restrict__ in,
                                                         uint8_t* __restrict__ out, int64_t T,
                                                         int64_t N, int64_t K) {
    const int64_t S = K / 256, per = N * (K / 32);
    const int64_t total = T * per;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
         p += (int64_t)gridDim.x * blockDim.x) {
        const int64_t tt = p / per, q = p - tt * per;
        const int l = (int)(q % 64), t = (int)((q / 64) % 4);
        const int64_t st = (q / 256) % S, b = q / (256 * S);
        const int64_t row = tt * N + 32 * b + l % 32;
        const v4u v = *reinterpret_cast<const v4u*>(in + row * (K / 2) + 128 * st +
                                                    16 * (4 * (l / 32) + t));
        *reinterpret_cast<v4u*>(out + 16 * p) = v;
    }
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
    return K % 512 == 0 && E <= tiled::GROUP_MAX_E && fits_buffer(total_M, K) &&
           fits_buffer(N, K) && total_M < ((int64_t)1 << 30) && bound < ((int64_t)1 << 30) &&
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
                             int64_t N, int64_t K, void* y, const uint16_t* bias,
                             bool out_bf16, hipStream_t stream) {
    // one 8-wave workgroup a tile, XCD-aware tile order (tile_coords): the
    // tiles a round of resident workgroups covers on an XCD form a compact
    // block, so its operand rows are read into that XCD's L2 once
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipErrorInvalidDevice;
    const int slots = cus / 8 > 0 ? cus / 8 : 1;   // resident workgroups per XCD
    auto run = [&](auto shape, auto halves_on) {
        using S = decltype(shape);
        constexpr bool H = decltype(halves_on)::value;
        const int tiles_m = (int)((M + S::BM - 1) / S::BM);
        const int tiles_n = (int)((N + S::BN - 1) / S::BN);
        const int per_xcd = (tiles_m * tiles_n + 7) / 8;
        // one round: the squarest block of tiles, rows first (8 x 4 at 32
        // slots); several rounds: half as many rows (4 x 8), measured faster
        // (28672 x 4096: 239 -> 234 us) at about the same L2 miss traffic
        const int gm = per_xcd > slots ? group_rows(tiles_m, slots / 4)
                                       : group_rows(tiles_m, per_xcd < slots ? per_xcd : slots);
        const int halves = H ? slots / 2 : 0;
        const dim3 grid((unsigned)((per_xcd + halves) * 8));
        auto go = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, grid, dim3(512), 0, stream, a_codes, a_scales, b_codes,
                               b_scales, M, N, K, y, gm, bias, halves);
        };
        if (bias)
            out_bf16 ? go(tiled::gemm_dense_kernel<true, true, S, H>)
                     : go(tiled::gemm_dense_kernel<false, true, S, H>);
        else
            out_bf16 ? go(tiled::gemm_dense_kernel<true, false, S, H>)
                     : go(tiled::gemm_dense_kernel<false, false, S, H>);
        return hipGetLastError();
    };
    using Off = std::false_type;
    // at most half the CUs' worth of 256 x 256 tiles: 128-row tiles, twice as
    // many (measured at K = 4096: M = 1024, N = 4096 25.3 -> 18.3 us; M = 2048
    // 28.6 -> 25.9 us; from 192 big tiles on the 256-row tiles are faster)
    const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
    if (2 * big_tiles <= (int64_t)cus) return run(tiled::DenseHalfShape{}, Off{});
    // more than one round with the last one at most half full: half tiles
    // (measured at K = 4096: M = 1536, N = 12288 58.5 -> 50.6 us; M = 5000,
    // N = 4096 59.7 -> 51.7 us; M = 3000, N = 28672 192.0 -> 181.5 us; with
    // the last round more than half full they were slower)
    const int64_t per_xcd = (big_tiles + 7) / 8, tail = per_xcd % slots;
    if (per_xcd > slots && tail != 0 && 2 * tail <= slots)
        return run(tiled::DenseShape{}, std::true_type{});
    return run(tiled::DenseShape{}, Off{});
}

// W4A8: MXFP8 activations [M][K] (one byte per element), MXFP4 weights.
bool tiled_w4a8_supported(int64_t M, int64_t N, int64_t K, const void* a_scales,
                          const void* b_scales) {
    return M >= 128 && K % 512 == 0 && M * K < ((int64_t)1 << 31) && fits_buffer(N, K) &&
           (reinterpret_cast<uintptr_t>(a_scales) % 4) == 0 &&
           (reinterpret_cast<uintptr_t>(b_scales) % 4) == 0;
}

hipError_t launch_gemm_tiled_w4a8(const uint8_t* a_codes, const uint8_t* a_scales,
                                  const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                  int64_t N, int64_t K, void* y, const uint16_t* bias,
                                  bool out_bf16, hipStream_t stream) {
    using S = tiled::W4A8Shape;
    const int tiles_m = (int)((M + S::BM - 1) / S::BM);
    const int tiles_n = (int)((N + S::BN - 1) / S::BN);
    const int per_xcd = (tiles_m * tiles_n + 7) / 8;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipErrorInvalidDevice;
    const int slots = cus / 8 > 0 ? cus / 8 : 1;   // resident workgroups per XCD
    if (per_xcd > slots && K >= 1024) {
        // more than one round: the persistent walk
        const int gm = group_rows(tiles_m, slots);
        const dim3 grid((unsigned)(slots * 8));
        auto go = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, a_codes, a_scales, b_codes,
                               b_scales, M, N, K, y, gm, bias);
        };
        if (bias)
            out_bf16 ? go(tiled::gemm_persistent_kernel<true, true, S>)
                     : go(tiled::gemm_persistent_kernel<false, true, S>);
        else
            out_bf16 ? go(tiled::gemm_persistent_kernel<true, false, S>)
                     : go(tiled::gemm_persistent_kernel<false, false, S>);
        return hipGetLastError();
    }
    const int gm = group_rows(tiles_m, per_xcd);
    const dim3 grid((unsigned)(per_xcd * 8));
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, a_codes, a_scales, b_codes,
                           b_scales, M, N, K, y, gm, bias);
    };
    if (bias)
        out_bf16 ? go(tiled::gemm_tiled_kernel<true, true, S>)
                 : go(tiled::gemm_tiled_kernel<false, true, S>);
    else
        out_bf16 ? go(tiled::gemm_tiled_kernel<true, false, S>)
                 : go(tiled::gemm_tiled_kernel<false, false, S>);
    return hipGetLastError();
}

// The register-streamed grouped kernel walks an item's stages four at a time.
static bool grouped_stream_ok(int64_t K) { return K % 1024 == 0; }

// Its activation tile: 160 rows when the experts average more than 96 rows
// (as MoE routing gives them: a spread around the mean that 128-row tiles
// would split, each part then reading the expert's weight tiles again),
// else 128.  ceil(r / 160) <= ceil(r / 128), so the wider tile never makes
// more items; the blocks past an expert's rows skip their MFMAs.
static bool grouped_wide_tile(int64_t E, int64_t total_M) { return total_M > 96 * E; }

bool grouped_stream_supported(int64_t E, int64_t total_M, int64_t N, int64_t K,
                              const void* a_scales, const void* b_scales) {
    return grouped_stream_ok(K) && N % 32 == 0 &&
           grouped_tiled_supported(E, total_M, N, K, a_scales, b_scales);
}

hipError_t launch_preshuffle(const uint8_t* in, uint8_t* out, int64_t T, int64_t N, int64_t K,
                             hipStream_t stream) {
    const int64_t pieces = T * N * (K / 32);
    const int64_t blocks = std::min<int64_t>((pieces + 255) / 256, 256 * 32);
    hipLaunchKernelGGL(tiled::preshuffle_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in,
                       out, T, N, K);
    return hipGetLastError();
}

// One persistent workgroup per CU (the tile's LDS allows no more), never
// more workgroups than the largest possible number of work items.
static hipError_t grouped_grid(int64_t E, int64_t total_M, int64_t N, dim3& grid) {
    using S = tiled::GroupShape;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipErrorInvalidDevice;
    const int64_t bound = ((total_M + S::BM - 1) / S::BM + E) * ((N + S::BN - 1) / S::BN);
    int64_t g = (int64_t)cus / 8 * 8;
    if (g < 8) g = 8;
    if (g > (bound + 7) / 8 * 8) g = (bound + 7) / 8 * 8;
    grid = dim3((unsigned)g);
    return hipSuccess;
}

hipError_t launch_grouped_gemm_tiled(const uint8_t* a_codes, const uint8_t* a_scales,
                                     const uint8_t* b_codes, const uint8_t* b_scales,
                                     const int32_t* offsets, int64_t E, int64_t total_M,
                                     int64_t N, int64_t K, void* y, bool out_bf16,
                                     bool b_shuffled, hipStream_t stream) {
    dim3 grid;
    const hipError_t e = grouped_grid(E, total_M, N, grid);
    if (e != hipSuccess) return e;
    uint8_t* const none = nullptr;
    if (grouped_stream_ok(K)) {
        auto go = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, a_codes, a_scales, b_codes,
                               b_scales, offsets, (int)E, (int)total_M, N, K, y, none);
        };
        using tiled::grouped_stream_kernel;
        const bool wide = grouped_wide_tile(E, total_M);
        if (b_shuffled) {
            if (wide)
                out_bf16 ? go(grouped_stream_kernel<5, true, false, false, true>)
                         : go(grouped_stream_kernel<5, false, false, false, true>);
            else
                out_bf16 ? go(grouped_stream_kernel<4, true, false, false, true>)
                         : go(grouped_stream_kernel<4, false, false, false, true>);
        } else {
            if (wide)
                out_bf16 ? go(grouped_stream_kernel<5, true, false, false, false>)
                         : go(grouped_stream_kernel<5, false, false, false, false>);
            else
                out_bf16 ? go(grouped_stream_kernel<4, true, false, false, false>)
                         : go(grouped_stream_kernel<4, false, false, false, false>);
        }
    } else {
        if (b_shuffled) return hipErrorInvalidValue;   // the caller checks this first
        auto go = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, a_codes, a_scales, b_codes,
                               b_scales, offsets, (int)E, (int)total_M, N, K, y, none);
        };
        out_bf16 ? go(tiled::grouped_tiled_kernel<true>) : go(tiled::grouped_tiled_kernel<false>);
    }
    return hipGetLastError();
}

bool grouped_glu_supported(int64_t E, int64_t total_M, int64_t N, int64_t K,
                           const void* a_scales, const void* b_scales) {
    return N % 64 == 0 && grouped_tiled_supported(E, total_M, N, K, a_scales, b_scales);
}

hipError_t launch_grouped_glu_quant(const uint8_t* a_codes, const uint8_t* a_scales,
                                    const uint8_t* b_codes, const uint8_t* b_scales,
                                    const int32_t* offsets, int64_t E, int64_t total_M,
                                    int64_t N, int64_t K, uint8_t* h_codes, uint8_t* h_scales,
                                    bool uos, bool b_shuffled, hipStream_t stream) {
    dim3 grid;
    const hipError_t e = grouped_grid(E, total_M, N, grid);
    if (e != hipSuccess) return e;
    if (grouped_stream_ok(K)) {
        auto go = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, a_codes, a_scales, b_codes,
                               b_scales, offsets, (int)E, (int)total_M, N, K,
                               static_cast<void*>(h_codes), h_scales);
        };
        using tiled::grouped_stream_kernel;
        const bool wide = grouped_wide_tile(E, total_M);
        if (b_shuffled) {
            if (wide)
                uos ? go(grouped_stream_kernel<5, true, true, true, true>)
                    : go(grouped_stream_kernel<5, true, true, false, true>);
            else
                uos ? go(grouped_stream_kernel<4, true, true, true, true>)
                    : go(grouped_stream_kernel<4, true, true, false, true>);
        } else {
            if (wide)
                uos ? go(grouped_stream_kernel<5, true, true, true, false>)
                    : go(grouped_stream_kernel<5, true, true, false, false>);
            else
                uos ? go(grouped_stream_kernel<4, true, true, true, false>)
                    : go(grouped_stream_kernel<4, true, true, false, false>);
        }
    } else {
        if (b_shuffled) return hipErrorInvalidValue;   // the caller checks this first
        auto go = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, a_codes, a_scales, b_codes,
                               b_scales, offsets, (int)E, (int)total_M, N, K,
                               static_cast<void*>(h_codes), h_scales);
        };
        uos ? go(tiled::grouped_tiled_kernel<true, true, true>)
            : go(tiled::grouped_tiled_kernel<true, true, false>);
    }
    return hipGetLastError();
}

}  // namespace mx
