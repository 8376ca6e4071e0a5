/*
 * mxfp4.h -- C ABI of the MI355X (gfx950) block-scaled 4-bit linear-layer
 * library: NVFP4 -> MXFP4 weight requant, dynamic MXFP4 activation
 * quantization, and the MXFP4 x MXFP4 GEMM (dense and grouped by expert).
 *
 * Formats (shared by every call):
 *   E2M1 code   4 bits: sign | 2-bit exponent (bias 1) | 1-bit mantissa;
 *               magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.  Two codes per
 *               byte, the even K-index in bits 3:0, the odd one in bits 7:4.
 *   MXFP4       codes [rows][K/2] u8 plus one E8M0 scale byte per 32
 *               consecutive K-elements, [rows][K/32] u8, value 2^(b-127),
 *               0xFF = NaN (vLLM-Omni "W4A4 MXFP4 Quantization", Overview;
 *               "Validation and Notes": raw uint8 scale bytes).
 *   NVFP4       codes [rows][K/2] u8 plus one float8_e4m3fn scale per 16
 *               K-elements, [rows][K/16] u8, plus one fp32 per-tensor scale
 *               (AMD blog "Efficiently Serving NVFP4 Models on AMD Instinct
 *               MI350X/MI355X ...", introduction; SGLang FP4 post, sections
 *               3-4: weight_packed / weight_scale / weight_global_scale).
 *
 * Conventions:
 *   - Every tensor pointer is a DEVICE pointer to row-major memory owned by
 *     the caller, except the host buffers of the layerwise load and the
 *     subset requant's tensor list (marked HOST).  No call allocates or frees
 *     device memory or synchronises the host; all work is enqueued on
 *     `stream`.  The only device memory the library holds is the static
 *     scratch of mxfp4_linear_bf16_noalloc.
 *   - Every call returns MXFP4_OK or a negative mxfp4_status.  Arguments are
 *     checked before anything is enqueued; on an error nothing is launched.
 *   - K must be a positive multiple of 32 (whole MX blocks).  A zero row
 *     count (M == 0, total_M == 0, T == 0) is a no-op returning MXFP4_OK.
 *   - Alignment, enforced with MXFP4_EALIGN: code pointers (u8 [rows][K/2])
 *     and bf16 activation pointers 16 bytes; fp32 outputs 4 bytes, bf16
 *     outputs 2 bytes; the requant's E4M3 scales (nv_scales) 2 bytes; the
 *     linear calls' weight scales (b_scales) 16 bytes; bias and Smooth
 *     vectors 16 bytes.  Other scale pointers may have any alignment, but
 *     the fast GEMM kernels need them aligned (16 bytes for the decode
 *     kernel, 4 for the tiled ones) and a call whose scale pointers are not
 *     falls back to the generic kernel: results within the same tolerance
 *     (the fp32 sums may round differently), slower.  Each GEMM call lists
 *     its kernel choice.
 *   - Results are bitwise reproducible from run to run (no atomics, fixed
 *     reduction order).
 */
#ifndef MXFP4_H
#define MXFP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MXFP4_OK = 0,
    MXFP4_EINVAL = -1,       /* bad size, null pointer, unknown flag/dtype    */
    MXFP4_EALIGN = -2,       /* a pointer or leading dimension misaligned     */
    MXFP4_EUNSUPPORTED = -3, /* valid request the library does not implement  */
    MXFP4_EHIP = -4,         /* the HIP runtime refused a launch              */
    MXFP4_ESCRATCH = -5      /* needs more than mxfp4_linear_bf16_noalloc's
                                static scratch (MXFP4_NOALLOC_SCRATCH_BYTES)  */
} mxfp4_status;

enum { MXFP4_OUT_BF16 = 0, MXFP4_OUT_FP32 = 1 };        /* out_dtype            */
enum { MXFP4_REQ_INTERMEDIATE_BF16 = 1u << 0 };         /* requant flags        */

/*
 * Scale-rule flag of every quantizing call (requant, act-quant, linear): the
 * UOS shared exponent of the vLLM-Omni guide, "Single-Scale Block Scaling",
 * setting 2 (Qmax = 7.25) in place of the OCP rule: the scale byte is
 * e + 127 for the smallest e with amax <= 7.25 * 2^e, clamped to [0, 254]
 * (the OCP byte, plus one when amax's binary fraction exceeds 1.8125).  The
 * largest scaled magnitude of a block is then at most 7.25 (below 8 under
 * OCP), so less of it saturates at 6; the codes' rounding and the NaN/Inf
 * rule are unchanged.  Both rules give ordinary MXFP4 data: the GEMMs take
 * no flag.
 */
enum { MXFP4_SCALE_UOS = 1u << 1 };
/* Grouped GEMM flag: b_codes are in the layout mxfp4_preshuffle_weights
   writes (see there). */
enum { MXFP4_B_PRESHUFFLED = 1u << 2 };

/*
 * NVFP4 -> MXFP4 requant of T same-shape weight tensors, the load-time step
 * of the AMD blog's pipeline section (Figure 1): dequantize, quantize to
 * MXFP4, write into a preallocated destination.  Per element the NVFP4 value
 * is v = fl32(fl32(e2m1(code) * e4m3(scale16)) * nv_global[t]) (one fp32
 * rounding; the product code*scale is exact), rounded once more to bf16 (RNE)
 * when MXFP4_REQ_INTERMEDIATE_BF16 is set.  Each 32-element block along K
 * (NVFP4 blocks 2j and 2j+1) is then quantized by the OCP MX rule (vLLM-Omni
 * guide, "Single-Scale Block Scaling", setting 0): scale byte =
 * floor(log2 amax) - 2 + 127 clamped to [0, 254]; codes = round-half-to-even
 * of v / 2^(byte-127) onto E2M1, saturating at +-6, sign kept.  A block
 * holding a NaN or Inf gets scale 0xFF and all-zero codes.
 *
 *   nv_codes   [T][N][K/2]  u8, device, read        (16-byte aligned)
 *   nv_scales  [T][N][K/16] u8 (float8_e4m3fn bits), device, read (2-byte
 *              aligned: the two E4M3 scales of an MX block are one load)
 *   nv_global  [T] fp32, device, read: the multiplier applied on dequant
 *              (a checkpoint that stores a divisor passes its reciprocal)
 *   mx_codes   [T][N][K/2]  u8, device, written     (16-byte aligned)
 *   mx_scales  [T][N][K/32] u8 (E8M0 bits), device, written
 *   flags      0, or MXFP4_REQ_INTERMEDIATE_BF16 and/or MXFP4_SCALE_UOS
 * Tensors a loader keeps in high precision are simply not passed (the blog's
 * note on producer excludes).  Source and destination must not overlap.
 */
int mxfp4_requant_from_nvfp4(const uint8_t* nv_codes, const uint8_t* nv_scales,
                             const float* nv_global, int64_t T, int64_t N, int64_t K,
                             uint8_t* mx_codes, uint8_t* mx_scales,
                             uint32_t flags, hipStream_t stream);

/*
 * The same requant of a chosen subset of the T tensors, in one launch: a
 * loader converting a layer whose excluded tensors (the blog's note on
 * producer excludes) break it into runs.  Arguments as above, plus
 *   tensors    [n_tensors] int32, HOST memory, read during the call: the
 *              tensor indices to convert, strictly increasing, each in
 *              [0, T); tensor t is read from slot t of the source and
 *              written to slot t of the destination, other slots untouched
 * Errors: MXFP4_EINVAL for a list out of range or not strictly increasing
 * (checked before anything is launched).  n_tensors == 0 is a no-op.
 */
int mxfp4_requant_from_nvfp4_subset(const uint8_t* nv_codes, const uint8_t* nv_scales,
                                    const float* nv_global, int64_t T, int64_t N, int64_t K,
                                    const int32_t* tensors, int64_t n_tensors,
                                    uint8_t* mx_codes, uint8_t* mx_scales,
                                    uint32_t flags, hipStream_t stream);

/*
 * The layerwise load (AMD blog, pipeline section under Figure 1: the NVFP4
 * checkpoint is requantized one layer at a time into a destination allocated
 * beforehand, so the load needs one layer's worth of extra memory; tensors
 * the producer excluded are skipped, per the blog's note on producer
 * excludes).  A part is one tensor kind of one layer: T same-shape NVFP4
 * tensors in HOST memory and their MXFP4 destination in DEVICE memory.
 *
 *   nv_codes   [T][N][K/2]  u8, host, read   (pinned, e.g. hipHostMalloc, for
 *   nv_scales  [T][N][K/16] u8, host, read    the copies to overlap the
 *   nv_global  [T] fp32, host, read           requant; pageable memory works
 *                                             but serialises them)
 *   excluded   [T] u8, host, read, or NULL: a non-zero entry leaves that
 *              tensor's destination slot untouched and its source unread
 *   mx_codes   [T][N][K/2]  u8, device, written (16-byte aligned)
 *   mx_scales  [T][N][K/32] u8, device, written
 *   T, N, K    T >= 0, N > 0, K a positive multiple of 32
 */
typedef struct {
    const uint8_t* nv_codes;
    const uint8_t* nv_scales;
    const float* nv_global;
    const uint8_t* excluded;
    uint8_t* mx_codes;
    uint8_t* mx_scales;
    int64_t T, N, K;
} mxfp4_load_part;

/*
 * One step of the load plan: tensors [t0, t1) of parts[part], staged in
 * scratch slot `slot` (0 or 1) at the given byte offsets from the scratch
 * base (codes of tensor t0 + i at codes_offset + i*N*K/2, its E4M3 scales at
 * scales_offset + i*N*K/16, its global at global_offset + 4i).  t0 and t1-1
 * are never excluded; excluded tensors between them are neither copied nor
 * converted.  Slot s spans [s * slot_bytes, (s+1) * slot_bytes).
 */
typedef struct {
    int64_t part;
    int64_t t0, t1;
    int64_t slot;
    uint64_t codes_offset, scales_offset, global_offset;
} mxfp4_load_chunk;

/*
 * The plan mxfp4_requant_layers_from_host follows, computed on the host
 * alone (no HIP call, no device pointer read; only the parts' sizes and
 * excluded lists matter).  The scratch is split into two slots of
 * slot_bytes = scratch_bytes / 2 rounded down to 256; each chunk is the
 * largest run of one part's tensors that fits a slot, parts in order, slots
 * alternating.  With chunks == NULL only *n_chunks (and *slot_bytes if not
 * NULL) is written.  Errors: MXFP4_EINVAL for a bad part, a slot too small
 * for one tensor of some part (N*K/2 and N*K/16 bytes each rounded up to
 * 256, plus 4), or max_chunks below the chunk count.
 */
int mxfp4_layerwise_plan(const mxfp4_load_part* parts, int64_t n_parts, size_t scratch_bytes,
                         mxfp4_load_chunk* chunks, int64_t max_chunks, int64_t* n_chunks,
                         uint64_t* slot_bytes);

/*
 * Runs the plan: for each chunk, the kept tensors' NVFP4 bytes are copied
 * host -> device into their slot on copy_stream, then converted on `stream`
 * by the requant of mxfp4_requant_from_nvfp4 into the destination; a slot is
 * refilled only after the requant that read it.  Every kept tensor of every
 * part is written exactly as mxfp4_requant_from_nvfp4 would write it; every
 * excluded slot is left alone.  The call only enqueues work: the host
 * buffers must stay valid, and the scratch unused by others, until `stream`
 * has finished it (which implies copy_stream has).  copy_stream may equal
 * stream (no overlap).  Besides the scratch it uses no device memory; it
 * creates and destroys four HIP events.
 *
 *   parts, n_parts   as for mxfp4_layerwise_plan, with every pointer set for
 *                    parts with T > 0
 *   scratch          device memory of scratch_bytes, 256-byte aligned; one
 *                    layer's NVFP4 bytes is enough for any layer
 *   flags            0, or MXFP4_REQ_INTERMEDIATE_BF16 and/or MXFP4_SCALE_UOS
 */
int mxfp4_requant_layers_from_host(const mxfp4_load_part* parts, int64_t n_parts,
                                   void* scratch, size_t scratch_bytes, uint32_t flags,
                                   hipStream_t copy_stream, hipStream_t stream);

/*
 * Dynamic per-call MXFP4 quantization of bf16 activations (AMD blog, closing
 * list: activations are quantized for each batch, no stored scales).  Row i
 * of the output is the OCP MX quantization (rule as above, amax over the 32
 * bf16 values of each block) of input row row_index[i], or of row i when
 * row_index is NULL (the gather serves expert-sorted MoE inputs).
 *
 *   x_bf16     [*][ldx] bf16, device, read; ldx >= K, ldx % 8 == 0,
 *              16-byte aligned.  Only the first K columns are read.
 *   row_index  [M] int32, device, read, or NULL.  Every entry must index an
 *              existing row of x (not checked: reading it would need a sync).
 *   codes      [M][K/2] u8, device, written   (16-byte aligned)
 *   scales     [M][K/32] u8, device, written
 *   flags      0 or MXFP4_SCALE_UOS
 */
int mxfp4_quantize_act(const void* x_bf16, int64_t ldx, const int32_t* row_index,
                       int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                       uint32_t flags, hipStream_t stream);

/*
 * MoE dispatch of the activations: each of the T token rows of x is quantized
 * once, exactly as mxfp4_quantize_act would quantize it (AMD blog, pipeline:
 * each batch quantized on the fly), and its codes and scale bytes are written
 * to output rows dest_rows[t*fan + j], j < fan: the expert-sorted rows the
 * grouped GEMM reads.  With dest_rows the inverse of a gather index (the
 * routing's token -> sorted-row table), the output equals mxfp4_quantize_act
 * with that gather index, bit for bit, and each token row is read once
 * instead of fan times.  Output rows no entry names are left as they are.
 *
 *   x_bf16      [T][ldx] bf16, device, read; ldx >= K, ldx % 8 == 0, 16-byte
 *               aligned
 *   dest_rows   [T][fan] int32, device, read; each entry is clamped to
 *               [0, R) in the kernel, so a bad table gives wrong rows but
 *               never a write outside the outputs
 *   fan         destinations per row, 1 .. 65536 (the MoE top-k)
 *   R           rows of the outputs
 *   codes       [R][K/2] u8, device, written (16-byte aligned)
 *   scales      [R][K/32] u8, device, written
 *   flags       0 or MXFP4_SCALE_UOS
 */
int mxfp4_quantize_act_scatter(const void* x_bf16, int64_t ldx, int64_t T, int64_t K,
                               const int32_t* dest_rows, int64_t fan, int64_t R, uint8_t* codes,
                               uint8_t* scales, uint32_t flags, hipStream_t stream);

/*
 * mxfp4_quantize_act with the Smooth pre-scale (vLLM-Omni guide, pre-quantized
 * single-scale weights: W4A4 and W4A8 quantize x * mul_scale, the Smooth
 * tensor held in the activation dtype): the values quantized are
 * h[k] = bf16_RNE(x[k] * smooth[k]), the product of the two bf16 values
 * formed in fp32.  Arguments as for mxfp4_quantize_act, plus
 *   smooth_bf16  [K] bf16, device, read, 16-byte aligned: the per-input-channel
 *                factor (a checkpoint's fp32 mul_scale rounded to bf16)
 *   flags        0 or MXFP4_SCALE_UOS
 */
int mxfp4_quantize_act_smooth(const void* x_bf16, int64_t ldx, const int32_t* row_index,
                              const void* smooth_bf16, int64_t M, int64_t K, uint8_t* codes,
                              uint8_t* scales, uint32_t flags, hipStream_t stream);

/*
 * Y = A * B^T over MXFP4 operands with fp32 accumulation on gfx950's
 * block-scaled MFMA (AMD blog, closing list: both operands MXFP4, no
 * separate dequantize step).  y[m][n] = sum_k A[m,k] * B[n,k] where
 * A[m,k] = e2m1 * 2^(a_scale - 127), likewise B.  Both operands are K-major.
 *
 *   a_codes, a_scales   [M][K/2], [M][K/32] u8, device, read
 *   b_codes, b_scales   [N][K/2], [N][K/32] u8, device, read
 *   y                   [M][N] bf16 (MXFP4_OUT_BF16, RNE of the fp32
 *                       accumulator) or fp32 (MXFP4_OUT_FP32), device, written
 *   workspace           reserved: the current kernels need none; pass NULL
 *                       and 0 (mxfp4_gemm_workspace_size returns 0)
 *   flags               must be 0
 * Kernel choice (every kernel meets the same tolerance; each is deterministic):
 *   M <= 64, K = 2048 or 4096, N >= 16, a_codes/a_scales/b_scales 16-byte
 *     aligned: the weight-streaming decode kernel;
 *   else K % 512 == 0 with K <= 16384, the same alignment, N >= 16 and
 *     M <= 64 (K <= 8192), 32 (K <= 12288) or 16 (K <= 16384): the
 *     weight-streaming kernel with ceil(K / 4096) super-steps a wave;
 *   64 < M <= 128 (M = 128 only under 64 tiles of 256 columns) at the K the
 *     two rules above take with 64 rows: those kernels once per 64-row slice;
 *   else M >= 128, K % 512 == 0, each operand's codes under 2 GiB, both scale
 *     pointers 4-byte aligned: the LDS-tiled MFMA kernel (8 wavefronts, one
 *     256 x 256 tile each; 128 x 256 tiles when the 256 x 256 ones would
 *     number at most half the CUs; when the tiles take more than one round
 *     of the CUs and the last round is at most half full, some tiles run
 *     as two 128-row halves, which changes no output bit);
 *   else the generic 16x16x128 MFMA kernel.
 */
int mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
               const uint8_t* b_codes, const uint8_t* b_scales,
               int64_t M, int64_t N, int64_t K, void* y, int out_dtype,
               void* workspace, size_t workspace_bytes,
               uint32_t flags, hipStream_t stream);

/*
 * Grouped GEMM for MoE experts (AMD blog, closing list: MoE experts run on
 * MXFP4 kernels).  For each expert e and each row r in [offsets[e],
 * offsets[e+1]): y[r][:] = A[r] * B_e^T.  A is expert-sorted.
 *
 *   a_codes, a_scales   [total_M][K/2], [total_M][K/32] u8, device, read
 *   b_codes, b_scales   [E][N][K/2], [E][N][K/32] u8, device, read
 *   offsets             [E+1] int32, device, read: non-decreasing,
 *                       offsets[0] = 0, offsets[E] = total_M.  Empty experts
 *                       are allowed.  The table is not checked on the host;
 *                       the kernel clamps every row range to [0, total_M), so
 *                       a bad table can give wrong rows but never a write
 *                       outside y.
 *   y                   [total_M][N] bf16 or fp32, device, written
 *   workspace           as for mxfp4_gemm
 *   flags               0 or MXFP4_B_PRESHUFFLED (b_codes pre-shuffled;
 *                       MXFP4_EUNSUPPORTED unless the register-streamed
 *                       kernel below applies and N % 32 == 0)
 * Kernel choice (same results): K % 512 == 0, E <= 2048, each operand's
 * codes under 2 GiB and both scale pointers 4-byte aligned: a persistent
 * kernel that walks the offset table, with the weights streamed straight
 * into registers when K % 1024 == 0 and staged in LDS otherwise; else the
 * generic kernel.
 */
int mxfp4_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                       const uint8_t* b_codes, const uint8_t* b_scales,
                       const int32_t* offsets, int64_t E, int64_t total_M,
                       int64_t N, int64_t K, void* y, int out_dtype,
                       void* workspace, size_t workspace_bytes,
                       uint32_t flags, hipStream_t stream);

/*
 * Rewrites T MXFP4 weight tensors [T][N][K/2] of E2M1 codes into the order
 * the grouped GEMMs' matrix-core operands are loaded in, for
 * MXFP4_B_PRESHUFFLED (a load-time step, like the requant; the scales are
 * unchanged).  Within each tensor, 16-byte piece p of the output is the
 * operand of lane l = p % 64 in K-step t = (p / 64) % 4 of K-stage
 * s = (p / 256) % (K/256) of the 32-row block b = p / (64 K): bytes
 * 128 s + 16 (4 (l / 32) + t) .. +15 of row 32 b + l % 32.
 *
 *   codes   [T][N][K/2] u8, device, read; 16-byte aligned
 *   out     [T][N][K/2] u8, device, written; 16-byte aligned, not
 *           overlapping codes
 *   N       a positive multiple of 32;  K  a positive multiple of 256
 */
int mxfp4_preshuffle_weights(const uint8_t* codes, uint8_t* out, int64_t T, int64_t N,
                             int64_t K, hipStream_t stream);

/* Workspace bytes mxfp4_gemm / mxfp4_grouped_gemm need (currently 0). */
size_t mxfp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * One linear layer on bf16 activations: the MXFP4 quantization of
 * mxfp4_quantize_act (row i of x, no gather) followed by mxfp4_gemm with B,
 * giving the same y bit for bit, plus an optional row bias (the SGLang FP4
 * post's apply_weights: quantize, GEMM, add bias; the vLLM-Omni guide's
 * W4A4/W4A8 notes: bf16 output with a bf16 row bias).  The bias joins each
 * fp32 sum before its one rounding: y[m][n] = round(sum_k A B + bias[n]).
 * For decode shapes (M <= 16, K = 2048 or 4096, N >= 16) it is one launch
 * whose workgroups quantize their own activation blocks while their weight
 * loads stream; for every other shape the two launches run through the
 * caller's workspace.  The choice depends on the shape alone, so
 * mxfp4_linear_workspace_size is exact.
 *
 *   x_bf16      [M][ldx] bf16, device, read (16-byte aligned, ldx % 8 == 0,
 *               ldx >= K)
 *   b_codes, b_scales, y, out_dtype   as for mxfp4_gemm, with b_scales
 *               16-byte aligned
 *   bias_bf16   [N] bf16, device, read, 16-byte aligned; or NULL for none
 *   workspace   device memory of at least mxfp4_linear_workspace_size(M, N,
 *               K) bytes (16-byte aligned; may be NULL when that is 0):
 *               the quantized activations of the two-launch form
 *   flags       0 or MXFP4_SCALE_UOS (the activations' scale rule)
 * Errors as for mxfp4_gemm; MXFP4_EINVAL also for a workspace smaller than
 * the two-launch form needs when that form is taken.
 */
int mxfp4_linear_bf16(const void* x_bf16, int64_t ldx, int64_t M, int64_t N, int64_t K,
                      const uint8_t* b_codes, const uint8_t* b_scales, const void* bias_bf16,
                      void* y, int out_dtype, void* workspace, size_t workspace_bytes,
                      uint32_t flags, hipStream_t stream);

/* Workspace bytes mxfp4_linear_bf16 needs: 0 for the one-launch shapes. */
size_t mxfp4_linear_workspace_size(int64_t M, int64_t N, int64_t K);

/* Bytes of the device scratch mxfp4_linear_bf16_noalloc holds on each GPU. */
#define MXFP4_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * mxfp4_linear_bf16 for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace: where mxfp4_linear_bf16 would quantize
 * the activations into the caller's workspace (shapes with
 * mxfp4_linear_workspace_size(M, N, K) > 0), it uses a device array of
 * MXFP4_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held from the
 * library's load until the process ends.  The call itself allocates and
 * frees nothing; the array's address on a device is looked up on the first
 * call made with that device current.
 *
 * Arguments, results and errors as for mxfp4_linear_bf16, plus
 * MXFP4_ESCRATCH when mxfp4_linear_workspace_size(M, N, K) exceeds
 * MXFP4_NOALLOC_SCRATCH_BYTES (M * K * 17/32 bytes, rounded up; 32 MiB holds
 * e.g. M = 4096 rows at K = 14336).  The device current at the call must be
 * the one that owns `stream` and the buffers.  Every call on one GPU shares
 * that GPU's array, so calls that may overlap on one GPU (other streams,
 * other threads) race on it: the caller orders them.  The array keeps the
 * last call's quantized activations; nothing in it needs clearing.
 */
int mxfp4_linear_bf16_noalloc(const void* x_bf16, int64_t ldx, int64_t M, int64_t N, int64_t K,
                              const uint8_t* b_codes, const uint8_t* b_scales,
                              const void* bias_bf16, void* y, int out_dtype, uint32_t flags,
                              hipStream_t stream);

/*
 * W4A8: MXFP8 activations with the same MXFP4 weights (vLLM-Omni guide,
 * "W4A8 fallback": activations quantized to float8_e4m3fn with the OCP MX
 * scale (scale_alg=0), block 32 along K, round to nearest even, never UOS;
 * the prepared MXFP4 weight and scale are shared with W4A4).  Per 32-element
 * block: scale byte = floor(log2 amax) - 8 + 127 clamped to [0, 254] (8 is
 * the exponent of E4M3's top binade, 448 = 1.75 * 2^8); each element is the
 * E4M3 value nearest to v / 2^(byte-127), ties to the even code, saturating
 * at +-448 (the NaN code 0x7F is never produced), sign kept.  A block holding
 * NaN or Inf gets scale 0xFF and zero codes.
 *
 *   x_bf16, ldx, row_index, M, K   as for mxfp4_quantize_act
 *   codes      [M][K] u8 (float8_e4m3fn bits, one per element), device,
 *              written (16-byte aligned)
 *   scales     [M][K/32] u8 (E8M0), device, written
 *   flags      must be 0
 */
int mxfp8_quantize_act(const void* x_bf16, int64_t ldx, const int32_t* row_index, int64_t M,
                       int64_t K, uint8_t* codes, uint8_t* scales, uint32_t flags,
                       hipStream_t stream);

/* mxfp8_quantize_act with the Smooth pre-scale (as mxfp4_quantize_act_smooth);
   flags must be 0. */
int mxfp8_quantize_act_smooth(const void* x_bf16, int64_t ldx, const int32_t* row_index,
                              const void* smooth_bf16, int64_t M, int64_t K, uint8_t* codes,
                              uint8_t* scales, uint32_t flags, hipStream_t stream);

/*
 * The mixed FP8 x FP4 GEMM of W4A8: y[m][n] = round(sum_k A[m,k] * B[n,k] +
 * bias[n]) with A = e4m3 * 2^(a_scale - 127) (MXFP8, as mxfp8_quantize_act
 * writes it) and B the MXFP4 weight of mxfp4_gemm, fp32 accumulation on the
 * block-scaled MFMA (E4M3 x E2M1 formats), bf16 or fp32 output (the guide
 * gives the mixed GEMM bf16 output and a bf16 row bias).
 *
 *   a_codes, a_scales   [M][K], [M][K/32] u8, device, read (16-byte aligned)
 *   b_codes, b_scales   [N][K/2], [N][K/32] u8, device, read
 *   bias_bf16           [N] bf16, device, read, 16-byte aligned; or NULL
 *   y, out_dtype        as for mxfp4_gemm
 *   flags               must be 0
 * Kernel choice as for mxfp4_gemm, the tiled kernel needing M * K < 2^31.
 */
int mxfp4_gemm_w4a8(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                    const uint8_t* b_scales, int64_t M, int64_t N, int64_t K,
                    const void* bias_bf16, void* y, int out_dtype, uint32_t flags,
                    hipStream_t stream);

/*
 * One W4A8 linear layer on bf16 activations: mxfp8_quantize_act then
 * mxfp4_gemm_w4a8, the same y bit for bit.  For the decode shapes of
 * mxfp4_linear_bf16 (M <= 16, K = 2048 or 4096, N >= 16) it is one launch
 * that quantizes the activations inside the GEMM kernel; otherwise the two
 * launches run through the caller's workspace
 * (mxfp4_linear_w4a8_workspace_size(M, N, K) bytes, 16-byte aligned), the
 * choice made by shape alone.  Arguments as for mxfp4_linear_bf16 (b_scales
 * 16-byte aligned); flags must be 0.
 */
int mxfp4_linear_w4a8_bf16(const void* x_bf16, int64_t ldx, int64_t M, int64_t N, int64_t K,
                           const uint8_t* b_codes, const uint8_t* b_scales,
                           const void* bias_bf16, void* y, int out_dtype, void* workspace,
                           size_t workspace_bytes, uint32_t flags, hipStream_t stream);

/* Workspace bytes mxfp4_linear_w4a8_bf16 needs: 0 for the one-launch shapes,
   else the MXFP8 activations. */
size_t mxfp4_linear_w4a8_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * The activation between an MoE layer's two grouped GEMMs, quantized for the
 * second (AMD blog, closing list: the MoE experts run as fused-MoE kernels on
 * MXFP4).  Each expert is a gate/up projection followed by a down projection;
 * the gate_up GEMM's output row holds the gate half g in columns [0, I) and
 * the up half u in [I, 2I).  The down projection's input is
 *   h = bf16_RNE(silu(g) * u),  silu(g) = g / (1 + e^-g),
 * evaluated in fp32 (exp, 1 + e, a reciprocal, two products), and is
 * quantized to MXFP4 exactly as mxfp4_quantize_act would quantize h.  The
 * exponential and reciprocal are gfx950's (within 2 ulp), so an h lying
 * within a few fp32 ulps of a bf16 rounding midpoint may round either way.
 * Rows stay in the order given (expert-sorted, as the grouped GEMM wrote
 * them).
 *
 *   gate_up_bf16  [M][ldg] bf16, device, read; ldg >= 2*I, ldg % 8 == 0,
 *                 16-byte aligned
 *   I             columns of h; a positive multiple of 32
 *   codes         [M][I/2] u8, device, written (16-byte aligned)
 *   scales        [M][I/32] u8, device, written
 *   flags         0 or MXFP4_SCALE_UOS
 */
int mxfp4_silu_mul_quantize(const void* gate_up_bf16, int64_t ldg, int64_t M, int64_t I,
                            uint8_t* codes, uint8_t* scales, uint32_t flags,
                            hipStream_t stream);

/*
 * The gate_up grouped GEMM of an MoE layer with the expert activation and its
 * MXFP4 quantization in the GEMM's epilogue (AMD blog, closing list: the MoE
 * experts run as fused-MoE kernels on MXFP4): one launch in place of
 * mxfp4_grouped_gemm (bf16 out) followed by mxfp4_silu_mul_quantize, and
 * without the bf16 gate_up output in HBM.  The result is the same, bit for
 * bit: each gate and up value is the bf16 (RNE) of its fp32 sum, then
 * h = bf16_RNE(silu(g) * u) is quantized by the act-quant rule.
 *
 * Layout: each expert's 2I weight rows are interleaved in groups of 64, 32
 * gate rows then the 32 up rows of the same columns of h: row 64q + r is the
 * gate row of h column 32q + r and row 64q + 32 + r its up row (r < 32).  A
 * caller holding [gate; up] stacked permutes the rows once, at load time.
 *
 *   a_codes, a_scales   [total_M][K/2], [total_M][K/32] u8, device, read
 *   b_codes, b_scales   [E][2I][K/2], [E][2I][K/32] u8, device, read,
 *                       interleaved as above
 *   offsets             [E+1] int32, device, read, as for mxfp4_grouped_gemm
 *   I                   columns of h; a positive multiple of 32
 *   h_codes, h_scales   [total_M][I/2], [total_M][I/32] u8, device, written
 *                       (h_codes 16-byte aligned)
 *   flags               0, MXFP4_SCALE_UOS and/or MXFP4_B_PRESHUFFLED (the
 *                       interleaved b_codes then pre-shuffled; needs
 *                       K % 1024 == 0)
 * Returns MXFP4_EUNSUPPORTED where the persistent grouped kernel does not
 * apply (K % 512 != 0, more than its expert table holds, operands over 2 GiB,
 * scale pointers not 4-byte aligned); the two calls above cover those shapes.
 */
int mxfp4_grouped_gemm_silu_quantize(const uint8_t* a_codes, const uint8_t* a_scales,
                                     const uint8_t* b_codes, const uint8_t* b_scales,
                                     const int32_t* offsets, int64_t E, int64_t total_M,
                                     int64_t I, int64_t K, uint8_t* h_codes,
                                     uint8_t* h_scales, uint32_t flags, hipStream_t stream);

/* Largest topk mxfp4_moe_combine accepts. */
enum { MXFP4_COMBINE_MAX_TOPK = 64 };

/*
 * The top-k combine that ends an MoE layer (AMD blog, closing list: MoE
 * experts): each token's output row is the weighted sum of its topk routed
 * expert-output rows,
 *   out[t][n] = sum_{j < topk} weights[t*topk + j] * y[rows[t*topk + j]][n],
 * accumulated in fp32 with one fused multiply-add per routed row, in the
 * order j = 0, 1, ..., then rounded once to the output type (RNE).  The
 * result is the same on every run.
 *
 *   y_bf16     [R][ldy] bf16, device, read: the down projection's output in
 *              expert-sorted row order; ldy >= H, ldy % 8 == 0, 16-byte aligned
 *   rows       [T][topk] int32, device, read: the sorted row holding token
 *              t's j-th expert output.  Not checked on the host (that would
 *              need a sync); the kernel clamps each index to [0, R), so a bad
 *              table gives wrong sums but never a read outside y.
 *   weights    [T][topk] fp32, device, read: the routing weights
 *   T, topk    tokens and experts per token (1 <= topk <= 64)
 *   H          columns; a positive multiple of 8
 *   out        [T][H] bf16 (MXFP4_OUT_BF16) or fp32 (MXFP4_OUT_FP32),
 *              device, written, 16-byte aligned; must not overlap y
 *   flags      0
 */
int mxfp4_moe_combine(const void* y_bf16, int64_t ldy, int64_t R, const int32_t* rows,
                      const float* weights, int64_t T, int64_t topk, int64_t H, void* out,
                      int out_dtype, uint32_t flags, hipStream_t stream);

/* Static description of a status code; never NULL. */
const char* mxfp4_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int mxfp4_version(void);

#ifdef __cplusplus
}
#endif
#endif
