// layerwise.cpp -- the layerwise load of an NVFP4 checkpoint into MXFP4
// (AMD blog "Efficiently Serving NVFP4 Models on AMD Instinct MI350X/MI355X
// ...", the pipeline section under Figure 1: requantize one layer at a time
// into a destination allocated beforehand, so that the load needs one
// layer's worth of extra memory; tensors the producer excluded are skipped).
//
// The NVFP4 source sits in host memory.  It is staged through a caller-owned
// device scratch buffer split into two slots: while the requant kernel
// converts the chunk in one slot, the copy engine fills the other.  A chunk is
// a run of tensors of one part (one tensor kind of one layer) that fits a
// slot; excluded tensors inside a chunk are neither copied nor converted.
//
// mxfp4_layerwise_plan is the whole schedule as plain host code (no HIP call),
// so it can be executed and checked without a GPU; the executor below walks
// the same plan with hipMemcpyAsync and the requant launcher.
#include "../../include/mxfp4.h"
#include "launch.h"

#include <stdint.h>

#include <vector>

namespace {

constexpr int64_t kSlots = 2;
constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

uint64_t codes_bytes(const mxfp4_load_part& p) { return (uint64_t)p.N * (uint64_t)(p.K / 2); }
uint64_t scales_bytes(const mxfp4_load_part& p) { return (uint64_t)p.N * (uint64_t)(p.K / 16); }

// Bytes a slot needs for c tensors of part p: codes, then E4M3 scales, then
// the fp32 globals, each region starting on a 256-byte boundary.
uint64_t chunk_bytes(const mxfp4_load_part& p, int64_t c) {
    return align_up((uint64_t)c * codes_bytes(p)) + align_up((uint64_t)c * scales_bytes(p)) +
           4u * (uint64_t)c;
}

bool excluded(const mxfp4_load_part& p, int64_t t) { return p.excluded && p.excluded[t]; }

int check_part(const mxfp4_load_part& p) {
    if (p.T < 0 || p.N <= 0 || p.K <= 0 || p.K % 32 != 0) return MXFP4_EINVAL;
    return MXFP4_OK;
}

// The plan: every chunk in the order the executor runs them.  Returns a
// status; on success fills `out` and the slot size.
int make_plan(const mxfp4_load_part* parts, int64_t n_parts, size_t scratch_bytes,
              std::vector<mxfp4_load_chunk>& out, uint64_t* slot_bytes_out) {
    if (n_parts < 0 || (n_parts > 0 && !parts)) return MXFP4_EINVAL;
    const uint64_t slot = (uint64_t)scratch_bytes / kSlots / kAlign * kAlign;
    for (int64_t i = 0; i < n_parts; ++i) {
        const int st = check_part(parts[i]);
        if (st != MXFP4_OK) return st;
        if (parts[i].T > 0 && chunk_bytes(parts[i], 1) > slot) return MXFP4_EINVAL;
    }
    out.clear();
    int64_t next_slot = 0;
    for (int64_t i = 0; i < n_parts; ++i) {
        const mxfp4_load_part& p = parts[i];
        // tensors per chunk: the most that fit one slot
        int64_t cap = 1;
        while (cap < p.T && chunk_bytes(p, cap * 2) <= slot) cap *= 2;
        for (int64_t step = cap / 2; step > 0; step /= 2)
            if (cap + step <= p.T && chunk_bytes(p, cap + step) <= slot) cap += step;
        int64_t t = 0;
        while (t < p.T) {
            while (t < p.T && excluded(p, t)) ++t;          // a chunk starts on a kept tensor
            if (t == p.T) break;
            int64_t t1 = t + cap < p.T ? t + cap : p.T;
            while (excluded(p, t1 - 1)) --t1;                // and ends on one
            mxfp4_load_chunk c;
            c.part = i;
            c.t0 = t;
            c.t1 = t1;
            c.slot = next_slot;
            const uint64_t base = (uint64_t)next_slot * slot;
            c.codes_offset = base;
            c.scales_offset = base + align_up((uint64_t)(t1 - t) * codes_bytes(p));
            c.global_offset = c.scales_offset + align_up((uint64_t)(t1 - t) * scales_bytes(p));
            out.push_back(c);
            next_slot = (next_slot + 1) % kSlots;
            t = t1;
        }
    }
    if (slot_bytes_out) *slot_bytes_out = slot;
    return MXFP4_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

int mxfp4_layerwise_plan(const mxfp4_load_part* parts, int64_t n_parts, size_t scratch_bytes,
                         mxfp4_load_chunk* chunks, int64_t max_chunks, int64_t* n_chunks,
                         uint64_t* slot_bytes) {
    if (!n_chunks || max_chunks < 0 || (max_chunks > 0 && !chunks)) return MXFP4_EINVAL;
    std::vector<mxfp4_load_chunk> plan;
    const int st = make_plan(parts, n_parts, scratch_bytes, plan, slot_bytes);
    if (st != MXFP4_OK) return st;
    *n_chunks = (int64_t)plan.size();
    if (chunks) {
        if ((int64_t)plan.size() > max_chunks) return MXFP4_EINVAL;
        for (size_t i = 0; i < plan.size(); ++i) chunks[i] = plan[i];
    }
    return MXFP4_OK;
}

int mxfp4_requant_layers_from_host(const mxfp4_load_part* parts, int64_t n_parts,
                                   void* scratch, size_t scratch_bytes, uint32_t flags,
                                   hipStream_t copy_stream, hipStream_t stream) {
    if ((flags & ~(uint32_t)(MXFP4_REQ_INTERMEDIATE_BF16 | MXFP4_SCALE_UOS)) != 0)
        return MXFP4_EINVAL;
    std::vector<mxfp4_load_chunk> plan;
    int st = make_plan(parts, n_parts, scratch_bytes, plan, nullptr);
    if (st != MXFP4_OK) return st;
    if (plan.empty()) return MXFP4_OK;
    if (!scratch) return MXFP4_EINVAL;
    if (!aligned(scratch, kAlign)) return MXFP4_EALIGN;
    for (int64_t i = 0; i < n_parts; ++i) {
        const mxfp4_load_part& p = parts[i];
        if (p.T == 0) continue;
        if (!p.nv_codes || !p.nv_scales || !p.nv_global || !p.mx_codes || !p.mx_scales)
            return MXFP4_EINVAL;
        if (!aligned(p.mx_codes, 16)) return MXFP4_EALIGN;
    }
    const bool bf16 = (flags & MXFP4_REQ_INTERMEDIATE_BF16) != 0;
    const bool uos = (flags & MXFP4_SCALE_UOS) != 0;

    // copied[s]: slot s holds its chunk; freed[s]: the requant of that chunk
    // has read it, so the slot may be refilled
    hipEvent_t copied[kSlots] = {}, freed[kSlots] = {};
    for (int64_t s = 0; s < kSlots && st == MXFP4_OK; ++s)
        if (hipEventCreateWithFlags(&copied[s], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&freed[s], hipEventDisableTiming) != hipSuccess)
            st = MXFP4_EHIP;
    uint8_t* base = static_cast<uint8_t*>(scratch);
    std::vector<int32_t> keep;
    for (size_t i = 0; i < plan.size() && st == MXFP4_OK; ++i) {
        const mxfp4_load_chunk& c = plan[i];
        const mxfp4_load_part& p = parts[c.part];
        const uint64_t cb = codes_bytes(p), sb = scales_bytes(p);
        hipError_t e = hipSuccess;
        if (i >= (size_t)kSlots) e = hipStreamWaitEvent(copy_stream, freed[c.slot], 0);
        // the kept tensors, copied run by run into their places in the slot
        keep.clear();
        for (int64_t t = c.t0; t < c.t1 && e == hipSuccess;) {
            if (excluded(p, t)) { ++t; continue; }
            int64_t r1 = t;
            while (r1 < c.t1 && !excluded(p, r1)) keep.push_back((int32_t)(r1++ - c.t0));
            const uint64_t n = (uint64_t)(r1 - t);
            e = hipMemcpyAsync(base + c.codes_offset + (uint64_t)(t - c.t0) * cb,
                               p.nv_codes + (uint64_t)t * cb, n * cb, hipMemcpyHostToDevice,
                               copy_stream);
            if (e == hipSuccess)
                e = hipMemcpyAsync(base + c.scales_offset + (uint64_t)(t - c.t0) * sb,
                                   p.nv_scales + (uint64_t)t * sb, n * sb,
                                   hipMemcpyHostToDevice, copy_stream);
            t = r1;
        }
        if (e == hipSuccess)
            e = hipMemcpyAsync(base + c.global_offset, p.nv_global + c.t0,
                               4u * (uint64_t)(c.t1 - c.t0), hipMemcpyHostToDevice, copy_stream);
        if (e == hipSuccess) e = hipEventRecord(copied[c.slot], copy_stream);
        if (e == hipSuccess) e = hipStreamWaitEvent(stream, copied[c.slot], 0);
        if (e == hipSuccess) {
            const int64_t T = c.t1 - c.t0;
            const bool all = (int64_t)keep.size() == T;
            e = mx::launch_requant(base + c.codes_offset, base + c.scales_offset,
                                   reinterpret_cast<const float*>(base + c.global_offset), T,
                                   p.N, p.K, all ? nullptr : keep.data(),
                                   all ? 0 : (int64_t)keep.size(),
                                   p.mx_codes + (uint64_t)c.t0 * cb,
                                   p.mx_scales + (uint64_t)c.t0 * (uint64_t)(p.N * (p.K / 32)),
                                   bf16, uos, stream);
        }
        if (e == hipSuccess) e = hipEventRecord(freed[c.slot], stream);
        if (e != hipSuccess) st = MXFP4_EHIP;
    }
    // destroying an event whose work is still pending is allowed (the
    // runtime releases it once the work is done); a failure is still reported
    for (int64_t s = 0; s < kSlots; ++s) {
        if (copied[s] && hipEventDestroy(copied[s]) != hipSuccess && st == MXFP4_OK) st = MXFP4_EHIP;
        if (freed[s] && hipEventDestroy(freed[s]) != hipSuccess && st == MXFP4_OK) st = MXFP4_EHIP;
    }
    return st;
}

}  // extern "C"
