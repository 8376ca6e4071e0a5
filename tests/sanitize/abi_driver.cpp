// Host sanitizer run of the C-ABI library's host code (test infrastructure):
// built with AddressSanitizer and UndefinedBehaviorSanitizer (no recovery)
// around the argument checks of every entry point and the layerwise load
// planner.  No GPU is used: each call here is rejected, or returns, before
// any HIP call.  The planner is run on random parts and its plan checked
// against the contract include/mxfp4.h states for it.
#include "mxfp4.h"

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

static int failures = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static uint64_t lcg = 0x243F6A8885A308D3ull;
static uint32_t rnd() {
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(lcg >> 33);
}

// never dereferenced: every call below is rejected (or has nothing to do)
// before a pointer is used
static const uint8_t* const FAKE = reinterpret_cast<const uint8_t*>(0x1000);
static const uint8_t* const ODD = reinterpret_cast<const uint8_t*>(0x1001);
static uint8_t* fake() { return const_cast<uint8_t*>(FAKE); }

static void argument_checks() {
    // GEMM
    CHECK(mxfp4_gemm(FAKE, FAKE, FAKE, FAKE, 16, 16, 48, fake(), 0, nullptr, 0, 0, nullptr) == MXFP4_EINVAL);
    CHECK(mxfp4_gemm(FAKE, FAKE, FAKE, FAKE, 16, 16, 64, fake(), 2, nullptr, 0, 0, nullptr) == MXFP4_EINVAL);
    CHECK(mxfp4_gemm(ODD, FAKE, FAKE, FAKE, 16, 16, 64, fake(), 0, nullptr, 0, 0, nullptr) == MXFP4_EALIGN);
    CHECK(mxfp4_gemm(nullptr, FAKE, FAKE, FAKE, 16, 16, 64, fake(), 0, nullptr, 0, 0, nullptr) == MXFP4_EINVAL);
    CHECK(mxfp4_gemm(FAKE, FAKE, FAKE, FAKE, 0, 16, 64, fake(), 0, nullptr, 0, 0, nullptr) == MXFP4_OK);
    // grouped GEMM and its fused form
    const int32_t* off = reinterpret_cast<const int32_t*>(FAKE);
    CHECK(mxfp4_grouped_gemm(FAKE, FAKE, FAKE, FAKE, off, 0, 64, 32, 64, fake(), 0, nullptr, 0, 0, nullptr) == MXFP4_EINVAL);
    CHECK(mxfp4_grouped_gemm(FAKE, FAKE, FAKE, FAKE, nullptr, 4, 64, 32, 64, fake(), 0, nullptr, 0, 0, nullptr) == MXFP4_EINVAL);
    CHECK(mxfp4_grouped_gemm(FAKE, FAKE, FAKE, FAKE, off, 4, 0, 32, 64, fake(), 0, nullptr, 0, 0, nullptr) == MXFP4_OK);
    CHECK(mxfp4_grouped_gemm_silu_quantize(FAKE, FAKE, FAKE, FAKE, off, 4, 64, 80, 512, fake(), fake(), 0, nullptr) == MXFP4_EINVAL);
    CHECK(mxfp4_grouped_gemm_silu_quantize(FAKE, FAKE, FAKE, FAKE, off, 4096, 64, 64, 512, fake(), fake(), 0, nullptr) == MXFP4_EUNSUPPORTED);
    CHECK(mxfp4_grouped_gemm_silu_quantize(FAKE, FAKE, FAKE, FAKE, off, 4, 0, 64, 512, fake(), fake(), 2, nullptr) == MXFP4_OK);
    // quantizers and requant
    const void* X = FAKE;
    CHECK(mxfp4_quantize_act(X, 32, nullptr, 4, 64, fake(), fake(), 0, nullptr) == MXFP4_EINVAL);
    CHECK(mxfp4_quantize_act(X, 68, nullptr, 4, 64, fake(), fake(), 0, nullptr) == MXFP4_EALIGN);
    CHECK(mxfp4_quantize_act(X, 64, nullptr, 0, 64, fake(), fake(), 2, nullptr) == MXFP4_OK);
    CHECK(mxfp8_quantize_act(X, 64, nullptr, 4, 64, fake(), fake(), 2, nullptr) == MXFP4_EINVAL);
    CHECK(mxfp4_quantize_act_scatter(X, 64, 4, 64, off, 0, 8, fake(), fake(), 0, nullptr) == MXFP4_EINVAL);
    CHECK(mxfp4_quantize_act_smooth(X, 64, nullptr, nullptr, 4, 64, fake(), fake(), 0, nullptr) == MXFP4_EINVAL);
    const float* G = reinterpret_cast<const float*>(FAKE);
    CHECK(mxfp4_requant_from_nvfp4(FAKE, FAKE, G, 1, 16, 48, fake(), fake(), 0, nullptr) == MXFP4_EINVAL);
    CHECK(mxfp4_requant_from_nvfp4(FAKE, ODD, G, 1, 16, 64, fake(), fake(), 0, nullptr) == MXFP4_EALIGN);
    const int32_t bad_order[3] = {0, 2, 2}, ok[3] = {0, 2, 5};
    CHECK(mxfp4_requant_from_nvfp4_subset(FAKE, FAKE, G, 6, 16, 64, bad_order, 3, fake(), fake(), 0, nullptr) == MXFP4_EINVAL);
    CHECK(mxfp4_requant_from_nvfp4_subset(FAKE, FAKE, G, 6, 16, 64, ok, 0, fake(), fake(), 3, nullptr) == MXFP4_OK);
    // linear layers, the epilogues, W4A8, the no-allocation call
    CHECK(mxfp4_linear_bf16(X, 4000, 1, 256, 4096, FAKE, FAKE, nullptr, fake(), 0, nullptr, 0, 0, nullptr) == MXFP4_EINVAL);
    CHECK(mxfp4_linear_bf16(X, 1024, 200, 256, 1024, FAKE, FAKE, nullptr, fake(), 0, nullptr, 0, 0, nullptr) == MXFP4_EINVAL);
    CHECK(mxfp4_linear_bf16(X, 4096, 1, 256, 4096, FAKE, FAKE + 4, nullptr, fake(), 0, nullptr, 0, 0, nullptr) == MXFP4_EALIGN);
    CHECK(mxfp4_silu_mul_quantize(X, 120, 4, 64, fake(), fake(), 0, nullptr) == MXFP4_EINVAL);
    CHECK(mxfp4_moe_combine(X, 64, 16, off, G, 2, 65, 64, fake(), 0, 0, nullptr) == MXFP4_EINVAL);
    CHECK(mxfp4_gemm_w4a8(FAKE, FAKE, FAKE, FAKE, 4, 16, 48, nullptr, fake(), 0, 0, nullptr) == MXFP4_EINVAL);
    CHECK(mxfp4_linear_w4a8_bf16(X, 4096, 17, 256, 4096, FAKE, FAKE, nullptr, fake(), 0, nullptr, 0, 0, nullptr) == MXFP4_EINVAL);
    const int64_t K = 14336, M = (int64_t)(MXFP4_NOALLOC_SCRATCH_BYTES / (K / 2 + K / 32)) + 1;
    CHECK(mxfp4_linear_bf16_noalloc(X, K, M, 256, K, FAKE, FAKE, nullptr, fake(), 0, 0, nullptr) == MXFP4_ESCRATCH);
    CHECK(mxfp4_linear_workspace_size(17, 512, 4096) > 0 && mxfp4_linear_workspace_size(0, 256, 1024) == 0);
    CHECK(mxfp4_gemm_workspace_size(64, 12288, 4096) == 0);
    for (int s : {0, -1, -2, -3, -4, -5, 7}) CHECK(mxfp4_status_string(s) != nullptr);
    CHECK(mxfp4_version() >= 100);
}

// The plan of random parts against the stated contract: chunks in part
// order, slots alternating, each chunk the largest run of its part's tensors
// that fits a slot (trimmed to start and end on kept tensors), its three
// regions inside its slot, and every kept tensor in exactly one chunk.
static uint64_t up256(uint64_t v) { return (v + 255) / 256 * 256; }

static void planner_fuzz(int cases) {
    for (int c = 0; c < cases; ++c) {
        const int n_parts = (int)(rnd() % 5);
        std::vector<mxfp4_load_part> parts(n_parts);
        std::vector<std::vector<uint8_t>> excl(n_parts);
        for (int i = 0; i < n_parts; ++i) {
            mxfp4_load_part& p = parts[i];
            p.T = rnd() % 9;
            p.N = 1 + rnd() % 300;
            p.K = 32 * (1 + rnd() % 64);
            excl[i].resize(p.T ? p.T : 1);
            for (int64_t t = 0; t < p.T; ++t) excl[i][t] = (rnd() % 4) == 0;
            p.excluded = (rnd() % 3) ? excl[i].data() : nullptr;
            p.nv_codes = p.nv_scales = FAKE;
            p.nv_global = reinterpret_cast<const float*>(FAKE);
            p.mx_codes = p.mx_scales = fake();
        }
        const size_t scratch = 512 + (size_t)(rnd() % (2u << 20));
        int64_t n = -1;
        uint64_t slot = 0;
        const int st = mxfp4_layerwise_plan(parts.data(), n_parts, scratch, nullptr, 0, &n, &slot);
        const uint64_t want_slot = scratch / 2 / 256 * 256;
        bool fits = true;
        for (auto& p : parts)
            if (p.T > 0 && up256((uint64_t)p.N * (p.K / 2)) + up256((uint64_t)p.N * (p.K / 16)) + 4 > want_slot)
                fits = false;
        if (!fits) {
            CHECK(st == MXFP4_EINVAL);
            continue;
        }
        CHECK(st == MXFP4_OK && slot == want_slot);
        if (st != MXFP4_OK) continue;
        std::vector<mxfp4_load_chunk> chunks((size_t)n + 1);
        int64_t n2 = -1;
        if (n > 0)
            CHECK(mxfp4_layerwise_plan(parts.data(), n_parts, scratch, chunks.data(), n - 1, &n2, nullptr) == MXFP4_EINVAL);
        CHECK(mxfp4_layerwise_plan(parts.data(), n_parts, scratch, chunks.data(), n, &n2, nullptr) == MXFP4_OK);
        CHECK(n2 == n);
        std::vector<std::vector<int>> seen(n_parts);
        for (int i = 0; i < n_parts; ++i) seen[i].assign(parts[i].T, 0);
        int64_t last_part = 0, last_t1 = 0;
        for (int64_t k = 0; k < n; ++k) {
            const mxfp4_load_chunk& ch = chunks[k];
            CHECK(ch.part >= 0 && ch.part < n_parts);
            if (ch.part < 0 || ch.part >= n_parts) break;
            const mxfp4_load_part& p = parts[ch.part];
            auto kept = [&](int64_t t) { return !(p.excluded && p.excluded[t]); };
            CHECK(0 <= ch.t0 && ch.t0 < ch.t1 && ch.t1 <= p.T);
            if (!(0 <= ch.t0 && ch.t0 < ch.t1 && ch.t1 <= p.T)) break;
            CHECK(kept(ch.t0) && kept(ch.t1 - 1));
            CHECK(ch.slot == k % 2);
            CHECK(ch.part > last_part || (ch.part == last_part && ch.t0 >= last_t1));
            last_part = ch.part, last_t1 = ch.t1;
            const uint64_t cnt = (uint64_t)(ch.t1 - ch.t0);
            const uint64_t cb = (uint64_t)p.N * (p.K / 2), sb = (uint64_t)p.N * (p.K / 16);
            CHECK(ch.codes_offset == (uint64_t)ch.slot * slot);
            CHECK(ch.scales_offset >= ch.codes_offset + cnt * cb && ch.scales_offset % 256 == 0);
            CHECK(ch.global_offset >= ch.scales_offset + cnt * sb && ch.global_offset % 256 == 0);
            CHECK(ch.global_offset + 4 * cnt <= (uint64_t)(ch.slot + 1) * slot);
            // the largest run that fits, from t0 (before trimming the end)
            int64_t cap = 0;
            while (cap < p.T && up256((cap + 1) * cb) + up256((cap + 1) * sb) + 4 * (cap + 1) <= slot) ++cap;
            int64_t t1 = ch.t0 + cap < p.T ? ch.t0 + cap : p.T;
            while (!kept(t1 - 1)) --t1;
            CHECK(ch.t1 == t1);
            for (int64_t t = ch.t0; t < ch.t1; ++t) seen[ch.part][t] += 1;
        }
        for (int i = 0; i < n_parts; ++i)
            for (int64_t t = 0; t < parts[i].T; ++t) {
                const bool kept = !(parts[i].excluded && parts[i].excluded[t]);
                if (kept) CHECK(seen[i][t] == 1);
                else CHECK(seen[i][t] <= 1);
            }
        // the executor rejects what the planner rejects, and has nothing to
        // do for parts without tensors, before any HIP call
        CHECK(mxfp4_requant_layers_from_host(parts.data(), n_parts, fake(), scratch, 4, nullptr, nullptr) == MXFP4_EINVAL);
    }
}

int main() {
    argument_checks();
    planner_fuzz(20000);
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("library host sanitizer run ok\n");
    return 0;
}
