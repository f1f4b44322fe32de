// kvq_plan.cpp -- which decode kernel runs, and how the context is split.
#include "kvq_internal.h"

namespace kvq {

Variant pick_variant(const kvq_cache& c, int Hq) {
    if (gqa_supported(c, Hq)) return V_GQA;
    if (mha_supported(c, Hq)) return V_MHA;
    if (mla_supported(c, Hq)) return V_MLA;
    return V_GENERIC;
}

const char* variant_name(Variant v) {
    switch (v) {
        case V_GENERIC: return "generic";
        case V_MHA: return "mha_mfma";
        case V_GQA: return "gqa_mfma";
        case V_MLA: return "mla_mfma";
    }
    return "unknown";
}

namespace {

int64_t clamp64(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Automatic split count: enough workgroups to fill 256 CUs several times
// over, but (matrix-core kernels) no shorter runs than 16 tiles (GQA) / 8
// tiles (MHA): at small batch more splits cost more in per-split start-up
// and in the merge than they gain (measured on MI355X, 32K-token GQA at one
// sequence: 255 splits 36 us per step, 32 splits 27 us).  Non-decreasing in
// ntiles, so the slot bound at full capacity covers every length.
//
// Workgroup targets (measured on MI355X, four interleaved runs per point):
// the 2-bit GQA kernel holds 8 workgroups per CU (2048 on the GPU); 6144 of
// them (three full rounds) beat 3072 (one and a half) by ~3% on the 32K
// batch-32 workload (150 vs 155 us) and on the 128K batch-4 one.  The 4-bit
// GQA kernel (6 per CU) was flat between 3072 and 8192.
int64_t wg_target(const kvq_cache_cfg& cfg, Variant v) {
    if (v == V_MHA) return 1536;
    if (v == V_GQA) return cfg.key.bits == 2 ? 6144 : 3072;
    return 2048;
}
}  // namespace

// The matrix-core kernels address a split's code run through a buffer
// resource with 32-bit byte offsets: a run holds at most 2^30 bytes of key
// or value codes (2^19 tiles of 64 tokens at 2 bits, 2^18 at 4 bits).
int64_t max_run_tiles(const kvq_cache_cfg& cfg) {
    const int64_t bits = cfg.key.bits > cfg.value.bits ? cfg.key.bits : cfg.value.bits;
    const int64_t dim = cfg.key.dim > cfg.value.dim ? cfg.key.dim : cfg.value.dim;
    return (int64_t(1) << 30) / (64 * dim * bits / 8);
}

bool runs_fit(const kvq_cache_cfg& cfg, int64_t ntiles, int64_t S_main) {
    return S_main < 1 || (ntiles + S_main - 1) / S_main <= max_run_tiles(cfg);
}

namespace {

int64_t auto_main(const kvq_cache& c, int Hq, Variant v, int64_t ntiles) {
    // MLA: one twelve-wave workgroup per CU, Hq / 64 of them per sequence and split
    if (v == V_MLA) return clamp64((256 * 64 / Hq + c.cfg.batch - 1) / c.cfg.batch, 1, KVQ_MAX_SPLITS);
    const bool tiled = v == V_GQA || v == V_MHA;
    const int64_t units = tiled ? int64_t(c.cfg.batch) * c.cfg.n_kv_heads : int64_t(c.cfg.batch) * Hq;
    // measured on MI355X: about 12 tiles per two-wave workgroup suit the MHA
    // kernel (64 tiles per sequence at 4K tokens)
    const int64_t target = wg_target(c.cfg, v);
    int64_t want = (target + units - 1) / units;
    if (tiled) {
        const int64_t min_run = v == V_MHA ? 8 : 16;
        want = want < (ntiles + min_run - 1) / min_run ? want : (ntiles + min_run - 1) / min_run;
        // and no run longer than a buffer resource addresses (at most 128
        // splits for the 2^31-token capacity limit)
        const int64_t max_run = max_run_tiles(c.cfg);
        const int64_t need = (ntiles + max_run - 1) / max_run;
        want = want > need ? want : need;
    }
    return clamp64(want, 1, KVQ_MAX_SPLITS);
}

}  // namespace

SplitPlan plan_splits(const kvq_cache& c, int Hq, int n_splits, int64_t T, int64_t nblk, Variant v) {
    SplitPlan sp;
    const int64_t G = c.cfg.key.group;
    const int64_t want = n_splits > 0 ? n_splits : auto_main(c, Hq, v, nblk * G / 64);
    if (v == V_GQA || v == V_MHA) {
        // whole 64-token tiles of quantized keys, then a tail slot for the rest
        const int64_t ntiles = nblk * G / 64;
        sp.ntiles = int(ntiles);
        // the merge pass reads at most KVQ_MAX_SPLITS slots, tail slot included
        sp.S_main = int(clamp64(clamp64(want, 0, KVQ_MAX_SPLITS - 1), 0, ntiles));
        sp.S = sp.S_main + (T > ntiles * 64 ? 1 : 0);
        return sp;
    }
    if (v == V_MLA) {
        // 16-token tiles over every token; the RoPE residual is read in place
        const int64_t ntiles = (T + 15) / 16;
        sp.ntiles = int(ntiles);
        sp.S_main = int(clamp64(want, 1, ntiles));
        sp.S = sp.S_main;
        return sp;
    }
    const int64_t R = T - nblk * G;
    const int64_t U = nblk + (R > 0 ? 1 : 0);
    sp.ntiles = 0;
    sp.S_main = int(clamp64(want, 1, U));
    sp.S = sp.S_main;
    return sp;
}

// ---- paged caches.  Lengths differ per sequence and live on the device, so
// the splits are planned for the caller's bound max_len: split s covers
// tiles (GQA) / key blocks (generic) [s * chunk, (s + 1) * chunk) of its
// sequence, and the splits past a shorter sequence's end write empty
// partials.
PagedPlan plan_paged(const kvq_paged& c, int Hq, int n_splits, int max_len, Variant v) {
    const int64_t G = c.cfg.key.group;
    PagedPlan pp;
    if (v == V_GQA || v == V_MHA) {
        const int64_t ntiles = int64_t(max_len) / G * G / 64;
        const int64_t units = int64_t(c.cfg.batch) * c.cfg.n_kv_heads;
        // as for a contiguous cache: fill the GPU, runs of at least 16 (GQA)
        // / 8 (MHA) tiles
        const int64_t target = wg_target(c.cfg, v), min_run = v == V_MHA ? 8 : 16;
        const int64_t fill = (target + units - 1) / units, runs = (ntiles + min_run - 1) / min_run;
        const int64_t want = n_splits > 0 ? n_splits : clamp64(fill < runs ? fill : runs, 1, KVQ_MAX_SPLITS - 1);
        int64_t chunk = ntiles > 0 ? (ntiles + want - 1) / want : 1;
        // the page numbers of a run sit one per lane: at most 64 key blocks
        chunk = clamp64(chunk, 1, G);
        pp.chunk = int(chunk);
        pp.S_main = int((ntiles + chunk - 1) / chunk);
        pp.S = pp.S_main + 1;   // + the tail slot (partial tile and residual keys)
        return pp;
    }
    const int64_t U = (int64_t(max_len) + G - 1) / G;   // key blocks, the residual one included
    const int64_t units = int64_t(c.cfg.batch) * Hq;
    const int64_t want = n_splits > 0 ? n_splits : clamp64((2048 + units - 1) / units, 1, KVQ_MAX_SPLITS);
    const int64_t s0 = clamp64(want, 1, U > 0 ? U : 1);
    const int64_t chunk = U > 0 ? (U + s0 - 1) / s0 : 1;
    pp.chunk = int(chunk);
    pp.S_main = int(U > 0 ? (U + chunk - 1) / chunk : 1);
    pp.S = pp.S_main;
    return pp;
}

Variant pick_paged_variant(const kvq_paged& c, int Hq, int n_splits, int max_len) {
    // the MFMA kernels while their main splits fit the merge's slot limit
    if (gqa_cfg_supported(c.cfg, Hq) && plan_paged(c, Hq, n_splits, max_len, V_GQA).S <= KVQ_MAX_SPLITS)
        return V_GQA;
    if (mha_cfg_supported(c.cfg, Hq) && plan_paged(c, Hq, n_splits, max_len, V_MHA).S <= KVQ_MAX_SPLITS)
        return V_MHA;
    return V_GENERIC;
}

const char* paged_variant_name(Variant v) {
    return v == V_GQA ? "gqa_mfma_paged" : v == V_MHA ? "mha_mfma_paged" : "generic_paged";
}

int max_slots(const kvq_cache& c, int Hq, int n_splits, Variant v) {
    const int64_t want = n_splits > 0 ? n_splits : auto_main(c, Hq, v, c.cfg.max_tokens / 64);
    if (v == V_GQA || v == V_MHA) return int(clamp64(want, 1, KVQ_MAX_SPLITS - 1) + 1);
    return int(want);
}

}  // namespace kvq
