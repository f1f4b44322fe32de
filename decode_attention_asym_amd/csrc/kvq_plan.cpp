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
// over.  It does not depend on T, so the slot bound below covers every T.
int64_t auto_main(const kvq_cache& c, int Hq, Variant v) {
    // MLA: one four-wave workgroup per CU, Hq / 64 of them per sequence and split
    if (v == V_MLA) return clamp64((256 * 64 / Hq + c.cfg.batch - 1) / c.cfg.batch, 1, KVQ_MAX_SPLITS);
    const bool tiled = v == V_GQA || v == V_MHA;
    const int64_t units = tiled ? int64_t(c.cfg.batch) * c.cfg.n_kv_heads : int64_t(c.cfg.batch) * Hq;
    // measured on MI355X: about 12 tiles per two-wave workgroup suit the MHA
    // kernel (64 tiles per sequence at 4K tokens), 6 waves per SIMD the GQA one
    const int64_t target = v == V_MHA ? 1536 : tiled ? 3072 : 2048;
    return clamp64((target + units - 1) / units, 1, KVQ_MAX_SPLITS);
}

}  // namespace

SplitPlan plan_splits(const kvq_cache& c, int Hq, int n_splits, int64_t T, int64_t nblk, Variant v) {
    SplitPlan sp;
    const int64_t G = c.cfg.key.group;
    const int64_t want = n_splits > 0 ? n_splits : auto_main(c, Hq, v);
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

int max_slots(const kvq_cache& c, int Hq, int n_splits, Variant v) {
    const int64_t want = n_splits > 0 ? n_splits : auto_main(c, Hq, v);
    if (v == V_GQA || v == V_MHA) return int(clamp64(want, 1, KVQ_MAX_SPLITS - 1) + 1);
    return int(want);
}

}  // namespace kvq
