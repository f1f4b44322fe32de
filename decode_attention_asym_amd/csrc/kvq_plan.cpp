// kvq_plan.cpp -- which decode kernel runs, and with how many splits.
#include "kvq_internal.h"

namespace kvq {

Variant pick_variant(const kvq_cache& c, int Hq) {
    (void)c;
    (void)Hq;
    return V_GENERIC;
}

const char* variant_name(Variant v) {
    switch (v) {
        case V_GENERIC: return "generic";
        case V_MHA: return "mha_valu";
        case V_GQA: return "gqa_mfma";
        case V_MLA: return "mla_mfma";
    }
    return "unknown";
}

// Automatic split count.  It must not decrease as T grows (the workspace
// query sizes for the full capacity); the caller clamps it to the number of
// work units.
int auto_splits(const kvq_cache& c, int Hq, int64_t T, Variant v) {
    (void)T;
    (void)v;
    const int64_t wgs = int64_t(c.cfg.batch) * Hq;
    int64_t S = (2048 + wgs - 1) / wgs;
    if (S > KVQ_MAX_SPLITS) S = KVQ_MAX_SPLITS;
    return int(S < 1 ? 1 : S);
}

}  // namespace kvq
