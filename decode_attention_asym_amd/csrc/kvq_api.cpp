// kvq_api.cpp -- host side of libkvq: argument validation (always before any
// HIP call), sizing, host counters, and the launch sequences behind the C ABI.
#include <stdlib.h>
#include <string.h>

#include <new>

#include "kvq_internal.h"

using namespace kvq;

namespace kvq {

Geom geom_of(const kvq_cache_cfg& c) {
    Geom g;
    g.B = c.batch;
    g.Hkv = c.n_kv_heads;
    g.kd = c.key.dim;
    g.kG = c.key.group;
    g.kbits = c.key.bits;
    g.kW = c.key.group * c.key.bits / 32;
    g.vd = c.value.dim;
    g.vG = c.value.group;
    g.vbits = c.value.bits;
    g.vWT = c.value.dim * c.value.bits / 32;
    g.vNG = c.value.dim / c.value.group;
    g.cap = c.max_tokens;
    g.nblk_cap = c.max_tokens / c.key.group;
    return g;
}

}  // namespace kvq

namespace {

hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kvq_status check_cfg(const kvq_cache_cfg* c) {
    if (!c) return KVQ_E_NULL;
    if (c->kind != KVQ_KIND_KIVI && c->kind != KVQ_KIND_MLA) return KVQ_E_SHAPE;
    if (c->reserved != 0) return KVQ_E_SHAPE;
    if (c->batch < 1 || c->n_kv_heads < 1) return KVQ_E_SHAPE;
    if (c->kind == KVQ_KIND_MLA && c->n_kv_heads != 1) return KVQ_E_SHAPE;
    const kvq_stream_cfg &k = c->key, &v = c->value;
    if ((k.bits != 2 && k.bits != 4) || (v.bits != 2 && v.bits != 4)) return KVQ_E_SHAPE;
    if (k.axis != KVQ_AXIS_PER_CHANNEL || v.axis != KVQ_AXIS_PER_TOKEN) return KVQ_E_UNSUPPORTED;
    if (k.dim < 32 || k.dim > 512 || k.dim % 32 != 0) return KVQ_E_SHAPE;
    if (v.dim < 32 || v.dim > 512 || v.dim % 32 != 0) return KVQ_E_SHAPE;
    if (k.group != 16 && k.group != 32 && k.group != 64 && k.group != 128) return KVQ_E_SHAPE;
    if (k.group * k.bits / 32 > 8) return KVQ_E_UNSUPPORTED;
    if (v.group != 32) return KVQ_E_UNSUPPORTED;
    if (c->kind == KVQ_KIND_KIVI && k.dim != v.dim) return KVQ_E_SHAPE;
    if (c->max_tokens < k.group || c->max_tokens % k.group != 0) return KVQ_E_SHAPE;
    if (c->max_tokens > (int64_t(1) << 31)) return KVQ_E_SHAPE;
    return KVQ_OK;
}

void sizes_of(const kvq_cache_cfg& c, kvq_buffer_sizes* s) {
    const Geom g = geom_of(c);
    const uint64_t bh = uint64_t(g.B) * g.Hkv;
    s->k_codes = bh * g.nblk_cap * g.kd * g.kW * 4;
    s->k_scale = bh * g.nblk_cap * g.kd * 2;
    s->k_zero = s->k_scale;
    s->k_resid = bh * g.kG * g.kd * 2;
    s->v_codes = bh * g.cap * g.vWT * 4;
    s->v_scale = bh * g.cap * g.vNG * 2;
    s->v_zero = s->v_scale;
}

kvq_status hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_E_HIP; }

// An explicit split count must keep every run of the matrix-core kernels
// within what their 32-bit buffer offsets address (nblk quantized blocks);
// the automatic plan always does.
bool splits_fit(const kvq_cache& c, Variant v, int n_splits, int64_t nblk) {
    if (n_splits == 0 || (v != V_GQA && v != V_MHA)) return true;
    const int64_t ntiles = nblk * c.cfg.key.group / 64;
    int64_t s = n_splits < KVQ_MAX_SPLITS - 1 ? n_splits : KVQ_MAX_SPLITS - 1;
    s = s < ntiles ? s : ntiles;
    return runs_fit(c.cfg, ntiles, s);
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

void paged_sizes_of(const kvq_cache_cfg& c, int32_t n_pages, kvq_buffer_sizes* s) {
    const Geom g = geom_of(c);
    const uint64_t ph = uint64_t(n_pages) * g.Hkv;   // (page, KV head) block rows
    s->k_codes = ph * g.kd * g.kW * 4;
    s->k_scale = ph * g.kd * 2;
    s->k_zero = s->k_scale;
    s->k_resid = uint64_t(g.B) * g.Hkv * g.kG * g.kd * 2;
    s->v_codes = ph * g.kG * g.vWT * 4;
    s->v_scale = ph * g.kG * g.vNG * 2;
    s->v_zero = s->v_scale;
}

PagedSeq paged_seq(const kvq_paged& c, const int32_t* table, const int32_t* lens, const int32_t* n_new) {
    PagedSeq ps;
    ps.table = table;
    ps.lens = lens;
    ps.n_new = n_new;
    ps.maxb = int(c.cfg.max_tokens / c.cfg.key.group);
    ps.n_pages = c.n_pages;
    return ps;
}

}  // namespace

namespace kvq {

kvq_status decode_workspace_now(const kvq_cache& c, int Hq, int n_splits, uint64_t* bytes) {
    if (Hq < 1 || Hq % c.cfg.n_kv_heads != 0) return KVQ_E_SHAPE;
    if (n_splits < 0 || n_splits > KVQ_MAX_SPLITS) return KVQ_E_SHAPE;
    const Variant v = pick_variant(c, Hq);
    if (!splits_fit(c, v, n_splits, c.nblk)) return KVQ_E_SHAPE;
    const SplitPlan sp = plan_splits(c, Hq, n_splits, c.T, c.nblk, v);
    *bytes = uint64_t(c.cfg.batch) * Hq * sp.S * (c.cfg.value.dim + 2) * 4;
    return KVQ_OK;
}

}  // namespace kvq

extern "C" {

const char* kvq_status_str(int32_t status) {
    // an int, not the enum: any value a caller passes is defined behaviour
    switch (status) {
        case KVQ_OK: return "ok";
        case KVQ_E_NULL: return "null pointer";
        case KVQ_E_SHAPE: return "bad shape";
        case KVQ_E_ALIGN: return "pointer not 16-byte aligned";
        case KVQ_E_CAPACITY: return "capacity exceeded";
        case KVQ_E_UNSUPPORTED: return "unsupported configuration";
        case KVQ_E_WORKSPACE: return "workspace too small";
        case KVQ_E_HIP: return "HIP launch failed";
        case KVQ_E_STATE: return "cache holds no tokens";
        case KVQ_E_SCRATCH: return "partials exceed the static scratch array";
    }
    return "unknown status";
}

kvq_status kv_cache_buffer_bytes(const kvq_cache_cfg* cfg, kvq_buffer_sizes* out) {
    if (!out) return KVQ_E_NULL;
    kvq_status st = check_cfg(cfg);
    if (st != KVQ_OK) return st;
    sizes_of(*cfg, out);
    return KVQ_OK;
}

kvq_status kv_cache_init(const kvq_cache_cfg* cfg, const kvq_cache_buffers* bufs, kvq_cache** out) {
    if (!out || !bufs) return KVQ_E_NULL;
    kvq_status st = check_cfg(cfg);
    if (st != KVQ_OK) return st;
    const void* ptrs[7] = {bufs->k_codes, bufs->k_scale, bufs->k_zero, bufs->k_resid,
                           bufs->v_codes, bufs->v_scale, bufs->v_zero};
    for (const void* p : ptrs) {
        if (!p) return KVQ_E_NULL;
        if (!aligned16(p)) return KVQ_E_ALIGN;
    }
    kvq_cache* c = new (std::nothrow) kvq_cache;
    if (!c) return KVQ_E_NULL;
    c->cfg = *cfg;
    c->buf = *bufs;
    c->T = 0;
    c->nblk = 0;
    *out = c;
    return KVQ_OK;
}

void kv_cache_destroy(kvq_cache* c) { delete c; }

kvq_status kv_cache_reset(kvq_cache* c) {
    if (!c) return KVQ_E_NULL;
    c->T = 0;
    c->nblk = 0;
    return KVQ_OK;
}

kvq_status kv_cache_state(const kvq_cache* c, int64_t* n_tokens, int32_t* n_resid) {
    if (!c) return KVQ_E_NULL;
    if (n_tokens) *n_tokens = c->T;
    if (n_resid) *n_resid = int32_t(c->T - c->nblk * c->cfg.key.group);
    return KVQ_OK;
}

kvq_status kv_quantize_append(kvq_cache* c, const void* k, const void* v, int64_t n,
                              uint32_t flags, void* stream) {
    if (!c) return KVQ_E_NULL;
    if (n < 0) return KVQ_E_SHAPE;
    if (flags & ~KVQ_APPEND_NO_AUTOFLUSH) return KVQ_E_SHAPE;
    if (n == 0) return KVQ_OK;
    if (!k || !v) return KVQ_E_NULL;
    if (!aligned16(k) || !aligned16(v)) return KVQ_E_ALIGN;
    const Geom g = geom_of(c->cfg);
    const int64_t G = g.kG;
    if (c->T + n > g.cap) return KVQ_E_CAPACITY;
    const int64_t R = c->T - c->nblk * G;
    const bool manual = (flags & KVQ_APPEND_NO_AUTOFLUSH) != 0;
    if (manual && R + n > G) return KVQ_E_CAPACITY;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t pending = R + n;           // keys not yet in a quantized block
    if (manual || pending < G) {
        // no block completes (with NO_AUTOFLUSH a full residual waits for
        // kv_flush_residual): values and residual keys in one launch
        if (launch_append_rows(*c, g, k, v, n, R, st) != hipSuccess) return KVQ_E_HIP;
        c->T += n;
        return KVQ_OK;
    }
    hipError_t e = launch_quant_values(*c, g, v, n, 0, n, c->T, st);
    if (e != hipSuccess) return KVQ_E_HIP;
    const int64_t full = pending / G;        // blocks that complete now (>= 1)
    const int64_t tail = pending - full * G; // keys left in the residual
    // block tokens < c->T come from the residual (rows t - nblk*G)
    e = launch_quant_keys(*c, g, k, n, c->T, c->nblk * G, c->nblk, full, st);
    if (e != hipSuccess) return KVQ_E_HIP;
    if (tail > 0) e = launch_resid_copy(*c, g, k, n, n - tail, 0, tail, st);
    if (e != hipSuccess) return KVQ_E_HIP;
    c->nblk += full;
    c->T += n;
    return KVQ_OK;
}

kvq_status kv_flush_residual(kvq_cache* c, void* stream, int32_t* flushed) {
    if (!c) return KVQ_E_NULL;
    if (flushed) *flushed = 0;
    const Geom g = geom_of(c->cfg);
    const int64_t R = c->T - c->nblk * g.kG;
    if (R != g.kG) return KVQ_OK;
    // every token of the block is a residual row; no input rows are read
    hipError_t e = launch_quant_keys(*c, g, nullptr, 0, c->T, c->nblk * g.kG, c->nblk, 1,
                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return KVQ_E_HIP;
    c->nblk += 1;
    if (flushed) *flushed = 1;
    return KVQ_OK;
}

kvq_status kv_decode_workspace_bytes(const kvq_cache* c, int32_t Hq, int32_t n_splits,
                                     uint64_t* bytes) {
    if (!c || !bytes) return KVQ_E_NULL;
    if (Hq < 1 || Hq % c->cfg.n_kv_heads != 0) return KVQ_E_SHAPE;
    if (n_splits < 0 || n_splits > KVQ_MAX_SPLITS) return KVQ_E_SHAPE;
    const Geom g = geom_of(c->cfg);
    const Variant v = pick_variant(*c, Hq);
    if (!splits_fit(*c, v, n_splits, g.nblk_cap)) return KVQ_E_SHAPE;
    const int S = max_slots(*c, Hq, n_splits, v);   // covers every length up to capacity
    *bytes = uint64_t(g.B) * Hq * S * (g.vd + 2) * 4;
    return KVQ_OK;
}

kvq_status kv_decode_attention(const kvq_cache* c, const void* q, int32_t Hq, float sigma,
                               int32_t n_splits, void* out, void* ws, uint64_t ws_bytes,
                               void* stream) {
    if (!c || !q || !out || !ws) return KVQ_E_NULL;
    if (Hq < 1 || Hq % c->cfg.n_kv_heads != 0) return KVQ_E_SHAPE;
    if (n_splits < 0 || n_splits > KVQ_MAX_SPLITS) return KVQ_E_SHAPE;
    if (!aligned16(q) || !aligned16(out) || !aligned16(ws)) return KVQ_E_ALIGN;
    if (c->T <= 0) return KVQ_E_STATE;
    DecodeArgs a{};
    a.c = c;
    a.g = geom_of(c->cfg);
    const Variant v = pick_variant(*c, Hq);
    if (!splits_fit(*c, v, n_splits, c->nblk)) return KVQ_E_SHAPE;
    a.q = q;
    a.Hq = Hq;
    a.sigma = sigma;
    a.out = out;
    a.T = c->T;
    a.nblk = c->nblk;
    a.R = int(c->T - c->nblk * a.g.kG);
    a.U = int(a.nblk + (a.R > 0 ? 1 : 0));
    const SplitPlan sp = plan_splits(*c, Hq, n_splits, a.T, a.nblk, v);
    a.S = sp.S;
    a.S_main = sp.S_main;
    a.ntiles = sp.ntiles;
    const uint64_t need = uint64_t(a.g.B) * Hq * a.S * (a.g.vd + 2) * 4;
    if (ws_bytes < need) return KVQ_E_WORKSPACE;
    a.ws_acc = static_cast<float*>(ws);
    a.ws_ml = a.ws_acc + uint64_t(a.g.B) * Hq * a.S * a.g.vd;

    a.ev_start = g_ev_before;
    a.ev_stop = g_ev_after;

    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    switch (v) {
        case V_GQA: e = launch_decode_gqa(a, st); break;
        case V_MHA: e = launch_decode_mha(a, st); break;
        case V_MLA: e = launch_decode_mla(a, st); break;
        default: e = launch_decode_generic(a, st); break;
    }
    if (e != hipSuccess) return KVQ_E_HIP;
    return hip_status(launch_merge(a, st));
}

// ------------------------------------------------------------------ paged

kvq_status kv_paged_buffer_bytes(const kvq_cache_cfg* cfg, int32_t n_pages, kvq_buffer_sizes* out) {
    if (!out) return KVQ_E_NULL;
    kvq_status st = check_cfg(cfg);
    if (st != KVQ_OK) return st;
    if (n_pages < 1) return KVQ_E_SHAPE;
    paged_sizes_of(*cfg, n_pages, out);
    return KVQ_OK;
}

kvq_status kv_paged_init(const kvq_cache_cfg* cfg, int32_t n_pages, const kvq_cache_buffers* bufs,
                         kvq_paged** out) {
    if (!out || !bufs) return KVQ_E_NULL;
    kvq_status st = check_cfg(cfg);
    if (st != KVQ_OK) return st;
    if (n_pages < 1) return KVQ_E_SHAPE;
    const void* ptrs[7] = {bufs->k_codes, bufs->k_scale, bufs->k_zero, bufs->k_resid,
                           bufs->v_codes, bufs->v_scale, bufs->v_zero};
    for (const void* p : ptrs) {
        if (!p) return KVQ_E_NULL;
        if (!aligned16(p)) return KVQ_E_ALIGN;
    }
    kvq_paged* c = new (std::nothrow) kvq_paged;
    if (!c) return KVQ_E_NULL;
    c->cfg = *cfg;
    c->buf = *bufs;
    c->n_pages = n_pages;
    *out = c;
    return KVQ_OK;
}

void kv_paged_destroy(kvq_paged* c) { delete c; }

kvq_status kv_paged_append(kvq_paged* c, const void* k, const void* v, int32_t n_max, const int32_t* n_new,
                           const int32_t* seq_lens, const int32_t* block_table, void* stream) {
    if (!c) return KVQ_E_NULL;
    if (n_max < 0) return KVQ_E_SHAPE;
    if (n_max == 0) return KVQ_OK;
    if (!k || !v || !seq_lens || !block_table) return KVQ_E_NULL;
    if (!aligned16(k) || !aligned16(v)) return KVQ_E_ALIGN;
    if (!aligned4(seq_lens) || !aligned4(block_table) || !aligned4(n_new)) return KVQ_E_ALIGN;
    if (n_max > c->cfg.max_tokens) return KVQ_E_CAPACITY;
    const Geom g = geom_of(c->cfg);
    const PagedSeq ps = paged_seq(*c, block_table, seq_lens, n_new);
    return hip_status(launch_paged_append(*c, g, k, v, n_max, ps, static_cast<hipStream_t>(stream)));
}

kvq_status kv_paged_workspace_bytes(const kvq_paged* c, int32_t Hq, int32_t max_len, int32_t n_splits,
                                    uint64_t* bytes) {
    if (!c || !bytes) return KVQ_E_NULL;
    if (Hq < 1 || Hq % c->cfg.n_kv_heads != 0) return KVQ_E_SHAPE;
    if (n_splits < 0 || n_splits > KVQ_MAX_SPLITS) return KVQ_E_SHAPE;
    if (max_len < 0 || max_len > c->cfg.max_tokens) return KVQ_E_SHAPE;
    const Variant v = pick_paged_variant(*c, Hq, n_splits, max_len);
    const PagedPlan pp = plan_paged(*c, Hq, n_splits, max_len, v);
    *bytes = uint64_t(c->cfg.batch) * Hq * pp.S * (c->cfg.value.dim + 2) * 4;
    return KVQ_OK;
}

kvq_status kv_paged_decode(const kvq_paged* c, const void* q, int32_t Hq, float sigma, const int32_t* seq_lens,
                           const int32_t* block_table, int32_t max_len, int32_t n_splits, void* out, void* ws,
                           uint64_t ws_bytes, void* stream) {
    if (!c || !q || !out || !ws || !seq_lens || !block_table) return KVQ_E_NULL;
    if (Hq < 1 || Hq % c->cfg.n_kv_heads != 0) return KVQ_E_SHAPE;
    if (n_splits < 0 || n_splits > KVQ_MAX_SPLITS) return KVQ_E_SHAPE;
    if (max_len < 0 || max_len > c->cfg.max_tokens) return KVQ_E_SHAPE;
    if (!aligned16(q) || !aligned16(out) || !aligned16(ws)) return KVQ_E_ALIGN;
    if (!aligned4(seq_lens) || !aligned4(block_table)) return KVQ_E_ALIGN;
    DecodeArgs a{};
    a.pc = c;
    a.g = geom_of(c->cfg);
    const Variant v = pick_paged_variant(*c, Hq, n_splits, max_len);
    const PagedPlan pp = plan_paged(*c, Hq, n_splits, max_len, v);
    a.q = q;
    a.Hq = Hq;
    a.sigma = sigma;
    a.out = out;
    a.S = pp.S;
    a.S_main = pp.S_main;
    a.chunk = pp.chunk;
    a.max_len = max_len;
    a.ps = paged_seq(*c, block_table, seq_lens, nullptr);
    const uint64_t need = uint64_t(a.g.B) * Hq * a.S * (a.g.vd + 2) * 4;
    if (ws_bytes < need) return KVQ_E_WORKSPACE;
    a.ws_acc = static_cast<float*>(ws);
    a.ws_ml = a.ws_acc + uint64_t(a.g.B) * Hq * a.S * a.g.vd;
    a.ev_start = g_ev_before;
    a.ev_stop = g_ev_after;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = v == V_GQA   ? launch_decode_gqa_paged(a, st)
                         : v == V_MHA ? launch_decode_mha_paged(a, st)
                                      : launch_decode_generic_paged(a, st);
    if (e != hipSuccess) return KVQ_E_HIP;
    return hip_status(launch_merge(a, st));
}

kvq_status kv_paged_decode_step(kvq_paged* c, const void* k, const void* v, const void* q, int32_t Hq, float sigma,
                                const int32_t* n_new, int32_t* seq_lens, const int32_t* block_table, int32_t max_len,
                                int32_t n_splits, uint32_t flags, void* out, void* ws, uint64_t ws_bytes,
                                void* stream) {
    if (!c || !k || !v || !q || !out || !ws || !seq_lens || !block_table) return KVQ_E_NULL;
    if (flags & ~KVQ_STEP_ADVANCE_LENGTHS) return KVQ_E_SHAPE;
    if (Hq < 1 || Hq % c->cfg.n_kv_heads != 0) return KVQ_E_SHAPE;
    if (n_splits < 0 || n_splits > KVQ_MAX_SPLITS) return KVQ_E_SHAPE;
    if (max_len < 1 || max_len > c->cfg.max_tokens) return KVQ_E_SHAPE;
    if (!aligned16(k) || !aligned16(v) || !aligned16(q) || !aligned16(out) || !aligned16(ws)) return KVQ_E_ALIGN;
    if (!aligned4(seq_lens) || !aligned4(block_table) || !aligned4(n_new)) return KVQ_E_ALIGN;
    const Variant v_ = pick_paged_variant(*c, Hq, n_splits, max_len);
    if (v_ != V_GQA && v_ != V_MHA) return KVQ_E_UNSUPPORTED;
    const PagedPlan pp = plan_paged(*c, Hq, n_splits, max_len, v_);
    DecodeArgs a{};
    a.pc = c;
    a.g = geom_of(c->cfg);
    a.q = q;
    a.Hq = Hq;
    a.sigma = sigma;
    a.out = out;
    a.S = pp.S;
    a.S_main = pp.S_main;
    a.chunk = pp.chunk;
    a.max_len = max_len;
    a.ps = paged_seq(*c, block_table, seq_lens, n_new);
    const uint64_t need = uint64_t(a.g.B) * Hq * a.S * (a.g.vd + 2) * 4;
    if (ws_bytes < need) return KVQ_E_WORKSPACE;
    a.ws_acc = static_cast<float*>(ws);
    a.ws_ml = a.ws_acc + uint64_t(a.g.B) * Hq * a.S * a.g.vd;
    a.ev_start = g_ev_before;
    a.ev_stop = g_ev_after;
    a.k_new = k;
    a.v_new = v;
    a.fuse = 1;
    a.lens_adv = (flags & KVQ_STEP_ADVANCE_LENGTHS) ? seq_lens : nullptr;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = v_ == V_GQA ? launch_decode_gqa_paged(a, st) : launch_decode_mha_paged(a, st);
    if (e != hipSuccess) return KVQ_E_HIP;
    return hip_status(launch_merge(a, st));
}

const char* kv_paged_variant(const kvq_paged* c, int32_t Hq, int32_t max_len) {
    if (!c || Hq < 1 || Hq % c->cfg.n_kv_heads != 0 || max_len < 0 || max_len > c->cfg.max_tokens)
        return "invalid";
    return paged_variant_name(pick_paged_variant(*c, Hq, 0, max_len));
}

kvq_status kv_decode_step(kvq_cache* c, const void* k, const void* v, const void* q, int32_t Hq, float sigma,
                          int32_t n_splits, void* out, void* ws, uint64_t ws_bytes, void* stream) {
    // everything both halves would check, before any HIP call
    if (!c || !k || !v || !q || !out || !ws) return KVQ_E_NULL;
    if (Hq < 1 || Hq % c->cfg.n_kv_heads != 0) return KVQ_E_SHAPE;
    if (n_splits < 0 || n_splits > KVQ_MAX_SPLITS) return KVQ_E_SHAPE;
    if (!aligned16(k) || !aligned16(v) || !aligned16(q) || !aligned16(out) || !aligned16(ws)) return KVQ_E_ALIGN;
    const Geom g = geom_of(c->cfg);
    if (c->T + 1 > g.cap) return KVQ_E_CAPACITY;
    const Variant v_ = pick_variant(*c, Hq);
    const int64_t R = c->T - c->nblk * g.kG;
    const int64_t T1 = c->T + 1;
    // the block count after the append (auto-flush when the key fills it)
    const int64_t nblk1 = c->nblk + (R + 1 >= g.kG ? 1 : 0);
    if (!splits_fit(*c, v_, n_splits, nblk1)) return KVQ_E_SHAPE;
    const SplitPlan sp = plan_splits(*c, Hq, n_splits, T1, nblk1, v_);
    const uint64_t need = uint64_t(g.B) * Hq * sp.S * (g.vd + 2) * 4;
    if (ws_bytes < need) return KVQ_E_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((v_ == V_GQA || v_ == V_MHA) && R + 1 < g.kG) {
        // no block completes: the tail workgroup of pass-1 appends the token
        // and attends over it, so the step is pass-1 + merge
        DecodeArgs a{};
        a.c = c;
        a.g = g;
        a.q = q;
        a.Hq = Hq;
        a.sigma = sigma;
        a.out = out;
        a.T = T1;
        a.nblk = c->nblk;
        a.R = int(R + 1);
        a.U = int(a.nblk + 1);
        a.S = sp.S;
        a.S_main = sp.S_main;
        a.ntiles = sp.ntiles;
        a.ws_acc = static_cast<float*>(ws);
        a.ws_ml = a.ws_acc + uint64_t(g.B) * Hq * a.S * g.vd;
        a.ev_start = g_ev_before;
        a.ev_stop = g_ev_after;
        a.k_new = k;
        a.v_new = v;
        a.fuse = 1;
        const hipError_t e = v_ == V_GQA ? launch_decode_gqa(a, st) : launch_decode_mha(a, st);
        if (e != hipSuccess) return KVQ_E_HIP;
        c->T = T1;
        return hip_status(launch_merge(a, st));
    }
    kvq_status r = kv_quantize_append(c, k, v, 1, 0, stream);
    if (r != KVQ_OK) return r;
    return kv_decode_attention(c, q, Hq, sigma, n_splits, out, ws, ws_bytes, stream);
}

kvq_status kv_prefill_attention(kvq_cache* c, const void* q, const void* k, const void* v, int64_t n, int32_t Hq,
                                float sigma, uint32_t flags, void* out, void* stream) {
    if (!c || !q || !k || !v || !out) return KVQ_E_NULL;
    if (flags & ~KVQ_PREFILL_ATTENTION_ONLY) return KVQ_E_SHAPE;
    // a (sequence, head) slice of the prompt is addressed with 32-bit byte offsets
    if (n < 1 || n > (int64_t(1) << 23)) return KVQ_E_SHAPE;
    if (Hq < 1 || Hq % c->cfg.n_kv_heads != 0) return KVQ_E_SHAPE;
    // one grid dimension of (query blocks) x (query heads) x (sequences) workgroups
    if (((n + 63) / 64) * int64_t(Hq) * c->cfg.batch > INT32_MAX) return KVQ_E_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return KVQ_E_ALIGN;
    if (!prefill_supported(c->cfg)) return KVQ_E_UNSUPPORTED;
    const bool quant = (flags & KVQ_PREFILL_ATTENTION_ONLY) == 0;
    const Geom g = geom_of(c->cfg);
    if (quant && c->T != 0) return KVQ_E_STATE;
    if (quant && n > g.cap) return KVQ_E_CAPACITY;
    PrefillArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.out = static_cast<uint16_t*>(out);
    a.B = g.B;
    a.Hq = Hq;
    a.Hkv = g.Hkv;
    a.T = int(n);
    a.sigma2 = sigma * 1.4426950408889634f;
    a.quant = quant ? 1 : 0;
    a.kc = static_cast<uint32_t*>(c->buf.k_codes);
    a.vc = static_cast<uint32_t*>(c->buf.v_codes);
    a.ks = static_cast<uint16_t*>(c->buf.k_scale);
    a.kz = static_cast<uint16_t*>(c->buf.k_zero);
    a.vs = static_cast<uint16_t*>(c->buf.v_scale);
    a.vz = static_cast<uint16_t*>(c->buf.v_zero);
    a.kr = static_cast<uint16_t*>(c->buf.k_resid);
    a.cap = g.cap;
    a.nblk_cap = g.nblk_cap;
    if (launch_prefill(a, c->cfg, static_cast<hipStream_t>(stream)) != hipSuccess) return KVQ_E_HIP;
    if (quant) {
        // what kv_quantize_append(c, k, v, n, 0) leaves on an empty cache
        c->nblk = n / g.kG;
        c->T = n;
    }
    return KVQ_OK;
}

kvq_status kv_set_timing_events(void* before, void* after) {
    if ((before == nullptr) != (after == nullptr)) return KVQ_E_NULL;
    g_ev_before = static_cast<hipEvent_t>(before);
    g_ev_after = static_cast<hipEvent_t>(after);
    return KVQ_OK;
}

const char* kv_decode_variant(const kvq_cache* c, int32_t Hq) {
    if (!c || Hq < 1 || Hq % c->cfg.n_kv_heads != 0) return "invalid";
    return variant_name(pick_variant(*c, Hq));
}

}  // extern "C"
