// kvq_internal.h -- shared between the host library (kvq_api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "../../include/kvq.h"

struct kvq_cache {
    kvq_cache_cfg cfg;
    kvq_cache_buffers buf;
    int64_t T;      // tokens held per sequence
    int64_t nblk;   // quantized key blocks; residual keys = T - nblk * G (0..G)
};

// Paged cache: pools of pages (one G-token key block plus the values of the
// same tokens, all KV heads) and one residual block per sequence slot.
struct kvq_paged {
    kvq_cache_cfg cfg;   // batch = sequence slots, max_tokens = per-sequence capacity
    kvq_cache_buffers buf;
    int32_t n_pages;
};

namespace kvq {

// Geometry derived from a validated configuration.
struct Geom {
    int B, Hkv;
    int kd, kG, kbits, kW;        // key stream: dim, tokens per block, bits, words per (block, channel)
    int vd, vG, vbits, vWT, vNG;  // value stream: dim, channels per group, bits, words per token, groups per token
    int64_t cap, nblk_cap;        // token capacity, block capacity
};

Geom geom_of(const kvq_cache_cfg& c);

// ---- quantize / append kernels (kvq_quant.hip) ----

// Per-token value quantization of n_tok input rows v_in [B][Hkv][n_in][vd],
// rows row0 .. row0 + n_tok - 1, stored at cache tokens t_dst0 ...
hipError_t launch_quant_values(const kvq_cache& c, const Geom& g, const void* v_in,
                               int64_t n_in, int64_t row0, int64_t n_tok, int64_t t_dst0,
                               hipStream_t st);

// Per-channel key quantization of blocks blk0 .. blk0 + nb - 1.  Key token t
// of a block comes from the residual row (t - res_tok0) when t < in_tok0,
// else from input row (t - in_tok0) of k_in [B][Hkv][n_in][kd].
hipError_t launch_quant_keys(const kvq_cache& c, const Geom& g, const void* k_in, int64_t n_in,
                             int64_t in_tok0, int64_t res_tok0, int64_t blk0, int64_t nb,
                             hipStream_t st);

// Copy m input key rows (from row src0) into residual rows dst0 ...
hipError_t launch_resid_copy(const kvq_cache& c, const Geom& g, const void* k_in, int64_t n_in,
                             int64_t src0, int64_t dst0, int64_t m, hipStream_t st);

// An append of n rows that completes no key block (R + n < G, R residual
// keys before it), in one launch: the n value rows are quantized at cache
// tokens c.T ... and the n key rows go to residual rows R ...
hipError_t launch_append_rows(const kvq_cache& c, const Geom& g, const void* k_in, const void* v_in,
                              int64_t n, int64_t R, hipStream_t st);

// ---- paged append (kvq_quant.hip) ----

// Sequence-side inputs of a paged call (device arrays owned by the caller).
struct PagedSeq {
    const int32_t* table;   // [B][maxb] page of block j of sequence b
    const int32_t* lens;    // [B] tokens of sequence b (before an append)
    const int32_t* n_new;   // [B] rows appended to sequence b, or null = n_max each
    int maxb;               // table row length = max_tokens / G
    int n_pages;
};

// Append up to n_max rows per sequence (inputs [B][Hkv][n_max][d]): values
// quantized into the pages of their blocks, keys into the residual, every
// block that fills quantized into its page.
hipError_t launch_paged_append(const kvq_paged& c, const Geom& g, const void* k_in, const void* v_in,
                               int n_max, const PagedSeq& ps, hipStream_t st);

// ---- decode kernels (kvq_decode*.hip) ----

enum Variant { V_GENERIC = 0, V_MHA = 1, V_GQA = 2, V_MLA = 3 };

struct DecodeArgs {
    const kvq_cache* c;
    Geom g;
    const void* q;
    int Hq, S;          // query heads, partial slots (main splits + tail slot)
    int S_main;         // splits over whole tiles (variants with a tail slot)
    int ntiles;         // whole 64-token tiles (KIVI MFMA variants); 16-token tiles (MLA)
    float sigma;
    void* out;
    float* ws_acc;      // [B][Hq][S][vd]
    float* ws_ml;       // [B][Hq][S][2]
    int64_t T, nblk;    // tokens, quantized blocks
    int R;              // residual keys
    int U;              // work units: nblk (+1 when R > 0)
    // optional profiling events; the pass-1 launch records its own start and
    // stop timestamps into them (hipExtLaunchKernel), with no extra packets
    hipEvent_t ev_start, ev_stop;
    // paged caches: the sequence inputs, the tile count of a main split
    // (chunk), and the length bound the splits were planned for
    const kvq_paged* pc;
    PagedSeq ps;
    int chunk;
    int max_len;
    // decode step with its append fused in (GQA / MHA kernels): T counts
    // the new token, whose key and value rows ([B][Hkv][1][D]) the tail
    // workgroup stores before attending
    const void *k_new, *v_new;
    int fuse;
    // paged decode step: lengths to advance in the merge launch (null = no)
    int32_t* lens_adv;
};

Variant pick_variant(const kvq_cache& c, int Hq);
const char* variant_name(Variant v);

// Split plan for a cache of T tokens with nblk quantized key blocks.
// n_splits == 0 picks automatically.  Returns the partial-slot count.
struct SplitPlan {
    int S_main, S, ntiles;
};
SplitPlan plan_splits(const kvq_cache& c, int Hq, int n_splits, int64_t T, int64_t nblk, Variant v);
// Upper bound of SplitPlan::S over every T <= capacity.
int max_slots(const kvq_cache& c, int Hq, int n_splits, Variant v);
// Longest run of 64-token tiles one split of a matrix-core kernel may take
// (its code bytes stay below 2^30), and whether S_main splits of ntiles
// tiles respect it.  The automatic plans always do; an explicit split count
// that does not is rejected.
int64_t max_run_tiles(const kvq_cache_cfg& cfg);
bool runs_fit(const kvq_cache_cfg& cfg, int64_t ntiles, int64_t S_main);

// Partial-slot bytes kv_decode_attention needs at the cache's current
// length (checks n_q_heads and n_splits as it does).
kvq_status decode_workspace_now(const kvq_cache& c, int Hq, int n_splits, uint64_t* bytes);

bool gqa_supported(const kvq_cache& c, int Hq);
bool gqa_cfg_supported(const kvq_cache_cfg& c, int Hq);
bool mha_supported(const kvq_cache& c, int Hq);
bool mla_supported(const kvq_cache& c, int Hq);
hipError_t launch_decode_generic(const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_gqa(const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_mha(const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t st);
hipError_t launch_merge(const DecodeArgs& a, hipStream_t st);

// Paged decode: variant choice, split plan over the length bound, launches.
Variant pick_paged_variant(const kvq_paged& c, int Hq, int n_splits, int max_len);
const char* paged_variant_name(Variant v);
struct PagedPlan {
    int S_main, S, chunk;   // main splits, slots (+1 tail), tiles (GQA) / blocks (generic) per main split
};
PagedPlan plan_paged(const kvq_paged& c, int Hq, int n_splits, int max_len, Variant v);
hipError_t launch_decode_gqa_paged(const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_mha_paged(const DecodeArgs& a, hipStream_t st);
bool mha_cfg_supported(const kvq_cache_cfg& c, int Hq);
hipError_t launch_decode_generic_paged(const DecodeArgs& a, hipStream_t st);

// ---- prefill attention fused with the bulk quantize (kvq_prefill.hip) ----
struct PrefillArgs {
    const uint16_t *q, *k, *v;   // q [B][Hq][T][128], k / v [B][Hkv][T][128] (fp16)
    uint16_t* out;               // [B][Hq][T][128] (fp16)
    int B, Hq, Hkv, T;
    float sigma2;                // softmax scale * log2(e)
    int quant;                   // also quantize the prompt into the cache
    uint32_t *kc, *vc;           // cache arrays (contiguous layout)
    uint16_t *ks, *kz, *vs, *vz, *kr;
    int64_t cap, nblk_cap;
};
bool prefill_supported(const kvq_cache_cfg& c);
hipError_t launch_prefill(const PrefillArgs& a, const kvq_cache_cfg& c, hipStream_t st);

}  // namespace kvq
