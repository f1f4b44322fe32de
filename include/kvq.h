/*
 * kvq.h -- C ABI of libkvq: KIVI-style asymmetric low-bit KV cache and
 * in-loop-dequant decode attention on AMD MI355X (gfx950).
 *
 * What the library computes (sources: page title + section):
 *   "Makale Bülteni -- KIVI" (cmlonder.com paper-to-prod), lead paragraph and
 *   section "İddia ve Gerçeklik: KIVI":
 *     - keys are quantized per channel, values per token, to asymmetric 2-bit
 *       codes (a zero point and a scale per group), with no calibration;
 *     - per-channel key statistics need future tokens, so keys are grouped in
 *       blocks of G = 32 or 64 tokens and the block that is not full yet stays
 *       in a full-precision (fp16) residual buffer;
 *     - decode attention reads the 2-bit cache, turning codes back into real
 *       numbers inside the attention computation.
 *   Section "Kod ve Entegrasyon Haritası": multi-query-head (GQA) models are
 *   supported.
 *   "QuantMLA: Düşük Bitli MLA KV Önbellekleme için Fonksiyon Uyumlu Çift
 *   Yollu Kuantizasyon", sections "Giriş ve Problem Analizi" and "QuantMLA
 *   Mimarisi ve Temel Bileşenleri": an MLA cache with a content latent at
 *   INT2 and a decoupled RoPE key at INT4, unpacked and dequantized inside a
 *   native attention kernel.
 *
 * Quantizer (one group of n values x_i, L = 2^bits - 1), computed in IEEE
 * binary32 with no fast-math: mn = min x, mx = max x (after -0 -> +0),
 * scale = (mx - mn) / L (true division), code_i = 0 if scale == 0 else
 * clamp(round_half_even((x_i - mn) / scale), 0, L).  Stored side values are
 * fp16(scale) (round to nearest even) and fp16(mn) (exact).  Dequantized
 * value: code * scale_h + zero_h.
 *
 * Layouts (row-major, last index fastest; "word" = little-endian uint32;
 * code i of a word sits in bits [bits*i, bits*i + bits)):
 *   key stream   (per channel, groups of G tokens, blocks start at token 0)
 *     k_codes  u32  [B][Hkv][max_tokens/G][kd][G*bits/32]
 *              word j of channel c holds tokens (32/bits)*j .. of the block
 *     k_scale, k_zero  fp16 [B][Hkv][max_tokens/G][kd]
 *     k_resid  fp16 [B][Hkv][G][kd]   residual keys, token-major
 *   value stream (per token, groups of Gv channels)
 *     v_codes  u32  [B][Hkv][max_tokens][vd*bits/32]
 *              word j of a token holds channels (32/bits)*j ..
 *     v_scale, v_zero  fp16 [B][Hkv][max_tokens][vd/Gv]
 *   KIVI: kd == vd == head dim; append inputs k, v are fp16 [B][Hkv][n][d];
 *         q is fp16 [B][Hq][d]; out is fp16 [B][Hq][d].
 *   MLA : Hkv == 1; key stream = RoPE key (kd), value stream = content
 *         latent (vd); append inputs k = RoPE [B][n][kd], v = content
 *         [B][n][vd]; q = fp16 [B][Hq][vd + kd] (content part, then RoPE
 *         part); out = fp16 [B][Hq][vd].
 *   Query head h reads KV head floor(h / (Hq / Hkv)).
 *
 * Ownership: the caller owns every device buffer (cache arrays, inputs,
 * outputs, workspace); the library never allocates device memory.  A
 * kvq_cache handle holds the device pointers plus host-side counters (tokens
 * held, quantized key blocks) and is the only host allocation.
 *
 * Errors: every argument is validated on the host before any HIP call; on
 * error nothing is launched and the handle is unchanged.  KVQ_E_HIP reports a
 * launch failure (hipGetLastError).  Faults while a kernel runs surface at the
 * caller's next synchronisation.  Calls are asynchronous on the given HIP
 * stream (hipStream_t passed as void*; NULL = the default stream).  Calls on
 * one handle must be ordered on one stream; a handle is not thread-safe.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
    KVQ_OK = 0,
    KVQ_E_NULL = -1,        /* a required pointer is NULL                    */
    KVQ_E_SHAPE = -2,       /* inconsistent or unsupported dimensions        */
    KVQ_E_ALIGN = -3,       /* a device pointer is not 16-byte aligned       */
    KVQ_E_CAPACITY = -4,    /* tokens would exceed max_tokens / the residual */
    KVQ_E_UNSUPPORTED = -5, /* valid request the library does not implement  */
    KVQ_E_WORKSPACE = -6,   /* workspace smaller than required               */
    KVQ_E_HIP = -7,         /* a HIP launch failed                           */
    KVQ_E_STATE = -8,       /* no tokens to attend over; prefill: not empty  */
    KVQ_E_SCRATCH = -9      /* the partials exceed the static scratch array  */
} kvq_status;

enum { KVQ_KIND_KIVI = 0, KVQ_KIND_MLA = 1 };
enum { KVQ_AXIS_PER_CHANNEL = 0,   /* groups of `group` tokens, one channel */
       KVQ_AXIS_PER_TOKEN = 1 };   /* groups of `group` channels, one token */

/* kv_quantize_append flag: do not quantize a key block when the residual
 * fills; the caller flushes it with kv_flush_residual. */
#define KVQ_APPEND_NO_AUTOFLUSH 1u

typedef struct kvq_stream_cfg {
    int32_t bits;    /* 2 or 4                                     */
    int32_t axis;    /* key stream: PER_CHANNEL, value: PER_TOKEN  */
    int32_t dim;     /* channels of the stream                     */
    int32_t group;   /* key: G tokens; value: Gv channels          */
} kvq_stream_cfg;

typedef struct kvq_cache_cfg {
    int32_t kind;          /* KVQ_KIND_KIVI or KVQ_KIND_MLA            */
    int32_t batch;         /* B                                         */
    int32_t n_kv_heads;    /* Hkv (MLA: 1)                              */
    int32_t reserved;      /* must be 0                                 */
    int64_t max_tokens;    /* capacity per sequence, a multiple of G    */
    kvq_stream_cfg key;    /* MLA: the RoPE key                         */
    kvq_stream_cfg value;  /* MLA: the content latent                   */
} kvq_cache_cfg;

typedef struct kvq_buffer_sizes {   /* bytes of each device array */
    uint64_t k_codes, k_scale, k_zero, k_resid, v_codes, v_scale, v_zero;
} kvq_buffer_sizes;

typedef struct kvq_cache_buffers {  /* caller-owned device arrays, 16-B aligned */
    void *k_codes, *k_scale, *k_zero, *k_resid, *v_codes, *v_scale, *v_zero;
} kvq_cache_buffers;

typedef struct kvq_cache kvq_cache;   /* opaque host handle */

/* Sizes of the seven device arrays for `cfg` (the layouts above).
 * Validates cfg: kind; batch, n_kv_heads >= 1 (MLA: n_kv_heads == 1);
 * bits in {2,4}; key axis PER_CHANNEL with G a multiple of 32/bits and
 * 16 <= G <= 128 and G*bits/32 in {1,2,4,8}; value axis PER_TOKEN with
 * Gv == 32; dims multiples of 32 and <= 512; KIVI: kd == vd; max_tokens >= G
 * and a multiple of G.  Returns KVQ_E_NULL / KVQ_E_SHAPE / KVQ_E_UNSUPPORTED. */
kvq_status kv_cache_buffer_bytes(const kvq_cache_cfg* cfg, kvq_buffer_sizes* out);

/* Create a handle over caller-owned device arrays (sizes from
 * kv_cache_buffer_bytes, 16-byte aligned, contents need not be initialised).
 * The cache starts empty.  Allocates the host handle only. */
kvq_status kv_cache_init(const kvq_cache_cfg* cfg, const kvq_cache_buffers* bufs,
                         kvq_cache** out);

/* Free the host handle (device arrays stay the caller's).  NULL is a no-op. */
void kv_cache_destroy(kvq_cache* cache);

/* Forget every token (host counters only; device contents are left). */
kvq_status kv_cache_reset(kvq_cache* cache);

/* Tokens held, and how many of them are residual (fp16) keys. */
kvq_status kv_cache_state(const kvq_cache* cache, int64_t* n_tokens, int32_t* n_resid);

/* Append n_tokens tokens per sequence ("İddia ve Gerçeklik: KIVI": values
 * quantized per token at once; keys join the residual and every block of G
 * keys that fills is quantized per channel).  k_fp16 / v_fp16 are device
 * arrays in the append layouts above; they are only read.  Without
 * KVQ_APPEND_NO_AUTOFLUSH the residual never holds a full block afterwards;
 * with it, R + n_tokens must be <= G (else KVQ_E_CAPACITY) and a residual
 * that reaches G waits for kv_flush_residual.  n_tokens == 0 is a no-op.
 * Errors: KVQ_E_NULL, KVQ_E_SHAPE (n_tokens < 0), KVQ_E_ALIGN,
 * KVQ_E_CAPACITY (T + n_tokens > max_tokens), KVQ_E_HIP. */
kvq_status kv_quantize_append(kvq_cache* cache, const void* k_fp16, const void* v_fp16,
                              int64_t n_tokens, uint32_t flags, void* hip_stream);

/* Quantize the residual as the next key block if it holds exactly G keys;
 * otherwise do nothing (a partial block is never quantized, which is why the
 * residual exists: "İddia ve Gerçeklik: KIVI" keeps the keys of the group
 * that is not full yet in full precision, since per-channel statistics need
 * all G of its tokens).  It serves appends made with KVQ_APPEND_NO_AUTOFLUSH;
 * the default append flushes by itself.  *n_blocks_flushed (may be NULL)
 * receives 1 or 0.  Errors: KVQ_E_NULL, KVQ_E_HIP. */
kvq_status kv_flush_residual(kvq_cache* cache, void* hip_stream, int32_t* n_blocks_flushed);

/* Split-K: the context is cut into n_splits contiguous token ranges handled
 * by independent workgroups and merged by a second pass.  0 = automatic. */
#define KVQ_MAX_SPLITS 256

/* Workspace bytes kv_decode_attention needs for n_q_heads and n_splits
 * (0 = automatic; the figure covers every cache length up to max_tokens).
 * The matrix-core kernels address one split's codes with 32-bit offsets: an
 * explicit n_splits that would give a split more than 2^30 bytes of key or
 * value codes at full capacity (2^25 tokens at 2 bits, 2^24 at 4 bits, for
 * dim 128) is rejected with KVQ_E_SHAPE; the automatic plan never does.
 * Errors: KVQ_E_NULL, KVQ_E_SHAPE. */
kvq_status kv_decode_workspace_bytes(const kvq_cache* cache, int32_t n_q_heads,
                                     int32_t n_splits, uint64_t* bytes);

/* Decode attention of one query per (sequence, query head) over every token
 * in the cache: logits sigma * q . khat_t over the quantized keys and the
 * fp16 residual keys (MLA: sigma * (q_content . chat_t + q_rope . khat_t)),
 * softmax, weighted sum of the dequantized values (MLA: of chat_t);
 * fp32 accumulation, fp16 output.  The 2-bit codes are unpacked and
 * dequantized inside the QK^T / softmax / PV loop ("İddia ve Gerçeklik:
 * KIVI"; "QuantMLA Mimarisi ve Temel Bileşenleri").  q_fp16, out_fp16 and
 * workspace are caller-owned device arrays, 16-byte aligned.
 * Errors: KVQ_E_NULL, KVQ_E_SHAPE (n_q_heads not a positive multiple of
 * Hkv, n_splits outside [0, KVQ_MAX_SPLITS], or an explicit n_splits whose
 * splits would exceed 2^30 bytes of codes each at the current length, as
 * for kv_decode_workspace_bytes), KVQ_E_ALIGN, KVQ_E_STATE (no tokens),
 * KVQ_E_WORKSPACE, KVQ_E_HIP. */
kvq_status kv_decode_attention(const kvq_cache* cache, const void* q_fp16, int32_t n_q_heads,
                               float softmax_scale, int32_t n_splits, void* out_fp16,
                               void* workspace, uint64_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------ paged cache
 * "Makale Bülteni -- KIVI", section "Kod ve Entegrasyon Haritası": the grouped
 * residual and the asymmetric layout do not fit a serving engine's paged
 * block manager as they are; serving a 2-bit asymmetric cache needs paged
 * 2-bit kernels.  Here a page holds one key block (G tokens, per-channel
 * codes, all KV heads) and the per-token value codes of the same G tokens;
 * each sequence slot keeps its own fp16 residual block.
 *
 * Layouts for P pages (same element types and word packing as above):
 *   k_codes  u32  [P][Hkv][kd][G*bits/32]    k_scale, k_zero fp16 [P][Hkv][kd]
 *   v_codes  u32  [P][Hkv][G][vd*bits/32]    v_scale, v_zero fp16 [P][Hkv][G][vd/Gv]
 *   k_resid  fp16 [B][Hkv][G][kd]            one residual block per sequence slot
 * Caller-owned int32 device arrays passed to each call (4-byte aligned):
 *   block_table [B][max_tokens/G]: page of key block j of sequence b.  The
 *     page of a block must be in the table before the block's first token is
 *     appended (its values go to that page at once).
 *   seq_lens [B]: tokens of sequence b.  Sequences are independent (ragged
 *     lengths); the library never changes these arrays.
 * Device-side entries are not seen by the host: an append skips every
 * sequence whose length, row count or capacity is out of range and every
 * row whose page number is outside [0, P); decode clamps lengths to
 * [0, max_len] and page numbers into [0, P), so bad entries give wrong
 * output but no access outside the arrays.
 * B (batch) in the configuration is the number of sequence slots and
 * max_tokens the capacity of one sequence. */
typedef struct kvq_paged kvq_paged;   /* opaque host handle */

/* Sizes of the seven device arrays of a paged cache with n_pages pages.
 * Validation of cfg as kv_cache_buffer_bytes; n_pages >= 1 (else
 * KVQ_E_SHAPE). */
kvq_status kv_paged_buffer_bytes(const kvq_cache_cfg* cfg, int32_t n_pages, kvq_buffer_sizes* out);

/* Handle over caller-owned paged arrays (sizes from kv_paged_buffer_bytes,
 * 16-byte aligned).  Holds no lengths: those are the caller's device array.
 * Errors: KVQ_E_NULL, KVQ_E_SHAPE, KVQ_E_ALIGN, KVQ_E_UNSUPPORTED. */
kvq_status kv_paged_init(const kvq_cache_cfg* cfg, int32_t n_pages, const kvq_cache_buffers* bufs,
                         kvq_paged** out);

/* Free the host handle.  NULL is a no-op. */
void kv_paged_destroy(kvq_paged* cache);

/* Append rows to every sequence: sequence b takes n_new[b] rows (all n_max
 * when n_new is NULL; 0 <= n_new[b] <= n_max) at tokens seq_lens[b] ..
 * ("İddia ve Gerçeklik: KIVI": values quantized per token at once, into the
 * page of their block; keys join the residual, and every block of G keys
 * that fills is quantized per channel into its page).  k_fp16 / v_fp16 are
 * [B][Hkv][n_max][d] (MLA: [B][n_max][d]).  seq_lens holds the lengths
 * before the append; the caller advances them afterwards.  n_max == 1 (the
 * decode step) is one launch; larger appends two.
 * Errors: KVQ_E_NULL, KVQ_E_SHAPE (n_max < 0), KVQ_E_ALIGN, KVQ_E_CAPACITY
 * (n_max > max_tokens), KVQ_E_HIP. */
kvq_status kv_paged_append(kvq_paged* cache, const void* k_fp16, const void* v_fp16, int32_t n_max,
                           const int32_t* n_new, const int32_t* seq_lens, const int32_t* block_table,
                           void* hip_stream);

/* Workspace bytes kv_paged_decode needs for n_q_heads, the length bound
 * max_len (0 <= max_len <= max_tokens) and n_splits (0 = automatic).
 * Errors: KVQ_E_NULL, KVQ_E_SHAPE. */
kvq_status kv_paged_workspace_bytes(const kvq_paged* cache, int32_t n_q_heads, int32_t max_len,
                                    int32_t n_splits, uint64_t* bytes);

/* Decode attention of one query per (sequence, query head) over the
 * seq_lens[b] tokens of each sequence, as kv_decode_attention computes it
 * for one sequence; max_len (host) bounds every length and sizes the split
 * plan.  A sequence of length 0 gets a zero output.
 * Errors: KVQ_E_NULL, KVQ_E_SHAPE (n_q_heads, n_splits, max_len out of
 * range), KVQ_E_ALIGN, KVQ_E_WORKSPACE, KVQ_E_HIP. */
kvq_status kv_paged_decode(const kvq_paged* cache, const void* q_fp16, int32_t n_q_heads, float softmax_scale,
                           const int32_t* seq_lens, const int32_t* block_table, int32_t max_len,
                           int32_t n_splits, void* out_fp16, void* workspace, uint64_t workspace_bytes,
                           void* hip_stream);

/* kv_paged_decode_step flag: advance seq_lens[b] by the row appended to
 * sequence b, on the device, after the step's reads of it (in the step's
 * last launch).  With it the step's arguments need not change from one step
 * to the next, so a caller can capture the step in a HIP graph and replay it
 * (no memset nodes, no host reads). */
#define KVQ_STEP_ADVANCE_LENGTHS 1u

/* One paged decode step ("Kod ve Entegrasyon Haritası": paged 2-bit
 * kernels for serving; "İddia ve Gerçeklik: KIVI": append and in-loop
 * dequantized attention on the decode path): sequence b with n_new[b] = 1
 * (or n_new NULL) appends one token (k_fp16 / v_fp16 [B][Hkv][1][d]) at
 * token seq_lens[b], then every sequence attends over its tokens, the new
 * one included.  Two launches: the attention kernel's tail workgroup stores
 * the value row and either the residual key or, when the key completes its
 * block, the block quantized per channel (the append kernels' own code), and
 * then attends; the merge follows.  Caches are bit-identical to
 * kv_paged_append + kv_paged_decode over the grown lengths; outputs too,
 * except for a sequence whose block completes in this step (its new block is
 * read on the tail path instead of a matrix-core tile; same tolerance).
 * max_len bounds every length after the step.  Only the shapes with a
 * matrix-core paged kernel (kv_paged_variant "gqa_mfma_paged" or
 * "mha_mfma_paged"); others return KVQ_E_UNSUPPORTED.
 * Errors: KVQ_E_NULL, KVQ_E_SHAPE (n_q_heads, n_splits, max_len, flags),
 * KVQ_E_ALIGN, KVQ_E_WORKSPACE, KVQ_E_UNSUPPORTED, KVQ_E_HIP. */
kvq_status kv_paged_decode_step(kvq_paged* cache, const void* k_fp16, const void* v_fp16, const void* q_fp16,
                                int32_t n_q_heads, float softmax_scale, const int32_t* n_new, int32_t* seq_lens,
                                const int32_t* block_table, int32_t max_len, int32_t n_splits, uint32_t flags,
                                void* out_fp16, void* workspace, uint64_t workspace_bytes, void* hip_stream);

/* Name of the kernel kv_paged_decode would launch (automatic splits). */
const char* kv_paged_variant(const kvq_paged* cache, int32_t n_q_heads, int32_t max_len);

/* One decode step: kv_quantize_append of one token per sequence (k_fp16 /
 * v_fp16 [B][Hkv][1][d], auto-flush) followed by kv_decode_attention, with
 * the same results bit for bit.  When the new key completes no block (G - 1
 * steps in G) and the cache runs the GQA or MHA matrix-core kernel, the
 * append happens inside the attention launch: the workgroup that handles
 * the tokens after the last whole tile stores the new key and value rows
 * (the same value quantizer as the append kernels) and then attends over
 * them, so the step is two launches (attention, merge) instead of three.
 * Otherwise it is the two calls.  ("İddia ve Gerçeklik: KIVI" puts the
 * residual append and the in-loop dequantized attention on the decode
 * path; the source names per-step latency at small batch as KIVI's cost.)
 * Every argument of both halves, the workspace size for the grown cache
 * included, is checked before any HIP call.
 * Errors: those of kv_quantize_append and kv_decode_attention. */
kvq_status kv_decode_step(kvq_cache* cache, const void* k_fp16, const void* v_fp16, const void* q_fp16,
                          int32_t n_q_heads, float softmax_scale, int32_t n_splits, void* out_fp16,
                          void* workspace, uint64_t workspace_bytes, void* hip_stream);

/* kv_prefill_attention flag: attention only; the cache is neither read nor
 * written (any length), e.g. to time the attention without the quantize. */
#define KVQ_PREFILL_ATTENTION_ONLY 1u

/* Prefill of an empty cache ("Makale Bülteni -- KIVI", section "Kod ve
 * Entegrasyon Haritası": the prefill phase runs ordinary attention over the
 * full-precision prompt; the cache is quantized from the same tensors).  One
 * kernel launch computes the causal attention of the n-token prompt,
 *   out[b][h][i] = sum_{j <= i} softmax_j(softmax_scale * q_i . k_j) v_j,
 * query head h reading KV head h / (n_q_heads / n_kv_heads), and appends the
 * prompt's keys and values to the cache exactly as kv_quantize_append(cache,
 * k, v, n, 0) would (every full key block quantized, the rest in the
 * residual; same bits), leaving T = n.
 *   q_fp16   [B][n_q_heads][n][128] (fp16, device, 16-B aligned)
 *   k_fp16, v_fp16 [B][n_kv_heads][n][128] (the kv_quantize_append layout)
 *   out_fp16 [B][n_q_heads][n][128]
 * Weights enter the PV product as fp16 (as FlashAttention does); sums in
 * fp32.  Needs key and value dim 128, key groups of 32 or 64 tokens, 2- or
 * 4-bit codes, 32-channel value groups (else KVQ_E_UNSUPPORTED) and, unless
 * KVQ_PREFILL_ATTENTION_ONLY, an empty cache (else KVQ_E_STATE).
 * Errors: KVQ_E_NULL, KVQ_E_SHAPE (n outside [1, 2^23], n_q_heads, flags,
 * grid limits),
 * KVQ_E_CAPACITY (n > max_tokens), KVQ_E_ALIGN, KVQ_E_STATE,
 * KVQ_E_UNSUPPORTED, KVQ_E_HIP. */
kvq_status kv_prefill_attention(kvq_cache* cache, const void* q_fp16, const void* k_fp16, const void* v_fp16,
                                int64_t n, int32_t n_q_heads, float softmax_scale, uint32_t flags, void* out_fp16,
                                void* hip_stream);

/* Bytes of the static device array (one per GPU, held until the process
 * ends) in which kv_decode_attention_noalloc keeps its split partials. */
#define KVQ_SCRATCH_BYTES (32u << 20)

/* kv_decode_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels, split plan and results bit for bit, with
 * the split partials in the library's static array of KVQ_SCRATCH_BYTES on
 * the current device instead of a caller workspace.  No device memory is
 * allocated or freed.  The array's address is looked up once per device, on
 * the first call made with that device current.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (two streams, two
 * threads) race and must be ordered by the caller.  Nothing needs clearing
 * between calls (each call writes every partial its merge reads).
 * Arguments as kv_decode_attention.  Errors: those of kv_decode_attention
 * except KVQ_E_WORKSPACE, and KVQ_E_SCRATCH when the partials,
 * B * n_q_heads * slots * (vd + 2) * 4 bytes, exceed KVQ_SCRATCH_BYTES
 * (fewer splits, a smaller batch or the workspace entry point then serve). */
kvq_status kv_decode_attention_noalloc(const kvq_cache* cache, const void* q_fp16, int32_t n_q_heads,
                                       float softmax_scale, int32_t n_splits, void* out_fp16, void* hip_stream);

/* Profiling hook: when both are non-NULL (hipEvent_t, created by the caller),
 * later kv_decode_attention / kv_decode_step / kv_paged_decode calls launch their split-K pass-1 kernel with
 * hipExtLaunchKernel so that the launch itself records its start and stop
 * timestamps into ev_before / ev_after (no separate event packets in the
 * stream).  NULL, NULL switches it off.  Process-wide. */
kvq_status kv_set_timing_events(void* ev_before, void* ev_after);

/* Name of the decode kernel variant kv_decode_attention would launch. */
const char* kv_decode_variant(const kvq_cache* cache, int32_t n_q_heads);

/* Static description of a status code (any int: values that are no
 * kvq_status give "unknown status"). */
const char* kvq_status_str(int32_t status);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
