/*
 * kvq_oracle.h -- plain, slow CPU oracle for KIVI-style asymmetric low-bit
 * KV-cache quantization and decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (libkvq.so and its Python binding) never links, loads or calls it, and this
 * code shares nothing with the HIP implementation.
 *
 * What it follows (page titles and sections of the source pages):
 *   - "Makale Bülteni -- KIVI" (cmlonder.com paper-to-prod), lead paragraph and
 *     section "İddia ve Gerçeklik: KIVI": keys are quantized per channel,
 *     values per token, asymmetric (min/zero + scale) 2-bit codes; keys are
 *     grouped over G = 32 or 64 tokens and the not-yet-full last group stays
 *     in a full-precision residual buffer.
 *   - "QuantMLA: Düşük Bitli MLA KV Önbellekleme için Fonksiyon Uyumlu Çift
 *     Yollu Kuantizasyon", sections "Giriş ve Problem Analizi" and "QuantMLA
 *     Mimarisi ve Temel Bileşenleri": an MLA cache holds a content latent and
 *     a decoupled RoPE key on two paths, content at INT2 and RoPE key at INT4.
 * The pages give no formulas; the readings used here (min-max asymmetric
 * quantizer with fp32 IEEE division, round-half-even, fp16 side arrays,
 * LSB-first packing, etc.) are listed in the repository's design notes.
 *
 * All fp16 data is passed as raw IEEE binary16 bit patterns (uint16_t).
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* exact binary16 -> binary32 */
float orc_half_to_float(uint16_t h);
/* binary32 -> binary16, round to nearest, ties to even (overflow -> inf) */
uint16_t orc_float_to_half(float f);
/* element-wise array forms of the two conversions */
void orc_half_to_float_n(const uint16_t* h, float* f, int64_t n);
void orc_float_to_half_n(const float* f, uint16_t* h, int64_t n);

/* Quantize one group of n fp16 values read at `stride` (elements).
 * L = 2^bits - 1.  Writes n codes (0..L), the fp16 scale and zero, and the
 * fp32 scale the codes were computed with.  Returns 0, or -1 on bad args /
 * non-finite input. */
int orc_quant_group(const uint16_t* x, int64_t n, int64_t stride, int bits,
                    uint8_t* codes, uint16_t* scale_h, uint16_t* zero_h,
                    float* scale32);

/* Pack codes LSB-first into 32-bit words: 32/bits codes per word.
 * n must be a multiple of 32/bits. */
void orc_pack(const uint8_t* codes, int64_t n, int bits, uint32_t* words);
void orc_unpack(const uint32_t* words, int64_t n, int bits, uint8_t* codes);

/* Key stream, per channel over blocks of G tokens (G tokens aligned to token 0).
 *   k      : fp16 [B][H][T][D]
 *   codes  : u32  [B][H][nblk_cap][D][G*bits/32]   (word j of channel c holds
 *            tokens (32/bits)*j .. of the block, LSB first)
 *   scale, zero : fp16 [B][H][nblk_cap][D]
 *   resid  : fp16 [B][H][G][D]  (tokens floor(T/G)*G .. T-1, token-major)
 * Returns R = T mod G (>= 0) or -1 on error. Untouched entries are left as is. */
int64_t orc_quantize_keys(const uint16_t* k, int64_t B, int64_t H, int64_t T,
                          int64_t D, int G, int bits, int64_t nblk_cap,
                          uint32_t* codes, uint16_t* scale, uint16_t* zero,
                          uint16_t* resid);

/* Value stream, per token over groups of Gv consecutive channels.
 *   v      : fp16 [B][H][T][D]
 *   codes  : u32  [B][H][tok_cap][D*bits/32]  (word j holds channels
 *            (32/bits)*j .., LSB first)
 *   scale, zero : fp16 [B][H][tok_cap][D/Gv]
 * Returns 0 or -1. */
int orc_quantize_values(const uint16_t* v, int64_t B, int64_t H, int64_t T,
                        int64_t D, int Gv, int bits, int64_t tok_cap,
                        uint32_t* codes, uint16_t* scale, uint16_t* zero);

/* A quantized cache as the oracle reads it (same layouts as above). */
typedef struct orc_cache {
    int64_t B, H, T;          /* batch, kv heads, tokens held */
    int64_t kq_blocks;        /* quantized key blocks; keys from kq_blocks*kG
                                 on are fp16 residual keys (at most kG of
                                 them); -1 means floor(T / kG)                */
    int64_t nblk_cap, tok_cap;/* capacities of the block and token axes   */
    int32_t kd, kG, kbits;    /* key stream: dim, token group, bits       */
    int32_t vd, vG, vbits;    /* value stream: dim, channel group, bits   */
    const uint32_t* k_codes; const uint16_t* k_scale; const uint16_t* k_zero;
    const uint16_t* k_resid;
    const uint32_t* v_codes; const uint16_t* v_scale; const uint16_t* v_zero;
} orc_cache;

/* Dequantized key / value rows of one (b, h) in fp64:
 *   khat: [T][kd], vhat: [T][vd] */
int orc_dequant_keys(const orc_cache* c, int64_t b, int64_t h, double* khat);
int orc_dequant_values(const orc_cache* c, int64_t b, int64_t h, double* vhat);

/* KIVI decode attention, fp64.
 *   q   : fp16 [B][Hq][kd] (kd == vd)
 *   out : fp64 [npairs][vd] if pairs != NULL, else [B][Hq][vd]
 *   pairs: optional list of (b, query head) pairs, 2*npairs int32
 * Query head h reads KV head h / (Hq/H).  nthreads <= 0 -> 1. */
int orc_attention_kivi(const orc_cache* c, const uint16_t* q, int32_t Hq,
                       float sigma, const int32_t* pairs, int64_t npairs,
                       double* out, int nthreads);

/* MLA absorbed decode attention, fp64.  H must be 1; the value stream is the
 * content latent (vd), the key stream is the RoPE key (kd).
 *   q   : fp16 [B][Hq][vd + kd]   (content part, then RoPE part)
 *   out : fp64 [npairs][vd] or [B][Hq][vd]
 * logit_t = sigma * (q_c . chat_t + q_r . khat_t), out = sum_t p_t chat_t. */
int orc_attention_mla(const orc_cache* c, const uint16_t* q, int32_t Hq,
                      float sigma, const int32_t* pairs, int64_t npairs,
                      double* out, int nthreads);

/* Causal prefill attention in fp64 over fp16 prompt tensors ("Makale Bülteni
 * -- KIVI", section "Kod ve Entegrasyon Haritası": ordinary attention over the
 * full-precision prompt in the prefill phase).
 *   q : fp16 [B][Hq][T][d], k : fp16 [B][Hkv][T][d], v : fp16 [B][Hkv][T][dv]
 *   rows : nrows triples (b, h, i); out : fp64 [nrows][dv]
 * out = sum_{j <= i} exp(s_j - max) v_j / sum_{j <= i} exp(s_j - max) with
 * s_j = sigma * q_i . k_j, KV head h / (Hq / Hkv).  Returns 0, or -1 on a bad
 * argument or row. */
int orc_prefill_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B, int64_t Hq,
                          int64_t Hkv, int64_t T, int32_t d, int32_t dv, double sigma, const int64_t* rows,
                          int64_t nrows, double* out, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
