/*
 * kvq_oracle.c -- plain, slow, obviously-correct CPU oracle (TEST
 * INFRASTRUCTURE ONLY; see kvq_oracle.h for who may use it).
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math
 *        -pthread kvq_oracle.c -lm
 * (no contraction into FMA, no reassociation: every fp32 step below is one
 * IEEE-754 binary32 operation in round-to-nearest-even, as written.)
 *
 * Method sources (page title + section):
 *   [KIVI] "Makale Bülteni -- KIVI", lead paragraph and section
 *          "İddia ve Gerçeklik: KIVI".
 *   [QMLA] "QuantMLA: Düşük Bitli MLA KV Önbellekleme için Fonksiyon Uyumlu
 *          Çift Yollu Kuantizasyon", sections "Giriş ve Problem Analizi" and
 *          "QuantMLA Mimarisi ve Temel Bileşenleri".
 */
#define _GNU_SOURCE
#include "kvq_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ fp16 */

float orc_half_to_float(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    uint32_t bits;
    if (e == 0) {                       /* zero / subnormal: m * 2^-24, exact */
        float v = (float)m * (1.0f / 16777216.0f);
        memcpy(&bits, &v, 4);
        bits |= sign;
    } else if (e == 31) {               /* inf / nan */
        bits = sign | 0x7f800000u | (m << 13);
    } else {                            /* normal: re-bias the exponent */
        bits = sign | ((e - 15u + 127u) << 23) | (m << 13);
    }
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

uint16_t orc_float_to_half(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    uint32_t ax = x & 0x7fffffffu;
    if (ax > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);   /* nan */
    if (ax >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);  /* >= 65520 */
    if (ax < 0x38800000u) {             /* below 2^-14: fp16 subnormal range */
        float af;
        memcpy(&af, &ax, 4);
        float units = nearbyintf(af * 16777216.0f);  /* exact scale, then RNE */
        return (uint16_t)(sign | (uint16_t)units);   /* 1024 encodes 2^-14 */
    }
    uint32_t e = (ax >> 23) - 127u + 15u, m = ax & 0x7fffffu;
    uint32_t h = (e << 10) | (m >> 13);
    uint32_t rem = m & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u; /* ties-even */
    return (uint16_t)(sign | h);
}

void orc_half_to_float_n(const uint16_t* h, float* f, int64_t n) {
    for (int64_t i = 0; i < n; ++i) f[i] = orc_half_to_float(h[i]);
}

void orc_float_to_half_n(const float* f, uint16_t* h, int64_t n) {
    for (int64_t i = 0; i < n; ++i) h[i] = orc_float_to_half(f[i]);
}

/* -------------------------------------------------------------- quantizer */

/* [KIVI] asymmetric quantization of one group: zero = group minimum,
 * scale = (max - min) / (2^bits - 1), code = round-half-even((x - min)/scale)
 * clamped to [0, 2^bits - 1].  All of it in binary32; the stored side values
 * are the fp16 roundings of scale and min. */
int orc_quant_group(const uint16_t* x, int64_t n, int64_t stride, int bits,
                    uint8_t* codes, uint16_t* scale_h, uint16_t* zero_h,
                    float* scale32) {
    if (!x || !codes || n <= 0 || (bits != 2 && bits != 4)) return -1;
    const float L = (float)((1 << bits) - 1);
    float mn = 0.0f, mx = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float v = orc_half_to_float(x[i * stride]) + 0.0f;   /* -0 -> +0 */
        if (!isfinite(v)) return -1;
        if (i == 0) { mn = v; mx = v; }
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    float range = mx - mn;
    float scale = range / L;
    for (int64_t i = 0; i < n; ++i) {
        float v = orc_half_to_float(x[i * stride]) + 0.0f;
        uint8_t c = 0;
        if (scale != 0.0f) {
            float d = v - mn;
            float qt = d / scale;
            float r = nearbyintf(qt);          /* ties to even */
            if (r < 0.0f) r = 0.0f;
            if (r > L) r = L;
            c = (uint8_t)r;
        }
        codes[i] = c;
    }
    if (scale_h) *scale_h = orc_float_to_half(scale);
    if (zero_h) *zero_h = orc_float_to_half(mn);
    if (scale32) *scale32 = scale;
    return 0;
}

void orc_pack(const uint8_t* codes, int64_t n, int bits, uint32_t* words) {
    const int per = 32 / bits;
    for (int64_t w = 0; w < n / per; ++w) {
        uint32_t acc = 0;
        for (int i = 0; i < per; ++i)
            acc |= (uint32_t)codes[w * per + i] << (bits * i);
        words[w] = acc;
    }
}

void orc_unpack(const uint32_t* words, int64_t n, int bits, uint8_t* codes) {
    const int per = 32 / bits;
    const uint32_t mask = (1u << bits) - 1u;
    for (int64_t i = 0; i < n; ++i)
        codes[i] = (uint8_t)((words[i / per] >> (bits * (i % per))) & mask);
}

/* [KIVI] keys: one group = one channel over G consecutive tokens of a block;
 * blocks start at token 0; the T mod G trailing tokens stay fp16. */
int64_t orc_quantize_keys(const uint16_t* k, int64_t B, int64_t H, int64_t T,
                          int64_t D, int G, int bits, int64_t nblk_cap,
                          uint32_t* codes, uint16_t* scale, uint16_t* zero,
                          uint16_t* resid) {
    if (!k || B <= 0 || H <= 0 || T < 0 || D <= 0 || G <= 0) return -1;
    if (bits != 2 && bits != 4) return -1;
    if ((G * bits) % 32 != 0) return -1;
    const int64_t W = (int64_t)G * bits / 32;
    const int64_t nblk = T / G, R = T - nblk * G;
    if (nblk > nblk_cap) return -1;
    uint8_t* tmp = (uint8_t*)malloc((size_t)G);
    if (!tmp) return -1;
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const uint16_t* kb = k + bh * T * D;
        for (int64_t blk = 0; blk < nblk; ++blk) {
            for (int64_t c = 0; c < D; ++c) {
                const int64_t side = (bh * nblk_cap + blk) * D + c;
                if (orc_quant_group(kb + blk * G * D + c, G, D, bits, tmp,
                                    &scale[side], &zero[side], NULL)) {
                    free(tmp);
                    return -1;
                }
                orc_pack(tmp, G, bits, codes + side * W);
            }
        }
        for (int64_t r = 0; r < R; ++r)
            for (int64_t c = 0; c < D; ++c)
                resid[(bh * G + r) * D + c] = kb[(nblk * G + r) * D + c];
    }
    free(tmp);
    return R;
}

/* [KIVI] values: one group = one token over Gv consecutive channels. */
int orc_quantize_values(const uint16_t* v, int64_t B, int64_t H, int64_t T,
                        int64_t D, int Gv, int bits, int64_t tok_cap,
                        uint32_t* codes, uint16_t* scale, uint16_t* zero) {
    if (!v || B <= 0 || H <= 0 || T < 0 || D <= 0 || Gv <= 0) return -1;
    if (bits != 2 && bits != 4) return -1;
    if (D % Gv != 0 || (Gv * bits) % 32 != 0 || T > tok_cap) return -1;
    const int64_t WT = D * bits / 32, NG = D / Gv, WG = (int64_t)Gv * bits / 32;
    uint8_t* tmp = (uint8_t*)malloc((size_t)Gv);
    if (!tmp) return -1;
    for (int64_t bh = 0; bh < B * H; ++bh) {
        for (int64_t t = 0; t < T; ++t) {
            const uint16_t* row = v + (bh * T + t) * D;
            for (int64_t g = 0; g < NG; ++g) {
                const int64_t side = (bh * tok_cap + t) * NG + g;
                if (orc_quant_group(row + g * Gv, Gv, 1, bits, tmp,
                                    &scale[side], &zero[side], NULL)) {
                    free(tmp);
                    return -1;
                }
                orc_pack(tmp, Gv, bits, codes + (bh * tok_cap + t) * WT + g * WG);
            }
        }
    }
    free(tmp);
    return 0;
}

/* ---------------------------------------------------------------- dequant */

/* code * scale + zero evaluated in binary64: exact, since the product of a
 * <=4-bit integer and an fp16 value has at most 15 significant bits. */
static int64_t quantized_keys(const orc_cache* c) {
    return (c->kq_blocks < 0 ? c->T / c->kG : c->kq_blocks) * c->kG;
}

static double key_at(const orc_cache* c, int64_t bh, int64_t t, int64_t ch) {
    const int64_t G = c->kG, per = 32 / c->kbits, W = G / per;
    const int64_t Tq = quantized_keys(c);
    if (t >= Tq)
        return (double)orc_half_to_float(c->k_resid[(bh * G + (t - Tq)) * c->kd + ch]);
    const int64_t blk = t / G, i = t % G;
    const int64_t side = (bh * c->nblk_cap + blk) * c->kd + ch;
    const uint32_t w = c->k_codes[side * W + i / per];
    const uint32_t code = (w >> (c->kbits * (i % per))) & ((1u << c->kbits) - 1u);
    return (double)code * (double)orc_half_to_float(c->k_scale[side]) +
           (double)orc_half_to_float(c->k_zero[side]);
}

static double value_at(const orc_cache* c, int64_t bh, int64_t t, int64_t ch) {
    const int64_t per = 32 / c->vbits, WT = c->vd / per, NG = c->vd / c->vG;
    const uint32_t w = c->v_codes[(bh * c->tok_cap + t) * WT + ch / per];
    const uint32_t code = (w >> (c->vbits * (ch % per))) & ((1u << c->vbits) - 1u);
    const int64_t side = (bh * c->tok_cap + t) * NG + ch / c->vG;
    return (double)code * (double)orc_half_to_float(c->v_scale[side]) +
           (double)orc_half_to_float(c->v_zero[side]);
}

static int cache_ok(const orc_cache* c) {
    if (!c || c->B <= 0 || c->H <= 0 || c->T < 0) return 0;
    if (c->T > c->tok_cap || quantized_keys(c) / c->kG > c->nblk_cap) return 0;
    if (c->kq_blocks >= 0 &&
        (c->kq_blocks * c->kG > c->T || c->T - c->kq_blocks * c->kG > c->kG)) return 0;
    if (!c->k_codes || !c->k_scale || !c->k_zero || !c->k_resid) return 0;
    if (!c->v_codes || !c->v_scale || !c->v_zero) return 0;
    return 1;
}

int orc_dequant_keys(const orc_cache* c, int64_t b, int64_t h, double* khat) {
    if (!cache_ok(c) || b < 0 || b >= c->B || h < 0 || h >= c->H) return -1;
    const int64_t bh = b * c->H + h;
    for (int64_t t = 0; t < c->T; ++t)
        for (int64_t ch = 0; ch < c->kd; ++ch) khat[t * c->kd + ch] = key_at(c, bh, t, ch);
    return 0;
}

int orc_dequant_values(const orc_cache* c, int64_t b, int64_t h, double* vhat) {
    if (!cache_ok(c) || b < 0 || b >= c->B || h < 0 || h >= c->H) return -1;
    const int64_t bh = b * c->H + h;
    for (int64_t t = 0; t < c->T; ++t)
        for (int64_t ch = 0; ch < c->vd; ++ch) vhat[t * c->vd + ch] = value_at(c, bh, t, ch);
    return 0;
}

/* -------------------------------------------------------------- attention */

typedef struct {
    const orc_cache* c; const uint16_t* q; int32_t Hq; double sigma;
    const int32_t* pairs; int64_t npairs; double* out; int mla;
    int64_t lo, hi; int err;
} att_job;

/* One (batch, query head): logits over all T tokens (quantized keys first,
 * then the fp16 residual), softmax with the maximum subtracted, weighted sum
 * of dequantized values; everything in binary64. */
static int attend_one(const att_job* J, int64_t b, int64_t hq, double* o, double* s) {
    const orc_cache* c = J->c;
    const int64_t group = J->Hq / c->H;
    const int64_t kvh = hq / group;
    const int64_t bh = b * c->H + kvh;
    const int64_t qd = J->mla ? (c->vd + c->kd) : c->kd;
    const uint16_t* qv = J->q + (b * J->Hq + hq) * qd;
    double mx = -INFINITY;
    for (int64_t t = 0; t < c->T; ++t) {
        double dot = 0.0;
        if (J->mla) {   /* [QMLA] content part uses the latent, RoPE part the key */
            for (int64_t ch = 0; ch < c->vd; ++ch)
                dot += (double)orc_half_to_float(qv[ch]) * value_at(c, bh, t, ch);
            for (int64_t ch = 0; ch < c->kd; ++ch)
                dot += (double)orc_half_to_float(qv[c->vd + ch]) * key_at(c, bh, t, ch);
        } else {
            for (int64_t ch = 0; ch < c->kd; ++ch)
                dot += (double)orc_half_to_float(qv[ch]) * key_at(c, bh, t, ch);
        }
        s[t] = J->sigma * dot;
        if (s[t] > mx) mx = s[t];
    }
    double l = 0.0;
    for (int64_t t = 0; t < c->T; ++t) { s[t] = exp(s[t] - mx); l += s[t]; }
    for (int64_t ch = 0; ch < c->vd; ++ch) o[ch] = 0.0;
    for (int64_t t = 0; t < c->T; ++t)
        for (int64_t ch = 0; ch < c->vd; ++ch) o[ch] += s[t] * value_at(c, bh, t, ch);
    for (int64_t ch = 0; ch < c->vd; ++ch) o[ch] /= l;
    return 0;
}

static void* att_worker(void* arg) {
    att_job* J = (att_job*)arg;
    double* s = (double*)malloc(sizeof(double) * (size_t)(J->c->T > 0 ? J->c->T : 1));
    if (!s) { J->err = -1; return NULL; }
    for (int64_t i = J->lo; i < J->hi; ++i) {
        int64_t b, hq;
        if (J->pairs) { b = J->pairs[2 * i]; hq = J->pairs[2 * i + 1]; }
        else { b = i / J->Hq; hq = i % J->Hq; }
        if (b < 0 || b >= J->c->B || hq < 0 || hq >= J->Hq) { J->err = -1; break; }
        attend_one(J, b, hq, J->out + i * J->c->vd, s);
    }
    free(s);
    return NULL;
}

static int run_attention(const orc_cache* c, const uint16_t* q, int32_t Hq, float sigma,
                         const int32_t* pairs, int64_t npairs, double* out,
                         int nthreads, int mla) {
    if (!cache_ok(c) || !q || !out || Hq <= 0 || Hq % c->H != 0 || c->T <= 0) return -1;
    if (!mla && c->kd != c->vd) return -1;
    if (mla && c->H != 1) return -1;
    const int64_t n = pairs ? npairs : c->B * (int64_t)Hq;
    if (n <= 0) return -1;
    if (nthreads <= 0) nthreads = 1;
    if (nthreads > n) nthreads = (int)n;
    att_job* jobs = (att_job*)calloc((size_t)nthreads, sizeof(att_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return -1; }
    for (int i = 0; i < nthreads; ++i) {
        att_job j = {c, q, Hq, (double)sigma, pairs, n, out, mla,
                     n * i / nthreads, n * (i + 1) / nthreads, 0};
        jobs[i] = j;
    }
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, att_worker, &jobs[i]);
    att_worker(&jobs[0]);
    int err = jobs[0].err;
    for (int i = 1; i < nthreads; ++i) { pthread_join(th[i], NULL); err |= jobs[i].err; }
    free(jobs);
    free(th);
    return err ? -1 : 0;
}

int orc_attention_kivi(const orc_cache* c, const uint16_t* q, int32_t Hq, float sigma,
                       const int32_t* pairs, int64_t npairs, double* out, int nthreads) {
    return run_attention(c, q, Hq, sigma, pairs, npairs, out, nthreads, 0);
}

int orc_attention_mla(const orc_cache* c, const uint16_t* q, int32_t Hq, float sigma,
                      const int32_t* pairs, int64_t npairs, double* out, int nthreads) {
    return run_attention(c, q, Hq, sigma, pairs, npairs, out, nthreads, 1);
}

/* ---------------------------------------------------------- prefill attention
 * "Makale Bülteni -- KIVI", section "Kod ve Entegrasyon Haritası": in the
 * prefill phase KIVI runs ordinary attention over the prompt's full-precision
 * keys and values (a FlashAttention kernel there); the cache is quantized from
 * those same fp16 tensors.  This is that attention written out: causal, every
 * query position i of a prompt attends to positions 0..i, query head h to KV
 * head h / (Hq / Hkv), in binary64 over the fp16 inputs. */

typedef struct {
    const uint16_t *q, *k, *v; int64_t Hq, Hkv, T; int32_t d, dv; double sigma;
    const int64_t* rows; int64_t lo, hi; double* out; int err;
} pf_job;

static void* pf_worker(void* arg) {
    pf_job* J = (pf_job*)arg;
    double* s = (double*)malloc(sizeof(double) * (size_t)J->T);
    if (!s) { J->err = -1; return NULL; }
    const int64_t group = J->Hq / J->Hkv;
    for (int64_t r = J->lo; r < J->hi; ++r) {
        const int64_t b = J->rows[3 * r], h = J->rows[3 * r + 1], i = J->rows[3 * r + 2];
        if (b < 0 || h < 0 || h >= J->Hq || i < 0 || i >= J->T) { J->err = -1; break; }
        const int64_t kvh = h / group;
        const uint16_t* qi = J->q + ((b * J->Hq + h) * J->T + i) * J->d;
        const uint16_t* kb = J->k + (b * J->Hkv + kvh) * J->T * J->d;
        const uint16_t* vb = J->v + (b * J->Hkv + kvh) * J->T * J->dv;
        double mx = -INFINITY;
        for (int64_t j = 0; j <= i; ++j) {
            double dot = 0.0;
            for (int32_t c = 0; c < J->d; ++c)
                dot += (double)orc_half_to_float(qi[c]) * (double)orc_half_to_float(kb[j * J->d + c]);
            s[j] = J->sigma * dot;
            if (s[j] > mx) mx = s[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j <= i; ++j) { s[j] = exp(s[j] - mx); l += s[j]; }
        double* o = J->out + r * J->dv;
        for (int32_t c = 0; c < J->dv; ++c) o[c] = 0.0;
        for (int64_t j = 0; j <= i; ++j)
            for (int32_t c = 0; c < J->dv; ++c) o[c] += s[j] * (double)orc_half_to_float(vb[j * J->dv + c]);
        for (int32_t c = 0; c < J->dv; ++c) o[c] /= l;
    }
    free(s);
    return NULL;
}

int orc_prefill_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B, int64_t Hq,
                          int64_t Hkv, int64_t T, int32_t d, int32_t dv, double sigma, const int64_t* rows,
                          int64_t nrows, double* out, int nthreads) {
    if (!q || !k || !v || !rows || !out || B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || T <= 0 ||
        d <= 0 || dv <= 0 || nrows <= 0)
        return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[3 * r] >= B) return -1;
    if (nthreads <= 0) nthreads = 1;
    if (nthreads > nrows) nthreads = (int)nrows;
    pf_job* jobs = (pf_job*)calloc((size_t)nthreads, sizeof(pf_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return -1; }
    for (int t = 0; t < nthreads; ++t) {
        pf_job j = {q, k, v, Hq, Hkv, T, d, dv, sigma, rows, nrows * t / nthreads, nrows * (t + 1) / nthreads, out, 0};
        jobs[t] = j;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, pf_worker, &jobs[t]);
    pf_worker(&jobs[0]);
    int err = jobs[0].err;
    for (int t = 1; t < nthreads; ++t) { pthread_join(th[t], NULL); err |= jobs[t].err; }
    free(jobs);
    free(th);
    return err ? -1 : 0;
}
