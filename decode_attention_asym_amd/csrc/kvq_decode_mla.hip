// kvq_decode_mla.hip -- split-K decode attention on MFMA for absorbed MLA
// caches: one latent KV head shared by 64 or 128 query heads; a 512-dim
// content latent in 2-bit per-token codes (32-channel groups) that serves as
// both key and value, and a 64-dim decoupled RoPE key in 4-bit per-channel
// codes over 64-token blocks (fp16 for the block that is not yet full).
//
// Method ("QuantMLA: Düşük Bitli MLA KV Önbellekleme için Fonksiyon Uyumlu
// Çift Yollu Kuantizasyon", sections "Giriş ve Problem Analizi" and "QuantMLA
// Mimarisi ve Temel Bileşenleri"): the content and RoPE caches are separate
// low-bit paths, unpacked and dequantized inside the attention kernel;
// logit = sigma (q_c . c_hat + q_r . k_hat_r), out = sum_t p_t c_hat_t (the
// absorbed form, the up-projection lies outside this kernel).  The per-token
// content quantizer and per-channel key quantizer are KIVI's ("Makale
// Bülteni -- KIVI", section "İddia ve Gerçeklik: KIVI").
//
// Every content element is reused by the 64 query heads of a workgroup, so
// it is dequantized once per workgroup and both contractions run on the
// matrix cores (128 heads take two workgroups):
//  * wave w owns latent channels [128w, 128w + 128).  Per 16-token tile it
//    dequantizes them (codes as exact fp16 integers via an exponent trick:
//    (bits & mask) | exponent(2^(10-2u)) is 2^(10-2u) + code), computing
//    c_hat = code * s + z with one fused fp16 FMA (the correctly rounded hi)
//    and the remainder c_hat - hi in fp32 (lo);
//  * QK^T: wave w takes 16 of the group's query heads over all 512 channels, reading the token-major hi copy of the whole tile from LDS
//    (v_mfma_f32_16x16x32_f16; Q stays in registers).  The RoPE term uses
//    exact 4-bit code operands (fp16 subnormals) against q' = q_r * s_k in
//    hi/lo rows plus the bias sum_c q_r z_k, or the fp16 residual keys;
//  * online softmax per head in log2 units (lazily moved maxima); the
//    weights go to LDS in fp16 and the row sums add up the same fp16 values;
//  * PV: O[heads][own channels] += P . (hi + lo) on v_mfma_f32_32x32x16_f16,
//    the accumulators in AGPRs.
// Tokens at or past T in the last tile get zero weight; their codes are read
// (they lie inside the caller's capacity) but never contribute.
#include <hip/hip_fp16.h>
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int VD = 512;      // content latent dim
constexpr int KD = 64;       // RoPE dim
constexpr int QD = VD + KD;  // query row
constexpr int GR = 64;       // RoPE key block (tokens)
constexpr int CHS = 260;     // dwords per token row of the hi tile (512 fp16 + pad)
constexpr int RCS = 68;      // dwords per word row of the RoPE code block (64 + pad)
constexpr int QRS = 36;      // dwords per head row of q' (64 fp16 + pad)
constexpr int PS = 12;       // dwords per head row of P (16 fp16 + pad)
constexpr float TAU = 8.0f;  // lazy-rescale threshold (log2 units)

struct MlaParams {
    const uint32_t* kc;          // RoPE codes [B][nblk_cap][64][8]
    const uint16_t *ks, *kz, *kr;
    const uint32_t* vc;          // content codes [B][cap][32]
    const uint16_t *vs, *vz;     // content side [B][cap][16]
    const uint16_t* q;           // [B][Hq][576]
    float *ws_acc, *ws_ml;
    int Hq, S, ntiles;           // ntiles = ceil(T / 16)
    int64_t T, nblk, cap, nblk_cap;
    float sigma2;                // softmax scale * log2(e)
};

template <int HQ>
struct Lds {
    uint32_t chi[16 * CHS];                        // content hi, token-major [token][512 fp16]
    uint32_t cst[4][8 * 16];                       // per wave: content codes [word][token]
    uint32_t sst[4][2 * 4 * 8];                    // per wave: content [scale|zero][group][16 fp16]
    uint32_t rc[8 * RCS];                          // RoPE codes of the block [word][channel]
    uint32_t rs[2 * 32];                           // RoPE [scale|zero][64 fp16]
    __attribute__((aligned(16))) uint32_t qr[HQ * 32];     // q_r fp16 [head][64]
    __attribute__((aligned(16))) uint32_t qrh[HQ * QRS];   // q' = q_r * s_k, hi [head][64 fp16]
    __attribute__((aligned(16))) uint32_t qrl[HQ * QRS];   // lo
    float rbp[256 / HQ][HQ];                       // partial sums q_r . z_k [channel chunk][head]
    __attribute__((aligned(16))) uint32_t pm[HQ * PS];     // weights fp16 [head][16 tokens]
    float alpha[HQ];                               // rescale factors of this tile
    int wflag[4];                                  // wave w moved some maxima this tile
};

__device__ __forceinline__ float lo_h(uint32_t w) { return float(__builtin_bit_cast(f16x2, w)[0]); }
__device__ __forceinline__ float hi_h(uint32_t w) { return float(__builtin_bit_cast(f16x2, w)[1]); }
__device__ __forceinline__ f16x8 as_f16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(f16x8, v);
}
__device__ __forceinline__ f16x8 as_f16x8(uint4 v) { return as_f16x8(v.x, v.y, v.z, v.w); }
__device__ __forceinline__ uint32_t pk_rtz(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}
__device__ __forceinline__ void split_prod2(float a0, float b0, float a1, float b1, uint32_t& hi,
                                            uint32_t& lo) {
    hi = pk_rtz(fmaf(a0, b0, 0.0f), fmaf(a1, b1, 0.0f));
    lo = pk_rtz(fmaf(a0, b0, -lo_h(hi)), fmaf(a1, b1, -hi_h(hi)));
}
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                 0xf, 0xf, false));
}
// over the 16 lanes of a row (quad xor 1, quad xor 2, half-row mirror, row mirror)
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp<0xb1>(x));
    x = fmaxf(x, dpp<0x4e>(x));
    x = fmaxf(x, dpp<0x141>(x));
    return fmaxf(x, dpp<0x140>(x));
}
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp<0xb1>(x);
    x += dpp<0x4e>(x);
    x += dpp<0x141>(x);
    return x + dpp<0x140>(x);
}
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}
// byte k of `lo_word` -> byte 0, of `hi_word` -> byte 2, bytes 1 and 3 zero
__device__ __forceinline__ uint32_t byte_pair_sel(int k) {
    return uint32_t(k) | (0x0cu << 8) | ((4u + uint32_t(k)) << 16) | (0x0cu << 24);
}

// fp16 pair c_hat = code * s + z, rounded once (fused), and its fp32 remainder.
// `h` holds (2^(10-2u) + code) in each half, `bias2` the pair (-2^(10-2u)).
__device__ __forceinline__ void dequant_pair(uint32_t h, uint32_t bias2, uint32_t s, uint32_t z,
                                             uint32_t& hi, uint32_t& lo) {
    const f16x2 c = __builtin_bit_cast(f16x2, h) + __builtin_bit_cast(f16x2, bias2);  // exact codes
    const f16x2 sv = __builtin_bit_cast(f16x2, s), zv = __builtin_bit_cast(f16x2, z);
    const f16x2 hv = __builtin_elementwise_fma(c, sv, zv);
    hi = __builtin_bit_cast(uint32_t, hv);
    const float d0 = fmaf(float(c[0]), float(sv[0]), float(zv[0]));
    const float d1 = fmaf(float(c[1]), float(sv[1]), float(zv[1]));
    lo = pk_rtz(d0 - float(hv[0]), d1 - float(hv[1]));
}

template <int HQ>
__global__ __launch_bounds__(256) void k_decode_mla(MlaParams p) {
    constexpr int QM = HQ / 64;      // 16-head MFMA rows per wave in QK^T
    constexpr int PM = HQ / 32;      // 32-head MFMA rows in PV
    constexpr int HW = HQ / 4;       // query heads per wave in QK^T
    constexpr int NC = 256 / HQ;     // RoPE channel chunks when forming q' (one head per thread)
    constexpr int CW = KD / NC;      // channels per chunk
    __shared__ Lds<HQ> L;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, kg = lane >> 4;        // 16x16x32 operand layout
    const int c32 = lane & 31, h32 = lane >> 5;     // 32x32x16 operand layout
    const int s = blockIdx.x, b = blockIdx.y;   // blockIdx.z: group of HQ query heads
    const int t_lo = int(int64_t(s) * p.ntiles / p.S);
    const int t_hi = int(int64_t(s + 1) * p.ntiles / p.S);
    const int hw0 = wave * HW;
    const int64_t qrow0 = int64_t(b) * p.Hq + int64_t(blockIdx.z) * HQ;

    // ---- q_r to LDS; this wave's content query rows as MFMA A operands
    for (int i = tid; i < HQ * 32; i += 256)
        L.qr[i] = reinterpret_cast<const uint32_t*>(p.q + (qrow0 + i / 32) * QD + VD)[i % 32];
    f16x8 QA[QM][16];
#pragma unroll
    for (int m = 0; m < QM; ++m)
#pragma unroll
        for (int ks = 0; ks < 16; ++ks)
            QA[m][ks] = as_f16x8(*reinterpret_cast<const uint4*>(
                p.q + (qrow0 + hw0 + 16 * m + n) * QD + 32 * ks + 8 * kg));

    f32x16 O[PM][4];
#pragma unroll
    for (int pm = 0; pm < PM; ++pm)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 16; ++e) O[pm][u][e] = 0.0f;
    // softmax state of rows (heads) hw0 + 16m + 4kg + j, this lane's column share
    float mrun[QM][4], lrun[QM][4];
#pragma unroll
    for (int m = 0; m < QM; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            mrun[m][j] = -INFINITY;
            lrun[m][j] = 0.0f;
        }

    // content tile loads (one ahead): codes of token t0 + (lane >> 2), words
    // 8w + 2(lane & 3), +1; side: scale (lanes < 32) / zero of token
    // t0 + ((lane >> 1) & 15), groups 4w + 2(lane & 1), +1
    const uint32_t* vcb = p.vc + int64_t(b) * p.cap * 32 + 8 * wave + 2 * (lane & 3);
    const uint16_t* vsb = (lane < 32 ? p.vs : p.vz) + int64_t(b) * p.cap * 16 + 4 * wave + 2 * (lane & 1);
    auto load_content = [&](int tile, uint2& cw, uint32_t& sw) {
        const int64_t t0 = int64_t(tile) * 16;
        cw = *reinterpret_cast<const uint2*>(vcb + (t0 + (lane >> 2)) * 32);
        sw = *reinterpret_cast<const uint32_t*>(vsb + (t0 + ((lane >> 1) & 15)) * 16);
    };
    // RoPE block loads: codes u32 pair 2*tid of the block; side (tid < 64)
    auto load_rope = [&](int64_t blk, uint2& rw, uint32_t& rsw) {
        rw = reinterpret_cast<const uint2*>(p.kc + (int64_t(b) * p.nblk_cap + blk) * GR * 8)[tid];
        rsw = tid < 64 ? reinterpret_cast<const uint32_t*>((tid < 32 ? p.ks : p.kz) +
                                                           (int64_t(b) * p.nblk_cap + blk) * KD)[tid & 31]
                       : 0u;
    };
    uint2 cw_n;
    uint32_t sw_n;
    load_content(t_lo, cw_n, sw_n);
    uint2 rw_n = make_uint2(0u, 0u);
    uint32_t rsw_n = 0u;
    if (int64_t(t_lo) * 16 / GR < p.nblk) load_rope(int64_t(t_lo) * 16 / GR, rw_n, rsw_n);
    __syncthreads();

    const uint32_t csel = byte_pair_sel(c32 & 3);         // content: byte of the lane's channels
    const uint32_t rsel = byte_pair_sel((n & 7) >> 1);    // RoPE: byte of the lane's token
    int64_t cur_blk = -1;

    for (int i = t_lo; i < t_hi; ++i) {
        const int64_t t0 = int64_t(i) * 16;
        const int64_t blk = t0 / GR;
        const bool qrope = blk < p.nblk;

        // ---- A0: entering a quantized RoPE block: codes, side, q' and bias
        if (qrope && blk != cur_blk) {
            L.rc[(2 * (tid & 3)) * RCS + (tid >> 2)] = rw_n.x;
            L.rc[(2 * (tid & 3) + 1) * RCS + (tid >> 2)] = rw_n.y;
            if (tid < 64) L.rs[tid] = rsw_n;
            cur_blk = blk;
            if (blk + 1 < p.nblk && (blk + 1) * GR < int64_t(t_hi) * 16) load_rope(blk + 1, rw_n, rsw_n);
            __syncthreads();
            const int h = tid % HQ, c0 = (tid / HQ) * CW;
            float bp = 0.0f;
#pragma unroll
            for (int k = 0; k < CW / 2; ++k) {
                const int cp = c0 / 2 + k;                      // channel pair
                const uint32_t qv = L.qr[h * 32 + cp], sv = L.rs[cp], zv = L.rs[32 + cp];
                uint32_t hi, lo;
                split_prod2(lo_h(qv), lo_h(sv), hi_h(qv), hi_h(sv), hi, lo);
                L.qrh[h * QRS + cp] = hi;
                L.qrl[h * QRS + cp] = lo;
                bp = fmaf(lo_h(qv), lo_h(zv), bp);
                bp = fmaf(hi_h(qv), hi_h(zv), bp);
            }
            L.rbp[tid / HQ][h] = bp;
        }

        // ---- A1: stage this wave's content codes and side values
        {
            const uint2 cw = cw_n;
            const uint32_t sw = sw_n;
            if (i + 1 < t_hi) load_content(i + 1, cw_n, sw_n);
            uint32_t* cs = L.cst[wave];
            cs[(2 * (lane & 3)) * 16 + (lane >> 2)] = cw.x;
            cs[(2 * (lane & 3) + 1) * 16 + (lane >> 2)] = cw.y;
            uint16_t* ss = reinterpret_cast<uint16_t*>(L.sst[wave]);
            const int sz = lane >> 5, tl = (lane >> 1) & 15, g0 = 2 * (lane & 1);
            ss[(sz * 4 + g0) * 16 + tl] = uint16_t(sw & 0xffffu);
            ss[(sz * 4 + g0 + 1) * 16 + tl] = uint16_t(sw >> 16);
        }
        wave_sync();

        // ---- A2: dequantize channels 128w + 4*c32 + u (u = 0..3) of tokens
        // 8*h32 .. 8*h32 + 7: PV operands hi/lo (token pairs per register) and
        // the token-major hi copy
        uint32_t PH[4][4], PL[4][4];   // [u][token pair]
        {
            const uint32_t* cs = L.cst[wave] + (c32 >> 2) * 16 + 8 * h32;
            const uint4 wa = *reinterpret_cast<const uint4*>(cs);
            const uint4 wb = *reinterpret_cast<const uint4*>(cs + 4);
            const uint32_t x[4] = {__builtin_amdgcn_perm(wa.y, wa.x, csel), __builtin_amdgcn_perm(wa.w, wa.z, csel),
                                   __builtin_amdgcn_perm(wb.y, wb.x, csel), __builtin_amdgcn_perm(wb.w, wb.z, csel)};
            const uint32_t* sp = L.sst[wave] + (c32 >> 3) * 8 + 4 * h32;
            const uint4 sv = *reinterpret_cast<const uint4*>(sp);
            const uint4 zv = *reinterpret_cast<const uint4*>(sp + 32);
            uint32_t sa[4] = {sv.x, sv.y, sv.z, sv.w}, za[4] = {zv.x, zv.y, zv.z, zv.w};
            if (t0 + 16 > p.T) {
                // tokens at or past T: scale and zero 0, so every value is 0
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2) {
                    const int64_t ta = t0 + 8 * h32 + 2 * q2;
                    const uint32_t keep = (ta < p.T ? 0x0000ffffu : 0u) | (ta + 1 < p.T ? 0xffff0000u : 0u);
                    sa[q2] &= keep;
                    za[q2] &= keep;
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t ex = uint32_t(25 - 2 * u) << 10;   // exponent of 2^(10-2u)
                const uint32_t mk = 0x00030003u << (2 * u);
                const uint32_t e2 = ex | (ex << 16);
                const uint32_t nb = e2 | 0x80008000u;             // (-2^(10-2u)) pair
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2)
                    dequant_pair((x[q2] & mk) | e2, nb, sa[q2], za[q2], PH[u][q2], PL[u][q2]);
            }
            // token-major: token 8*h32 + 2*q2 (+1), channels 4*c32 .. 4*c32 + 3
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
                const uint32_t a0 = __builtin_amdgcn_perm(PH[1][q2], PH[0][q2], 0x05040100u);
                const uint32_t a1 = __builtin_amdgcn_perm(PH[3][q2], PH[2][q2], 0x05040100u);
                const uint32_t b0 = __builtin_amdgcn_perm(PH[1][q2], PH[0][q2], 0x07060302u);
                const uint32_t b1 = __builtin_amdgcn_perm(PH[3][q2], PH[2][q2], 0x07060302u);
                uint32_t* row = L.chi + (8 * h32 + 2 * q2) * CHS + 64 * wave + 2 * c32;
                *reinterpret_cast<uint2*>(row) = make_uint2(a0, a1);
                *reinterpret_cast<uint2*>(row + CHS) = make_uint2(b0, b1);
            }
        }
        __syncthreads();   // hi tile, q' and bias complete

        // ---- B: logits of heads hw0 .. hw0 + HW - 1, online softmax, weights to LDS
        {
            f32x4 Sc[QM], Sr[QM];
#pragma unroll
            for (int m = 0; m < QM; ++m) {
                Sc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
                Sr[m] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) {
                const f16x8 Bv = as_f16x8(*reinterpret_cast<const uint4*>(L.chi + n * CHS + 16 * ks + 4 * kg));
#pragma unroll
                for (int m = 0; m < QM; ++m)
                    Sc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(QA[m][ks], Bv, Sc[m], 0, 0, 0);
            }
            float rf = 1.0f;   // scale of the RoPE partial logits of this lane's column
            if (qrope) {
                const int wr = 2 * int((t0 % GR) / 16) + (n >> 3);   // code word of token n
                const uint32_t nm = (n & 1) ? 0x00f000f0u : 0x000f000fu;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const uint32_t* src = L.rc + wr * RCS + 32 * ks + 8 * kg;
                    const uint4 w0 = *reinterpret_cast<const uint4*>(src);
                    const uint4 w1 = *reinterpret_cast<const uint4*>(src + 4);
                    const f16x8 Bv = as_f16x8(__builtin_amdgcn_perm(w0.y, w0.x, rsel) & nm,
                                              __builtin_amdgcn_perm(w0.w, w0.z, rsel) & nm,
                                              __builtin_amdgcn_perm(w1.y, w1.x, rsel) & nm,
                                              __builtin_amdgcn_perm(w1.w, w1.z, rsel) & nm);
#pragma unroll
                    for (int m = 0; m < QM; ++m) {
                        const int hr = hw0 + 16 * m + n;
                        const f16x8 Ah = as_f16x8(*reinterpret_cast<const uint4*>(L.qrh + hr * QRS + 16 * ks + 4 * kg));
                        const f16x8 Al = as_f16x8(*reinterpret_cast<const uint4*>(L.qrl + hr * QRS + 16 * ks + 4 * kg));
                        Sr[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Bv, Sr[m], 0, 0, 0);
                        Sr[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, Bv, Sr[m], 0, 0, 0);
                    }
                }
                rf = __builtin_ldexpf(1.0f, (n & 1) ? 20 : 24);
            } else {
                // residual keys, fp16: row t0 + n - nblk*64 of the residual
                const int64_t r = t0 + n - p.nblk * GR;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    uint4 kv = make_uint4(0u, 0u, 0u, 0u);
                    if (r < GR && t0 + n < p.T)
                        kv = *reinterpret_cast<const uint4*>(p.kr + (int64_t(b) * GR + r) * KD + 32 * ks + 8 * kg);
                    const f16x8 Bv = as_f16x8(kv);
#pragma unroll
                    for (int m = 0; m < QM; ++m) {
                        const int hr = hw0 + 16 * m + n;
                        const f16x8 Aq = as_f16x8(*reinterpret_cast<const uint4*>(L.qr + hr * 32 + 16 * ks + 4 * kg));
                        Sr[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aq, Bv, Sr[m], 0, 0, 0);
                    }
                }
            }
            const bool valid = t0 + n < p.T;
            float x[QM][4];
            bool over = false;
#pragma unroll
            for (int m = 0; m < QM; ++m)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int h = hw0 + 16 * m + 4 * kg + j;
                    float bias = 0.0f;
                    if (qrope) {
#pragma unroll
                        for (int cc = 0; cc < NC; ++cc) bias += L.rbp[cc][h];
                    }
                    const float lg = (Sc[m][j] + fmaf(Sr[m][j], rf, bias)) * p.sigma2;
                    x[m][j] = valid ? lg : -INFINITY;
                    over = over || x[m][j] > mrun[m][j] + TAU;
                }
            const bool moved = __builtin_amdgcn_ballot_w64(over) != 0;
            if (moved) {
#pragma unroll
                for (int m = 0; m < QM; ++m)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float mn = fmaxf(mrun[m][j], row_max16(x[m][j]));
                        const float a = __builtin_amdgcn_exp2f(mrun[m][j] - mn);
                        mrun[m][j] = mn;
                        lrun[m][j] *= a;
                        if (n == 0) L.alpha[hw0 + 16 * m + 4 * kg + j] = a;
                    }
            }
            if (lane == 0) L.wflag[wave] = moved ? 1 : 0;
            uint16_t* pw = reinterpret_cast<uint16_t*>(L.pm);
#pragma unroll
            for (int m = 0; m < QM; ++m)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float pv = valid ? __builtin_amdgcn_exp2f(x[m][j] - mrun[m][j]) : 0.0f;
                    const _Float16 ph = _Float16(pv);
                    lrun[m][j] += float(ph);
                    pw[(hw0 + 16 * m + 4 * kg + j) * (2 * PS) + n] = __builtin_bit_cast(uint16_t, ph);
                }
        }
        __syncthreads();   // weights and rescale factors complete

        // ---- C: rescale, then O += P . (hi + lo) for this wave's channels
        {
            const int f0 = L.wflag[0], f1 = L.wflag[1], f2 = L.wflag[2], f3 = L.wflag[3];
            if ((f0 | f1 | f2 | f3) != 0) {
#pragma unroll
                for (int pm = 0; pm < PM; ++pm)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int h = 32 * pm + 8 * (e >> 2) + 4 * h32 + (e & 3);
                        const int hw = h / HW;
                        const int fl = hw == 0 ? f0 : hw == 1 ? f1 : hw == 2 ? f2 : f3;
                        const float a = fl ? L.alpha[h] : 1.0f;
#pragma unroll
                        for (int u = 0; u < 4; ++u) O[pm][u][e] *= a;
                    }
            }
#pragma unroll
            for (int pm = 0; pm < PM; ++pm) {
                const f16x8 A = as_f16x8(*reinterpret_cast<const uint4*>(L.pm + (32 * pm + c32) * PS + 4 * h32));
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    O[pm][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        A, as_f16x8(PH[u][0], PH[u][1], PH[u][2], PH[u][3]), O[pm][u], 0, 0, 0);
                    O[pm][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        A, as_f16x8(PL[u][0], PL[u][1], PL[u][2], PL[u][3]), O[pm][u], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue: running maxima and row sums per head, partial outputs
#pragma unroll
    for (int m = 0; m < QM; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float l = row_sum16(lrun[m][j]);
            if (n == 0) {
                const int64_t slot = (qrow0 + hw0 + 16 * m + 4 * kg + j) * p.S + s;
                p.ws_ml[slot * 2] = mrun[m][j];
                p.ws_ml[slot * 2 + 1] = l;
            }
        }
#pragma unroll
    for (int pm = 0; pm < PM; ++pm)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int h = 32 * pm + 8 * (e >> 2) + 4 * h32 + (e & 3);
            float4 v = make_float4(O[pm][0][e], O[pm][1][e], O[pm][2][e], O[pm][3][e]);
            *reinterpret_cast<float4*>(p.ws_acc + ((qrow0 + h) * p.S + s) * VD + 128 * wave + 4 * c32) = v;
        }
}

}  // namespace

bool mla_supported(const kvq_cache& c, int Hq) {
    const kvq_cache_cfg& g = c.cfg;
    return g.kind == KVQ_KIND_MLA && g.n_kv_heads == 1 && g.key.bits == 4 && g.key.dim == KD &&
           g.key.group == GR && g.value.bits == 2 && g.value.dim == VD && g.value.group == 32 &&
           (Hq == 64 || Hq == 128);
}

hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t st) {
    const kvq_cache& c = *a.c;
    MlaParams p;
    p.kc = static_cast<const uint32_t*>(c.buf.k_codes);
    p.ks = static_cast<const uint16_t*>(c.buf.k_scale);
    p.kz = static_cast<const uint16_t*>(c.buf.k_zero);
    p.kr = static_cast<const uint16_t*>(c.buf.k_resid);
    p.vc = static_cast<const uint32_t*>(c.buf.v_codes);
    p.vs = static_cast<const uint16_t*>(c.buf.v_scale);
    p.vz = static_cast<const uint16_t*>(c.buf.v_zero);
    p.q = static_cast<const uint16_t*>(a.q);
    p.ws_acc = a.ws_acc;
    p.ws_ml = a.ws_ml;
    p.Hq = a.Hq;
    p.S = a.S;
    p.ntiles = a.ntiles;
    p.T = a.T;
    p.nblk = a.nblk;
    p.cap = a.g.cap;
    p.nblk_cap = a.g.nblk_cap;
    p.sigma2 = a.sigma * 1.4426950408889634f;
    // 64 query heads per workgroup (the register budget of one wave per SIMD)
    const dim3 grid(a.S, a.g.B, a.Hq / 64);
    hipLaunchKernelGGL(k_decode_mla<64>, grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace kvq
