// kvq_decode_mla.hip -- split-K decode attention on MFMA for absorbed MLA
// caches: one latent KV head shared by 64 or 128 query heads; a 512-dim
// content latent in 2- or 4-bit per-token codes (32-channel groups) that
// serves as both key and value, and a 64-dim decoupled RoPE key in 4-bit
// per-channel codes over 64-token blocks (fp16 for the block that is not yet
// full).  QuantMLA's INT2 and INT4 content paths are both served.
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
// One workgroup of 8 waves (two per SIMD) takes 64 query heads of one
// sequence over a run of 16-token tiles; 128 heads take two workgroups.
// Wave w owns latent channels [64w, 64w + 64) and does all the work on
// them, so every content element is dequantized once per workgroup:
//  * dequant: codes become exact fp16 integers by an exponent trick
//    ((bits & mask) | exponent of 2^(10-b u) is 2^(10-b u) + code for the
//    b-bit code at position u of its byte);
//    c_hat = code * s + z is one fused fp16 FMA (the correctly rounded hi)
//    plus the fp32 remainder c_hat - hi (lo);
//  * QK^T: partial logits of all 64 heads over the wave's own channels
//    (v_mfma_f32_16x16x32_f16, Q in registers, the hi tile transposed to
//    token-major through a wave-private LDS block); the RoPE term of one
//    (16-head, 32-channel) block per wave uses exact 4-bit code operands
//    (the codes as fp16 integers) against q' = q_r * s_k in hi/lo rows plus the bias
//    sum_c q_r z_k, or the fp16 residual keys;
//  * softmax: wave w sums the 8 partials of heads [8w, 8w + 8), runs the
//    online softmax in log2 units (lazily moved maxima) and writes fp16
//    weights; the row sums add up the same fp16 values;
//  * PV: O[64 heads][own channels] += P . (hi + lo) on
//    v_mfma_f32_32x32x16_f16.
// Three tiles are in flight: a step does PV of tile i-2, the softmax of tile
// i-1 and dequant + QK^T of tile i, with one workgroup barrier, so the matrix
// work of one wave overlaps the vector work of the other.
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
constexpr int HQ = 64;       // query heads per workgroup
constexpr int NW = 8;        // waves per workgroup
constexpr int CWS = 36;      // dwords per token row of a wave's hi block (64 fp16 + pad)
constexpr int SXS = 68;      // floats per token row of a partial-logit block (64 heads + pad)
constexpr int RCS = 68;      // dwords per word row of the RoPE code block (64 + pad)
constexpr int QRS = 36;      // dwords per head row of q' (64 fp16 + pad)
constexpr int PS = 12;       // dwords per head row of P (16 fp16 + pad)
constexpr float TAU = 8.0f;  // lazy-rescale threshold (log2 units)

struct MlaParams {
    const uint32_t* kc;          // RoPE codes [B][nblk_cap][64][8]
    const uint16_t *ks, *kz, *kr;
    const uint32_t* vc;          // content codes [B][cap][16 * bits]
    const uint16_t *vs, *vz;     // content side [B][cap][16]
    const uint16_t* q;           // [B][Hq][576]
    float *ws_acc, *ws_ml;
    int Hq, S, ntiles;           // ntiles = ceil(T / 16)
    int64_t T, nblk, cap, nblk_cap;
    float sigma2;                // softmax scale * log2(e)
    float neg1;                  // -1, kept opaque so c*s + z - hi stays one mixed FMA
};

struct Lds {
    __attribute__((aligned(16))) float sx[2][NW][16 * SXS];  // partial logits [buf][wave][token][head]
    __attribute__((aligned(16))) float srx[2][NW][16 * 20];  // RoPE partials [buf][wave][token][16 heads]
    __attribute__((aligned(16))) uint32_t chw[NW][16 * CWS]; // per wave: hi, token-major [token][64 fp16]
    __attribute__((aligned(16))) uint32_t cst[NW][8 * 16];   // per wave: content codes [word][token] (4 or 8 words)
    __attribute__((aligned(16))) uint32_t sst[NW][2 * 2 * 8];  // per wave: [scale|zero][group][16 fp16]
    __attribute__((aligned(16))) uint32_t pm[2][HQ * PS];    // weights fp16 [buf][head][16 tokens]
    __attribute__((aligned(16))) uint32_t rc[8 * RCS];       // RoPE codes of the block [word][channel]
    uint32_t rs[2 * 32];                                     // RoPE [scale|zero][64 fp16]
    __attribute__((aligned(16))) uint32_t qr[HQ * 32];       // q_r fp16 [head][64]
    __attribute__((aligned(16))) uint32_t qrh[HQ * QRS];     // q' = q_r * s_k, hi [head][64 fp16]
    __attribute__((aligned(16))) uint32_t qrl[HQ * QRS];     // lo
    float rbias[HQ];                                         // RoPE zero bias of the block per head
    float alpha[2][HQ];                                      // rescale factors [buf][head]
    __attribute__((aligned(16))) int wflag[2][NW];           // softmax wave w moved some maxima
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

// fp16 pair c_hat = code * s + z, rounded once (fused), and its remainder.
// `h` holds (2^(10-2u) + code) in each half, `bias2` the pair -2^(10-2u).
__device__ __forceinline__ void dequant_pair(uint32_t h, uint32_t bias2, uint32_t s, uint32_t z,
                                             float neg1, uint32_t& hi, uint32_t& lo) {
    const f16x2 c = __builtin_bit_cast(f16x2, h) + __builtin_bit_cast(f16x2, bias2);  // exact codes
    const f16x2 sv = __builtin_bit_cast(f16x2, s), zv = __builtin_bit_cast(f16x2, z);
    const f16x2 hv = __builtin_elementwise_fma(c, sv, zv);
    hi = __builtin_bit_cast(uint32_t, hv);
    // c*s + z in fp32 (one rounding), minus hi (exact): both fp16-operand FMAs
    const float d0 = fmaf(float(c[0]), float(sv[0]), float(zv[0]));
    const float d1 = fmaf(float(c[1]), float(sv[1]), float(zv[1]));
    const f16x2 lv = {_Float16(fmaf(float(hv[0]), neg1, d0)), _Float16(fmaf(float(hv[1]), neg1, d1))};
    lo = __builtin_bit_cast(uint32_t, lv);
}

struct Frags {
    uint32_t h[2][4], l[2][4];   // [channel 2*c32 + v][token pair]
};

// Content code width VB (2 or 4): a wave's 64 channels are CW words per token.
template <int VB>
__global__ __launch_bounds__(512) void k_decode_mla(MlaParams p) {
    constexpr int CW = 64 * VB / 32;    // own code words per token
    constexpr int VWT = VD * VB / 32;   // code words per token
    __shared__ Lds L;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, kg = lane >> 4;        // 16x16x32 operand layout
    const int c32 = lane & 31, h32 = lane >> 5;     // 32x32x16 operand layout
    const int tq = lane & 15, hp = lane >> 4;       // softmax: token, head pair
    const int s = blockIdx.x, b = blockIdx.y;       // blockIdx.z: group of 64 query heads
    const int t_lo = int(int64_t(s) * p.ntiles / p.S);
    const int t_hi = int(int64_t(s + 1) * p.ntiles / p.S);
    const int64_t qrow0 = int64_t(b) * p.Hq + int64_t(blockIdx.z) * HQ;
    const int ch0 = 64 * wave;                      // first own latent channel

    // ---- q_r to LDS; content query rows of the own channels as A operands
    for (int i = tid; i < HQ * 32; i += 512)
        L.qr[i] = reinterpret_cast<const uint32_t*>(p.q + (qrow0 + i / 32) * QD + VD)[i % 32];
    f16x8 QA[4][2];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            QA[m][ks] = as_f16x8(*reinterpret_cast<const uint4*>(
                p.q + (qrow0 + 16 * m + n) * QD + ch0 + 32 * ks + 8 * kg));

    f32x16 O[2][2];   // [32-head row block][channel 2*c32 + v]
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
            for (int e = 0; e < 16; ++e) O[m][v][e] = 0.0f;
    // softmax state of heads 8w + 2hp + e, this lane's token share
    float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.0f, 0.0f};

    // per-lane dequant constants: channels ch0 + 2*c32 + v sit at code
    // position u = 2(c32 & 1) + v of byte (c32 & 7) >> 1 of word c32 >> 3
    // (2 bits), or in nibble v of byte c32 & 3 of word c32 >> 2 (4 bits)
    uint32_t dmk[2], de2[2], dnb[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
        const int u = VB == 2 ? 2 * (c32 & 1) + v : v;
        const uint32_t ex = uint32_t(25 - VB * u) << 10;   // exponent field of 2^(10-VB*u)
        dmk[v] = (VB == 2 ? 0x00030003u : 0x000F000Fu) << (VB * u);
        de2[v] = ex | (ex << 16);
        dnb[v] = de2[v] | 0x80008000u;
    }
    const uint32_t csel = byte_pair_sel(VB == 2 ? (c32 & 7) >> 1 : c32 & 3);
    const int cword = VB == 2 ? c32 >> 3 : c32 >> 2;      // own word of the lane's channels
    const uint32_t rsel = byte_pair_sel((n & 7) >> 1);    // RoPE: byte of the lane's token
    // (its code is the low nibble for even n, the high one for odd n)
    const int mr = wave >> 1, kr = wave & 1;              // this wave's RoPE block

    // content loads (two tiles ahead): code words CW/4 * (lane & 3) .. of the
    // own CW words of token t0 + (lane >> 2) (one word at 2 bits, two at 4);
    // side (lanes < 32): scale (lanes < 16) / zero pair of the own 2 groups of
    // token t0 + (lane & 15)
    const uint32_t* vcb = p.vc + int64_t(b) * p.cap * VWT + CW * wave + (CW / 4) * (lane & 3);
    const uint16_t* vsb = ((lane & 16) ? p.vz : p.vs) + int64_t(b) * p.cap * 16 + 2 * wave;
    auto load_content = [&](int tile, uint2& cw, uint32_t& sw) {
        const int64_t t0 = int64_t(tile) * 16;
        const uint32_t* src = vcb + (t0 + (lane >> 2)) * VWT;
        cw = VB == 2 ? make_uint2(src[0], 0u) : *reinterpret_cast<const uint2*>(src);
        sw = lane < 32 ? *reinterpret_cast<const uint32_t*>(vsb + (t0 + (lane & 15)) * 16) : 0u;
    };
    // RoPE block loads: code word tid of the block; side (tid < 64)
    auto load_rope = [&](int64_t blk, uint32_t& rw, uint32_t& rsw) {
        rw = p.kc[(int64_t(b) * p.nblk_cap + blk) * GR * 8 + tid];
        rsw = tid < 64 ? reinterpret_cast<const uint32_t*>((tid < 32 ? p.ks : p.kz) +
                                                           (int64_t(b) * p.nblk_cap + blk) * KD)[tid & 31]
                       : 0u;
    };
    // tile i's content words in slot (i - t_lo) & 1
    uint2 cwq[2] = {make_uint2(0u, 0u), make_uint2(0u, 0u)};
    uint32_t swq[2] = {0u, 0u}, rw_n = 0u, rsw_n = 0u;
    load_content(t_lo, cwq[0], swq[0]);
    if (t_lo + 1 < t_hi) load_content(t_lo + 1, cwq[1], swq[1]);
    if (int64_t(t_lo) * 16 / GR < p.nblk) load_rope(int64_t(t_lo) * 16 / GR, rw_n, rsw_n);
    __syncthreads();

    Frags F[2];        // tile i's operands in F[(i - t_lo) & 1]
    int64_t cur_blk = -1;

    // ---- stage 1 of tile i: dequant, QK^T partials -> sx[i & 1]
    auto front = [&](int i, Frags& fr, uint2& cwr, uint32_t& swr) {
        const int64_t t0 = int64_t(i) * 16;
        const int64_t blk = t0 / GR;
        const bool qrope = blk < p.nblk;
        if (qrope && blk != cur_blk) {
            // entering a quantized RoPE block: codes, side, q' = q_r * s_k, bias
            L.rc[(tid & 7) * RCS + (tid >> 3)] = rw_n;
            if (tid < 64) L.rs[tid] = rsw_n;
            cur_blk = blk;
            if (blk + 1 < p.nblk && (blk + 1) * GR < int64_t(t_hi) * 16) load_rope(blk + 1, rw_n, rsw_n);
            __syncthreads();
            // lane (cp = lane & 31) takes channel pair cp of heads 2*(tid >> 6)
            // + (lane >> 5) + 16k; the bias sum runs over the 32 lanes of a head
            const int cp = lane & 31;
            const uint32_t sv = L.rs[cp], zv = L.rs[32 + cp];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int h = 2 * wave + (lane >> 5) + 16 * k;
                const uint32_t qv = L.qr[h * 32 + cp];
                uint32_t hi, lo;
                split_prod2(lo_h(qv), lo_h(sv), hi_h(qv), hi_h(sv), hi, lo);
                L.qrh[h * QRS + cp] = hi;
                L.qrl[h * QRS + cp] = lo;
                float bp = fmaf(hi_h(qv), hi_h(zv), lo_h(qv) * lo_h(zv));
                bp = row_sum16(bp);
                bp += __shfl_xor(bp, 16);
                if (cp == 0) L.rbias[h] = bp;
            }
        }
        // stage the own codes and side values, prefetch tile i + 2
        {
            const uint2 cw = cwr;
            const uint32_t sw = swr;
            if (i + 2 < t_hi) load_content(i + 2, cwr, swr);
            L.cst[wave][(CW / 4) * (lane & 3) * 16 + (lane >> 2)] = cw.x;
            if (VB == 4) L.cst[wave][(2 * (lane & 3) + 1) * 16 + (lane >> 2)] = cw.y;
            // lane (sz, tl) holds groups (0, 1) of token tl; even tl writes
            // group 0 of tokens (tl, tl + 1), odd tl group 1
            const uint32_t other = uint32_t(__builtin_amdgcn_update_dpp(0, int(sw), 0xb1, 0xf, 0xf, false));
            const int sz = (lane >> 4) & 1, tl = lane & 15;
            const bool odd = (tl & 1) != 0;
            const uint32_t wv = odd ? __builtin_amdgcn_perm(sw, other, 0x07060302u)
                                    : __builtin_amdgcn_perm(other, sw, 0x05040100u);
            if (lane < 32) L.sst[wave][(sz * 2 + (odd ? 1 : 0)) * 8 + (tl >> 1)] = wv;
        }
        wave_sync();
        // dequant channels ch0 + 2*c32 + v of tokens 8*h32 .. 8*h32 + 7
        {
            const uint32_t* cs = L.cst[wave] + cword * 16 + 8 * h32;
            const uint4 wa = *reinterpret_cast<const uint4*>(cs);
            const uint4 wb = *reinterpret_cast<const uint4*>(cs + 4);
            const uint32_t x[4] = {__builtin_amdgcn_perm(wa.y, wa.x, csel), __builtin_amdgcn_perm(wa.w, wa.z, csel),
                                   __builtin_amdgcn_perm(wb.y, wb.x, csel), __builtin_amdgcn_perm(wb.w, wb.z, csel)};
            const uint32_t* sp = L.sst[wave] + (c32 >> 4) * 8 + 4 * h32;
            const uint4 sv = *reinterpret_cast<const uint4*>(sp);
            const uint4 zv = *reinterpret_cast<const uint4*>(sp + 16);
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
            for (int v = 0; v < 2; ++v)
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2)
                    dequant_pair((x[q2] & dmk[v]) | de2[v], dnb[v], sa[q2], za[q2], p.neg1, fr.h[v][q2],
                                 fr.l[v][q2]);
            // token-major hi: token 8*h32 + 2*q2 (+1), channels 2*c32, 2*c32 + 1
            uint32_t* cw = L.chw[wave];
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
                cw[(8 * h32 + 2 * q2) * CWS + c32] = __builtin_amdgcn_perm(fr.h[1][q2], fr.h[0][q2], 0x05040100u);
                cw[(8 * h32 + 2 * q2 + 1) * CWS + c32] = __builtin_amdgcn_perm(fr.h[1][q2], fr.h[0][q2], 0x07060302u);
            }
        }
        wave_sync();
        // partial logits of all 64 heads over the own channels
        f32x4 Sc[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) Sc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const f16x8 Bv = as_f16x8(*reinterpret_cast<const uint4*>(L.chw[wave] + n * CWS + 16 * ks + 4 * kg));
#pragma unroll
            for (int m = 0; m < 4; ++m) Sc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(QA[m][ks], Bv, Sc[m], 0, 0, 0);
        }
        // RoPE partial of heads 16mr .. 16mr + 15 over channels 32kr .. 32kr + 31
        // to srx: A = q' hi, lo against the codes as exact fp16 integers (low
        // nibble: (bits | exponent of 2^10) is 2^10 + code, high nibble: 2^6 +
        // code), or q_r against the fp16 residual keys
        const int hr = 16 * mr + n;
        f32x4 Sr = f32x4{0.f, 0.f, 0.f, 0.f};
        if (qrope) {
            const int wr = 2 * int((t0 % GR) / 16) + (n >> 3);   // code word of token n
            const bool hin = (n & 1) != 0;
            const uint32_t nm = hin ? 0x00f000f0u : 0x000f000fu;
            const uint32_t ne = hin ? 0x54005400u : 0x64006400u;   // 2^6 | 2^10 exponent pairs
            const f16x2 nb = __builtin_bit_cast(f16x2, hin ? 0xd400d400u : 0xe400e400u);
            const uint32_t* src = L.rc + wr * RCS + 32 * kr + 8 * kg;
            const uint4 w0 = *reinterpret_cast<const uint4*>(src);
            const uint4 w1 = *reinterpret_cast<const uint4*>(src + 4);
            auto code2 = [&](uint32_t hw, uint32_t lw) {
                const uint32_t x = (__builtin_amdgcn_perm(hw, lw, rsel) & nm) | ne;
                return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, x) + nb);
            };
            const f16x8 Bv = as_f16x8(code2(w0.y, w0.x), code2(w0.w, w0.z), code2(w1.y, w1.x), code2(w1.w, w1.z));
            const f16x8 Ah = as_f16x8(*reinterpret_cast<const uint4*>(L.qrh + hr * QRS + 16 * kr + 4 * kg));
            const f16x8 Al = as_f16x8(*reinterpret_cast<const uint4*>(L.qrl + hr * QRS + 16 * kr + 4 * kg));
            Sr = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Bv, Sr, 0, 0, 0);
            Sr = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, Bv, Sr, 0, 0, 0);
        } else {
            // residual keys, fp16: row t0 + n - nblk*64 of the residual
            const int64_t r = t0 + n - p.nblk * GR;
            uint4 kv = make_uint4(0u, 0u, 0u, 0u);
            if (r < GR && t0 + n < p.T)
                kv = *reinterpret_cast<const uint4*>(p.kr + (int64_t(b) * GR + r) * KD + 32 * kr + 8 * kg);
            const f16x8 Aq = as_f16x8(*reinterpret_cast<const uint4*>(L.qr + hr * 32 + 16 * kr + 4 * kg));
            Sr = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aq, as_f16x8(kv), Sr, 0, 0, 0);
        }
        *reinterpret_cast<f32x4*>(L.srx[i & 1][wave] + n * 20 + 4 * kg) = Sr;
        // partial logits to sx[i & 1][wave][token n][heads 16m + 4kg .. +3]
        float* dst = L.sx[i & 1][wave] + n * SXS + 4 * kg;
#pragma unroll
        for (int m = 0; m < 4; ++m) *reinterpret_cast<f32x4*>(dst + 16 * m) = Sc[m];
    };

    // ---- stage 2 of tile i: sum the partials of heads 8w + 2hp + e, softmax,
    // weights -> pm[i & 1], rescale factors -> alpha[i & 1], wflag[i & 1]
    auto softmax = [&](int i) {
        const int64_t t0 = int64_t(i) * 16;
        const bool qrope = t0 / GR < p.nblk;
        const int bf = i & 1;
        const int h0 = 8 * wave + 2 * hp;
        float x[2] = {0.0f, 0.0f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float2 v = *reinterpret_cast<const float2*>(L.sx[bf][w] + tq * SXS + h0);
            x[0] += v.x;
            x[1] += v.y;
        }
        // RoPE partials of heads h0, h0 + 1: waves 2(h0 >> 4) and 2(h0 >> 4) + 1
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const float2 v = *reinterpret_cast<const float2*>(L.srx[bf][2 * (h0 >> 4) + r] + tq * 20 + (h0 & 15));
            x[0] += v.x;
            x[1] += v.y;
        }
        const bool valid = t0 + tq < p.T;
        bool over = false;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float bias = qrope ? L.rbias[h0 + e] : 0.0f;
            x[e] = valid ? (x[e] + bias) * p.sigma2 : -INFINITY;
            over = over || x[e] > mrun[e] + TAU;
        }
        const bool moved = __builtin_amdgcn_ballot_w64(over) != 0;
        if (moved) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float mn = fmaxf(mrun[e], row_max16(x[e]));
                const float a = __builtin_amdgcn_exp2f(mrun[e] - mn);
                mrun[e] = mn;
                lrun[e] *= a;
                if (tq == 0) L.alpha[bf][h0 + e] = a;
            }
        }
        if (lane == 0) L.wflag[bf][wave] = moved ? 1 : 0;
        _Float16 ph[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float pv = valid ? __builtin_amdgcn_exp2f(x[e] - mrun[e]) : 0.0f;
            ph[e] = _Float16(pv);
            lrun[e] += float(ph[e]);
        }
        // even tq writes tokens (tq, tq + 1) of head h0, odd tq those of h0 + 1
        const uint32_t mine = __builtin_bit_cast(uint32_t, f16x2{ph[0], ph[1]});
        const uint32_t other = uint32_t(__builtin_amdgcn_update_dpp(0, int(mine), 0xb1, 0xf, 0xf, false));
        const bool odd = (tq & 1) != 0;
        const uint32_t wv = odd ? __builtin_amdgcn_perm(mine, other, 0x07060302u)
                                : __builtin_amdgcn_perm(other, mine, 0x05040100u);
        L.pm[bf][(h0 + (odd ? 1 : 0)) * PS + (tq >> 1)] = wv;
    };

    // ---- stage 3 of tile i: rescale, O += P . (hi + lo)
    auto pv_stage = [&](int i, const Frags& fr) {
        const int bf = i & 1;
        const int4 fa = *reinterpret_cast<const int4*>(L.wflag[bf]);
        const int4 fb = *reinterpret_cast<const int4*>(L.wflag[bf] + 4);
        if ((fa.x | fa.y | fa.z | fa.w | fb.x | fb.y | fb.z | fb.w) != 0) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    // row e of block m is head 32m + 8(e >> 2) + 4h32 + (e & 3),
                    // whose softmax ran on wave 4m + (e >> 2)
                    const int h = 32 * m + 8 * (e >> 2) + 4 * h32 + (e & 3);
                    const int hw = 4 * m + (e >> 2);
                    const int fl = hw == 0 ? fa.x : hw == 1 ? fa.y : hw == 2 ? fa.z : hw == 3 ? fa.w
                                 : hw == 4 ? fb.x : hw == 5 ? fb.y : hw == 6 ? fb.z : fb.w;
                    const float a = fl ? L.alpha[bf][h] : 1.0f;
                    O[m][0][e] *= a;
                    O[m][1][e] *= a;
                }
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const f16x8 A = as_f16x8(*reinterpret_cast<const uint4*>(L.pm[bf] + (32 * m + c32) * PS + 4 * h32));
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                O[m][v] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    A, as_f16x8(fr.h[v][0], fr.h[v][1], fr.h[v][2], fr.h[v][3]), O[m][v], 0, 0, 0);
                O[m][v] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    A, as_f16x8(fr.l[v][0], fr.l[v][1], fr.l[v][2], fr.l[v][3]), O[m][v], 0, 0, 0);
            }
        }
    };

    // step k: PV of tile t_lo + k - 2, softmax of t_lo + k - 1, front of
    // t_lo + k; the operands of tile i live in F[(i - t_lo) & 1]
    const int nt = t_hi - t_lo;
    // Waves w and w + 4 share a SIMD; the second one runs its softmax before
    // its PV so that the two overlap matrix and vector work.
    const bool sm_first = wave >= 4;
    for (int k = 0; k < nt + 2; k += 2) {
        if (sm_first && k >= 1 && k - 1 < nt) softmax(t_lo + k - 1);
        if (k >= 2) pv_stage(t_lo + k - 2, F[0]);
        if (!sm_first && k >= 1 && k - 1 < nt) softmax(t_lo + k - 1);
        if (k < nt) front(t_lo + k, F[0], cwq[0], swq[0]);
        __syncthreads();
        if (k + 1 >= nt + 2) break;
        if (sm_first && k < nt) softmax(t_lo + k);
        if (k >= 1) pv_stage(t_lo + k - 1, F[1]);
        if (!sm_first && k < nt) softmax(t_lo + k);
        if (k + 1 < nt) front(t_lo + k + 1, F[1], cwq[1], swq[1]);
        __syncthreads();
    }

    // ---- epilogue: running maxima and row sums, partial outputs
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const float l = row_sum16(lrun[e]);
        if (tq == 0) {
            const int64_t slot = (qrow0 + 8 * wave + 2 * hp + e) * p.S + s;
            p.ws_ml[slot * 2] = mrun[e];
            p.ws_ml[slot * 2 + 1] = l;
        }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int h = 32 * m + 8 * (e >> 2) + 4 * h32 + (e & 3);
            *reinterpret_cast<float2*>(p.ws_acc + ((qrow0 + h) * p.S + s) * VD + ch0 + 2 * c32) =
                make_float2(O[m][0][e], O[m][1][e]);
        }
}

}  // namespace

bool mla_supported(const kvq_cache& c, int Hq) {
    const kvq_cache_cfg& g = c.cfg;
    return g.kind == KVQ_KIND_MLA && g.n_kv_heads == 1 && g.key.bits == 4 && g.key.dim == KD &&
           g.key.group == GR && (g.value.bits == 2 || g.value.bits == 4) && g.value.dim == VD &&
           g.value.group == 32 && (Hq == 64 || Hq == 128);
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
    p.neg1 = -1.0f;
    const dim3 grid(a.S, a.g.B, a.Hq / HQ);
    if (c.cfg.value.bits == 4)
        hipExtLaunchKernelGGL(k_decode_mla<4>, grid, dim3(64 * NW), 0, st, a.ev_start, a.ev_stop, 0, p);
    else
        hipExtLaunchKernelGGL(k_decode_mla<2>, grid, dim3(64 * NW), 0, st, a.ev_start, a.ev_stop, 0, p);
    return hipGetLastError();
}

}  // namespace kvq
