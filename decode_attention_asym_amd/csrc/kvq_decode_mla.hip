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
// Arithmetic:
//  * dequant: codes become exact fp16 integers by an exponent trick
//    ((bits & mask) | exponent of 2^(10-f) is 2^(10-f) + code for the code
//    in bit field f of its byte); c_hat = code * s + z is one fused fp16 FMA
//    (the correctly rounded hi) plus the fp32 remainder c_hat - hi (lo);
//  * QK^T with the hi latent (v_mfma_f32_16x16x32_f16); the RoPE term uses
//    exact 4-bit code operands (the codes as fp16 integers) against
//    q' = q_r * s_k in hi/lo rows plus the bias sum_c q_r z_k, or the fp16
//    residual keys;
//  * online softmax in log2 units (maxima moved lazily, by more than TAU),
//    fp16 weights whose row sums add up the same fp16 values;
//  * PV: O += P . (hi + lo) on v_mfma_f32_32x32x16_f16.
//
// Work split.  One workgroup of four waves, one per SIMD, takes 64 query
// heads of one sequence over a run of 16-token tiles (128 heads take two
// workgroups).  One wave per SIMD gets 512 registers: the 64 x 128 PV
// accumulators of a wave and its 16 heads' content query rows (the QK^T A
// operands, which the matrix instructions read there directly) sit in its
// accumulation registers, the dequantized latent of two tiles in its vector
// registers.
//  * QK^T and the softmax by heads: wave w owns heads [16w, 16w + 16) of the
//    workgroup over the whole 576-wide contraction; the tile's hi latent is
//    read token-major from LDS as the B operand.  A logit needs no sum
//    across waves.
//  * PV by latent channels: wave w owns channels [128w, 128w + 128), which it
//    dequantized itself, for the workgroup's 64 heads (the weights read from
//    LDS as A operands).  Column j of channel block u is channel
//    128w + 4j + u: a lane's four channels are the four codes of one 2-bit
//    code byte.
// Software pipeline, one workgroup barrier per tile: step k runs PV of tile
// k - 1, QK^T of tile k and the dequant of tile k + 1, then the softmax of
// tile k, the RoPE operands of tile k + 1's block, the staging of tile k + 2
// into LDS and the global loads of tile k + 4.
#include <hip/hip_fp16.h>
#include <math.h>

#include <type_traits>

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
constexpr int QRS = 36;      // dwords per head row of q' (64 fp16 + pad)
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

constexpr int HW = 64;      // query heads per workgroup
constexpr int NW4 = 4;      // waves per workgroup
constexpr int CHS = 260;    // dwords per token row of a hi tile (512 fp16 + pad)
constexpr int PS2 = 12;     // dwords per head row of P (16 fp16 + pad)
constexpr int RRS = 512;    // dwords per staged RoPE record

struct Lds4w {
    __attribute__((aligned(16))) uint32_t ch[2][16 * CHS];       // hi latent [tile parity][token][512 fp16]
    __attribute__((aligned(16))) uint32_t pm[2][HW * PS2];       // weights fp16 [tile parity][head][16 tokens]
    __attribute__((aligned(16))) uint32_t cst[2][NW4][16 * 16];  // per wave: content codes [parity][word][token]
    __attribute__((aligned(16))) uint32_t sst[2][NW4][64];       // per wave: [parity][scale|zero][group][token pair]
    // RoPE record of a tile [tile mod 4]: quantized block: codes [word][64
    // channels] (dwords 0..127), the block's scales and zeros (128..191);
    // residual block: the tile's 16 fp16 key rows (dwords 0..511)
    __attribute__((aligned(16))) uint32_t rr[4][RRS];
    __attribute__((aligned(16))) uint32_t qr[HW * QRS];          // q_r fp16 [head][64 + pad]
    __attribute__((aligned(16))) uint4 qa[NW4][4][64];           // per lane: q' hi/lo A operands [kr][hl]
    __attribute__((aligned(16))) float alpha[2][HW];             // rescale factors [tile parity][head]
    __attribute__((aligned(16))) int wflag[2][NW4];              // wave w moved some of its maxima
};

struct Frags {
    uint32_t h[4][4], l[4][4];   // [channel block u][token pair]
};

// One tile's global loads, two steps ahead of their staging into LDS.
struct Pre {
    uint4 cw;       // own content code words of token t0 + (lane >> 2)
    uint32_t sw;    // content scale or zero pair of token t0 + (lane & 15)
    uint2 rw;       // RoPE record dwords tid, tid + 256
};

template <int VB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_decode_mla(MlaParams p) {
    constexpr int CW = 128 * VB / 32;   // own code words per token (8 or 16)
    constexpr int VWT = VD * VB / 32;   // code words per token
    __shared__ Lds4w L;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, kg = lane >> 4;        // 16x16x32 operand layout
    const int c32 = lane & 31, h32 = lane >> 5;     // 32x32x16 operand layout
    const int s = blockIdx.x, b = blockIdx.y;
    const int t_lo = int(int64_t(s) * p.ntiles / p.S);
    const int t_hi = int(int64_t(s + 1) * p.ntiles / p.S);
    const int64_t qrow0 = int64_t(b) * p.Hq + HW * blockIdx.z;   // first query row of the workgroup
    const int hw0 = 16 * wave;    // first own head (QK^T, softmax)
    const int ch0 = 128 * wave;   // first own latent channel (PV)
    if (t_lo >= t_hi) {
        // an empty run (the split plans make none): an empty partial
        for (int i = tid; i < HW * VD; i += 256) p.ws_acc[((qrow0 + i / VD) * p.S + s) * VD + i % VD] = 0.0f;
        if (tid < HW) {
            p.ws_ml[((qrow0 + tid) * p.S + s) * 2] = -INFINITY;
            p.ws_ml[((qrow0 + tid) * p.S + s) * 2 + 1] = 0.0f;
        }
        return;
    }

    // ---- q_r of the 64 heads to LDS; the own heads' content rows as A
    // operands: QA[ks] = channels 32ks + 8kg .. + 7 of head hw0 + n
    // (8 dwords per thread, all loads issued before the first store)
    static_assert(HW * 32 % 256 == 0, "q_r dwords per thread");
    uint32_t qrv[HW * 32 / 256];
#pragma unroll
    for (int j = 0; j < HW * 32 / 256; ++j) {
        const int i = tid + 256 * j;
        qrv[j] = reinterpret_cast<const uint32_t*>(p.q + (qrow0 + (i >> 5)) * QD + VD)[i & 31];
    }
#pragma unroll
    for (int j = 0; j < HW * 32 / 256; ++j) {
        const int i = tid + 256 * j;
        L.qr[(i >> 5) * QRS + (i & 31)] = qrv[j];
    }
    // (kept in accumulation registers, which the matrix instructions read
    // directly: the vector registers hold the dequantized latent)
    // All 16 loads are issued before the first register constraint: with
    // the constraint next to each load, every load waited for the previous
    // one (16 memory latencies in a row at the start of each workgroup).
    f16x8 QA[16];
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
        QA[ks] = as_f16x8(*reinterpret_cast<const uint4*>(p.q + (qrow0 + hw0 + n) * QD + 32 * ks + 8 * kg));
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) asm volatile("" : "+a"(QA[ks]));

    f32x16 O[2][4];   // [32-head row block m][channel block u]
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 16; ++e) O[m][u][e] = 0.0f;
    // softmax state of heads hw0 + 4kg + j, and this lane's token share of
    // their row sums
    float mrun[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY}, lrun[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 rb = f32x4{0.f, 0.f, 0.f, 0.f};   // RoPE bias of the block, rows 4kg + j

    // Dequant layout: lane (c32, h32) takes channels ch0 + 4c32 + u of tokens
    // 8h32 .. 8h32 + 7.  2 bits: code u of byte c32 & 3 of own word c32 >> 2;
    // 4 bits: nibble u & 1 of byte 2(c32 & 1) + (u >> 1) of own word c32 >> 1
    const int cword = VB == 2 ? c32 >> 2 : c32 >> 1;
    const uint32_t csel0 = byte_pair_sel(VB == 2 ? c32 & 3 : 2 * (c32 & 1));
    const uint32_t csel1 = byte_pair_sel(VB == 2 ? c32 & 3 : 2 * (c32 & 1) + 1);
    const uint32_t rsel = byte_pair_sel((n & 7) >> 1);   // RoPE: byte of the lane's token

    // ---- global loads of tile t (clamped to the last tile: a load past the
    // run reads valid memory and is never used).  Content: own words
    // (CW / 4)(lane & 3) .. of token t0 + (lane >> 2); lane (sz, gp, tl)
    // takes the scale (sz = 0) or zero pair of own groups 2gp, 2gp + 1 of
    // token t0 + tl.  RoPE record dwords tid and tid + 256.
    const uint32_t* vcb = p.vc + int64_t(b) * p.cap * VWT + CW * wave + (CW / 4) * (lane & 3);
    const uint16_t* vsb = ((lane & 32) ? p.vz : p.vs) + int64_t(b) * p.cap * 16 + 4 * wave + 2 * ((lane >> 4) & 1);
    auto load = [&](int t, Pre& P) __attribute__((always_inline)) {
        t = t < p.ntiles ? t : p.ntiles - 1;
        const int64_t t0 = int64_t(t) * 16;
        const uint32_t* src = vcb + (t0 + (lane >> 2)) * VWT;
        if (VB == 2) {
            const uint2 w = *reinterpret_cast<const uint2*>(src);
            P.cw = make_uint4(w.x, w.y, 0u, 0u);
        } else {
            P.cw = *reinterpret_cast<const uint4*>(src);
        }
        P.sw = *reinterpret_cast<const uint32_t*>(vsb + (t0 + (lane & 15)) * 16);
        const int64_t blk = t0 / GR;
        const uint32_t *ax, *ay;
        if (blk < p.nblk) {
            // codes: dword tid < 128 is word 2(t mod 4) + (tid >> 6) of
            // channel tid & 63; dwords 128..191 the scales, then the zeros
            const int64_t row = int64_t(b) * p.nblk_cap + blk;
            const uint32_t* kc = p.kc + row * GR * 8;
            ax = tid < 128 ? kc + (tid & 63) * 8 + 2 * (t & 3) + (tid >> 6)
                 : tid < 192 ? reinterpret_cast<const uint32_t*>(((tid & 32) ? p.kz : p.ks) + row * KD) + (tid & 31)
                             : kc;
            ay = kc;
        } else {
            // the residual key rows t0 - 64 nblk .. + 15 (inside its 64 rows)
            const uint32_t* kr = reinterpret_cast<const uint32_t*>(p.kr + (int64_t(b) * GR + (t0 - p.nblk * GR)) * KD);
            ax = kr + tid;
            ay = kr + tid + 256;
        }
        P.rw = make_uint2(*ax, *ay);
    };
    // ---- staging of tile t into LDS (content: wave-private; RoPE record:
    // shared).  Tokens at or past T get scale and zero 0, so they dequantize
    // to exact zeros.
    auto stage = [&](int t, const Pre& P) __attribute__((always_inline)) {
        uint32_t* cst = L.cst[t & 1][wave];
        const int tk = lane >> 2, w0 = (CW / 4) * (lane & 3);
        cst[w0 * 16 + tk] = P.cw.x;
        cst[(w0 + 1) * 16 + tk] = P.cw.y;
        if (VB == 4) {
            cst[(w0 + 2) * 16 + tk] = P.cw.z;
            cst[(w0 + 3) * 16 + tk] = P.cw.w;
        }
        const int sz = lane >> 5, gp = (lane >> 4) & 1, tl = lane & 15;
        const uint32_t sw = int64_t(t) * 16 + tl < p.T ? P.sw : 0u;
        // lane (sz, gp, tl) holds groups (2gp, 2gp + 1) of token tl; even tl
        // writes group 2gp of tokens (tl, tl + 1), odd tl group 2gp + 1
        const uint32_t other = uint32_t(__builtin_amdgcn_update_dpp(0, int(sw), 0xb1, 0xf, 0xf, false));
        const bool odd = (tl & 1) != 0;
        const uint32_t wv = odd ? __builtin_amdgcn_perm(sw, other, 0x07060302u)
                                : __builtin_amdgcn_perm(other, sw, 0x05040100u);
        L.sst[t & 1][wave][(sz * 4 + 2 * gp + (odd ? 1 : 0)) * 8 + (tl >> 1)] = wv;
        L.rr[t & 3][tid] = P.rw.x;
        L.rr[t & 3][tid + 256] = P.rw.y;
    };

    // ---- q' = q_r * s_k (hi/lo A operands, lane-private) and the bias of
    // the own heads for the quantized block of tile t (record staged)
    auto fold = [&](int t) __attribute__((always_inline)) {
        const uint32_t* rec = L.rr[t & 3];
#pragma unroll
        for (int kr = 0; kr < 2; ++kr) {
            const uint4 sv = *reinterpret_cast<const uint4*>(rec + 128 + 16 * kr + 4 * kg);
            const uint4 zv = *reinterpret_cast<const uint4*>(rec + 160 + 16 * kr + 4 * kg);
            const uint4 qv = *reinterpret_cast<const uint4*>(L.qr + (hw0 + n) * QRS + 16 * kr + 4 * kg);
            const uint32_t sa[4] = {sv.x, sv.y, sv.z, sv.w};
            const uint32_t qa[4] = {qv.x, qv.y, qv.z, qv.w};
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) split_prod2(lo_h(qa[e]), lo_h(sa[e]), hi_h(qa[e]), hi_h(sa[e]), hi[e], lo[e]);
            L.qa[wave][kr * 2][lane] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            L.qa[wave][kr * 2 + 1][lane] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
            // bias sum_c q_r z_k: every column of B holds the zeros
            rb = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(qv), as_f16x8(zv), kr ? rb : f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        }
    };

    // ---- dequant of tile t (codes staged): hi token-major into its LDS tile
    // for QK^T, hi and lo of the own channels into F for PV
    auto dequant = [&](int t, Frags& F) __attribute__((always_inline)) {
        const uint32_t* cs = L.cst[t & 1][wave] + cword * 16 + 8 * h32;
        const uint4 wa = *reinterpret_cast<const uint4*>(cs);
        const uint4 wb = *reinterpret_cast<const uint4*>(cs + 4);
        const uint32_t wt[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
        const uint32_t* sp = L.sst[t & 1][wave] + (c32 >> 3) * 8 + 4 * h32;
        const uint4 sv = *reinterpret_cast<const uint4*>(sp);
        const uint4 zv = *reinterpret_cast<const uint4*>(sp + 32);
        const uint32_t sa[4] = {sv.x, sv.y, sv.z, sv.w}, za[4] = {zv.x, zv.y, zv.z, zv.w};
        uint32_t* chb = L.ch[t & 1];
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
            // code bytes of tokens 8h32 + 2q2 (low half) and + 1 (high half)
            const uint32_t x0 = __builtin_amdgcn_perm(wt[2 * q2 + 1], wt[2 * q2], csel0);
            const uint32_t x1 = VB == 2 ? x0 : __builtin_amdgcn_perm(wt[2 * q2 + 1], wt[2 * q2], csel1);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                // field f of the code in its byte; (bits & mask) | exponent of
                // 2^(10 - f) is the fp16 2^(10 - f) + code
                const int f = VB == 2 ? 2 * u : 4 * (u & 1);
                const uint32_t mk = (VB == 2 ? 0x00030003u : 0x000F000Fu) << f;
                const uint32_t ex = uint32_t(25 - f) << 10;
                const uint32_t x = (VB == 2 || u < 2) ? x0 : x1;
                dequant_pair((x & mk) | ex | (ex << 16), ex | (ex << 16) | 0x80008000u, sa[q2], za[q2], p.neg1,
                             F.h[u][q2], F.l[u][q2]);
            }
            // hi, token-major: channels ch0 + 4c32 .. + 3 of the two tokens
            uint32_t* row = chb + (8 * h32 + 2 * q2) * CHS + 64 * wave + 2 * c32;
            *reinterpret_cast<uint2*>(row) = make_uint2(__builtin_amdgcn_perm(F.h[1][q2], F.h[0][q2], 0x05040100u),
                                                        __builtin_amdgcn_perm(F.h[3][q2], F.h[2][q2], 0x05040100u));
            *reinterpret_cast<uint2*>(row + CHS) =
                make_uint2(__builtin_amdgcn_perm(F.h[1][q2], F.h[0][q2], 0x07060302u),
                           __builtin_amdgcn_perm(F.h[3][q2], F.h[2][q2], 0x07060302u));
        }
    };

    // ---- content part of the logits of the own 16 heads over tile t
    auto qk_content = [&](int t) __attribute__((always_inline)) {
        f32x4 S = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint32_t* chr = L.ch[t & 1] + n * CHS + 4 * kg;
        // B operands requested in batches ahead of their products
        constexpr int NB = 4;
#pragma unroll
        for (int kb = 0; kb < 16; kb += NB) {
            uint4 Bk[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) Bk[j] = *reinterpret_cast<const uint4*>(chr + 16 * (kb + j));
#pragma unroll
            for (int j = 0; j < NB; ++j) S = __builtin_amdgcn_mfma_f32_16x16x32_f16(QA[kb + j], as_f16x8(Bk[j]), S, 0, 0, 0);
        }
        return S;
    };

    // ---- RoPE part of the logits over tile t, softmax, weights to LDS
    auto qk_rope_softmax = [&](int t, f32x4 S) __attribute__((always_inline)) {
        const int64_t t0 = int64_t(t) * 16;
        const bool qrope = t0 / GR < p.nblk;
        const uint32_t* rec = L.rr[t & 3];
        if (qrope) {
            // q' hi, lo against the codes as exact fp16 integers: channel c
            // of token n is nibble n & 1 of byte (n & 7) >> 1 of word
            // (n >> 3) of the tile's two
            const bool hin = (n & 1) != 0;
            const uint32_t nm = hin ? 0x00f000f0u : 0x000f000fu;
            const uint32_t ne = hin ? 0x54005400u : 0x64006400u;   // 2^6 | 2^10 exponent pairs
            const f16x2 nbias = __builtin_bit_cast(f16x2, hin ? 0xd400d400u : 0xe400e400u);
            auto code2 = [&](uint32_t hw, uint32_t lw) __attribute__((always_inline)) {
                const uint32_t xx = (__builtin_amdgcn_perm(hw, lw, rsel) & nm) | ne;
                return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, xx) + nbias);
            };
#pragma unroll
            for (int kr = 0; kr < 2; ++kr) {
                const uint32_t* src = rec + (n >> 3) * 64 + 32 * kr + 8 * kg;
                const uint4 w0 = *reinterpret_cast<const uint4*>(src);
                const uint4 w1 = *reinterpret_cast<const uint4*>(src + 4);
                const f16x8 Bv = as_f16x8(code2(w0.y, w0.x), code2(w0.w, w0.z), code2(w1.y, w1.x), code2(w1.w, w1.z));
                S = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(L.qa[wave][kr * 2][lane]), Bv, S, 0, 0, 0);
                S = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(L.qa[wave][kr * 2 + 1][lane]), Bv, S, 0, 0, 0);
            }
        } else {
            // q_r against the fp16 residual key rows of the record
#pragma unroll
            for (int kr = 0; kr < 2; ++kr) {
                const f16x8 Bv = as_f16x8(*reinterpret_cast<const uint4*>(rec + n * 32 + 16 * kr + 4 * kg));
                const f16x8 Aq = as_f16x8(*reinterpret_cast<const uint4*>(L.qr + (hw0 + n) * QRS + 16 * kr + 4 * kg));
                S = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aq, Bv, S, 0, 0, 0);
            }
        }
        // ---- softmax of rows 4kg + j (head hw0 + 4kg + j), column n (token t0 + n)
        const bool valid = t0 + n < p.T;
        float x[4];
        bool over = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = valid ? (S[j] + (qrope ? rb[j] : 0.0f)) * p.sigma2 : -INFINITY;
            over = over || x[j] > mrun[j] + TAU;
        }
        const bool moved = __builtin_amdgcn_ballot_w64(over) != 0;
        float a[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if (moved) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float mn = fmaxf(mrun[j], row_max16(x[j]));
                a[j] = __builtin_amdgcn_exp2f(mrun[j] - mn);
                mrun[j] = mn;
                lrun[j] *= a[j];
            }
        }
        if (n == 0) *reinterpret_cast<float4*>(L.alpha[t & 1] + hw0 + 4 * kg) = make_float4(a[0], a[1], a[2], a[3]);
        if (lane == 0) L.wflag[t & 1][wave] = moved ? 1 : 0;
        _Float16* pmh = reinterpret_cast<_Float16*>(L.pm[t & 1]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const _Float16 ph = _Float16(valid ? __builtin_amdgcn_exp2f(x[j] - mrun[j]) : 0.0f);
            lrun[j] += float(ph);
            pmh[(hw0 + 4 * kg + j) * (2 * PS2) + n] = ph;
        }
    };

    // ---- O *= alpha per head when some maximum moved at tile t (not on the
    // run's first tile, where O is still zero).  Row e of block m is head
    // 32m + 8(e >> 2) + 4h32 + (e & 3).  Each accumulator is scaled where it
    // lives, in its accumulation register (read, multiply, write back), so
    // that they stay there for the whole loop; the matrix instructions that
    // last wrote them finished a barrier ago.
    auto rescale = [&](int t) __attribute__((always_inline)) {
        const int4 fl = *reinterpret_cast<const int4*>(L.wflag[t & 1]);
        if (t > t_lo && (fl.x | fl.y | fl.z | fl.w) != 0) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float f = L.alpha[t & 1][32 * m + 8 * (e >> 2) + 4 * h32 + (e & 3)];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        float tmp;
                        asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                                     : "+a"(O[m][u][e]), "=&v"(tmp)
                                     : "v"(f));
                    }
                }
            // wait states between these writes and the matrix instructions
            // that read the same registers next
            asm volatile("s_nop 7");
        }
    };

    // ---- O += P . (hi + lo) for the 64 heads over the own channels, tile t
    auto pv_mfma = [&](int t, const Frags& F) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const f16x8 A = as_f16x8(*reinterpret_cast<const uint4*>(L.pm[t & 1] + (32 * m + c32) * PS2 + 4 * h32));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                O[m][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    A, as_f16x8(F.h[u][0], F.h[u][1], F.h[u][2], F.h[u][3]), O[m][u], 0, 0, 0);
                O[m][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    A, as_f16x8(F.l[u][0], F.l[u][1], F.l[u][2], F.l[u][3]), O[m][u], 0, 0, 0);
            }
        }
    };

    // ---- step k: PV of tile k - 1 (fragments Fc), QK^T of tile k and the
    // dequant of tile k + 1 (into Fc: tiles k - 1 and k + 1 share a slot),
    // then the softmax of tile k, the RoPE operands of tile k + 1, the staging
    // of tile k + 2 (from Ps) and the loads of tile k + 4 (into Ps).  Past
    // the run's last tile the dequant, staging and loads work on clamped
    // (valid, unused) data, so every step has the same shape.
    auto step = [&](int k, auto pv_on, Frags& Fc, Pre& Ps) __attribute__((always_inline)) {
        if constexpr (decltype(pv_on)::value) {
            rescale(k - 1);
            pv_mfma(k - 1, Fc);
        }
        const f32x4 S = qk_content(k);
        dequant(k + 1, Fc);
        qk_rope_softmax(k, S);
        const int64_t t1 = int64_t(k + 1) * 16;
        if (k + 1 < t_hi && t1 / GR < p.nblk && t1 % GR == 0) fold(k + 1);
        stage(k + 2, Ps);
        load(k + 4, Ps);
        __syncthreads();
    };

    // ---- prologue: tiles t_lo, t_lo + 1 staged, t_lo's RoPE operands and
    // dequant; tiles t_lo + 2, + 3 in flight
    Frags F0, F1;
    Pre P0, P1;
    load(t_lo, P0);
    load(t_lo + 1, P1);
    __syncthreads();   // L.qr
    stage(t_lo, P0);
    stage(t_lo + 1, P1);
    load(t_lo + 2, P0);
    load(t_lo + 3, P1);
    __syncthreads();
    if (int64_t(t_lo) * 16 / GR < p.nblk) fold(t_lo);
    dequant(t_lo, F0);
    __syncthreads();

    // tile t's fragments sit in F0 when t - t_lo is even, else in F1
    step(t_lo, std::false_type{}, F1, P0);
    int k = t_lo + 1;
    for (; k + 1 < t_hi; k += 2) {
        step(k, std::true_type{}, F0, P1);
        step(k + 1, std::true_type{}, F1, P0);
    }
    if (k < t_hi) {
        step(k, std::true_type{}, F0, P1);
        rescale(k);
        pv_mfma(k, F1);
    } else {
        rescale(k - 1);
        pv_mfma(k - 1, F0);
    }

    // ---- epilogue: running maxima and row sums, partial outputs
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float l = row_sum16(lrun[j]);
        if (n == 0) {
            const int64_t slot = (qrow0 + hw0 + 4 * kg + j) * p.S + s;
            p.ws_ml[slot * 2] = mrun[j];
            p.ws_ml[slot * 2 + 1] = l;
        }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int h = 32 * m + 8 * (e >> 2) + 4 * h32 + (e & 3);
            *reinterpret_cast<float4*>(p.ws_acc + ((qrow0 + h) * p.S + s) * VD + ch0 + 4 * c32) =
                make_float4(O[m][0][e], O[m][1][e], O[m][2][e], O[m][3][e]);
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
    const dim3 grid(a.S, a.g.B, a.Hq / HW);
    if (c.cfg.value.bits == 4)
        hipExtLaunchKernelGGL(k_decode_mla<4>, grid, dim3(64 * NW4), 0, st, a.ev_start, a.ev_stop, 0, p);
    else
        hipExtLaunchKernelGGL(k_decode_mla<2>, grid, dim3(64 * NW4), 0, st, a.ev_start, a.ev_stop, 0, p);
    return hipGetLastError();
}

}  // namespace kvq
