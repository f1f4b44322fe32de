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
// Work split.  One workgroup of twelve waves (three per SIMD, 168 vector
// registers each) takes 64 query heads of one sequence over a run of 16-token
// tiles (128 heads take two workgroups).  The waves have two roles:
//  * waves 0..7 dequantize and run PV by latent channels: wave v owns
//    channels [64v, 64v + 64) for the workgroup's 64 heads.  Its lanes
//    dequantize those channels of the tile (hi and lo stay in its registers
//    as the PV B operands, hi is also written token-major to LDS) and read
//    the weights from LDS as A operands.  Column j of channel block u is
//    channel 64v + 2j + u, so a lane's two channels share one code byte;
//  * waves 8..11 run QK^T and the softmax by heads: wave w owns heads
//    [16w, 16w + 16) over the whole 576-wide contraction, its content query
//    rows in registers as A operands, the tile's hi latent read from LDS as
//    the B operand.  A logit needs no sum across waves.  They issue at a
//    raised priority: their chain (LDS reads, QK^T, softmax, weights to LDS)
//    sets the pace of a step, and the dequant and PV waves fill the gaps.
//    Measured on MI355X, B64 x 128 heads x 16K tokens: 612-618 us per launch
//    against 849-855 us for a four-wave kernel in which every wave did both
//    roles (one wave per SIMD, no other wave to hide its latencies), and
//    630-650 us without the raised priority.
// Software pipeline, one workgroup barrier per tile: in step k the dequant
// waves run PV of tile k - 1 (weights written in step k - 1), the dequant of
// tile k + 1, the staging of their codes of tile k + 2 and the loads of tile
// k + 4; the softmax waves run QK^T and the softmax of tile k (hi written in
// step k - 1), the RoPE operands of tile k + 1's block, the staging of tile
// k + 2's RoPE record and its loads of tile k + 4.
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
constexpr int CHS = 264;    // dwords per token row of a hi tile (512 fp16 + pad)
constexpr int PS2 = 12;     // dwords per head row of P (16 fp16 + pad)
constexpr int RRS = 512;    // dwords per staged RoPE record

constexpr int NVW = 8;      // dequant + PV waves (64 latent channels each)
constexpr int NQW = 4;      // QK^T + softmax waves (16 heads each)

// What the PV waves touch comes first, within 64 KB of the start (the reach
// of an LDS instruction's immediate offset from one base register).
struct LdsMla {
    __attribute__((aligned(16))) uint32_t ch[2][16 * CHS];       // hi latent [tile parity][token][512 fp16]
    __attribute__((aligned(16))) uint32_t pm[2][HW * PS2];       // weights fp16 [tile parity][head][16 tokens]
    __attribute__((aligned(16))) uint32_t cst[2][NVW][8 * 16];   // per PV wave: content codes [parity][word][token]
    __attribute__((aligned(16))) uint32_t sst[2][NVW][32];       // per PV wave: [parity][scale|zero][group][token pair]
    __attribute__((aligned(16))) float alpha[2][HW];             // rescale factors [tile parity][head]
    __attribute__((aligned(16))) int wflag[2][NQW];              // softmax wave w moved some of its maxima
    // RoPE record of a tile [tile mod 4]: quantized block: codes [word][64
    // channels] (dwords 0..127), the block's scales and zeros (128..191);
    // residual block: the tile's 16 fp16 key rows (dwords 0..511)
    __attribute__((aligned(16))) uint32_t rr[4][RRS];
    __attribute__((aligned(16))) uint32_t qr[HW * QRS];          // q_r fp16 [head][64 + pad]
    __attribute__((aligned(16))) uint4 qa[NQW][4][64];           // per softmax-wave lane: q' hi/lo A operands [kr][hl]
};

struct Frags {
    uint32_t h[2][4], l[2][4];   // [channel block u][token pair]
};

template <int VB>
__global__ __launch_bounds__(64 * (NVW + NQW)) __attribute__((amdgpu_waves_per_eu(3, 3)))
void k_decode_mla(MlaParams p) {
    constexpr int CWv = 64 * VB / 32;   // own code words per token (4 or 8)
    constexpr int VWT = VD * VB / 32;   // code words per token
    __shared__ LdsMla L;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const bool vrole = wave < NVW;
    const int n = lane & 15, kg = lane >> 4;        // 16x16x32 operand layout
    const int c32 = lane & 31, h32 = lane >> 5;     // 32x32x16 operand layout
    const int s = blockIdx.x, b = blockIdx.y;
    const int t_lo = int(int64_t(s) * p.ntiles / p.S);
    const int t_hi = int(int64_t(s + 1) * p.ntiles / p.S);
    const int64_t qrow0 = int64_t(b) * p.Hq + HW * blockIdx.z;   // first query row of the workgroup
    if (t_lo >= t_hi) {
        for (int i = tid; i < HW * VD; i += 64 * (NVW + NQW))
            p.ws_acc[((qrow0 + i / VD) * p.S + s) * VD + i % VD] = 0.0f;
        if (tid < HW) {
            p.ws_ml[((qrow0 + tid) * p.S + s) * 2] = -INFINITY;
            p.ws_ml[((qrow0 + tid) * p.S + s) * 2 + 1] = 0.0f;
        }
        return;
    }

    if (vrole) {
        // ================= dequant + PV: latent channels [ch0, ch0 + 64)
        const int vw = wave, ch0 = 64 * vw;
        f32x16 O[2][2];   // [32-head row block m][channel block u]: column j is channel ch0 + 2j + u
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int e = 0; e < 16; ++e) O[m][u][e] = 0.0f;
        // lane (c32, h32) dequantizes channels ch0 + 2c32 + u of tokens
        // 8h32 .. 8h32 + 7.  2 bits: own word c32 >> 3, byte (c32 & 7) >> 1,
        // field 4(c32 & 1) + 2u; 4 bits: own word c32 >> 2, byte c32 & 3,
        // field 4u
        const int cword = VB == 2 ? c32 >> 3 : c32 >> 2;
        const uint32_t csel = byte_pair_sel(VB == 2 ? (c32 & 7) >> 1 : c32 & 3);
        const int f0 = VB == 2 ? 4 * (c32 & 1) : 0;
        uint32_t mk[2], exx[2], bias2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int f = f0 + (VB == 2 ? 2 : 4) * u;
            const uint32_t m1 = (VB == 2 ? 3u : 15u) << f;
            const uint32_t ex = uint32_t(25 - f) << 10;
            mk[u] = m1 | (m1 << 16);
            exx[u] = ex | (ex << 16);
            bias2[u] = exx[u] | 0x80008000u;
        }
        // loads: lane (token lane >> 2, words (CWv / 4)(lane & 3) ..) of the
        // own code words; lane (sz = lane >> 5, tl = lane & 15) the scale
        // (sz = 0) or zero pair of the own groups of token tl
        const uint32_t* vcb = p.vc + int64_t(b) * p.cap * VWT + CWv * vw + (CWv / 4) * (lane & 3);
        const uint16_t* vsb = ((lane & 32) ? p.vz : p.vs) + int64_t(b) * p.cap * 16 + 2 * vw;
        struct PreV {
            uint2 cw;
            uint32_t sw;
        };
        // (a load past the run is clamped to the last tile: it reads valid
        // memory and is never used)
        auto load = [&](int t, PreV& P) __attribute__((always_inline)) {
            t = t < p.ntiles ? t : p.ntiles - 1;
            const int64_t t0 = int64_t(t) * 16;
            const uint32_t* src = vcb + (t0 + (lane >> 2)) * VWT;
            if (VB == 2) P.cw = make_uint2(*src, 0u);
            else P.cw = *reinterpret_cast<const uint2*>(src);
            P.sw = *reinterpret_cast<const uint32_t*>(vsb + (t0 + (lane & 15)) * 16);
        };
        // staging into the wave's own LDS slots; tokens at or past T get scale
        // and zero 0, so they dequantize to exact zeros.  Lane (sz, tl) with
        // even tl writes the first own group of tokens (tl, tl + 1), odd tl
        // the second group of tokens (tl - 1, tl)
        auto stage = [&](int t, const PreV& P) __attribute__((always_inline)) {
            uint32_t* cst = L.cst[t & 1][vw];
            const int tk = lane >> 2, wd = (CWv / 4) * (lane & 3);
            cst[wd * 16 + tk] = P.cw.x;
            if (VB == 4) cst[(wd + 1) * 16 + tk] = P.cw.y;
            const int sz = lane >> 5, tl = lane & 15;
            const uint32_t sw = int64_t(t) * 16 + tl < p.T ? P.sw : 0u;
            const uint32_t other = uint32_t(__builtin_amdgcn_update_dpp(0, int(sw), 0xb1, 0xf, 0xf, false));
            const bool odd = (tl & 1) != 0;
            const uint32_t wv = odd ? __builtin_amdgcn_perm(sw, other, 0x07060302u)
                                    : __builtin_amdgcn_perm(other, sw, 0x05040100u);
            if ((lane & 16) == 0) L.sst[t & 1][vw][(sz * 2 + (odd ? 1 : 0)) * 8 + (tl >> 1)] = wv;
        };
        // dequant of tile t (codes staged): hi and lo of the own channels into
        // F, hi token-major into the LDS tile that the softmax waves read
        auto dequant = [&](int t, Frags& F) __attribute__((always_inline)) {
            const uint32_t* cs = L.cst[t & 1][vw] + cword * 16 + 8 * h32;
            const uint4 wa = *reinterpret_cast<const uint4*>(cs);
            const uint4 wb = *reinterpret_cast<const uint4*>(cs + 4);
            const uint32_t wt[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
            const uint32_t* sp = L.sst[t & 1][vw] + (c32 >> 4) * 8 + 4 * h32;
            const uint4 sv = *reinterpret_cast<const uint4*>(sp);
            const uint4 zv = *reinterpret_cast<const uint4*>(sp + 16);
            const uint32_t sa[4] = {sv.x, sv.y, sv.z, sv.w}, za[4] = {zv.x, zv.y, zv.z, zv.w};
            uint32_t* chb = L.ch[t & 1];
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
                // code bytes of tokens 8h32 + 2q2 (low half) and + 1 (high half)
                const uint32_t x = __builtin_amdgcn_perm(wt[2 * q2 + 1], wt[2 * q2], csel);
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    dequant_pair((x & mk[u]) | exx[u], bias2[u], sa[q2], za[q2], p.neg1, F.h[u][q2], F.l[u][q2]);
                // hi, token-major: channels ch0 + 2c32, + 1 of the two tokens
                uint32_t* row = chb + (8 * h32 + 2 * q2) * CHS + 32 * vw + c32;
                row[0] = __builtin_amdgcn_perm(F.h[1][q2], F.h[0][q2], 0x05040100u);
                row[CHS] = __builtin_amdgcn_perm(F.h[1][q2], F.h[0][q2], 0x07060302u);
            }
        };
        // O *= alpha per head when some maximum moved at tile t (not on the
        // run's first tile, where O is still zero).  Row e of block m is head
        // 32m + 8(e >> 2) + 4h32 + (e & 3): four factors per LDS read, one
        // group of rows at a time (the factors of all rows at once would not
        // fit the register budget)
        auto rescale = [&](int t) __attribute__((always_inline)) {
            const int4 fl = *reinterpret_cast<const int4*>(L.wflag[t & 1]);
            if (t > t_lo && (fl.x | fl.y | fl.z | fl.w) != 0) {
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float4 f = *reinterpret_cast<const float4*>(L.alpha[t & 1] + 32 * m + 8 * g + 4 * h32);
                        const float fa[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int u = 0; u < 2; ++u) O[m][u][4 * g + i] *= fa[i];
                        __builtin_amdgcn_sched_barrier(0);
                    }
            }
        };
        // O += P . (hi + lo) for the 64 heads over the own channels, tile t
        auto pv_mfma = [&](int t, const Frags& F) __attribute__((always_inline)) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const f16x8 A = as_f16x8(*reinterpret_cast<const uint4*>(L.pm[t & 1] + (32 * m + c32) * PS2 + 4 * h32));
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    O[m][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        A, as_f16x8(F.h[u][0], F.h[u][1], F.h[u][2], F.h[u][3]), O[m][u], 0, 0, 0);
                    O[m][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        A, as_f16x8(F.l[u][0], F.l[u][1], F.l[u][2], F.l[u][3]), O[m][u], 0, 0, 0);
                }
            }
        };
        // step k: PV of tile k - 1 (weights written by the softmax waves in
        // step k - 1), the dequant of tile k + 1 into the same slot, the
        // staging of tile k + 2 and the loads of tile k + 4
        auto step = [&](int k, auto pv_on, Frags& Fc, PreV& Ps) __attribute__((always_inline)) {
            if constexpr (decltype(pv_on)::value) {
                rescale(k - 1);
                pv_mfma(k - 1, Fc);
                // the slot's old fragments are dead once the products are issued
                __builtin_amdgcn_sched_barrier(0);
            }
            dequant(k + 1, Fc);
            stage(k + 2, Ps);
            load(k + 4, Ps);
            __syncthreads();
        };
        // prologue: tiles t_lo, t_lo + 1 staged and t_lo dequantized; tiles
        // t_lo + 2, + 3 in flight.  Tile t's fragments sit in F0 when t - t_lo
        // is even, else in F1 (tiles k - 1 and k + 1 share a slot)
        Frags F0, F1;
        PreV P0, P1;
        load(t_lo, P0);
        load(t_lo + 1, P1);
        __syncthreads();   // (1) L.qr
        stage(t_lo, P0);
        stage(t_lo + 1, P1);
        load(t_lo + 2, P0);
        load(t_lo + 3, P1);
        __syncthreads();   // (2) staged
        dequant(t_lo, F0);
        __syncthreads();   // (3) hi of tile t_lo, q' of its block
        step(t_lo, std::false_type{}, F1, P0);
        int k = t_lo + 1;
        for (; k + 1 < t_hi; k += 2) {
            step(k, std::true_type{}, F0, P1);
            step(k + 1, std::true_type{}, F1, P0);
        }
        // PV of tile k - 1, and when tile k is the run's last, the last step:
        // nothing past the run is dequantized, staged or loaded
        rescale(k - 1);
        pv_mfma(k - 1, F0);
        if (k < t_hi) {
            __syncthreads();
            rescale(k);
            pv_mfma(k, F1);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int h = 32 * m + 8 * (e >> 2) + 4 * h32 + (e & 3);
                *reinterpret_cast<float2*>(p.ws_acc + ((qrow0 + h) * p.S + s) * VD + ch0 + 2 * c32) =
                    make_float2(O[m][0][e], O[m][1][e]);
            }
    } else {
        // ================= QK^T + softmax: heads [hw0, hw0 + 16)
        const int qw = wave - NVW, rtid = tid - 64 * NVW;
        // these waves set the pace of a step: they issue first
        __builtin_amdgcn_s_setprio(2);
        const int hw0 = 16 * qw;
        const uint32_t rsel = byte_pair_sel((n & 7) >> 1);   // RoPE: byte of the lane's token
        static_assert(HW * 32 % 256 == 0, "q_r dwords per thread");
        uint32_t qrv[HW * 32 / 256];
#pragma unroll
        for (int j = 0; j < HW * 32 / 256; ++j) {
            const int i = rtid + 256 * j;
            qrv[j] = reinterpret_cast<const uint32_t*>(p.q + (qrow0 + (i >> 5)) * QD + VD)[i & 31];
        }
#pragma unroll
        for (int j = 0; j < HW * 32 / 256; ++j) {
            const int i = rtid + 256 * j;
            L.qr[(i >> 5) * QRS + (i & 31)] = qrv[j];
        }
        // the own heads' content rows as A operands: QA[ks] = channels
        // 32ks + 8kg .. + 7 of head hw0 + n
        f16x8 QA[16];
#pragma unroll
        for (int ks = 0; ks < 16; ++ks)
            QA[ks] = as_f16x8(*reinterpret_cast<const uint4*>(p.q + (qrow0 + hw0 + n) * QD + 32 * ks + 8 * kg));
        float mrun[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY}, lrun[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        f32x4 rb = f32x4{0.f, 0.f, 0.f, 0.f};   // RoPE bias of the block, rows 4kg + j
        // loads of tile t's RoPE record, dwords rtid and rtid + 256 (clamped
        // to the last tile like the content loads).  Quantized block: dword
        // rtid < 128 is word 2(t mod 4) + (rtid >> 6) of channel rtid & 63,
        // dwords 128..191 the scales, then the zeros; residual block: the
        // key rows t0 - 64 nblk .. + 15
        auto load = [&](int t, uint2& rw) __attribute__((always_inline)) {
            t = t < p.ntiles ? t : p.ntiles - 1;
            const int64_t t0 = int64_t(t) * 16;
            const int64_t blk = t0 / GR;
            const uint32_t *ax, *ay;
            if (blk < p.nblk) {
                const int64_t row = int64_t(b) * p.nblk_cap + blk;
                const uint32_t* kc = p.kc + row * GR * 8;
                ax = rtid < 128 ? kc + (rtid & 63) * 8 + 2 * (t & 3) + (rtid >> 6)
                     : rtid < 192 ? reinterpret_cast<const uint32_t*>(((rtid & 32) ? p.kz : p.ks) + row * KD) + (rtid & 31)
                                  : kc;
                ay = kc;
            } else {
                const uint32_t* kr = reinterpret_cast<const uint32_t*>(p.kr + (int64_t(b) * GR + (t0 - p.nblk * GR)) * KD);
                ax = kr + rtid;
                ay = kr + rtid + 256;
            }
            rw = make_uint2(*ax, *ay);
        };
        auto stage = [&](int t, const uint2& rw) __attribute__((always_inline)) {
            L.rr[t & 3][rtid] = rw.x;
            L.rr[t & 3][rtid + 256] = rw.y;
        };
        // q' = q_r * s_k (hi/lo A operands, lane-private) and the bias of the
        // own heads for the quantized block of tile t (record staged)
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
                L.qa[qw][kr * 2][lane] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                L.qa[qw][kr * 2 + 1][lane] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
                // bias sum_c q_r z_k: every column of B holds the zeros
                rb = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(qv), as_f16x8(zv), kr ? rb : f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            }
        };
        // content part of the logits of the own 16 heads over tile t, the B
        // operands requested in batches ahead of their products
        auto qk_content = [&](int t) __attribute__((always_inline)) {
            f32x4 S = f32x4{0.f, 0.f, 0.f, 0.f};
            const uint32_t* chr = L.ch[t & 1] + n * CHS + 4 * kg;
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
        // RoPE part of the logits over tile t, softmax, weights to LDS
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
                const uint32_t ne = hin ? 0x54005400u : 0x64006400u;
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
                    S = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(L.qa[qw][kr * 2][lane]), Bv, S, 0, 0, 0);
                    S = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(L.qa[qw][kr * 2 + 1][lane]), Bv, S, 0, 0, 0);
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
            // softmax of rows 4kg + j (head hw0 + 4kg + j), column n (token t0 + n)
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
            if (lane == 0) L.wflag[t & 1][qw] = moved ? 1 : 0;
            _Float16* pmh = reinterpret_cast<_Float16*>(L.pm[t & 1]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const _Float16 ph = _Float16(valid ? __builtin_amdgcn_exp2f(x[j] - mrun[j]) : 0.0f);
                lrun[j] += float(ph);
                pmh[(hw0 + 4 * kg + j) * (2 * PS2) + n] = ph;
            }
        };
        // step k: QK^T and softmax of tile k (its hi latent dequantized in
        // step k - 1), the RoPE operands of tile k + 1's block, the staging
        // of tile k + 2's RoPE record and the loads of tile k + 4's
        auto step = [&](int k, uint2& Rs) __attribute__((always_inline)) {
            const f32x4 S = qk_content(k);
            qk_rope_softmax(k, S);
            const int64_t t1 = int64_t(k + 1) * 16;
            if (k + 1 < t_hi && t1 / GR < p.nblk && t1 % GR == 0) fold(k + 1);
            stage(k + 2, Rs);
            load(k + 4, Rs);
            __syncthreads();
        };
        // prologue: records of tiles t_lo, t_lo + 1 staged, the RoPE operands
        // of t_lo's block; tiles t_lo + 2, + 3 in flight
        uint2 R0, R1;
        load(t_lo, R0);
        load(t_lo + 1, R1);
        __syncthreads();   // (1) L.qr
        stage(t_lo, R0);
        stage(t_lo + 1, R1);
        load(t_lo + 2, R0);
        load(t_lo + 3, R1);
        __syncthreads();   // (2) staged
        if (int64_t(t_lo) * 16 / GR < p.nblk) fold(t_lo);
        __syncthreads();   // (3)
        step(t_lo, R0);
        int k = t_lo + 1;
        for (; k + 1 < t_hi; k += 2) {
            step(k, R1);
            step(k + 1, R0);
        }
        if (k < t_hi) step(k, R1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float l = row_sum16(lrun[j]);
            if (n == 0) {
                const int64_t slot = (qrow0 + hw0 + 4 * kg + j) * p.S + s;
                p.ws_ml[slot * 2] = mrun[j];
                p.ws_ml[slot * 2 + 1] = l;
            }
        }
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
        hipExtLaunchKernelGGL(k_decode_mla<4>, grid, dim3(64 * (NVW + NQW)), 0, st, a.ev_start, a.ev_stop, 0, p);
    else
        hipExtLaunchKernelGGL(k_decode_mla<2>, grid, dim3(64 * (NVW + NQW)), 0, st, a.ev_start, a.ev_stop, 0, p);
    return hipGetLastError();
}

}  // namespace kvq
