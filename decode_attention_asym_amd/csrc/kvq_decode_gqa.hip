// kvq_decode_gqa.hip -- split-K decode attention on MFMA for GQA caches:
// 4 query heads per KV head, head dim 128, 2-bit keys (G = 32 or 64) and
// 2-bit values (32-channel groups).
//
// Method ("Makale Bülteni -- KIVI", section "İddia ve Gerçeklik: KIVI"):
// logits over the per-channel-quantized keys and the fp16 residual keys,
// softmax, weighted sum of the per-token-quantized values; the codes are
// unpacked and dequantized inside this loop, never written back as fp16.
// GQA: four query heads share each KV head (section "Kod ve Entegrasyon
// Haritası"), which makes QK^T and PV dense enough for the matrix cores.
//
// How the contractions reach v_mfma_f32_16x16x32_f16 exactly:
//  * a 2-bit code c placed in bits [2u, 2u+1] of an fp16 lane (all other bits
//    zero) is the subnormal c * 4^u * 2^-24: exact, and gfx950 MFMA consumes
//    fp16 subnormals exactly.  One v_perm_b32 gathers one code byte from
//    each of two words into the two fp16 halves of a register; one AND per
//    code position then yields an operand register.  The power-of-two
//    factors are undone on the fp32 results.
//  * keys: khat = code * s + z with s, z per (block, channel).  The scale is
//    folded into the query (q' = q * s, exact in fp32) which is fed as two
//    fp16 rows hi + lo (q' - hi), so logits keep ~22 bits; the zero term
//    sum_c q_c z_c is a per-(head, block) bias computed on the VALU.
//  * values: vhat = code * s + z with s, z per (token, 32-channel group).
//    The scale is folded into the softmax weights (p' = p * s) as hi/lo
//    rows; sum_t p_t z_t per (head, group) is accumulated on the VALU.
//  * online softmax in log2 units; the running maximum only moves when a
//    tile exceeds it by more than 2^8 (weights stay <= 256, fp16-safe).
// One 64-lane workgroup handles one contiguous run of 64-token tiles of one
// (sequence, KV head); the work of the next tile's global loads overlaps the
// current tile.  The keys of a trailing partial tile and the residual are
// handled by one extra workgroup per (sequence, KV head) on the VALU.
#include <hip/hip_fp16.h>
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int HG = 4;       // query heads per KV head
constexpr int D = 128;      // head dim
constexpr int KSTR = 136;   // dwords per row of the key-code tile in LDS
constexpr int VSTR = 76;    // dwords per row of the value-code tile in LDS
constexpr int QSTR = 68;    // dwords per q' row (128 fp16 + pad)
constexpr int ASTR = 36;    // dwords per p' row (64 fp16 + pad)
constexpr int PSTR = 68;    // floats per row of the weight tile in LDS
constexpr float TAU = 8.0f; // lazy-rescale threshold (log2 units)

struct GqaParams {
    const uint32_t* kc;
    const uint16_t *ks, *kz, *kr;
    const uint32_t* vc;
    const uint16_t *vs, *vz;
    const uint16_t* q;
    float *ws_acc, *ws_ml;
    int Hq, Hkv, S, S_main, ntiles, G;
    int64_t T, nblk, cap, nblk_cap;
    float sigma2;  // softmax scale * log2(e)
};

struct Tile {
    uint4 k0, k1, v0, v1;     // 2 KB of key codes and 2 KB of value codes, 32 B per lane
    uint4 ks;                 // key scale (lanes 0..31) / zero (lanes 32..63) of the tile's blocks
    uint4 vs;                 // value scale (lanes 0..31) / zero (lanes 32..63) of the tile's tokens
};

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
__device__ __forceinline__ float lo_h(uint32_t w) { return float(__builtin_bit_cast(f16x2, w)[0]); }
__device__ __forceinline__ float hi_h(uint32_t w) { return float(__builtin_bit_cast(f16x2, w)[1]); }

__device__ __forceinline__ f16x8 as_f16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(f16x8, v);
}

__device__ __forceinline__ uint32_t pk_rtz(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// fp16 hi/lo split of two fp32 values: (hi, lo) with hi + lo == x to ~2^-22
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    hi = pk_rtz(x0, x1);
    lo = pk_rtz(x0 - lo_h(hi), x1 - hi_h(hi));
}

// hi/lo split of the products a0*b0, a1*b1 (a fp32, b an fp16 half): the
// remainders are single fused operations a*b - hi
__device__ __forceinline__ void split_prod2(float a0, float b0, float a1, float b1, uint32_t& hi,
                                            uint32_t& lo) {
    // fma(a, b, +0) is one v_fma_mix with the fp16 operand read in place
    // (it cannot become a plain multiply: they differ for a*b == -0)
    hi = pk_rtz(fmaf(a0, b0, 0.0f), fmaf(a1, b1, 0.0f));
    lo = pk_rtz(fmaf(a0, b0, -lo_h(hi)), fmaf(a1, b1, -hi_h(hi)));
}

__device__ __forceinline__ float xor_max16(float x) {
    x = fmaxf(x, __shfl_xor(x, 1));
    x = fmaxf(x, __shfl_xor(x, 2));
    x = fmaxf(x, __shfl_xor(x, 4));
    return fmaxf(x, __shfl_xor(x, 8));
}
__device__ __forceinline__ float xor_sum16(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    return x + __shfl_xor(x, 8);
}

__device__ __forceinline__ float pick4(const float* v, int i) {
    return i == 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : v[3];
}

// All global loads of one 64-token tile, 16-byte aligned, no lane reads
// what another lane reads: codes 2 x 2 KB, key side 512 B (G = 64) or 1 KB
// (G = 32), value side 1 KB.
template <int G>
__device__ __forceinline__ void load_tile(const GqaParams& p, int64_t bh, int64_t tt, int lane, Tile& r) {
    constexpr int NBT = 64 / G, W = G / 16;
    const uint4* kb = reinterpret_cast<const uint4*>(p.kc + (bh * p.nblk_cap + tt * NBT) * D * W);
    r.k0 = kb[lane];
    r.k1 = kb[lane + 64];
    const uint4* vb = reinterpret_cast<const uint4*>(p.vc + (bh * p.cap + tt * 64) * 8);
    r.v0 = vb[lane];
    r.v1 = vb[lane + 64];
    const uint16_t* kside = (lane < 32 ? p.ks : p.kz) + (bh * p.nblk_cap + tt * NBT) * D;
    if (G == 64) {
        const uint2 v = reinterpret_cast<const uint2*>(kside)[lane & 31];
        r.ks = make_uint4(v.x, v.y, 0u, 0u);
    } else {
        r.ks = reinterpret_cast<const uint4*>(kside)[lane & 31];
    }
    const uint16_t* vside = (lane < 32 ? p.vs : p.vz) + (bh * p.cap + tt * 64) * 4;
    r.vs = reinterpret_cast<const uint4*>(vside)[lane & 31];
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float key_hat(const GqaParams& p, int64_t bh, int64_t t, int c) {
    const int64_t Tq = p.nblk * p.G;
    if (t >= Tq) return h2f(p.kr[(bh * p.G + (t - Tq)) * D + c]);
    const int64_t blk = t / p.G;
    const int i = int(t - blk * p.G);
    const int64_t side = (bh * p.nblk_cap + blk) * D + c;
    const uint32_t w = p.kc[side * (p.G / 16) + i / 16];
    return fmaf(float((w >> (2 * (i & 15))) & 3u), h2f(p.ks[side]), h2f(p.kz[side]));
}

__device__ __forceinline__ float value_hat(const GqaParams& p, int64_t bh, int64_t t, int c) {
    const int64_t row = bh * p.cap + t;
    const uint32_t w = p.vc[row * 8 + c / 16];
    const int64_t side = row * 4 + c / 32;
    return fmaf(float((w >> (2 * (c & 15))) & 3u), h2f(p.vs[side]), h2f(p.vz[side]));
}

// Trailing tokens [ntiles*64, T): partial key block and fp16 residual keys,
// one token per lane for the logits, two channels per lane for the values.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__device__ void tail_split(const GqaParams& p, int b, int kvh, int s, float* qf, float* pl) {
    const int lane = threadIdx.x;
    const int64_t bh = int64_t(b) * p.Hkv + kvh;
    const int hq0 = kvh * HG;
    for (int i = lane; i < HG * D; i += 64) qf[i] = h2f(p.q[(int64_t(b) * p.Hq + hq0) * D + i]);
    wave_sync();
    const int64_t t0 = int64_t(p.ntiles) * 64;
    const int n_tail = int(p.T - t0);
    const int64_t t = t0 + lane;
    const bool valid = lane < n_tail;
    float sc[HG] = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
        for (int c = 0; c < D; ++c) {
            const float kh = key_hat(p, bh, t, c);
#pragma unroll
            for (int h = 0; h < HG; ++h) sc[h] = fmaf(qf[h * D + c], kh, sc[h]);
        }
    }
    float m[HG], l[HG];
#pragma unroll
    for (int h = 0; h < HG; ++h) {
        float x = valid ? sc[h] * p.sigma2 : -INFINITY;
        float mx = x;
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        const float pv = valid ? exp2f(x - mx) : 0.0f;
        float sum = pv;
        for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
        m[h] = mx;
        l[h] = sum;
        pl[h * PSTR + lane] = pv;
    }
    wave_sync();
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int c = lane + 64 * half;
        float acc[HG] = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < n_tail; ++j) {
            const float vh = value_hat(p, bh, t0 + j, c);
#pragma unroll
            for (int h = 0; h < HG; ++h) acc[h] = fmaf(pl[h * PSTR + j], vh, acc[h]);
        }
#pragma unroll
        for (int h = 0; h < HG; ++h)
            p.ws_acc[((int64_t(b) * p.Hq + hq0 + h) * p.S + s) * D + c] = acc[h];
    }
    if (lane < HG) {
        const int64_t slot = (int64_t(b) * p.Hq + hq0 + lane) * p.S + s;
        p.ws_ml[slot * 2] = pick4(m, lane);
        p.ws_ml[slot * 2 + 1] = pick4(l, lane);
    }
}

// Row-of-16 reductions with DPP (quad xor 1, quad xor 2, half-row mirror,
// row mirror): afterwards every lane of the 16-lane row holds the result.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                 0xf, 0xf, false));
}
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
__device__ __forceinline__ float sel4(int i, float a, float b, float c, float d) {
    return (i & 2) ? ((i & 1) ? d : c) : ((i & 1) ? b : a);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float readlane_f(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// ---------------------------------------------------------------------------
// Two specialised waves per workgroup, software-pipelined by one tile:
//   wave 0 (keys)   tile i: stage key codes, q' = q * s_k, S = q' . codes on
//                   MFMA, online softmax -> weights p(i) and the rescale
//                   factors alpha(i) into handoff buffer i & 1;
//   wave 1 (values) tile i-1: stage value codes, rescale its accumulators by
//                   alpha(i-1), p' = p * s_v, O += p' . codes on MFMA.
// One workgroup barrier per iteration hands buffer i & 1 from wave 0 to
// wave 1; each wave prefetches its own next tile into registers right
// after staging the current one.

struct LdsK {
    uint32_t kl[4 * KSTR];                                  // key codes [word row][channel]
    __attribute__((aligned(16))) uint32_t qa[2 * 8 * QSTR];  // q' rows (fp16) per key block
    __attribute__((aligned(16))) uint32_t ksl[2 * 2 * 64];   // key [scale|zero][block][128 fp16]
    float bias[8];                                          // sigma2 * sum_c q z_k per (block, head)
};

struct LdsV {
    uint32_t vl[8 * VSTR];                                  // value codes [word][token]
    __attribute__((aligned(16))) uint32_t pa[2 * 16 * ASTR];  // p' rows (fp16) per pass
    __attribute__((aligned(16))) uint32_t vsl[2 * 128];      // value [scale|zero][token][4 fp16]
};

struct Handoff {
    __attribute__((aligned(16))) float pl[HG * PSTR];  // softmax weights [head][token]
    float alpha[HG];                                  // rescale of earlier accumulations
};

struct Lds {
    LdsK k;
    LdsV v;
    Handoff hb[2];
    float misc[64];
};

struct KTile {
    uint4 k0, k1;   // 2 KB of key codes, 32 B per lane
    uint4 ks;       // key scale (lanes 0..31) / zero (lanes 32..63)
};
struct VTile {
    uint4 v0, v1;   // 2 KB of value codes
    uint4 vs;       // value scale (lanes 0..31) / zero (lanes 32..63)
};

template <int G>
__device__ __forceinline__ void load_ktile(const GqaParams& p, int64_t bh, int64_t tt, int lane, KTile& r) {
    constexpr int NBT = 64 / G, W = G / 16;
    const uint4* kb = reinterpret_cast<const uint4*>(p.kc + (bh * p.nblk_cap + tt * NBT) * D * W);
    r.k0 = kb[lane];
    r.k1 = kb[lane + 64];
    const uint16_t* kside = (lane < 32 ? p.ks : p.kz) + (bh * p.nblk_cap + tt * NBT) * D;
    if (G == 64) {
        const uint2 v = reinterpret_cast<const uint2*>(kside)[lane & 31];
        r.ks = make_uint4(v.x, v.y, 0u, 0u);
    } else {
        r.ks = reinterpret_cast<const uint4*>(kside)[lane & 31];
    }
}

__device__ __forceinline__ void load_vtile(const GqaParams& p, int64_t bh, int64_t tt, int lane, VTile& r) {
    const uint4* vb = reinterpret_cast<const uint4*>(p.vc + (bh * p.cap + tt * 64) * 8);
    r.v0 = vb[lane];
    r.v1 = vb[lane + 64];
    const uint16_t* vside = (lane < 32 ? p.vs : p.vz) + (bh * p.cap + tt * 64) * 4;
    r.vs = reinterpret_cast<const uint4*>(vside)[lane & 31];
}

struct KState {
    float m0, m1, m2, m3;   // running maxima per head (log2 units, wave-uniform)
};

// Key side of one tile: produces p and alpha in `hb`.
template <int G>
__device__ __forceinline__ void key_tile(const GqaParams& p, KTile& cur, KState& st, LdsK& L,
                                         Handoff& hb, const float* qv, uint32_t sel, int lane,
                                         int64_t bh, int nxt, int end) {
    constexpr int NBT = 64 / G;
    const int n = lane & 15, kg = lane >> 4;
    const int hh = lane >> 4, chunk = lane & 15;

    // ---- stage key codes transposed to [word row][channel], and the side values
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint4 kw = half ? cur.k1 : cur.k0;
        const int i = lane + 64 * half;
        if (G == 64) {
            L.kl[0 * KSTR + i] = kw.x;
            L.kl[1 * KSTR + i] = kw.y;
            L.kl[2 * KSTR + i] = kw.z;
            L.kl[3 * KSTR + i] = kw.w;
        } else {
            const int be = i >> 6, c = 2 * (i & 63);
            *reinterpret_cast<uint2*>(L.kl + (2 * be) * KSTR + c) = make_uint2(kw.x, kw.z);
            *reinterpret_cast<uint2*>(L.kl + (2 * be + 1) * KSTR + c) = make_uint2(kw.y, kw.w);
        }
    }
    if (G == 64)
        *reinterpret_cast<uint2*>(L.ksl + (lane >> 5) * 128 + 2 * (lane & 31)) = make_uint2(cur.ks.x, cur.ks.y);
    else
        *reinterpret_cast<uint4*>(L.ksl + (lane >> 5) * 128 + 4 * (lane & 31)) = cur.ks;
    if (nxt < end) load_ktile<G>(p, bh, nxt, lane, cur);
    wave_sync();

    // ---- q' = q * s_k as fp16 hi/lo rows, sigma2 * sum_c q z_k per (block, head)
#pragma unroll
    for (int be = 0; be < NBT; ++be) {
        uint32_t hi[4], lo[4];
        float bias = 0.0f;
        const uint4 swv = *reinterpret_cast<const uint4*>(L.ksl + be * 64 + 4 * chunk);
        const uint4 zwv = *reinterpret_cast<const uint4*>(L.ksl + 128 + be * 64 + 4 * chunk);
        const uint32_t sw[4] = {swv.x, swv.y, swv.z, swv.w};
        const uint32_t zw[4] = {zwv.x, zwv.y, zwv.z, zwv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            split_prod2(qv[2 * i], lo_h(sw[i]), qv[2 * i + 1], hi_h(sw[i]), hi[i], lo[i]);
            bias = fmaf(qv[2 * i], lo_h(zw[i]), bias);
            bias = fmaf(qv[2 * i + 1], hi_h(zw[i]), bias);
        }
        uint32_t* row = L.qa + (be * 8 + 2 * hh) * QSTR + 4 * chunk;
        *reinterpret_cast<uint4*>(row) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *reinterpret_cast<uint4*>(row + QSTR) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        bias = row_sum16(bias);
        if (chunk == 0) L.bias[be * 4 + hh] = bias * p.sigma2;
    }
    wave_sync();

    // ---- S = q' . codes: 4 MFMA tiles of 16 tokens x 4 K-steps of 32 channels.
    // Rows 8..15 of the A operand repeat rows 0..7.
    f32x4 S[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) S[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ksx = 0; ksx < 4; ++ksx) {
#pragma unroll
        for (int be = 0; be < NBT; ++be) {
            const uint4 a = *reinterpret_cast<const uint4*>(L.qa + (be * 8 + (n & 7)) * QSTR + 16 * ksx + 4 * kg);
            const f16x8 A = as_f16x8(a.x, a.y, a.z, a.w);
            const int r = G == 64 ? (n >> 2) : (2 * be + ((n & 7) >> 2));
            const uint4* src = reinterpret_cast<const uint4*>(L.kl + r * KSTR + 32 * ksx + 8 * kg);
            const uint4 w0 = src[0], w1 = src[1];
            const uint32_t x0 = __builtin_amdgcn_perm(w0.y, w0.x, sel);
            const uint32_t x1 = __builtin_amdgcn_perm(w0.w, w0.z, sel);
            const uint32_t x2 = __builtin_amdgcn_perm(w1.y, w1.x, sel);
            const uint32_t x3 = __builtin_amdgcn_perm(w1.w, w1.z, sel);
            if (G == 64) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t mk = 0x00030003u << (2 * u);
                    S[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        A, as_f16x8(x0 & mk, x1 & mk, x2 & mk, x3 & mk), S[u], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const uint32_t mk = 0x00030003u << (2 * (2 * v + (n >> 3)));
                    S[2 * be + v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        A, as_f16x8(x0 & mk, x1 & mk, x2 & mk, x3 & mk), S[2 * be + v], 0, 0, 0);
                }
            }
        }
    }

    // ---- softmax.  Lane (n, kg) holds rows 4kg..4kg+3; rows 8..15 repeat
    // rows 0..7, so lanes kg and kg+2 see heads 2(kg&1), 2(kg&1)+1 (hi/lo row
    // pairs) and split the tiles: kg < 2 take tiles 0, 1 and kg >= 2 tiles 2, 3.
    const bool odd = (kg & 1) != 0;
    const int u0 = 2 * (kg >> 1);
    float sA[2], sB[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
        // element-wise selects keep the accumulators in registers
        const bool up2 = (kg >> 1) != 0;
        float Sv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) Sv[e] = up2 ? S[2 + v][e] : S[v][e];
        const int up = G == 64 ? u0 + v : 2 * v + (n >> 3);
        const int be = G == 64 ? 0 : (kg >> 1);
        const float f = p.sigma2 * __builtin_ldexpf(1.0f, 24 - 2 * up);
        sA[v] = fmaf(Sv[0] + Sv[1], f, L.bias[be * 4 + 2 * (kg & 1)]);
        sB[v] = fmaf(Sv[2] + Sv[3], f, L.bias[be * 4 + 2 * (kg & 1) + 1]);
    }
    // the running maxima move only when some logit exceeds them by more than
    // TAU; each lane tests its logits and one ballot decides
    float a0 = 1.0f, a1 = 1.0f, a2 = 1.0f, a3 = 1.0f;
    const float thA = (odd ? st.m2 : st.m0) + TAU, thB = (odd ? st.m3 : st.m1) + TAU;
    const bool over = fmaxf(sA[0], sA[1]) > thA || fmaxf(sB[0], sB[1]) > thB;
    if (__builtin_amdgcn_ballot_w64(over) != 0) {
        const float mA = row_max16(fmaxf(sA[0], sA[1]));
        const float mB = row_max16(fmaxf(sB[0], sB[1]));
        const float t0 = fmaxf(readlane_f(mA, 0), readlane_f(mA, 32));
        const float t1 = fmaxf(readlane_f(mB, 0), readlane_f(mB, 32));
        const float t2 = fmaxf(readlane_f(mA, 16), readlane_f(mA, 48));
        const float t3 = fmaxf(readlane_f(mB, 16), readlane_f(mB, 48));
        const float n0 = fmaxf(st.m0, t0), n1 = fmaxf(st.m1, t1);
        const float n2 = fmaxf(st.m2, t2), n3 = fmaxf(st.m3, t3);
        a0 = fast_exp2(st.m0 - n0);
        a1 = fast_exp2(st.m1 - n1);
        a2 = fast_exp2(st.m2 - n2);
        a3 = fast_exp2(st.m3 - n3);
        st.m0 = n0;
        st.m1 = n1;
        st.m2 = n2;
        st.m3 = n3;
    }
    const float mrA = odd ? st.m2 : st.m0, mrB = odd ? st.m3 : st.m1;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
        sA[v] = fast_exp2(sA[v] - mrA);
        sB[v] = fast_exp2(sB[v] - mrB);
    }
    const int hA = 2 * (kg & 1), hB = hA + 1;
    if (G == 64) {
        *reinterpret_cast<float2*>(hb.pl + hA * PSTR + 4 * n + u0) = make_float2(sA[0], sA[1]);
        *reinterpret_cast<float2*>(hb.pl + hB * PSTR + 4 * n + u0) = make_float2(sB[0], sB[1]);
    } else {
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int t = 32 * (kg >> 1) + 16 * ((n & 7) >> 2) + 4 * (n & 3) + 2 * v + (n >> 3);
            hb.pl[hA * PSTR + t] = sA[v];
            hb.pl[hB * PSTR + t] = sB[v];
        }
    }
    if (lane < HG) hb.alpha[lane] = sel4(lane, a0, a1, a2, a3);
}

struct VState {
    f32x4 O[2][4];   // PV accumulators [pass][channel tile]
    float lsum;      // this lane's share of sum p for head (lane >> 4)
    float vb[4];     // this lane's share of sum p z_v per group, head (lane >> 4)
};

// Value side of one tile, reading p and alpha from `hb`.
__device__ __forceinline__ void value_tile(const GqaParams& p, VTile& cur, VState& st, LdsV& L,
                                           const Handoff& hb, uint32_t sel, int lane, int64_t bh,
                                           int nxt, int end) {
    const int n = lane & 15, kg = lane >> 4;
    const int hh = lane >> 4, chunk = lane & 15;
    // ---- stage value codes transposed to [word][token], and the side values
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint4 vw = half ? cur.v1 : cur.v0;
        const int i = lane + 64 * half;
        const int tok = i >> 1, w0 = 4 * (i & 1);
        L.vl[(w0 + 0) * VSTR + tok] = vw.x;
        L.vl[(w0 + 1) * VSTR + tok] = vw.y;
        L.vl[(w0 + 2) * VSTR + tok] = vw.z;
        L.vl[(w0 + 3) * VSTR + tok] = vw.w;
    }
    *reinterpret_cast<uint4*>(L.vsl + (lane >> 5) * 128 + 4 * (lane & 31)) = cur.vs;
    if (nxt < end) load_vtile(p, bh, nxt, lane, cur);

    // ---- rescale what was accumulated with the previous maxima
    const float a0 = hb.alpha[0], a1 = hb.alpha[1], a2 = hb.alpha[2], a3 = hb.alpha[3];
    if (fminf(fminf(a0, a1), fminf(a2, a3)) < 1.0f) {
        const bool odd = (kg & 1) != 0;
        const float aA = odd ? a2 : a0, aB = odd ? a3 : a1;
#pragma unroll
        for (int P = 0; P < 2; ++P)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                st.O[P][u][0] *= aA;
                st.O[P][u][1] *= aA;
                st.O[P][u][2] *= aB;
                st.O[P][u][3] *= aB;
            }
        const float ah = sel4(hh, a0, a1, a2, a3);
        st.lsum *= ah;
#pragma unroll
        for (int g = 0; g < 4; ++g) st.vb[g] *= ah;
    }
    wave_sync();

    // ---- p' = p * s_v as fp16 hi/lo rows per value group; sum_t p, sum_t p z_v
    {
        const float4 pv4 = *reinterpret_cast<const float4*>(hb.pl + hh * PSTR + 4 * chunk);
        const float pv[4] = {pv4.x, pv4.y, pv4.z, pv4.w};
        st.lsum += (pv[0] + pv[1]) + (pv[2] + pv[3]);
        // scale / zero halves of token t (0..3), group g (0..3) at half index 4t + g
        const uint4* svp = reinterpret_cast<const uint4*>(L.vsl + 8 * chunk);
        const uint4* zvp = reinterpret_cast<const uint4*>(L.vsl + 128 + 8 * chunk);
        const uint4 s0 = svp[0], s1 = svp[1], z0 = zvp[0], z1 = zvp[1];
        const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const uint32_t zw[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float sv[4], zv[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int hidx = 4 * t + g;
                sv[t] = (hidx & 1) ? hi_h(sw[hidx >> 1]) : lo_h(sw[hidx >> 1]);
                zv[t] = (hidx & 1) ? hi_h(zw[hidx >> 1]) : lo_h(zw[hidx >> 1]);
            }
            uint32_t h01, l01, h23, l23;
            split_prod2(pv[0], sv[0], pv[1], sv[1], h01, l01);
            split_prod2(pv[2], sv[2], pv[3], sv[3], h23, l23);
            // row ((pass*2 + gsel)*4 + head)*2 + hl; 64 tokens = 32 dwords per row
            uint32_t* rowp = L.pa + ((((g >> 1) * 2 + (g & 1)) * 4 + hh) * 2) * ASTR + 2 * chunk;
            *reinterpret_cast<uint2*>(rowp) = make_uint2(h01, h23);
            *reinterpret_cast<uint2*>(rowp + ASTR) = make_uint2(l01, l23);
            float z = st.vb[g];
#pragma unroll
            for (int t = 0; t < 4; ++t) z = fmaf(pv[t], zv[t], z);
            st.vb[g] = z;
        }
    }
    wave_sync();

    // ---- O += p' . codes: 2 passes x 4 channel tiles x 2 K-steps of 32 tokens
#pragma unroll
    for (int P = 0; P < 2; ++P) {
        const int wi = 4 * P + 2 * (n >> 3) + ((n & 7) >> 2);
#pragma unroll
        for (int ksx = 0; ksx < 2; ++ksx) {
            const uint4 a = *reinterpret_cast<const uint4*>(L.pa + (P * 16 + n) * ASTR + 16 * ksx + 4 * kg);
            const f16x8 A = as_f16x8(a.x, a.y, a.z, a.w);
            const uint4* src = reinterpret_cast<const uint4*>(L.vl + wi * VSTR + 32 * ksx + 8 * kg);
            const uint4 w0 = src[0], w1 = src[1];
            const uint32_t x0 = __builtin_amdgcn_perm(w0.y, w0.x, sel);
            const uint32_t x1 = __builtin_amdgcn_perm(w0.w, w0.z, sel);
            const uint32_t x2 = __builtin_amdgcn_perm(w1.y, w1.x, sel);
            const uint32_t x3 = __builtin_amdgcn_perm(w1.w, w1.z, sel);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t mk = 0x00030003u << (2 * u);
                st.O[P][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    A, as_f16x8(x0 & mk, x1 & mk, x2 & mk, x3 & mk), st.O[P][u], 0, 0, 0);
            }
        }
    }
}

template <int G>
__global__ __launch_bounds__(128) void k_decode_gqa(GqaParams p) {
    __shared__ Lds L;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = lane & 15, kg = lane >> 4;
    const int hh = lane >> 4, chunk = lane & 15;
    const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int64_t bh = int64_t(b) * p.Hkv + kvh;
    const int hq0 = kvh * HG;
    if (s >= p.S_main) {
        if (wave == 0) tail_split(p, b, kvh, s, reinterpret_cast<float*>(L.k.qa), L.hb[0].pl);
        return;
    }
    const int t_lo = int(int64_t(s) * p.ntiles / p.S_main);
    const int t_hi = int(int64_t(s + 1) * p.ntiles / p.S_main);
    const int ntl = t_hi - t_lo;
    // v_perm selector: byte (n & 3) of the low-channel (or low-token) word ->
    // byte 0, of the high one -> byte 2, zero bytes 1 and 3
    const uint32_t bsel = uint32_t(n & 3);
    const uint32_t sel = bsel | (0x0cu << 8) | ((4u + bsel) << 16) | (0x0cu << 24);

    if (wave == 0) {
        float qv[8];
        {
            const uint4 raw = *reinterpret_cast<const uint4*>(p.q + ((int64_t(b) * p.Hq + hq0 + hh) * D + 8 * chunk));
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qv[2 * i] = lo_h(w[i]);
                qv[2 * i + 1] = hi_h(w[i]);
            }
        }
        KState st;
        st.m0 = st.m1 = st.m2 = st.m3 = -INFINITY;
        // two register tiles in flight: tile t is staged from set (t & 1),
        // which then receives tile t + 2
        KTile ta, tb;
        load_ktile<G>(p, bh, t_lo, lane, ta);
        if (ntl > 1) load_ktile<G>(p, bh, t_lo + 1, lane, tb);
        for (int it = 0; it <= ntl; it += 2) {
            if (it < ntl) key_tile<G>(p, ta, st, L.k, L.hb[0], qv, sel, lane, bh, t_lo + it + 2, t_hi);
            if (it == ntl && lane < HG) L.misc[lane] = sel4(lane, st.m0, st.m1, st.m2, st.m3);
            __syncthreads();
            if (it + 1 > ntl) break;
            if (it + 1 < ntl) key_tile<G>(p, tb, st, L.k, L.hb[1], qv, sel, lane, bh, t_lo + it + 3, t_hi);
            if (it + 1 == ntl && lane < HG) L.misc[lane] = sel4(lane, st.m0, st.m1, st.m2, st.m3);
            __syncthreads();
        }
    } else {
        VState st;
        st.lsum = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) st.vb[g] = 0.0f;
#pragma unroll
        for (int P = 0; P < 2; ++P)
#pragma unroll
            for (int u = 0; u < 4; ++u) st.O[P][u] = f32x4{0.f, 0.f, 0.f, 0.f};
        // value work trails the key work by one tile (tile it - 1 at step it)
        VTile ta, tb;
        load_vtile(p, bh, t_lo, lane, ta);
        if (ntl > 1) load_vtile(p, bh, t_lo + 1, lane, tb);
        for (int it = 0; it <= ntl; it += 2) {
            if (it >= 1) value_tile(p, tb, st, L.v, L.hb[1], sel, lane, bh, t_lo + it + 1, t_hi);
            __syncthreads();
            if (it + 1 > ntl) break;
            value_tile(p, ta, st, L.v, L.hb[0], sel, lane, bh, t_lo + it + 2, t_hi);
            __syncthreads();
        }
        // ---- epilogue: l and the value-zero sums over the 16 lanes of a head
        const float lsum = row_sum16(st.lsum);
        float vbs[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) vbs[g] = row_sum16(st.vb[g]);
        if (chunk == 0) {
            L.misc[16 + hh] = lsum;
#pragma unroll
            for (int g = 0; g < 4; ++g) L.misc[32 + hh * 4 + g] = vbs[g];
        }
        wave_sync();
        if ((kg >> 1) == (n >> 3)) {
#pragma unroll
            for (int P = 0; P < 2; ++P)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int c = 64 * P + 32 * (n >> 3) + 4 * (n & 7) + u;
                    const int g = 2 * P + (n >> 3);
                    const float f = __builtin_ldexpf(1.0f, 24 - 2 * u);
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int h = 2 * (kg & 1) + j;
                        const float acc = fmaf(st.O[P][u][2 * j] + st.O[P][u][2 * j + 1], f, L.misc[32 + h * 4 + g]);
                        p.ws_acc[((int64_t(b) * p.Hq + hq0 + h) * p.S + s) * D + c] = acc;
                    }
                }
        }
        if (lane < HG) {
            const int64_t slot = (int64_t(b) * p.Hq + hq0 + lane) * p.S + s;
            p.ws_ml[slot * 2] = L.misc[lane];
            p.ws_ml[slot * 2 + 1] = L.misc[16 + lane];
        }
    }
}

}  // namespace

bool gqa_supported(const kvq_cache& c, int Hq) {
    const kvq_cache_cfg& g = c.cfg;
    return g.kind == KVQ_KIND_KIVI && g.key.bits == 2 && g.value.bits == 2 && g.key.dim == D &&
           g.value.dim == D && g.value.group == 32 && (g.key.group == 32 || g.key.group == 64) &&
           Hq == HG * g.n_kv_heads;
}

hipError_t launch_decode_gqa(const DecodeArgs& a, hipStream_t st) {
    const kvq_cache& c = *a.c;
    GqaParams p;
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
    p.Hkv = a.g.Hkv;
    p.S = a.S;
    p.S_main = a.S_main;
    p.ntiles = a.ntiles;
    p.G = a.g.kG;
    p.T = a.T;
    p.nblk = a.nblk;
    p.cap = a.g.cap;
    p.nblk_cap = a.g.nblk_cap;
    p.sigma2 = a.sigma * 1.4426950408889634f;
    const dim3 grid(a.S, a.g.Hkv, a.g.B);
    if (a.g.kG == 64)
        hipLaunchKernelGGL(k_decode_gqa<64>, grid, dim3(128), 0, st, p);
    else
        hipLaunchKernelGGL(k_decode_gqa<32>, grid, dim3(128), 0, st, p);
    return hipGetLastError();
}

}  // namespace kvq
