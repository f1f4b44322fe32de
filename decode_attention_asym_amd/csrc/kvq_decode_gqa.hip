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
constexpr int VSTR = 72;    // dwords per row of the value-code tile in LDS
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
    uint4 ksc[2], kze[2];     // key scale / zero of 8 channels, per block of the tile
    uint4 vsc[2], vze[2];     // value scale / zero of 4 tokens x 4 groups
};

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
__device__ __forceinline__ float lo_h(uint32_t w) { return h2f(uint16_t(w & 0xffffu)); }
__device__ __forceinline__ float hi_h(uint32_t w) { return h2f(uint16_t(w >> 16)); }

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

template <int G>
__device__ __forceinline__ void load_tile(const GqaParams& p, int64_t bh, int64_t tt, int lane,
                                          Tile& r) {
    constexpr int NBT = 64 / G, W = G / 16;
    const int chunk = lane & 15;
    const uint4* kb = reinterpret_cast<const uint4*>(p.kc + (bh * p.nblk_cap + tt * NBT) * D * W);
    r.k0 = kb[lane];
    r.k1 = kb[lane + 64];
    const uint4* vb = reinterpret_cast<const uint4*>(p.vc + (bh * p.cap + tt * 64) * 8);
    r.v0 = vb[lane];
    r.v1 = vb[lane + 64];
#pragma unroll
    for (int be = 0; be < NBT; ++be) {
        const int64_t side = (bh * p.nblk_cap + tt * NBT + be) * D + 8 * chunk;
        r.ksc[be] = *reinterpret_cast<const uint4*>(p.ks + side);
        r.kze[be] = *reinterpret_cast<const uint4*>(p.kz + side);
    }
    const int64_t vside = (bh * p.cap + tt * 64 + 4 * chunk) * 4;
    r.vsc[0] = reinterpret_cast<const uint4*>(p.vs + vside)[0];
    r.vsc[1] = reinterpret_cast<const uint4*>(p.vs + vside)[1];
    r.vze[0] = reinterpret_cast<const uint4*>(p.vz + vside)[0];
    r.vze[1] = reinterpret_cast<const uint4*>(p.vz + vside)[1];
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
__device__ void tail_split(const GqaParams& p, int b, int kvh, int s, float* qf, float* pl) {
    const int lane = threadIdx.x;
    const int64_t bh = int64_t(b) * p.Hkv + kvh;
    const int hq0 = kvh * HG;
    for (int i = lane; i < HG * D; i += 64) qf[i] = h2f(p.q[(int64_t(b) * p.Hq + hq0) * D + i]);
    __syncthreads();
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
    __syncthreads();
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

template <int G>
__global__ __launch_bounds__(64) void k_decode_gqa(GqaParams p) {
    constexpr int NBT = 64 / G;   // key blocks per 64-token tile
    __shared__ uint32_t kl[4 * KSTR];
    __shared__ uint32_t vl[8 * VSTR];
    __shared__ __attribute__((aligned(16))) uint32_t ab[1024];  // q' rows, later p' rows (fp16)
    __shared__ __attribute__((aligned(16))) float pl[HG * PSTR];
    __shared__ float misc[64];

    const int lane = threadIdx.x;
    const int n = lane & 15, kg = lane >> 4;   // MFMA operand lane roles
    const int hh = lane >> 4, chunk = lane & 15;  // q' / p' lane roles
    const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int64_t bh = int64_t(b) * p.Hkv + kvh;
    const int hq0 = kvh * HG;
    if (s >= p.S_main) {
        tail_split(p, b, kvh, s, reinterpret_cast<float*>(ab), pl);
        return;
    }
    const int t_lo = int(int64_t(s) * p.ntiles / p.S_main);
    const int t_hi = int(int64_t(s + 1) * p.ntiles / p.S_main);

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
    // v_perm selector: byte (n & 3) of the low-channel word -> byte 0, of the
    // high-channel word -> byte 2, zero bytes 1 and 3
    const uint32_t bsel = uint32_t(n & 3);
    const uint32_t sel = bsel | (0x0cu << 8) | ((4u + bsel) << 16) | (0x0cu << 24);

    float m_run[HG] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    float lsum = 0.0f;
    float vb[4] = {0.f, 0.f, 0.f, 0.f};
    f32x4 O[2][4];
#pragma unroll
    for (int P = 0; P < 2; ++P)
#pragma unroll
        for (int u = 0; u < 4; ++u) O[P][u] = f32x4{0.f, 0.f, 0.f, 0.f};

    Tile cur, nxt;
    load_tile<G>(p, bh, t_lo, lane, cur);
    for (int tt = t_lo; tt < t_hi; ++tt) {
        if (tt + 1 < t_hi) load_tile<G>(p, bh, tt + 1, lane, nxt);

        // ---- 1. stage the code tiles in LDS, transposed to [word row][channel | token]
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint4 kw = half ? cur.k1 : cur.k0;
            const int i = lane + 64 * half;
            if (G == 64) {
#pragma unroll
                for (int j = 0; j < 4; ++j) kl[j * KSTR + i] = word_of(kw, j);
            } else {
                const int be = i >> 6, c = 2 * (i & 63);
                kl[(2 * be) * KSTR + c] = kw.x;
                kl[(2 * be + 1) * KSTR + c] = kw.y;
                kl[(2 * be) * KSTR + c + 1] = kw.z;
                kl[(2 * be + 1) * KSTR + c + 1] = kw.w;
            }
            const uint4 vw = half ? cur.v1 : cur.v0;
            const int tok = i >> 1, w0 = 4 * (i & 1);
#pragma unroll
            for (int e = 0; e < 4; ++e) vl[(w0 + e) * VSTR + tok] = word_of(vw, e);
        }

        // ---- 2. q' = q * s_k (hi/lo rows) and the zero bias per (head, block)
#pragma unroll
        for (int be = 0; be < NBT; ++be) {
            uint32_t hi[4], lo[4];
            float bias = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t sw = word_of(cur.ksc[be], i), zw = word_of(cur.kze[be], i);
                split2(qv[2 * i] * lo_h(sw), qv[2 * i + 1] * hi_h(sw), hi[i], lo[i]);
                bias = fmaf(qv[2 * i], lo_h(zw), bias);
                bias = fmaf(qv[2 * i + 1], hi_h(zw), bias);
            }
            uint4* row = reinterpret_cast<uint4*>(ab + (be * 8 + 2 * hh) * 64 + 4 * chunk);
            row[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            row[16] = make_uint4(lo[0], lo[1], lo[2], lo[3]);   // next row (64 dwords on)
            bias = xor_sum16(bias);
            if (chunk == 0) misc[be * 4 + hh] = bias * p.sigma2;
        }
        __syncthreads();

        // ---- 3. S = q' . codes on MFMA: 4 tiles of 16 tokens x 4 K-steps of 32 channels
        f32x4 S[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) S[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ksx = 0; ksx < 4; ++ksx) {
            f16x8 A[NBT];
#pragma unroll
            for (int be = 0; be < NBT; ++be) {
                if (n < 8) {
                    const uint4 a = *reinterpret_cast<const uint4*>(ab + (be * 8 + n) * 64 + 16 * ksx + 4 * kg);
                    A[be] = as_f16x8(a.x, a.y, a.z, a.w);
                } else {
                    A[be] = as_f16x8(0u, 0u, 0u, 0u);
                }
            }
#pragma unroll
            for (int be = 0; be < NBT; ++be) {
                const int r = G == 64 ? (n >> 2) : (2 * be + ((n & 7) >> 2));
                const uint4* src = reinterpret_cast<const uint4*>(kl + r * KSTR + 32 * ksx + 8 * kg);
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
                            A[0], as_f16x8(x0 & mk, x1 & mk, x2 & mk, x3 & mk), S[u], 0, 0, 0);
                    }
                } else {
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        const int up = 2 * v + (n >> 3);
                        const uint32_t mk = 0x00030003u << (2 * up);
                        S[2 * be + v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            A[be], as_f16x8(x0 & mk, x1 & mk, x2 & mk, x3 & mk), S[2 * be + v], 0, 0, 0);
                    }
                }
            }
        }

        // ---- 4. softmax: lane (n, kg<2) holds heads 2kg (rows 0,1) and 2kg+1 (rows 2,3)
        const int hA = 2 * (kg & 1), hB = hA + 1;
        float sA[4], sB[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int up = G == 64 ? u : 2 * (u & 1) + (n >> 3);
            const int be = G == 64 ? 0 : (u >> 1);
            const float f = p.sigma2 * __builtin_ldexpf(1.0f, 24 - 2 * up);
            sA[u] = fmaf(S[u][0] + S[u][1], f, misc[be * 4 + hA]);
            sB[u] = fmaf(S[u][2] + S[u][3], f, misc[be * 4 + hB]);
        }
        const float mA = xor_max16(fmaxf(fmaxf(sA[0], sA[1]), fmaxf(sA[2], sA[3])));
        const float mB = xor_max16(fmaxf(fmaxf(sB[0], sB[1]), fmaxf(sB[2], sB[3])));
        float tmax[HG];
        tmax[0] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mA), 0));
        tmax[1] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mB), 0));
        tmax[2] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mA), 16));
        tmax[3] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mB), 16));
        bool resc = false;
#pragma unroll
        for (int h = 0; h < HG; ++h) resc |= tmax[h] > m_run[h] + TAU;
        if (resc) {
            float alpha[HG];
#pragma unroll
            for (int h = 0; h < HG; ++h) {
                const float mn = fmaxf(m_run[h], tmax[h]);
                alpha[h] = exp2f(m_run[h] - mn);
                m_run[h] = mn;
            }
            const float a0 = pick4(alpha, 2 * (kg & 1)), a1 = pick4(alpha, 2 * (kg & 1) + 1);
#pragma unroll
            for (int P = 0; P < 2; ++P)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    O[P][u][0] *= a0;
                    O[P][u][1] *= a0;
                    O[P][u][2] *= a1;
                    O[P][u][3] *= a1;
                }
            const float ah = pick4(alpha, hh);
            lsum *= ah;
#pragma unroll
            for (int g = 0; g < 4; ++g) vb[g] *= ah;
        }
        const float mrA = pick4(m_run, hA), mrB = pick4(m_run, hB);
        if (kg < 2) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                sA[u] = exp2f(sA[u] - mrA);
                sB[u] = exp2f(sB[u] - mrB);
            }
            if (G == 64) {
                *reinterpret_cast<float4*>(pl + hA * PSTR + 4 * n) = make_float4(sA[0], sA[1], sA[2], sA[3]);
                *reinterpret_cast<float4*>(pl + hB * PSTR + 4 * n) = make_float4(sB[0], sB[1], sB[2], sB[3]);
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int t = 32 * (u >> 1) + 16 * ((n & 7) >> 2) + 4 * (n & 3) + 2 * (u & 1) + (n >> 3);
                    pl[hA * PSTR + t] = sA[u];
                    pl[hB * PSTR + t] = sB[u];
                }
            }
        }
        __syncthreads();

        // ---- 5. p' = p * s_v (hi/lo rows) per value group; sum_t p and sum_t p z_v
        {
            const float4 pv4 = *reinterpret_cast<const float4*>(pl + hh * PSTR + 4 * chunk);
            const float pv[4] = {pv4.x, pv4.y, pv4.z, pv4.w};
            lsum += (pv[0] + pv[1]) + (pv[2] + pv[3]);
            // scale / zero halves: token t (0..3), group g at half index 4t + g
            float sv[4][4], zv[4][4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int g = 0; g < 4; g += 2) {
                    const int hidx = 4 * t + g;
                    const uint32_t sw = word_of(cur.vsc[hidx >> 3], (hidx & 7) >> 1);
                    const uint32_t zw = word_of(cur.vze[hidx >> 3], (hidx & 7) >> 1);
                    sv[t][g] = lo_h(sw);
                    sv[t][g + 1] = hi_h(sw);
                    zv[t][g] = lo_h(zw);
                    zv[t][g + 1] = hi_h(zw);
                }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint32_t h01, l01, h23, l23;
                split2(pv[0] * sv[0][g], pv[1] * sv[1][g], h01, l01);
                split2(pv[2] * sv[2][g], pv[3] * sv[3][g], h23, l23);
                // row ((pass*2 + gsel)*4 + head)*2 + hl, 64 tokens = 32 dwords per row
                uint32_t* rowp = ab + ((((g >> 1) * 2 + (g & 1)) * 4 + hh) * 2) * 32 + 2 * chunk;
                *reinterpret_cast<uint2*>(rowp) = make_uint2(h01, h23);
                *reinterpret_cast<uint2*>(rowp + 32) = make_uint2(l01, l23);
                vb[g] = fmaf(pv[0], zv[0][g], vb[g]);
                vb[g] = fmaf(pv[1], zv[1][g], vb[g]);
                vb[g] = fmaf(pv[2], zv[2][g], vb[g]);
                vb[g] = fmaf(pv[3], zv[3][g], vb[g]);
            }
        }
        __syncthreads();

        // ---- 6. O += p' . codes on MFMA: 2 passes x 4 channel tiles x 2 K-steps of 32 tokens
#pragma unroll
        for (int P = 0; P < 2; ++P) {
            const int wi = 4 * P + 2 * (n >> 3) + ((n & 7) >> 2);
#pragma unroll
            for (int ksx = 0; ksx < 2; ++ksx) {
                const uint4 a = *reinterpret_cast<const uint4*>(ab + (P * 16 + n) * 32 + 16 * ksx + 4 * kg);
                const f16x8 A = as_f16x8(a.x, a.y, a.z, a.w);
                const uint4* src = reinterpret_cast<const uint4*>(vl + wi * VSTR + 32 * ksx + 8 * kg);
                const uint4 w0 = src[0], w1 = src[1];
                const uint32_t x0 = __builtin_amdgcn_perm(w0.y, w0.x, sel);
                const uint32_t x1 = __builtin_amdgcn_perm(w0.w, w0.z, sel);
                const uint32_t x2 = __builtin_amdgcn_perm(w1.y, w1.x, sel);
                const uint32_t x3 = __builtin_amdgcn_perm(w1.w, w1.z, sel);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t mk = 0x00030003u << (2 * u);
                    O[P][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        A, as_f16x8(x0 & mk, x1 & mk, x2 & mk, x3 & mk), O[P][u], 0, 0, 0);
                }
            }
        }
        __syncthreads();
        cur = nxt;
    }

    // ---- epilogue: reduce l and the value-zero sums over the 16 lanes of a head
    lsum = xor_sum16(lsum);
#pragma unroll
    for (int g = 0; g < 4; ++g) vb[g] = xor_sum16(vb[g]);
    if (chunk == 0) {
        misc[16 + hh] = lsum;
#pragma unroll
        for (int g = 0; g < 4; ++g) misc[32 + hh * 4 + g] = vb[g];
    }
    __syncthreads();
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
                    const float acc = fmaf(O[P][u][2 * j] + O[P][u][2 * j + 1], f, misc[32 + h * 4 + g]);
                    p.ws_acc[((int64_t(b) * p.Hq + hq0 + h) * p.S + s) * D + c] = acc;
                }
            }
    }
    if (lane < HG) {
        const int64_t slot = (int64_t(b) * p.Hq + hq0 + lane) * p.S + s;
        p.ws_ml[slot * 2] = pick4(m_run, lane);
        p.ws_ml[slot * 2 + 1] = misc[16 + lane];
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
        hipLaunchKernelGGL(k_decode_gqa<64>, grid, dim3(64), 0, st, p);
    else
        hipLaunchKernelGGL(k_decode_gqa<32>, grid, dim3(64), 0, st, p);
    return hipGetLastError();
}

}  // namespace kvq
