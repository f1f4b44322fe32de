// kvq_mfma_tiles.h -- device pieces shared by the MFMA decode kernels for
// KIVI caches with head dim 128, 2-bit keys (G = 32 or 64) and 2-bit values
// in 32-channel groups: tile loads, LDS staging, register helpers and the
// VALU path for the trailing tokens.  Included by kvq_decode_gqa.hip and
// kvq_decode_mha.hip only.
//
// Method ("Makale Bülteni -- KIVI", section "İddia ve Gerçeklik: KIVI"):
// khat = code * s + z with s, z per (key block, channel); vhat = code * s + z
// with s, z per (token, 32-channel group); the keys of the block that is not
// yet full are fp16.
#pragma once

#include <hip/hip_fp16.h>
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Streaming loads: every cache byte is read once per decode step, so the
// loads carry the non-temporal hint and do not displace other lines from
// the L2 and the Infinity Cache (measured on MI355X: a load pattern of this
// shape streams at ~6.8 TB/s with the hint and ~5.7 TB/s without).
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream(const uint2* p) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v.x, v.y);
}

constexpr int D = 128;      // head dim
constexpr int KSTR = 136;   // dwords per row of the key-code tile in LDS
constexpr int VSTR = 76;    // dwords per row of the value-code tile in LDS
constexpr int QSTR = 68;    // dwords per q' row (128 fp16 + pad)
constexpr int ASTR = 36;    // dwords per p' row (64 fp16 + pad)
constexpr int PSTR = 68;    // floats per row of the weight tile in LDS
constexpr float TAU = 8.0f; // lazy-rescale threshold (log2 units)

struct MfmaParams {
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

inline MfmaParams mfma_params(const DecodeArgs& a) {
    const kvq_cache& c = *a.c;
    MfmaParams p;
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
    return p;
}

// The shapes these kernels take: KIVI, D = 128, 2-bit keys and values,
// 32-channel value groups, G in {32, 64}.
inline bool mfma_shape_ok(const kvq_cache& c) {
    const kvq_cache_cfg& g = c.cfg;
    return g.kind == KVQ_KIND_KIVI && g.key.bits == 2 && g.value.bits == 2 && g.key.dim == D &&
           g.value.dim == D && g.value.group == 32 && (g.key.group == 32 || g.key.group == 64);
}

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

// hi/lo split of the products a0*b0, a1*b1 (a fp32, b an fp16 half): the
// remainders are single fused operations a*b - hi
__device__ __forceinline__ void split_prod2(float a0, float b0, float a1, float b1, uint32_t& hi,
                                            uint32_t& lo) {
    // fma(a, b, +0) is one v_fma_mix with the fp16 operand read in place
    // (it cannot become a plain multiply: they differ for a*b == -0)
    hi = pk_rtz(fmaf(a0, b0, 0.0f), fmaf(a1, b1, 0.0f));
    lo = pk_rtz(fmaf(a0, b0, -lo_h(hi)), fmaf(a1, b1, -hi_h(hi)));
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
// sum over the whole wave, returned to every lane
__device__ __forceinline__ float wave_sum(float x) {
    x = row_sum16(x);
    return (readlane_f(x, 0) + readlane_f(x, 16)) + (readlane_f(x, 32) + readlane_f(x, 48));
}

// Orders this wave's LDS accesses (the waves of a workgroup are otherwise
// only ordered by the workgroup barriers).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// ---- one 64-token tile in registers, 16-byte loads, no lane reads what
// another lane reads: key codes 2 KB, key side 512 B (G = 64) or 1 KB
// (G = 32); value codes 2 KB, value side 1 KB.

struct KTile {
    uint4 k0, k1;   // key codes, 32 B per lane
    uint4 ks;       // key scale (lanes 0..31) / zero (lanes 32..63)
};
struct VTile {
    uint4 v0, v1;   // value codes
    uint4 vs;       // value scale (lanes 0..31) / zero (lanes 32..63)
};

template <int G>
__device__ __forceinline__ void load_ktile(const MfmaParams& p, int64_t bh, int64_t tt, int lane, KTile& r) {
    constexpr int NBT = 64 / G, W = G / 16;
    const uint4* kb = reinterpret_cast<const uint4*>(p.kc + (bh * p.nblk_cap + tt * NBT) * D * W);
    r.k0 = ld_stream(kb + lane);
    r.k1 = ld_stream(kb + lane + 64);
    const uint16_t* kside = (lane < 32 ? p.ks : p.kz) + (bh * p.nblk_cap + tt * NBT) * D;
    if (G == 64) {
        const uint2 v = ld_stream(reinterpret_cast<const uint2*>(kside) + (lane & 31));
        r.ks = make_uint4(v.x, v.y, 0u, 0u);
    } else {
        r.ks = ld_stream(reinterpret_cast<const uint4*>(kside) + (lane & 31));
    }
}

__device__ __forceinline__ void load_vtile(const MfmaParams& p, int64_t bh, int64_t tt, int lane, VTile& r) {
    const uint4* vb = reinterpret_cast<const uint4*>(p.vc + (bh * p.cap + tt * 64) * 8);
    r.v0 = ld_stream(vb + lane);
    r.v1 = ld_stream(vb + lane + 64);
    const uint16_t* vside = (lane < 32 ? p.vs : p.vz) + (bh * p.cap + tt * 64) * 4;
    r.vs = ld_stream(reinterpret_cast<const uint4*>(vside) + (lane & 31));
}

// Key codes transposed to kl [word row][channel] (a word row holds 16 tokens
// of every channel; G = 32 tiles hold two blocks, rows 2be and 2be + 1), and
// the side values to ksl [scale | zero][block][128 fp16].
template <int G>
__device__ __forceinline__ void stage_keys(const KTile& cur, uint32_t* kl, uint32_t* ksl, int lane) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint4 kw = half ? cur.k1 : cur.k0;
        const int i = lane + 64 * half;
        if (G == 64) {
            kl[0 * KSTR + i] = kw.x;
            kl[1 * KSTR + i] = kw.y;
            kl[2 * KSTR + i] = kw.z;
            kl[3 * KSTR + i] = kw.w;
        } else {
            const int be = i >> 6, c = 2 * (i & 63);
            *reinterpret_cast<uint2*>(kl + (2 * be) * KSTR + c) = make_uint2(kw.x, kw.z);
            *reinterpret_cast<uint2*>(kl + (2 * be + 1) * KSTR + c) = make_uint2(kw.y, kw.w);
        }
    }
    if (G == 64)
        *reinterpret_cast<uint2*>(ksl + (lane >> 5) * 128 + 2 * (lane & 31)) = make_uint2(cur.ks.x, cur.ks.y);
    else
        *reinterpret_cast<uint4*>(ksl + (lane >> 5) * 128 + 4 * (lane & 31)) = cur.ks;
}

// Value codes transposed to vl [word][token], and the side values to
// vsl [scale | zero][token][4 fp16].
__device__ __forceinline__ void stage_values(const VTile& cur, uint32_t* vl, uint32_t* vsl, int lane) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint4 vw = half ? cur.v1 : cur.v0;
        const int i = lane + 64 * half;
        const int tok = i >> 1, w0 = 4 * (i & 1);
        vl[(w0 + 0) * VSTR + tok] = vw.x;
        vl[(w0 + 1) * VSTR + tok] = vw.y;
        vl[(w0 + 2) * VSTR + tok] = vw.z;
        vl[(w0 + 3) * VSTR + tok] = vw.w;
    }
    *reinterpret_cast<uint4*>(vsl + (lane >> 5) * 128 + 4 * (lane & 31)) = cur.vs;
}

// v_perm selector: byte (n & 3) of the low-channel (or low-token) word ->
// byte 0, of the high one -> byte 2, zero bytes 1 and 3
__device__ __forceinline__ uint32_t perm_selector(int n) {
    const uint32_t bsel = uint32_t(n & 3);
    return bsel | (0x0cu << 8) | ((4u + bsel) << 16) | (0x0cu << 24);
}

// ---- trailing tokens [ntiles*64, T) on the VALU: partial key block and the
// fp16 residual keys, one token per lane for the logits, two channels per
// lane for the values.  Runs on one wave; qf holds HG*D floats, pl HG*PSTR.

__device__ __forceinline__ float key_hat(const MfmaParams& p, int64_t bh, int64_t t, int c) {
    const int64_t Tq = p.nblk * p.G;
    if (t >= Tq) return h2f(p.kr[(bh * p.G + (t - Tq)) * D + c]);
    const int64_t blk = t / p.G;
    const int i = int(t - blk * p.G);
    const int64_t side = (bh * p.nblk_cap + blk) * D + c;
    const uint32_t w = p.kc[side * (p.G / 16) + i / 16];
    return fmaf(float((w >> (2 * (i & 15))) & 3u), h2f(p.ks[side]), h2f(p.kz[side]));
}

__device__ __forceinline__ float value_hat(const MfmaParams& p, int64_t bh, int64_t t, int c) {
    const int64_t row = bh * p.cap + t;
    const uint32_t w = p.vc[row * 8 + c / 16];
    const int64_t side = row * 4 + c / 32;
    return fmaf(float((w >> (2 * (c & 15))) & 3u), h2f(p.vs[side]), h2f(p.vz[side]));
}

template <int HG>
__device__ void tail_split(const MfmaParams& p, int b, int kvh, int s, float* qf, float* pl) {
    const int lane = threadIdx.x & 63;
    const int64_t bh = int64_t(b) * p.Hkv + kvh;
    const int hq0 = kvh * HG;
    for (int i = lane; i < HG * D; i += 64) qf[i] = h2f(p.q[(int64_t(b) * p.Hq + hq0) * D + i]);
    wave_sync();
    const int64_t t0 = int64_t(p.ntiles) * 64;
    const int n_tail = int(p.T - t0);
    const int64_t t = t0 + lane;
    const bool valid = lane < n_tail;
    float sc[HG];
#pragma unroll
    for (int h = 0; h < HG; ++h) sc[h] = 0.0f;
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
        float acc[HG];
#pragma unroll
        for (int h = 0; h < HG; ++h) acc[h] = 0.0f;
        for (int j = 0; j < n_tail; ++j) {
            const float vh = value_hat(p, bh, t0 + j, c);
#pragma unroll
            for (int h = 0; h < HG; ++h) acc[h] = fmaf(pl[h * PSTR + j], vh, acc[h]);
        }
#pragma unroll
        for (int h = 0; h < HG; ++h)
            p.ws_acc[((int64_t(b) * p.Hq + hq0 + h) * p.S + s) * D + c] = acc[h];
    }
#pragma unroll
    for (int h = 0; h < HG; ++h) {
        if (lane == h) {
            const int64_t slot = (int64_t(b) * p.Hq + hq0 + h) * p.S + s;
            p.ws_ml[slot * 2] = m[h];
            p.ws_ml[slot * 2 + 1] = l[h];
        }
    }
}

}  // namespace
}  // namespace kvq
