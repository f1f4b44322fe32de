// kvq_quant.hip -- quantize / pack kernels of the KIVI-style cache on gfx950.
//
// "Makale Bülteni -- KIVI", section "İddia ve Gerçeklik: KIVI": values are
// quantized per token, keys per channel over blocks of G tokens, both as
// asymmetric 2-bit codes (zero = group minimum, scale = range / 3); the
// unfilled key block stays fp16 in the residual.  "QuantMLA ...", section
// "QuantMLA Mimarisi ve Temel Bileşenleri": the same per-token rule serves the
// INT2 content latent and the per-channel rule the INT4 RoPE key.
//
// Exactness: codes must equal round_half_even(fl32(fl32(x - mn) / scale32))
// with an IEEE binary32 division.  A correctly rounded division costs ~10
// VALU instructions, so each code is first taken from q = fl32(x - mn) *
// rcp(scale) (v_rcp_f32, <= 1 ulp).  |q - fl32(true quotient)| <= 6.6e-7 for
// quotients <= 2^bits - 1, so whenever q lies more than 2^-19 from a
// half-integer both round to the same integer; a group with any code closer
// than that to a tie is recomputed with the IEEE division.
#include <hip/hip_fp16.h>

#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr float kTieBand = 0.5f - 0x1p-19f;

__device__ __forceinline__ float half_bits_to_float(uint32_t h16) {
    return __half2float(__ushort_as_half(static_cast<unsigned short>(h16)));
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
    return __half_as_ushort(__float2half_rn(f));
}

// binary32 value of an fp16 input, with -0 canonicalised to +0
__device__ __forceinline__ float canon(uint32_t h16) { return half_bits_to_float(h16) + 0.0f; }

struct GroupQ {
    float mn, scale, rcp;
};

__device__ __forceinline__ GroupQ make_group(float mn, float mx, float L) {
    GroupQ q;
    q.mn = mn;
    q.scale = (mx - mn) / L;   // IEEE division (HIP default: correctly rounded)
    q.rcp = q.scale == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(q.scale);
    return q;
}

__device__ __forceinline__ uint32_t code_fast(float x, const GroupQ& q, float L, bool& tie) {
    const float qa = (x - q.mn) * q.rcp;
    const float k = __builtin_rintf(qa);
    tie |= __builtin_fabsf(qa - k) > kTieBand;
    return static_cast<uint32_t>(__builtin_fminf(k, L));
}

__device__ __forceinline__ uint32_t code_exact(float x, const GroupQ& q, float L) {
    if (q.scale == 0.0f) return 0u;
    const float d = x - q.mn;
    const float qt = d / q.scale;
    const float k = __builtin_rintf(qt);
    return static_cast<uint32_t>(__builtin_fminf(__builtin_fmaxf(k, 0.0f), L));
}

// ------------------------------------------------------------------ values
// One thread = 8 consecutive channels of one token (one 16-byte load); four
// neighbouring lanes form a 32-channel group and reduce min/max by shuffles.
template <int BITS>
__global__ __launch_bounds__(256) void k_quant_values(
    const uint16_t* __restrict__ vin, int64_t n_in, int64_t row0, int64_t n_tok,
    int64_t t_dst0, int vd, int64_t cap, int BH, uint32_t* __restrict__ codes,
    uint16_t* __restrict__ scale, uint16_t* __restrict__ zero) {
    constexpr float L = float((1 << BITS) - 1);
    const int tpt = vd / 8;
    const int64_t total = int64_t(BH) * n_tok * tpt;
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= total) return;
    const int sub = int(idx % tpt);
    const int64_t tok = (idx / tpt) % n_tok;
    const int64_t bh = idx / tpt / n_tok;

    const uint4 raw = *reinterpret_cast<const uint4*>(vin + ((bh * n_in) + row0 + tok) * vd + sub * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = canon(w[i] & 0xffffu);
        x[2 * i + 1] = canon(w[i] >> 16);
    }
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        mn = __builtin_fminf(mn, x[i]);
        mx = __builtin_fmaxf(mx, x[i]);
    }
    mn = __builtin_fminf(mn, __shfl_xor(mn, 1));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 1));
    mn = __builtin_fminf(mn, __shfl_xor(mn, 2));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 2));
    const GroupQ q = make_group(mn, mx, L);

    uint32_t c[8];
    bool tie = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = code_fast(x[i], q, L, tie);
    if (tie) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = code_exact(x[i], q, L);
    }
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= c[i] << (BITS * i);

    const int64_t t = t_dst0 + tok;
    const int vWT = vd * BITS / 32;
    uint32_t* wrow = codes + (bh * cap + t) * vWT;
    if (BITS == 2) {
        const uint32_t other = __shfl_xor(packed, 1);
        if ((sub & 1) == 0) wrow[sub >> 1] = packed | (other << 16);
    } else {
        wrow[sub] = packed;
    }
    if ((sub & 3) == 0) {
        const int64_t side = (bh * cap + t) * (vd / 32) + (sub >> 2);
        scale[side] = float_to_half_bits(q.scale);
        zero[side] = float_to_half_bits(q.mn);
    }
}

// -------------------------------------------------------------------- keys
// One thread = 2 adjacent channels of one G-token block: it reads the G
// token rows (4 bytes each; a wave covers 128 channels = 256 contiguous bytes
// per row), reduces min/max per channel, and writes each channel's G codes
// as G*BITS/32 consecutive words.
template <int W>
struct WordVec;
template <> struct WordVec<1> { static __device__ void st(uint32_t* p, const uint32_t* w) { p[0] = w[0]; } };
template <> struct WordVec<2> {
    static __device__ void st(uint32_t* p, const uint32_t* w) { *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]); }
};
template <> struct WordVec<4> {
    static __device__ void st(uint32_t* p, const uint32_t* w) {
        *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    }
};
template <> struct WordVec<8> {
    static __device__ void st(uint32_t* p, const uint32_t* w) {
        reinterpret_cast<uint4*>(p)[0] = make_uint4(w[0], w[1], w[2], w[3]);
        reinterpret_cast<uint4*>(p)[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
};

template <int G, int BITS>
__global__ __launch_bounds__(256) void k_quant_keys(
    const uint16_t* __restrict__ kin, int64_t n_in, int64_t in_tok0,
    const uint16_t* __restrict__ resid, int64_t res_tok0, int64_t blk0, int nb, int kd,
    int64_t nblk_cap, int BH, uint32_t* __restrict__ codes, uint16_t* __restrict__ scale,
    uint16_t* __restrict__ zero) {
    constexpr float L = float((1 << BITS) - 1);
    constexpr int PER = 32 / BITS;
    constexpr int W = G / PER;
    const int tpb = kd / 2;
    const int64_t total = int64_t(BH) * nb * tpb;
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= total) return;
    const int cp = int(idx % tpb);
    const int64_t blk = blk0 + (idx / tpb) % nb;
    const int64_t bh = idx / tpb / nb;

    uint32_t raw[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int64_t tok = blk * G + i;
        const uint16_t* row = tok < in_tok0 ? resid + (bh * G + (tok - res_tok0)) * kd
                                            : kin + (bh * n_in + (tok - in_tok0)) * kd;
        raw[i] = *reinterpret_cast<const uint32_t*>(row + 2 * cp);
    }
    GroupQ q[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        float mn = canon((raw[0] >> (16 * e)) & 0xffffu), mx = mn;
#pragma unroll
        for (int i = 1; i < G; ++i) {
            const float x = canon((raw[i] >> (16 * e)) & 0xffffu);
            mn = __builtin_fminf(mn, x);
            mx = __builtin_fmaxf(mx, x);
        }
        q[e] = make_group(mn, mx, L);
    }
    const int64_t side = (bh * nblk_cap + blk) * kd + 2 * cp;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        uint32_t words[W];
#pragma unroll
        for (int j = 0; j < W; ++j) words[j] = 0;
        bool tie = false;
#pragma unroll
        for (int i = 0; i < G; ++i)
            words[i / PER] |= code_fast(canon((raw[i] >> (16 * e)) & 0xffffu), q[e], L, tie)
                              << (BITS * (i % PER));
        if (tie) {
#pragma unroll
            for (int j = 0; j < W; ++j) words[j] = 0;
#pragma unroll
            for (int i = 0; i < G; ++i)
                words[i / PER] |= code_exact(canon((raw[i] >> (16 * e)) & 0xffffu), q[e], L)
                                  << (BITS * (i % PER));
        }
        WordVec<W>::st(codes + (side + e) * W, words);
    }
    *reinterpret_cast<uint32_t*>(scale + side) =
        uint32_t(float_to_half_bits(q[0].scale)) | (uint32_t(float_to_half_bits(q[1].scale)) << 16);
    *reinterpret_cast<uint32_t*>(zero + side) =
        uint32_t(float_to_half_bits(q[0].mn)) | (uint32_t(float_to_half_bits(q[1].mn)) << 16);
}

// ---------------------------------------------------------- residual copy
__global__ __launch_bounds__(256) void k_resid_copy(const uint16_t* __restrict__ kin, int64_t n_in,
                                                    int64_t src0, int64_t dst0, int64_t m, int kd,
                                                    int G, int BH, uint16_t* __restrict__ resid) {
    const int vpr = kd / 8;
    const int64_t total = int64_t(BH) * m * vpr;
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= total) return;
    const int v = int(idx % vpr);
    const int64_t r = (idx / vpr) % m;
    const int64_t bh = idx / vpr / m;
    *reinterpret_cast<uint4*>(resid + (bh * G + dst0 + r) * kd + v * 8) =
        *reinterpret_cast<const uint4*>(kin + (bh * n_in + src0 + r) * kd + v * 8);
}

inline unsigned grid_of(int64_t threads) { return unsigned((threads + 255) / 256); }

template <int G, int BITS>
hipError_t launch_keys_t(const kvq_cache& c, const Geom& g, const void* k_in, int64_t n_in,
                         int64_t in_tok0, int64_t res_tok0, int64_t blk0, int64_t nb,
                         hipStream_t st) {
    const int BH = g.B * g.Hkv;
    const int64_t threads = int64_t(BH) * nb * (g.kd / 2);
    hipLaunchKernelGGL((k_quant_keys<G, BITS>), dim3(grid_of(threads)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(k_in), n_in, in_tok0,
                       static_cast<const uint16_t*>(c.buf.k_resid), res_tok0, blk0, int(nb), g.kd,
                       g.nblk_cap, BH, static_cast<uint32_t*>(c.buf.k_codes),
                       static_cast<uint16_t*>(c.buf.k_scale), static_cast<uint16_t*>(c.buf.k_zero));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_values(const kvq_cache& c, const Geom& g, const void* v_in, int64_t n_in,
                               int64_t row0, int64_t n_tok, int64_t t_dst0, hipStream_t st) {
    if (n_tok <= 0) return hipSuccess;
    const int BH = g.B * g.Hkv;
    const int64_t threads = int64_t(BH) * n_tok * (g.vd / 8);
    const auto* vin = static_cast<const uint16_t*>(v_in);
    auto* codes = static_cast<uint32_t*>(c.buf.v_codes);
    auto* sc = static_cast<uint16_t*>(c.buf.v_scale);
    auto* ze = static_cast<uint16_t*>(c.buf.v_zero);
    if (g.vbits == 2)
        hipLaunchKernelGGL(k_quant_values<2>, dim3(grid_of(threads)), dim3(256), 0, st, vin, n_in,
                           row0, n_tok, t_dst0, g.vd, g.cap, BH, codes, sc, ze);
    else
        hipLaunchKernelGGL(k_quant_values<4>, dim3(grid_of(threads)), dim3(256), 0, st, vin, n_in,
                           row0, n_tok, t_dst0, g.vd, g.cap, BH, codes, sc, ze);
    return hipGetLastError();
}

hipError_t launch_quant_keys(const kvq_cache& c, const Geom& g, const void* k_in, int64_t n_in,
                             int64_t in_tok0, int64_t res_tok0, int64_t blk0, int64_t nb,
                             hipStream_t st) {
    if (nb <= 0) return hipSuccess;
#define KVQ_KEYS(GG, BB)                                                                      \
    if (g.kG == GG && g.kbits == BB)                                                          \
        return launch_keys_t<GG, BB>(c, g, k_in, n_in, in_tok0, res_tok0, blk0, nb, st);
    KVQ_KEYS(16, 2)
    KVQ_KEYS(32, 2)
    KVQ_KEYS(64, 2)
    KVQ_KEYS(128, 2)
    KVQ_KEYS(16, 4)
    KVQ_KEYS(32, 4)
    KVQ_KEYS(64, 4)
#undef KVQ_KEYS
    return hipErrorInvalidValue;
}

hipError_t launch_resid_copy(const kvq_cache& c, const Geom& g, const void* k_in, int64_t n_in,
                             int64_t src0, int64_t dst0, int64_t m, hipStream_t st) {
    if (m <= 0) return hipSuccess;
    const int BH = g.B * g.Hkv;
    const int64_t threads = int64_t(BH) * m * (g.kd / 8);
    hipLaunchKernelGGL(k_resid_copy, dim3(grid_of(threads)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(k_in), n_in, src0, dst0, m, g.kd, g.kG, BH,
                       static_cast<uint16_t*>(c.buf.k_resid));
    return hipGetLastError();
}

}  // namespace kvq
