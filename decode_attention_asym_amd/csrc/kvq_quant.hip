// kvq_quant.hip -- quantize / pack kernels of the KIVI-style cache on gfx950.
//
// "Makale Bülteni -- KIVI", section "İddia ve Gerçeklik: KIVI": values are
// quantized per token, keys per channel over blocks of G tokens, both as
// asymmetric 2-bit codes (zero = group minimum, scale = range / 3); the
// unfilled key block stays fp16 in the residual.  "QuantMLA ...", section
// "QuantMLA Mimarisi ve Temel Bileşenleri": the same per-token rule serves the
// INT2 content latent and the per-channel rule the INT4 RoPE key.
//
// Exactness: codes must equal round_half_even(fl32(fl32(x - mn) / scale))
// with an IEEE binary32 division.  A correctly rounded division costs ~10
// VALU instructions, so each code is first taken from q = fl32(x - mn) *
// rcp(scale) (v_rcp_f32, <= 1 ulp).  |q - fl32(true quotient)| <= 6.6e-7 for
// quotients <= 2^bits - 1, so whenever q lies more than 2^-19 from a
// half-integer both round to the same integer; a code closer than that to a
// tie takes the IEEE division (a branch per code: on fp16 data about 1 code
// in 10^4 does, so a wave almost never executes the division).
// No clamp is needed: 0 <= fl32(x - mn) <= fl32(max - mn), so both quotients
// round into [0, 2^bits - 1].
#include <hip/hip_fp16.h>

#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr float kTieBand = 0.5f - 0x1p-19f;

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f16x2 as_h2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }

// The fp16 inputs are read exactly once: non-temporal loads keep them from
// displacing other lines (measured: +4..5% on the bulk quantize; the same
// hint on the code stores made it slower).
typedef unsigned int qu4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_once4(const uint16_t* p) {
    const qu4 v = __builtin_nontemporal_load(reinterpret_cast<const qu4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_once1(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// fl32(x - mn) for the fp16 half HALF of w, in one instruction: v_fma_mix
// converts the fp16 operand exactly and rounds x * 1 + (-mn) once
template <int HALF>
__device__ __forceinline__ float sub_half(uint32_t w, float neg_mn) {
    float d;
    if (HALF == 0)
        asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(w), "v"(neg_mn));
    else
        asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(w), "v"(neg_mn));
    return d;
}

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

// code of d = fl32(x - mn): round-half-even of d * rcp, or of the IEEE
// quotient d / scale when the product lies within the tie band (scale == 0
// gives rcp == 0, product 0, never in the band)
__device__ __forceinline__ uint32_t code_of(float d, const GroupQ& q) {
    const float qa = d * q.rcp;
    float k = __builtin_rintf(qa);
    if (__builtin_fabsf(qa - k) > kTieBand) k = __builtin_rintf(d / q.scale);
    return static_cast<uint32_t>(k);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h16) {
    return __half2float(__ushort_as_half(static_cast<unsigned short>(h16)));
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
    return __half_as_ushort(__float2half_rn(f));
}

// ------------------------------------------------------------------ values
// One thread = 8 consecutive channels (one 16-byte load) of VT consecutive
// tokens, all loads issued first; four neighbouring lanes form a 32-channel
// group and reduce min/max by shuffles.
constexpr int VT = 4;

struct ValueArgs {
    const uint16_t* vin;
    int64_t n_in, row0, n_tok, t_dst0, cap;
    int vd, BH;
    uint32_t* codes;
    uint16_t *scale, *zero;
};

// threads that quantize n_tok value rows: BH * ceil(n_tok / VT) * (vd / 8),
// a multiple of 4 (vd / 8 is)
__host__ __device__ inline int64_t value_threads(int BH, int64_t n_tok, int vd) { return int64_t(BH) * ((n_tok + VT - 1) / VT) * (vd / 8); }

// Thread idx < value_threads(...) quantizes 8 channels of up to VT rows;
// the 4 threads of a 32-channel group are adjacent lanes and exchange their
// min / max by shuffles, so callers keep whole 4-lane groups together.
template <int BITS>
__device__ __forceinline__ void quant_values_thread(const ValueArgs& a, int64_t idx) {
    const uint16_t* __restrict__ vin = a.vin;
    const int64_t n_in = a.n_in, row0 = a.row0, n_tok = a.n_tok, t_dst0 = a.t_dst0, cap = a.cap;
    const int vd = a.vd;
    uint32_t* __restrict__ codes = a.codes;
    uint16_t* __restrict__ scale = a.scale;
    uint16_t* __restrict__ zero = a.zero;
    constexpr float L = float((1 << BITS) - 1);
    const int tpt = vd / 8;
    const int64_t nq = (n_tok + VT - 1) / VT;
    const int sub = int(idx % tpt);
    const int64_t tq = (idx / tpt) % nq;
    const int64_t bh = idx / tpt / nq;

    uint4 raw[VT];
#pragma unroll
    for (int j = 0; j < VT; ++j) {
        const int64_t tok = tq * VT + j;
        raw[j] = tok < n_tok ? ld_once4(vin + ((bh * n_in) + row0 + tok) * vd + sub * 8)
                             : make_uint4(0u, 0u, 0u, 0u);
    }
    const int vWT = vd * BITS / 32;
#pragma unroll
    for (int j = 0; j < VT; ++j) {
        const int64_t tok = tq * VT + j;
        const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
        // min / max of the 8 values (packed fp16, exact; -0 is canonicalised after)
        f16x2 mn2 = __builtin_elementwise_min(__builtin_elementwise_min(as_h2(w[0]), as_h2(w[1])),
                                              __builtin_elementwise_min(as_h2(w[2]), as_h2(w[3])));
        f16x2 mx2 = __builtin_elementwise_max(__builtin_elementwise_max(as_h2(w[0]), as_h2(w[1])),
                                              __builtin_elementwise_max(as_h2(w[2]), as_h2(w[3])));
        float mn = __builtin_fminf(float(mn2[0]), float(mn2[1]));
        float mx = __builtin_fmaxf(float(mx2[0]), float(mx2[1]));
        mn = __builtin_fminf(mn, __shfl_xor(mn, 1));
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 1));
        mn = __builtin_fminf(mn, __shfl_xor(mn, 2));
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 2));
        const GroupQ q = make_group(mn + 0.0f, mx + 0.0f, L);

        uint32_t packed = 0;
        const float nmn = -q.mn;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            packed |= code_of(sub_half<0>(w[i], nmn), q) << (BITS * (2 * i));
            packed |= code_of(sub_half<1>(w[i], nmn), q) << (BITS * (2 * i + 1));
        }
        const int64_t t = t_dst0 + tok;
        uint32_t* wrow = codes + (bh * cap + t) * vWT;
        const bool valid = tok < n_tok;
        if (BITS == 2) {
            const uint32_t other = __shfl_xor(packed, 1);
            if (valid && (sub & 1) == 0) wrow[sub >> 1] = packed | (other << 16);
        } else if (valid) {
            wrow[sub] = packed;
        }
        if (valid && (sub & 3) == 0) {
            const int64_t side = (bh * cap + t) * (vd / 32) + (sub >> 2);
            scale[side] = float_to_half_bits(q.scale);
            zero[side] = float_to_half_bits(q.mn);
        }
    }
}

template <int BITS>
__global__ __launch_bounds__(256) void k_quant_values(ValueArgs a) {
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= value_threads(a.BH, a.n_tok, a.vd)) return;   // whole 4-lane groups leave together
    quant_values_thread<BITS>(a, idx);
}

// -------------------------------------------------------------------- keys
// One thread = 2 adjacent channels over up to 32 rows of one G-token block
// (4-byte loads; lanes side by side read contiguous bytes of a row); for
// G > 32 the SPL = G/32 threads of a channel pair sit in one wave and merge
// their min/max by shuffles.  Each thread writes its rows' codes as
// consecutive words of the channel's G*BITS/32.
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
    constexpr int W = G / PER;                 // words per (block, channel)
    constexpr int TG = G < 32 ? G : 32;        // rows per thread
    constexpr int SPL = G / TG;                // threads per channel pair
    constexpr int CPW = 64 / SPL;              // channel pairs per wave (SPL > 1)
    constexpr int WT = TG / PER;               // words per thread and channel
    const int tpb = kd / 2;
    const int64_t total = int64_t(BH) * nb * tpb * SPL;
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= total) return;   // whole waves: total is a multiple of 64 when SPL > 1
    int cp, sp;
    int64_t blk, bh;
    if (SPL == 1) {
        sp = 0;
        cp = int(idx % tpb);
        blk = blk0 + (idx / tpb) % nb;
        bh = idx / tpb / nb;
    } else {
        // a wave holds the SPL row ranges of CPW consecutive channel pairs
        const int lane = int(idx & 63);
        const int64_t wv = idx >> 6;
        const int chunks = tpb / CPW;
        sp = lane / CPW;
        cp = int(wv % chunks) * CPW + lane % CPW;
        blk = blk0 + (wv / chunks) % nb;
        bh = wv / chunks / nb;
    }

    uint32_t raw[TG];
#pragma unroll
    for (int i = 0; i < TG; ++i) {
        const int64_t tok = blk * G + sp * TG + i;
        const uint16_t* row = tok < in_tok0 ? resid + (bh * G + (tok - res_tok0)) * kd
                                            : kin + (bh * n_in + (tok - in_tok0)) * kd;
        raw[i] = ld_once1(row + 2 * cp);
    }
    // per-channel min / max over the rows, both channels at once (packed
    // fp16, exact; -0 is canonicalised after), then across the row ranges
    f16x2 mn2 = as_h2(raw[0]), mx2 = mn2;
#pragma unroll
    for (int i = 1; i < TG; ++i) {
        mn2 = __builtin_elementwise_min(mn2, as_h2(raw[i]));
        mx2 = __builtin_elementwise_max(mx2, as_h2(raw[i]));
    }
#pragma unroll
    for (int o = CPW; o < 64 && SPL > 1; o <<= 1) {
        mn2 = __builtin_elementwise_min(mn2, as_h2(__shfl_xor(__builtin_bit_cast(uint32_t, mn2), o)));
        mx2 = __builtin_elementwise_max(mx2, as_h2(__shfl_xor(__builtin_bit_cast(uint32_t, mx2), o)));
    }
    GroupQ q[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) q[e] = make_group(float(mn2[e]) + 0.0f, float(mx2[e]) + 0.0f, L);
    const int64_t side = (bh * nblk_cap + blk) * kd + 2 * cp;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        uint32_t words[WT];
#pragma unroll
        for (int j = 0; j < WT; ++j) words[j] = 0;
        const float nmn = -q[e].mn;
#pragma unroll
        for (int i = 0; i < TG; ++i) {
            const float d = e == 0 ? sub_half<0>(raw[i], nmn) : sub_half<1>(raw[i], nmn);
            words[i / PER] |= code_of(d, q[e]) << (BITS * (i % PER));
        }
        WordVec<WT>::st(codes + (side + e) * W + sp * WT, words);
    }
    if (sp == 0) {
        *reinterpret_cast<uint32_t*>(scale + side) =
            uint32_t(float_to_half_bits(q[0].scale)) | (uint32_t(float_to_half_bits(q[1].scale)) << 16);
        *reinterpret_cast<uint32_t*>(zero + side) =
            uint32_t(float_to_half_bits(q[0].mn)) | (uint32_t(float_to_half_bits(q[1].mn)) << 16);
    }
}

// ---------------------------------------------------------- residual copy
struct ResidArgs {
    const uint16_t* kin;
    int64_t n_in, src0, dst0, m;
    int kd, G, BH;
    uint16_t* resid;
};

__host__ __device__ inline int64_t resid_threads(const ResidArgs& a) { return int64_t(a.BH) * a.m * (a.kd / 8); }

// thread idx < resid_threads(...) copies 8 channels of one key row into the residual
__device__ __forceinline__ void resid_copy_thread(const ResidArgs& a, int64_t idx) {
    const int vpr = a.kd / 8;
    const int v = int(idx % vpr);
    const int64_t r = (idx / vpr) % a.m;
    const int64_t bh = idx / vpr / a.m;
    *reinterpret_cast<uint4*>(a.resid + (bh * a.G + a.dst0 + r) * a.kd + v * 8) =
        *reinterpret_cast<const uint4*>(a.kin + (bh * a.n_in + a.src0 + r) * a.kd + v * 8);
}

__global__ __launch_bounds__(256) void k_resid_copy(ResidArgs a) {
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= resid_threads(a)) return;
    resid_copy_thread(a, idx);
}

// An append that completes no key block: the value rows are quantized and
// the key rows land in the residual, in one launch (value threads first;
// their count is a multiple of 4, so no 4-lane group is split).
template <int BITS>
__global__ __launch_bounds__(256) void k_append_rows(ValueArgs va, ResidArgs ka) {
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t nv = value_threads(va.BH, va.n_tok, va.vd);
    if (idx < nv)
        quant_values_thread<BITS>(va, idx);
    else if (idx - nv < resid_threads(ka))
        resid_copy_thread(ka, idx - nv);
}

inline unsigned grid_of(int64_t threads) { return unsigned((threads + 255) / 256); }

template <int G, int BITS>
hipError_t launch_keys_t(const kvq_cache& c, const Geom& g, const void* k_in, int64_t n_in,
                         int64_t in_tok0, int64_t res_tok0, int64_t blk0, int64_t nb,
                         hipStream_t st) {
    const int BH = g.B * g.Hkv;
    const int64_t threads = int64_t(BH) * nb * (g.kd / 2) * (G > 32 ? G / 32 : 1);
    hipLaunchKernelGGL((k_quant_keys<G, BITS>), dim3(grid_of(threads)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(k_in), n_in, in_tok0,
                       static_cast<const uint16_t*>(c.buf.k_resid), res_tok0, blk0, int(nb), g.kd,
                       g.nblk_cap, BH, static_cast<uint32_t*>(c.buf.k_codes),
                       static_cast<uint16_t*>(c.buf.k_scale), static_cast<uint16_t*>(c.buf.k_zero));
    return hipGetLastError();
}

}  // namespace

namespace {
ValueArgs value_args(const kvq_cache& c, const Geom& g, const void* v_in, int64_t n_in, int64_t row0,
                     int64_t n_tok, int64_t t_dst0) {
    ValueArgs a;
    a.vin = static_cast<const uint16_t*>(v_in);
    a.n_in = n_in;
    a.row0 = row0;
    a.n_tok = n_tok;
    a.t_dst0 = t_dst0;
    a.cap = g.cap;
    a.vd = g.vd;
    a.BH = g.B * g.Hkv;
    a.codes = static_cast<uint32_t*>(c.buf.v_codes);
    a.scale = static_cast<uint16_t*>(c.buf.v_scale);
    a.zero = static_cast<uint16_t*>(c.buf.v_zero);
    return a;
}
ResidArgs resid_args(const kvq_cache& c, const Geom& g, const void* k_in, int64_t n_in, int64_t src0,
                     int64_t dst0, int64_t m) {
    ResidArgs a;
    a.kin = static_cast<const uint16_t*>(k_in);
    a.n_in = n_in;
    a.src0 = src0;
    a.dst0 = dst0;
    a.m = m;
    a.kd = g.kd;
    a.G = g.kG;
    a.BH = g.B * g.Hkv;
    a.resid = static_cast<uint16_t*>(c.buf.k_resid);
    return a;
}
}  // namespace

hipError_t launch_quant_values(const kvq_cache& c, const Geom& g, const void* v_in, int64_t n_in,
                               int64_t row0, int64_t n_tok, int64_t t_dst0, hipStream_t st) {
    if (n_tok <= 0) return hipSuccess;
    const ValueArgs a = value_args(c, g, v_in, n_in, row0, n_tok, t_dst0);
    const unsigned grid = grid_of(value_threads(a.BH, n_tok, a.vd));
    if (g.vbits == 2)
        hipLaunchKernelGGL(k_quant_values<2>, dim3(grid), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(k_quant_values<4>, dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_append_rows(const kvq_cache& c, const Geom& g, const void* k_in, const void* v_in,
                              int64_t n, int64_t R, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const ValueArgs va = value_args(c, g, v_in, n, 0, n, c.T);
    const ResidArgs ka = resid_args(c, g, k_in, n, 0, R, n);
    const unsigned grid = grid_of(value_threads(va.BH, n, va.vd) + resid_threads(ka));
    if (g.vbits == 2)
        hipLaunchKernelGGL(k_append_rows<2>, dim3(grid), dim3(256), 0, st, va, ka);
    else
        hipLaunchKernelGGL(k_append_rows<4>, dim3(grid), dim3(256), 0, st, va, ka);
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
    const ResidArgs a = resid_args(c, g, k_in, n_in, src0, dst0, m);
    hipLaunchKernelGGL(k_resid_copy, dim3(grid_of(resid_threads(a))), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace kvq
