// kvq_quant_dev.h -- the quantizers as device code (per-token values,
// per-channel key blocks), shared by the quantize kernels (kvq_quant.hip) and
// the decode kernels that append a token inside their tail workgroup
// (kvq_mfma_tiles.h), so that both write the same bits.  Also the
// destination-row policies of the contiguous and paged layouts.
//
// "Makale Bülteni -- KIVI", section "İddia ve Gerçeklik: KIVI": values are
// quantized per token, as asymmetric low-bit codes (zero = group minimum,
// scale = range / (2^bits - 1)).
//
// Exactness: codes must equal round_half_even(fl32(fl32(x - mn) / scale))
// with an IEEE binary32 division.  A correctly rounded division costs ~10
// VALU instructions, so each code is first taken from q = fl32(d * r) with
// d = fl32(x - mn) and r = rcp(scale) (v_rcp_f32: within 1 ulp of 1/scale).
// With Q = d / scale <= L = 2^bits - 1, r = (1 + e1) / scale, |e1| <= 2^-23,
// q = d r (1 + e2) and fl32(Q) = Q (1 + e3), |e2|, |e3| <= 2^-24, so
// |q - fl32(Q)| <= Q (2^-23 + 2^-24 + 2^-24) (1 + 2^-22) ~ L * 2^-22:
// 7.2e-7 at 2 bits, 3.6e-6 at 4 bits.  Whenever q lies farther than a band
// above that bound from a half-integer -- 2^-19 (1.9e-6) at 2 bits, 2^-17
// (7.6e-6) at 4 bits -- both round to the same integer; a code within its
// band of a tie takes the IEEE division (a branch per code: on N(0, 1) fp16
// groups of 32, 1.4e-4 (2 bits) / 2.5e-4 (4 bits) of the codes do, so a
// wave rarely executes the division).
// No clamp is needed: 0 <= fl32(x - mn) <= fl32(max - mn), so both quotients
// round into [0, 2^bits - 1].  Floating-point contraction is off in every
// function here (the including file's setting does not matter).
#pragma once

#include <hip/hip_fp16.h>

#include "kvq_internal.h"

namespace kvq {
namespace {
namespace qdev {

// |q - k| above this sends a code to the IEEE division (see above)
template <int BITS>
constexpr float tie_band() { return BITS == 2 ? 0.5f - 0x1p-19f : 0.5f - 0x1p-17f; }
static_assert(3.0 * 0x1p-22 * (1 + 0x1p-20) < 0x1p-19 && 15.0 * 0x1p-22 * (1 + 0x1p-20) < 0x1p-17,
              "tie bands must exceed the reciprocal path's error bound L * 2^-22");

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
typedef unsigned int qu2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ld_once2(const uint16_t* p) {
    const qu2 v = __builtin_nontemporal_load(reinterpret_cast<const qu2*>(p));
    return make_uint2(v.x, v.y);
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
#pragma clang fp contract(off)
    GroupQ q;
    q.mn = mn;
    q.scale = (mx - mn) / L;   // IEEE division (HIP default: correctly rounded)
    q.rcp = q.scale == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(q.scale);
    return q;
}

// code of d = fl32(x - mn): round-half-even of d * rcp, or of the IEEE
// quotient d / scale when the product lies within the tie band (scale == 0
// gives rcp == 0, product 0, never in the band).  qa - k is exact (both lie
// in one binade's grid, |qa - k| <= 1/2).
template <int BITS>
__device__ __forceinline__ uint32_t code_of(float d, const GroupQ& q) {
#pragma clang fp contract(off)
    const float qa = d * q.rcp;
    float k = __builtin_rintf(qa);
    if (__builtin_fabsf(qa - k) > tie_band<BITS>()) k = __builtin_rintf(d / q.scale);
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
    const uint16_t* vin;   // [BH][n_in][vd]
    int64_t n_in, row0, n_tok;
    int vd, BH;
    uint32_t* codes;
    uint16_t *scale, *zero;
};

// Destination rows of the value stream.  Contiguous cache: token t of
// (b, kvh) is row bh * cap + t.
struct ContigRows {
    int64_t cap, t_dst0, n_tok;
    __device__ int64_t count(int64_t) const { return n_tok; }
    __device__ int64_t row(int64_t bh, int64_t tok) const { return bh * cap + t_dst0 + tok; }
};

// Paged cache: rows appended to sequence b (0 when its length, row count or
// capacity is out of range, so nothing is written for it)
__device__ __forceinline__ int seq_rows(const PagedSeq& ps, int b, int n_max, int G) {
    const int pos = ps.lens[b];
    const int n = ps.n_new ? ps.n_new[b] : n_max;
    if (pos < 0 || n < 0 || n > n_max || int64_t(pos) + n > int64_t(ps.maxb) * G) return 0;
    return n;
}
// block row page * Hkv + kvh of block j of sequence b, or -1 when the table
// names a page outside the pool
__device__ __forceinline__ int64_t paged_block_row(const PagedSeq& ps, int b, int kvh, int Hkv, int64_t j) {
    const int pg = ps.table[int64_t(b) * ps.maxb + j];
    return (pg < 0 || pg >= ps.n_pages) ? -1 : int64_t(pg) * Hkv + kvh;
}
// value row of token t: block row * G + t mod G
struct PagedRows {
    PagedSeq ps;
    int Hkv, G, n_max;
    __device__ int64_t count(int64_t bh) const { return seq_rows(ps, int(bh / Hkv), n_max, G); }
    __device__ int64_t row(int64_t bh, int64_t tok) const {
        const int b = int(bh / Hkv), kvh = int(bh % Hkv);
        const int64_t t = ps.lens[b] + tok;
        const int64_t r = paged_block_row(ps, b, kvh, Hkv, t / G);
        return r < 0 ? -1 : r * G + t % G;
    }
};

// threads that quantize n_tok value rows: BH * ceil(n_tok / VT) * (vd / 8),
// a multiple of 4 (vd / 8 is)
__host__ __device__ inline int64_t value_threads(int BH, int64_t n_tok, int vd) { return int64_t(BH) * ((n_tok + VT - 1) / VT) * (vd / 8); }

// Where a value row comes from: input row row0 + tok of (b, kvh) in global
// memory (read once), or a tile staged in LDS.
struct GlobalValueSrc {
    const uint16_t* vin;
    int64_t n_in, row0;
    int vd;
    __device__ uint4 row8(int64_t bh, int64_t tok, int sub) const {
        return ld_once4(vin + ((bh * n_in) + row0 + tok) * vd + sub * 8);
    }
};

// Thread idx < value_threads(...) quantizes 8 channels of up to VT rows;
// the 4 threads of a 32-channel group are adjacent lanes and exchange their
// min / max by shuffles, so callers keep whole 4-lane groups together.
// Rows tok < rows.count(bh) are quantized into rows.row(bh, tok) (skipped
// when that is negative); src.row8(bh, tok, sub) supplies channels
// 8 sub .. 8 sub + 7 of row tok.
template <int BITS, class Rows, class Src>
__device__ __forceinline__ void quant_values_thread(const ValueArgs& a, const Rows& rows, int64_t idx, const Src& src) {
#pragma clang fp contract(off)
    const int vd = a.vd;
    uint32_t* __restrict__ codes = a.codes;
    uint16_t* __restrict__ scale = a.scale;
    uint16_t* __restrict__ zero = a.zero;
    constexpr float L = float((1 << BITS) - 1);
    const int tpt = vd / 8;
    const int64_t nq = (a.n_tok + VT - 1) / VT;
    const int sub = int(idx % tpt);
    const int64_t tq = (idx / tpt) % nq;
    const int64_t bh = idx / tpt / nq;
    const int64_t cnt = rows.count(bh);

    uint4 raw[VT];
#pragma unroll
    for (int j = 0; j < VT; ++j) {
        const int64_t tok = tq * VT + j;
        raw[j] = tok < cnt ? src.row8(bh, tok, sub) : make_uint4(0u, 0u, 0u, 0u);
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
            packed |= code_of<BITS>(sub_half<0>(w[i], nmn), q) << (BITS * (2 * i));
            packed |= code_of<BITS>(sub_half<1>(w[i], nmn), q) << (BITS * (2 * i + 1));
        }
        // the same for the 4 lanes of a group (same bh, same token)
        const int64_t row = tok < cnt ? rows.row(bh, tok) : -1;
        const bool valid = row >= 0;
        if (BITS == 2) {
            const uint32_t other = __shfl_xor(packed, 1);
            if (valid && (sub & 1) == 0) codes[row * vWT + (sub >> 1)] = packed | (other << 16);
        } else if (valid) {
            codes[row * vWT + sub] = packed;
        }
        if (valid && (sub & 3) == 0) {
            const int64_t side = row * (vd / 32) + (sub >> 2);
            scale[side] = float_to_half_bits(q.scale);
            zero[side] = float_to_half_bits(q.mn);
        }
    }
}

template <int BITS, class Rows>
__device__ __forceinline__ void quant_values_thread(const ValueArgs& a, const Rows& rows, int64_t idx) {
    quant_values_thread<BITS>(a, rows, idx, GlobalValueSrc{a.vin, a.n_in, a.row0, a.vd});
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

// A thread takes CPT = 2 or 4 adjacent channels (one 4- or 8-byte load per
// row) of up to 32 rows of a block.
template <int G, int BITS>
struct KeyShape {
    static constexpr int PER = 32 / BITS;
    static constexpr int W = G / PER;            // words per (block, channel)
    static constexpr int TG = G < 32 ? G : 32;   // rows per thread
    static constexpr int SPL = G / TG;           // threads per channel unit
    static constexpr int CPW = 64 / SPL;         // channel units per wave (SPL > 1)
    static constexpr int WT = TG / PER;          // words per thread and channel
};

// Threads per (sequence, KV head, block).  With SPL > 1 a wave holds the SPL
// row ranges of CPW channel pairs, so the count is rounded up to whole waves;
// lanes past the last pair (kd / 2 < CPW) take part in the shuffles only.
template <int G, int BITS, int CPT = 2>
__host__ __device__ inline int64_t key_threads_per_block(int kd) {
    using S = KeyShape<G, BITS>;
    const int tpb = kd / CPT;
    return S::SPL == 1 ? tpb : int64_t((tpb + S::CPW - 1) / S::CPW) * 64;
}

// thread idx -> (block unit, channel unit, row range)
template <int G, int BITS, int CPT = 2>
__device__ __forceinline__ void key_thread_coords(int64_t idx, int kd, int64_t& unit, int& cp, int& sp) {
    using S = KeyShape<G, BITS>;
    const int tpb = kd / CPT;
    if (S::SPL == 1) {
        sp = 0;
        cp = int(idx % tpb);
        unit = idx / tpb;
    } else {
        const int lane = int(idx & 63);
        const int64_t wv = idx >> 6;
        const int chunks = (tpb + S::CPW - 1) / S::CPW;
        sp = lane / S::CPW;
        cp = int(wv % chunks) * S::CPW + lane % S::CPW;
        unit = wv / chunks;
    }
}

// One key block as a thread sees it: token tok < in_tok0 is residual row
// tok - res_tok0, later ones input row tok - in_tok0; codes go to block row
// dst (codes at dst * kd * W, side values at dst * kd).
struct KeyJob {
    const uint16_t* kin;     // input rows of this (sequence, KV head)
    const uint16_t* resid;   // residual rows of this (sequence, KV head)
    int64_t blk_tok0, in_tok0, res_tok0;
    int64_t dst;
};

// Where a key row comes from: the job's residual / input rows in global
// memory (read once), or a tile staged in LDS.  pair(tok, cp) = channels
// 2 cp, 2 cp + 1 of token tok; quad(tok, cq) = channels 4 cq .. 4 cq + 3.
struct GlobalKeySrc {
    const KeyJob& j;
    int kd;
    __device__ const uint16_t* row(int64_t tok) const {
        return tok < j.in_tok0 ? j.resid + (tok - j.res_tok0) * kd : j.kin + (tok - j.in_tok0) * kd;
    }
    __device__ uint32_t pair(int64_t tok, int cp) const { return ld_once1(row(tok) + 2 * cp); }
    __device__ uint2 quad(int64_t tok, int cq) const { return ld_once2(row(tok) + 4 * cq); }
};

template <int G, int BITS, int CPT = 2, class Src>
__device__ __forceinline__ void quant_key_pair(const KeyJob& j, int kd, int cp, int sp,
                                               uint32_t* __restrict__ codes, uint16_t* __restrict__ scale,
                                               uint16_t* __restrict__ zero, const Src& src) {
#pragma clang fp contract(off)
    static_assert(CPT == 2 || CPT == 4, "two or four channels per thread");
    using S = KeyShape<G, BITS>;
    constexpr int NP = CPT / 2;   // channel pairs per thread
    constexpr float L = float((1 << BITS) - 1);
    const bool active = cp < kd / CPT;
    uint32_t raw[S::TG][NP];
#pragma unroll
    for (int i = 0; i < S::TG; ++i) {
        const int64_t tok = j.blk_tok0 + sp * S::TG + i;
        if constexpr (CPT == 2) {
            raw[i][0] = active ? src.pair(tok, cp) : 0u;
        } else {
            const uint2 w = active ? src.quad(tok, cp) : make_uint2(0u, 0u);
            raw[i][0] = w.x;
            raw[i][1] = w.y;
        }
    }
    // per-channel min / max over the rows, a channel pair at once (packed
    // fp16, exact; -0 is canonicalised after), then across the row ranges
    f16x2 mn2[NP], mx2[NP];
#pragma unroll
    for (int c = 0; c < NP; ++c) {
        mn2[c] = as_h2(raw[0][c]);
        mx2[c] = mn2[c];
#pragma unroll
        for (int i = 1; i < S::TG; ++i) {
            mn2[c] = __builtin_elementwise_min(mn2[c], as_h2(raw[i][c]));
            mx2[c] = __builtin_elementwise_max(mx2[c], as_h2(raw[i][c]));
        }
#pragma unroll
        for (int o = S::CPW; o < 64 && S::SPL > 1; o <<= 1) {
            mn2[c] = __builtin_elementwise_min(mn2[c], as_h2(__shfl_xor(__builtin_bit_cast(uint32_t, mn2[c]), o)));
            mx2[c] = __builtin_elementwise_max(mx2[c], as_h2(__shfl_xor(__builtin_bit_cast(uint32_t, mx2[c]), o)));
        }
    }
    if (!active) return;
    GroupQ q[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) q[e] = make_group(float(mn2[e >> 1][e & 1]) + 0.0f, float(mx2[e >> 1][e & 1]) + 0.0f, L);
    const int64_t side = j.dst * kd + CPT * cp;
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
        uint32_t words[S::WT];
#pragma unroll
        for (int w = 0; w < S::WT; ++w) words[w] = 0;
        const float nmn = -q[e].mn;
#pragma unroll
        for (int i = 0; i < S::TG; ++i) {
            const float d = (e & 1) == 0 ? sub_half<0>(raw[i][e >> 1], nmn) : sub_half<1>(raw[i][e >> 1], nmn);
            words[i / S::PER] |= code_of<BITS>(d, q[e]) << (BITS * (i % S::PER));
        }
        WordVec<S::WT>::st(codes + (side + e) * S::W + sp * S::WT, words);
    }
    if (sp == 0) {
        uint32_t sv[NP], zv[NP];
#pragma unroll
        for (int c = 0; c < NP; ++c) {
            sv[c] = uint32_t(float_to_half_bits(q[2 * c].scale)) | (uint32_t(float_to_half_bits(q[2 * c + 1].scale)) << 16);
            zv[c] = uint32_t(float_to_half_bits(q[2 * c].mn)) | (uint32_t(float_to_half_bits(q[2 * c + 1].mn)) << 16);
        }
        WordVec<NP>::st(reinterpret_cast<uint32_t*>(scale + side), sv);
        WordVec<NP>::st(reinterpret_cast<uint32_t*>(zero + side), zv);
    }
}

template <int G, int BITS, int CPT = 2>
__device__ __forceinline__ void quant_key_pair(const KeyJob& j, int kd, int cp, int sp,
                                               uint32_t* __restrict__ codes, uint16_t* __restrict__ scale,
                                               uint16_t* __restrict__ zero) {
    quant_key_pair<G, BITS, CPT>(j, kd, cp, sp, codes, scale, zero, GlobalKeySrc{j, kd});
}

}  // namespace qdev
}  // namespace
}  // namespace kvq
