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
#include "kvq_quant_dev.h"

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
constexpr int KTILE_DW = 512;   // key-code tile in LDS (dwords): the cache layout, copied
constexpr int VTILE_DW = 528;   // value-code tile in LDS (dwords): the cache layout + pad
// q' and p' rows are read as 16-byte A operands, lane n taking row n: with
// these strides rows 0..7 start on eight distinct multiples of 8 banks
// (mod 64), which the LDS bank-conflict counter showed to serve such reads
// with the fewest conflicts (68- and 36-dword rows measured 2.5x the cycles)
constexpr int QSTR = 72;    // dwords per q' row (128 fp16 + pad)
constexpr int ASTR = 40;    // dwords per p' row (64 fp16 + pad)
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
    float neg1;    // -1, kept opaque so p - fp16(p) stays one mixed FMA
    // paged caches: block table [B][maxb], lengths [B] (clamped to
    // [0, max_len]), pool size, tiles per main split
    const int32_t *table, *lens;
    int maxb, npages, chunk, max_len;
    // fused append of token T - 1 (see fused_append), or for a paged cache
    // of token lens[b] of each sequence (fused_append_paged; n_new: rows per
    // sequence, 0 or 1, null = 1)
    const uint16_t *k_new, *v_new;
    uint32_t *vc_w, *kc_w;
    uint16_t *vs_w, *vz_w, *kr_w, *ks_w, *kz_w;
    const int32_t* n_new;
    int fuse;
};

inline MfmaParams mfma_params(const DecodeArgs& a) {
    const kvq_cache_buffers& buf = a.pc ? a.pc->buf : a.c->buf;
    MfmaParams p;
    p.kc = static_cast<const uint32_t*>(buf.k_codes);
    p.ks = static_cast<const uint16_t*>(buf.k_scale);
    p.kz = static_cast<const uint16_t*>(buf.k_zero);
    p.kr = static_cast<const uint16_t*>(buf.k_resid);
    p.vc = static_cast<const uint32_t*>(buf.v_codes);
    p.vs = static_cast<const uint16_t*>(buf.v_scale);
    p.vz = static_cast<const uint16_t*>(buf.v_zero);
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
    p.neg1 = -1.0f;
    p.table = a.ps.table;
    p.lens = a.ps.lens;
    p.maxb = a.ps.maxb;
    p.npages = a.ps.n_pages;
    p.chunk = a.chunk;
    p.max_len = a.max_len;
    p.k_new = static_cast<const uint16_t*>(a.k_new);
    p.v_new = static_cast<const uint16_t*>(a.v_new);
    p.vc_w = static_cast<uint32_t*>(buf.v_codes);
    p.vs_w = static_cast<uint16_t*>(buf.v_scale);
    p.vz_w = static_cast<uint16_t*>(buf.v_zero);
    p.kr_w = static_cast<uint16_t*>(buf.k_resid);
    p.kc_w = static_cast<uint32_t*>(buf.k_codes);
    p.ks_w = static_cast<uint16_t*>(buf.k_scale);
    p.kz_w = static_cast<uint16_t*>(buf.k_zero);
    p.n_new = a.ps.n_new;
    p.fuse = a.fuse;
    return p;
}

// The shapes these kernels take: KIVI, D = 128, 2-bit keys and values,
// 32-channel value groups, G in {32, 64}.
inline bool mfma_cfg_ok(const kvq_cache_cfg& g) {
    return g.kind == KVQ_KIND_KIVI && g.key.bits == 2 && g.value.bits == 2 && g.key.dim == D &&
           g.value.dim == D && g.value.group == 32 && (g.key.group == 32 || g.key.group == 64);
}
inline bool mfma_shape_ok(const kvq_cache& c) { return mfma_cfg_ok(c.cfg); }
// the same shapes with 4-bit keys and values (GQA kernel, contiguous cache)
inline bool mfma_cfg_ok4(const kvq_cache_cfg& g) {
    return g.kind == KVQ_KIND_KIVI && g.key.bits == 4 && g.value.bits == 4 && g.key.dim == D &&
           g.value.dim == D && g.value.group == 32 && (g.key.group == 32 || g.key.group == 64);
}

// ---- where key block j of (sequence b, KV head kvh) lives: its block row r
// (key codes at r * D * G/16 words, key side values at r * D, value rows
// r * G + i).  Contiguous: (b * Hkv + kvh) * nblk_cap + j; paged:
// page * Hkv + kvh with the page from the block table (clamped into the pool,
// so a bad entry reads the wrong page but never outside the arrays).
__device__ __forceinline__ int page_of(const MfmaParams& p, int b, int64_t j) {
    const int pg = p.table[int64_t(b) * p.maxb + j];
    return pg < 0 ? 0 : (pg >= p.npages ? p.npages - 1 : pg);
}
struct ContigBlocks {
    __device__ int64_t operator()(const MfmaParams& p, int b, int kvh, int64_t j) const {
        return (int64_t(b) * p.Hkv + kvh) * p.nblk_cap + j;
    }
};
struct PagedBlocks {
    __device__ int64_t operator()(const MfmaParams& p, int b, int kvh, int64_t j) const {
        return int64_t(page_of(p, b, j)) * p.Hkv + kvh;
    }
};
// tokens of sequence b in a paged call
__device__ __forceinline__ int seq_len(const MfmaParams& p, int b) {
    const int l = p.lens[b];
    return l < 0 ? 0 : (l > p.max_len ? p.max_len : l);
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

// ---- packed fp16 products (v_pk_mul_f16, v_pk_fma_f16, v_dot2_f32_f16)
__device__ __forceinline__ f16x2 as_h2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }
__device__ __forceinline__ uint32_t as_u32(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

// a * b (fp16 pairs) as hi + lo: hi = fp16(a b), lo = a b - hi, which is
// exact in fp16 (the rounding error of a product of two 11-bit significands
// fits in 11 bits, barring underflow), so the pair carries a b to ~22 bits
__device__ __forceinline__ void split_prod_h(uint32_t a, uint32_t b, uint32_t& hi, uint32_t& lo) {
    const f16x2 h = as_h2(a) * as_h2(b);
    hi = as_u32(h);
    lo = as_u32(__builtin_elementwise_fma(as_h2(a), as_h2(b), -h));
}

// (ah + al) * b as hi + lo: hi = fp16(ah b), lo = fp16(al b + (ah b - hi))
// with ah b - hi exact as above and one rounding in the outer fma
__device__ __forceinline__ void split_prod_hl(uint32_t ah, uint32_t al, uint32_t b, uint32_t& hi,
                                              uint32_t& lo) {
    const f16x2 h = as_h2(ah) * as_h2(b);
    hi = as_u32(h);
    lo = as_u32(__builtin_elementwise_fma(as_h2(al), as_h2(b),
                                          __builtin_elementwise_fma(as_h2(ah), as_h2(b), -h)));
}

// c + a.x b.x + a.y b.y in fp32 with fp16 operands read in place (two
// v_fma_mix).  v_dot2_f32_f16 would be one instruction, but on MI355X it is
// not correctly rounded (measured: ~11% of random inputs off, relative error
// up to 1.5e-3), too coarse for the zero-point sums.
__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float c) {
    return fmaf(hi_h(a), hi_h(b), fmaf(lo_h(a), lo_h(b), c));
}

// fp32 values hi + lo of two fp16 hi/lo pairs (exact: the halves of lo lie
// below the last bit of hi); neg1 = -1 keeps each a single v_fma_mix
__device__ __forceinline__ float join_lo(uint32_t hi, uint32_t lo, float neg1) {
    return -fmaf(lo_h(hi), neg1, -lo_h(lo));
}
__device__ __forceinline__ float join_hi(uint32_t hi, uint32_t lo, float neg1) {
    return -fmaf(hi_h(hi), neg1, -hi_h(lo));
}

// two fp32 values as fp16 hi + lo (hi = fp16(x), lo = fp16(x - hi); x - hi
// is exact in fp32)
__device__ __forceinline__ void split_f32(float a, float b, float neg1, uint32_t& hi, uint32_t& lo) {
    const f16x2 h = {_Float16(a), _Float16(b)};
    hi = as_u32(h);
    const f16x2 l = {_Float16(fmaf(float(h[0]), neg1, a)), _Float16(fmaf(float(h[1]), neg1, b))};
    lo = as_u32(l);
}

// halves (x.lo, y.lo) and (x.hi, y.hi): the K dimension of every contraction
// here runs in the quad order 0, 2, 1, 3 (see code_operands)
__device__ __forceinline__ uint32_t pair_lo(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x07060302u); }

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
//
// The code tiles of a workgroup's run [t_lo, t_hi) are read through buffer
// resources that span exactly that run: the prefetches that run past its
// end (every path issues the same loads, see the kernels) then return zeros
// without touching memory.  The small side-value loads are clamped to the
// last tile instead.
struct KTile {
    uint4 k0, k1;   // key codes, 32 B per lane
    uint4 ks;       // key scale (lanes 0..31) / zero (lanes 32..63)
};
struct VTile {
    uint4 v0, v1;   // value codes
    uint4 vs;       // value scale (lanes 0..31) / zero (lanes 32..63) of two tokens
};

struct TileRun {
    __amdgpu_buffer_rsrc_t kc, vc;
    int t0, t_last;
};

template <int G>
__device__ __forceinline__ TileRun tile_run(const MfmaParams& p, int64_t bh, int t_lo, int t_hi) {
    constexpr int NBT = 64 / G, W = G / 16;
    constexpr int FLAGS = 0x00020000;   // raw 32-bit buffer (gfx9 descriptor word 3)
    TileRun r;
    const int bytes = (t_hi - t_lo) * 2048;
    r.kc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(p.kc + (bh * p.nblk_cap + int64_t(t_lo) * NBT) * D * W),
                                             0, bytes, FLAGS);
    r.vc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(p.vc + (bh * p.cap + int64_t(t_lo) * 64) * 8), 0,
                                             bytes, FLAGS);
    r.t0 = t_lo;
    r.t_last = t_hi - 1;
    return r;
}

// 16-byte streaming load at byte offset off of a run (non-temporal)
__device__ __forceinline__ uint4 ld_run(__amdgpu_buffer_rsrc_t rs, int off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2);
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int G>
__device__ __forceinline__ void load_ktile(const MfmaParams& p, const TileRun& run, int64_t bh, int tt, int lane,
                                           KTile& r) {
    constexpr int NBT = 64 / G;
    const int off = (tt - run.t0) * 2048 + 16 * lane;
    r.k0 = ld_run(run.kc, off);
    r.k1 = ld_run(run.kc, off + 1024);
    const int ts = tt < run.t_last ? tt : run.t_last;
    const uint16_t* kside = (lane < 32 ? p.ks : p.kz) + (bh * p.nblk_cap + int64_t(ts) * NBT) * D;
    if (G == 64) {
        const uint2 v = ld_stream(reinterpret_cast<const uint2*>(kside) + (lane & 31));
        r.ks = make_uint4(v.x, v.y, 0u, 0u);
    } else {
        r.ks = ld_stream(reinterpret_cast<const uint4*>(kside) + (lane & 31));
    }
}

__device__ __forceinline__ void load_vtile(const MfmaParams& p, const TileRun& run, int64_t bh, int tt, int lane,
                                           VTile& r) {
    const int off = (tt - run.t0) * 2048 + 16 * lane;
    r.v0 = ld_run(run.vc, off);
    r.v1 = ld_run(run.vc, off + 1024);
    const int64_t ts = tt < run.t_last ? tt : run.t_last;
    // lane l (mod 32) takes tokens t = 4(l >> 1) + (l & 1) and t + 2: a pair
    // in the quad order of the K dimension
    const uint16_t* vside = (lane < 32 ? p.vs : p.vz) + (bh * p.cap + ts * 64) * 4;
    const int t = 4 * ((lane & 31) >> 1) + (lane & 1);
    const uint2 a = ld_stream(reinterpret_cast<const uint2*>(vside + 4 * t));
    const uint2 b = ld_stream(reinterpret_cast<const uint2*>(vside + 4 * (t + 2)));
    r.vs = make_uint4(a.x, a.y, b.x, b.y);
}

// ---- 4-bit tiles: 4 KB of key codes and 4 KB of value codes per 64-token
// tile (16 words per token, G/8 words per key block and channel); side
// values as for 2 bits.  A code nibble alone in bits 6..9 of an fp16 lane
// is the exact subnormal code * 2^-18 (code_operands, code_slice4), so each
// code byte feeds two MFMAs instead of four: twice the bytes and transposed
// reads per tile, the same MFMA and AND counts.
struct KTile4 {
    uint4 k[4];   // key codes, 64 B per lane
    uint4 ks;     // key scale (lanes 0..31) / zero (lanes 32..63)
};
struct VTile4 {
    uint4 v[4];   // value codes
    uint4 vs;     // value scale / zero of two tokens
};

constexpr int KTILE4_DW = 1088;   // key-code tile in LDS (dwords), padded (kdw4_64)
constexpr int VTILE4_DW = 1088;   // value-code tile in LDS (dwords), padded (vdw4)

template <int G>
__device__ __forceinline__ TileRun tile_run4(const MfmaParams& p, int64_t bh, int t_lo, int t_hi) {
    constexpr int NBT = 64 / G, W = G / 8;
    constexpr int FLAGS = 0x00020000;
    TileRun r;
    const int bytes = (t_hi - t_lo) * 4096;
    r.kc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(p.kc + (bh * p.nblk_cap + int64_t(t_lo) * NBT) * D * W),
                                             0, bytes, FLAGS);
    r.vc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(p.vc + (bh * p.cap + int64_t(t_lo) * 64) * 16), 0,
                                             bytes, FLAGS);
    r.t0 = t_lo;
    r.t_last = t_hi - 1;
    return r;
}

template <int G>
__device__ __forceinline__ void load_ktile4(const MfmaParams& p, const TileRun& run, int64_t bh, int tt, int lane,
                                            KTile4& r) {
    constexpr int NBT = 64 / G;
    const int off = (tt - run.t0) * 4096 + 16 * lane;
#pragma unroll
    for (int q = 0; q < 4; ++q) r.k[q] = ld_run(run.kc, off + 1024 * q);
    const int ts = tt < run.t_last ? tt : run.t_last;
    const uint16_t* kside = (lane < 32 ? p.ks : p.kz) + (bh * p.nblk_cap + int64_t(ts) * NBT) * D;
    if (G == 64) {
        const uint2 v = ld_stream(reinterpret_cast<const uint2*>(kside) + (lane & 31));
        r.ks = make_uint4(v.x, v.y, 0u, 0u);
    } else {
        r.ks = ld_stream(reinterpret_cast<const uint4*>(kside) + (lane & 31));
    }
}

__device__ __forceinline__ void load_vtile4(const MfmaParams& p, const TileRun& run, int64_t bh, int tt, int lane,
                                            VTile4& r) {
    const int off = (tt - run.t0) * 4096 + 16 * lane;
#pragma unroll
    for (int q = 0; q < 4; ++q) r.v[q] = ld_run(run.vc, off + 1024 * q);
    const int64_t ts = tt < run.t_last ? tt : run.t_last;
    const uint16_t* vside = (lane < 32 ? p.vs : p.vz) + (bh * p.cap + ts * 64) * 4;
    const int t = 4 * ((lane & 31) >> 1) + (lane & 1);
    const uint2 a = ld_stream(reinterpret_cast<const uint2*>(vside + 4 * t));
    const uint2 b = ld_stream(reinterpret_cast<const uint2*>(vside + 4 * (t + 2)));
    r.vs = make_uint4(a.x, a.y, b.x, b.y);
}

// dword of word w (0..7) of channel c in the staged G = 64 key tile: the
// cache layout with 4 dwords of pad after every 8 channels, so that the two
// 16-lane groups of a transposed read hit different banks
__device__ __forceinline__ int kdw4_64(int c, int w) { return 8 * c + w + 4 * (c >> 3); }
// dword of word w (0..15) of token t in the staged value tile: 4 dwords of
// pad after every 4 tokens (16 consecutive tokens on distinct banks)
__device__ __forceinline__ int vdw4(int t, int w) { return 16 * t + w + 4 * (t >> 2); }

// Key codes staged: G = 64 in kdw4_64 order; G = 32 in the cache layout
// (block be, channel c at dwords 512be + 4c .. 4c + 3).  Side values as for
// 2 bits.
template <int G>
__device__ __forceinline__ void stage_keys4(const KTile4& cur, uint32_t* kl, uint32_t* ksl, int lane) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = 64 * q + lane;   // 16-byte piece of the tile
        *reinterpret_cast<uint4*>(kl + (G == 64 ? kdw4_64(i >> 1, 4 * (i & 1)) : 4 * i)) = cur.k[q];
    }
    if (G == 64)
        *reinterpret_cast<uint2*>(ksl + (lane >> 5) * 128 + 2 * (lane & 31)) =
            make_uint2(pair_lo(cur.ks.x, cur.ks.y), pair_hi(cur.ks.x, cur.ks.y));
    else
        *reinterpret_cast<uint4*>(ksl + (lane >> 5) * 128 + 4 * (lane & 31)) =
            make_uint4(pair_lo(cur.ks.x, cur.ks.y), pair_hi(cur.ks.x, cur.ks.y),
                       pair_lo(cur.ks.z, cur.ks.w), pair_hi(cur.ks.z, cur.ks.w));
}

// Value codes staged in vdw4 order, side values as for 2 bits.
__device__ __forceinline__ void stage_values4(const VTile4& cur, uint32_t* vl, uint32_t* vsl, int lane) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = 64 * q + lane;
        *reinterpret_cast<uint4*>(vl + vdw4(i >> 2, 4 * (i & 3))) = cur.v[q];
    }
    uint32_t* row = vsl + (lane >> 5) * 128 + (lane & 31);
    row[0] = pair_lo(cur.vs.x, cur.vs.z);
    row[32] = pair_hi(cur.vs.x, cur.vs.z);
    row[64] = pair_lo(cur.vs.y, cur.vs.w);
    row[96] = pair_hi(cur.vs.y, cur.vs.w);
}

// Key row named by lane n of group kg for K-step ksx and half r (tokens
// 32r .. 32r + 31 of the tile; the block r for G = 32): lanes 2e, 2e + 1
// name channel 32ksx + 8kg + e, bytes 0-7 and 8-15 of that half.  Lane n
// then holds tokens 32r + 2n (low nibble) and 32r + 2n + 1 (high nibble) of
// the 8 channels.
template <int G>
__device__ __forceinline__ int key_row_dw4(int ksx, int r, int kg, int n) {
    const int c = 32 * ksx + 8 * kg + (n >> 1);
    return G == 64 ? kdw4_64(c, 4 * r + 2 * (n & 1)) : 512 * r + 4 * c + 2 * (n & 1);
}

// Value row named by lane n of group kg for K-step ksx (32 tokens) and pass
// P (words 4P .. 4P + 3 = channels 32P .. 32P + 31, one value group): lane
// n then holds channels 32P + 8(n >> 2) + 2(n & 3) (low nibble) and + 1
// (high nibble) of the 8 tokens.
__device__ __forceinline__ int value_row_dw4(int ksx, int P, int kg, int n) {
    return vdw4(32 * ksx + 8 * kg + (n >> 1), 4 * P + 2 * (n & 1));
}

// Paged runs: the tiles of a run lie in the pages the block table names.
// Lane l holds the page of block NBT * t_lo + l (a run spans at most 64
// blocks); each tile's code loads go through buffer resources over its own
// page(s), empty past the run, so the same branch-free prefetch works.
struct PagedRun {
    int pg;   // this lane's page
    int t0, t_last, kvh;
};

// The page numbers of the p.chunk tiles from t_lo (those inside the table
// row): they do not depend on the sequence length, so this load is issued
// alongside the length's instead of after it (two dependent round trips
// before the first tile arrives, not three).  t_last is set once the length
// is known.
template <int G>
__device__ __forceinline__ PagedRun paged_run(const MfmaParams& p, int b, int kvh, int t_lo, int lane) {
    constexpr int NBT = 64 / G;
    PagedRun r;
    const int64_t j = int64_t(t_lo) * NBT + lane;
    r.pg = lane < p.chunk * NBT && j < p.maxb ? page_of(p, b, j) : 0;
    r.t0 = t_lo;
    r.t_last = t_lo - 1;
    r.kvh = kvh;
    return r;
}

// block row of block e (0 .. NBT-1) of tile tt (clamped into the run); the
// lane index is wave-uniform
template <int G>
__device__ __forceinline__ int64_t paged_row(const MfmaParams& p, const PagedRun& run, int tt, int e) {
    constexpr int NBT = 64 / G;
    const int ic = (tt <= run.t_last ? tt : run.t_last) - run.t0;
    return int64_t(__builtin_amdgcn_readlane(run.pg, ic * NBT + e)) * p.Hkv + run.kvh;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint32_t* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(base), 0, bytes, 0x00020000);
}

template <int G>
__device__ __forceinline__ void load_ktile(const MfmaParams& p, const PagedRun& run, int64_t, int tt, int lane,
                                           KTile& r) {
    constexpr int W = G / 16;
    const bool in = tt <= run.t_last;
    const int64_t ra = paged_row<G>(p, run, tt, 0);
    const uint16_t* side = lane < 32 ? p.ks : p.kz;
    if (G == 64) {
        const __amdgpu_buffer_rsrc_t rs = page_rsrc(p.kc + ra * D * W, in ? 2048 : 0);
        r.k0 = ld_run(rs, 16 * lane);
        r.k1 = ld_run(rs, 16 * lane + 1024);
        const uint2 v = ld_stream(reinterpret_cast<const uint2*>(side + ra * D) + (lane & 31));
        r.ks = make_uint4(v.x, v.y, 0u, 0u);
    } else {
        const int64_t rb = paged_row<G>(p, run, tt, 1);
        r.k0 = ld_run(page_rsrc(p.kc + ra * D * W, in ? 1024 : 0), 16 * lane);
        r.k1 = ld_run(page_rsrc(p.kc + rb * D * W, in ? 1024 : 0), 16 * lane);
        r.ks = ld_stream(reinterpret_cast<const uint4*>(side + ((lane & 16) ? rb : ra) * D) + (lane & 15));
    }
}

template <int G>
__device__ __forceinline__ void load_vtile(const MfmaParams& p, const PagedRun& run, int64_t, int tt, int lane,
                                           VTile& r) {
    const bool in = tt <= run.t_last;
    const int64_t ra = paged_row<G>(p, run, tt, 0);
    // lane l (mod 32) takes tokens t = 4(l >> 1) + (l & 1) and t + 2 (same block)
    const int t = 4 * ((lane & 31) >> 1) + (lane & 1);
    int64_t vrow;
    if (G == 64) {
        const __amdgpu_buffer_rsrc_t rs = page_rsrc(p.vc + ra * 64 * 8, in ? 2048 : 0);
        r.v0 = ld_run(rs, 16 * lane);
        r.v1 = ld_run(rs, 16 * lane + 1024);
        vrow = ra * 64 + t;
    } else {
        const int64_t rb = paged_row<G>(p, run, tt, 1);
        r.v0 = ld_run(page_rsrc(p.vc + ra * 32 * 8, in ? 1024 : 0), 16 * lane);
        r.v1 = ld_run(page_rsrc(p.vc + rb * 32 * 8, in ? 1024 : 0), 16 * lane);
        vrow = t < 32 ? ra * 32 + t : rb * 32 + (t - 32);
    }
    const uint16_t* vside = (lane < 32 ? p.vs : p.vz) + vrow * 4;
    const uint2 a = ld_stream(reinterpret_cast<const uint2*>(vside));
    const uint2 b = ld_stream(reinterpret_cast<const uint2*>(vside + 8));
    r.vs = make_uint4(a.x, a.y, b.x, b.y);
}

// the code-tile run of a main split: contiguous (one buffer resource per
// run) or paged (per-tile resources over the pages of the block table,
// loaded at the kernel's start)
template <int G, bool PAGED>
__device__ __forceinline__ auto pick_run(const MfmaParams& p, const PagedRun& prun, int64_t bh, int t_lo, int t_hi) {
    if constexpr (PAGED)
        return prun;
    else
        return tile_run<G>(p, bh, t_lo, t_hi);
}

// 4-bit tiles over pages: G = 64, one 4 KB page block per tile; G = 32, two
// 2 KB blocks (tokens 0..31, 32..63), as the contiguous layout splits them
template <int G>
__device__ __forceinline__ void load_ktile4(const MfmaParams& p, const PagedRun& run, int64_t, int tt, int lane,
                                            KTile4& r) {
    constexpr int W = G / 8;
    const bool in = tt <= run.t_last;
    const int64_t ra = paged_row<G>(p, run, tt, 0);
    const uint16_t* side = lane < 32 ? p.ks : p.kz;
    if (G == 64) {
        const __amdgpu_buffer_rsrc_t rs = page_rsrc(p.kc + ra * D * W, in ? 4096 : 0);
#pragma unroll
        for (int q = 0; q < 4; ++q) r.k[q] = ld_run(rs, 16 * lane + 1024 * q);
        const uint2 v = ld_stream(reinterpret_cast<const uint2*>(side + ra * D) + (lane & 31));
        r.ks = make_uint4(v.x, v.y, 0u, 0u);
    } else {
        const int64_t rb = paged_row<G>(p, run, tt, 1);
        const __amdgpu_buffer_rsrc_t rsa = page_rsrc(p.kc + ra * D * W, in ? 2048 : 0);
        const __amdgpu_buffer_rsrc_t rsb = page_rsrc(p.kc + rb * D * W, in ? 2048 : 0);
        r.k[0] = ld_run(rsa, 16 * lane);
        r.k[1] = ld_run(rsa, 16 * lane + 1024);
        r.k[2] = ld_run(rsb, 16 * lane);
        r.k[3] = ld_run(rsb, 16 * lane + 1024);
        r.ks = ld_stream(reinterpret_cast<const uint4*>(side + ((lane & 16) ? rb : ra) * D) + (lane & 15));
    }
}

template <int G>
__device__ __forceinline__ void load_vtile4(const MfmaParams& p, const PagedRun& run, int64_t, int tt, int lane,
                                            VTile4& r) {
    const bool in = tt <= run.t_last;
    const int64_t ra = paged_row<G>(p, run, tt, 0);
    const int t = 4 * ((lane & 31) >> 1) + (lane & 1);
    int64_t vrow;
    if (G == 64) {
        const __amdgpu_buffer_rsrc_t rs = page_rsrc(p.vc + ra * 64 * 16, in ? 4096 : 0);
#pragma unroll
        for (int q = 0; q < 4; ++q) r.v[q] = ld_run(rs, 16 * lane + 1024 * q);
        vrow = ra * 64 + t;
    } else {
        const int64_t rb = paged_row<G>(p, run, tt, 1);
        const __amdgpu_buffer_rsrc_t rsa = page_rsrc(p.vc + ra * 32 * 16, in ? 2048 : 0);
        const __amdgpu_buffer_rsrc_t rsb = page_rsrc(p.vc + rb * 32 * 16, in ? 2048 : 0);
        r.v[0] = ld_run(rsa, 16 * lane);
        r.v[1] = ld_run(rsa, 16 * lane + 1024);
        r.v[2] = ld_run(rsb, 16 * lane);
        r.v[3] = ld_run(rsb, 16 * lane + 1024);
        vrow = t < 32 ? ra * 32 + t : rb * 32 + (t - 32);
    }
    const uint16_t* vside = (lane < 32 ? p.vs : p.vz) + vrow * 4;
    const uint2 a = ld_stream(reinterpret_cast<const uint2*>(vside));
    const uint2 b = ld_stream(reinterpret_cast<const uint2*>(vside + 8));
    r.vs = make_uint4(a.x, a.y, b.x, b.y);
}

// 4-bit runs: contiguous or paged
template <int G, bool PAGED>
__device__ __forceinline__ auto pick_run4(const MfmaParams& p, const PagedRun& prun, int64_t bh, int t_lo, int t_hi) {
    if constexpr (PAGED)
        return prun;
    else
        return tile_run4<G>(p, bh, t_lo, t_hi);
}
// the contiguous value loader with the paged overload's call shape
template <int G>
__device__ __forceinline__ void load_vtile4(const MfmaParams& p, const TileRun& run, int64_t bh, int tt, int lane,
                                            VTile4& r) {
    load_vtile4(p, run, bh, tt, lane, r);
}

// contiguous runs, same call shape as the paged overload
template <int G>
__device__ __forceinline__ void load_vtile(const MfmaParams& p, const TileRun& run, int64_t bh, int tt, int lane,
                                           VTile& r) {
    load_vtile(p, run, bh, tt, lane, r);
}

// Key codes staged in their cache layout: G = 64, channel c of the tile at
// dwords 4c..4c+3 (word j = tokens 16j..16j+15); G = 32, block be, channel c
// at dwords 256be + 2c, +1.  Side values to ksl [scale | zero][block][128 fp16]
// in quad order.
template <int G>
__device__ __forceinline__ void stage_keys(const KTile& cur, uint32_t* kl, uint32_t* ksl, int lane) {
    *reinterpret_cast<uint4*>(kl + 4 * lane) = cur.k0;
    *reinterpret_cast<uint4*>(kl + 4 * (lane + 64)) = cur.k1;
    // side values with the channels of each quad in the order 0, 2, 1, 3
    if (G == 64)
        *reinterpret_cast<uint2*>(ksl + (lane >> 5) * 128 + 2 * (lane & 31)) =
            make_uint2(pair_lo(cur.ks.x, cur.ks.y), pair_hi(cur.ks.x, cur.ks.y));
    else
        *reinterpret_cast<uint4*>(ksl + (lane >> 5) * 128 + 4 * (lane & 31)) =
            make_uint4(pair_lo(cur.ks.x, cur.ks.y), pair_hi(cur.ks.x, cur.ks.y),
                       pair_lo(cur.ks.z, cur.ks.w), pair_hi(cur.ks.z, cur.ks.w));
}

// dword of word w of token t in the staged value tile: the cache layout
// (8 words per token) with 16 bytes of pad before every odd group of 8
// tokens (group g starts 4 * ((g + 1) >> 1) dwords late), so that the two
// 16-lane groups of a transposed read (groups 2k, 2k + 1) hit different banks
__device__ __forceinline__ int vtile_dw(int t, int w) { return 8 * t + w + 4 * (((t >> 3) + 1) >> 1); }

// Value codes staged in the cache layout (padded as above), side values to
// vsl [scale | zero][group][32 token pairs]: dword 2k + j of a group row
// holds tokens 4k + j, 4k + j + 2 (the quad order of the K dimension).
__device__ __forceinline__ void stage_values(const VTile& cur, uint32_t* vl, uint32_t* vsl, int lane) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int i = lane + 64 * half;
        *reinterpret_cast<uint4*>(vl + vtile_dw(i >> 1, 4 * (i & 1))) = half ? cur.v1 : cur.v0;
    }
    uint32_t* row = vsl + (lane >> 5) * 128 + (lane & 31);
    row[0] = pair_lo(cur.vs.x, cur.vs.z);
    row[32] = pair_hi(cur.vs.x, cur.vs.z);
    row[64] = pair_lo(cur.vs.y, cur.vs.w);
    row[96] = pair_hi(cur.vs.y, cur.vs.w);
}

// ds_read_b64_tr_b8: within each group of 16 lanes, lane i names an 8-byte
// row; lane j receives byte (j & 7) of the rows named by lanes
// 2e + (j >> 3), e = 0..7 (in that order).  The operand builders below use
// it so that each lane reads only the code bytes its MFMA column needs.
typedef int lds_v2i __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ld_tr8(const uint32_t* p) {
    const lds_v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) lds_v2i*)(p));
    return make_uint2(uint32_t(r.x), uint32_t(r.y));
}

// Key-code row named by lane n of group kg for K-step ksx (32 channels):
// lanes 2e, 2e + 1 name channel 32ksx + 8kg + e, words 0-1 and 2-3 (G = 64),
// or both its two words in block be (G = 32).  Lane n then holds byte n & 3
// of word row n >> 2 (G = 64) or (n >> 2) & 1 (G = 32) for the 8 channels.
template <int G>
__device__ __forceinline__ int key_row_dw(int ksx, int be, int kg, int n) {
    const int c = 32 * ksx + 8 * kg + (n >> 1);
    return G == 64 ? 4 * c + 2 * (n & 1) : 256 * be + 2 * c;
}

// Value-code row named by lane n of group kg for K-step ksx (32 tokens) and
// channel half P: lanes 2e, 2e + 1 name token 32ksx + 8kg + e, words
// 4P + 0-1 and 4P + 2-3.  Lane n then holds byte n & 3 of word 4P + (n >> 2)
// for the 8 tokens.
__device__ __forceinline__ int value_row_dw(int ksx, int P, int kg, int n) {
    return vtile_dw(32 * ksx + 8 * kg + (n >> 1), 4 * P + 2 * (n & 1));
}

// The 8 code bytes e = 0..7 of a transposed read as MFMA operand registers.
// An fp16 lane whose only set bits are one code field is the subnormal
// code * 2^(f - 24), f the field's lowest bit: an exact operand.  But the
// matrix cores align the 32 products of a dot product to the largest
// product's nominal exponent, and a subnormal operand counts with the
// exponent of 2^-14 whatever its leading zeros: a field low in the mantissa
// loses that many bits of the sum's precision (measured on gfx950
// v_mfma_f32_16x16x32_f16: codes at bits 0..1 gave sums off by ~2^12 ulps
// of the largest product; single products are exact).  So each code is read
// from a copy of the bytes shifted to put its field at bits 6..9 of its fp16
// half (at most 2 leading zeros below the top mantissa bit):
//   a: bytes at bit 6 of each half -- 2-bit positions u = 0, 1 (fields 6..7,
//      8..9) and the low 4-bit nibble (field 6..9);
//   b: bytes at bit 2 -- 2-bit positions u = 2, 3 and the high nibble.
// Register j of a set holds bytes (0, 2), (1, 3), (4, 6), (5, 7) in its two
// halves (a shift spills neighbouring bytes only outside the fields), so
// the K index runs over e in the quad order 0, 2, 1, 3; the A operands (q',
// p') are laid out in the same order.  Results carry a factor
// 2^-(24 - f): code_unscale2 / code_unscale4 undo it.
// The shifts run on the 8 bytes as one 64-bit word: v_lshlrev_b64 /
// v_lshrrev_b64 issue at the rate of 32-bit shifts on gfx950 (an in-bounds
// probe timed 8 of each per loop at the same 1.27 ms), so four of them
// replace eight.  The bits that cross between the two words land at bits
// 0..5 or 10..15 of a half, outside every field.  The shift counts come from
// opaque scalar registers: with constant counts the compiler splits each
// 64-bit shift into two 32-bit ones.
struct CodeRegs {
    uint32_t a[4], b[4];
};
__device__ __forceinline__ CodeRegs code_operands(uint2 r) {
    const uint64_t w = (uint64_t(r.y) << 32) | r.x;
    uint32_t s2, s6;
    asm("s_mov_b32 %0, 2" : "=s"(s2));
    asm("s_mov_b32 %0, 6" : "=s"(s6));
    const uint64_t l6 = w << s6, r2 = w >> s2, l2 = w << s2, r6 = w >> s6;
    return CodeRegs{{uint32_t(l6), uint32_t(r2), uint32_t(l6 >> 32), uint32_t(r2 >> 32)},
                    {uint32_t(l2), uint32_t(r6), uint32_t(l2 >> 32), uint32_t(r6 >> 32)}};
}
// 2-bit code position u (0..3) of every byte; `lanes_mk` variant: the set
// (u >> 1) is uniform and the field (u & 1) may differ per lane
__device__ __forceinline__ uint32_t code_mask2(int u) { return 0x00030003u << (6 + 2 * (u & 1)); }
__device__ __forceinline__ f16x8 code_slice_set(const CodeRegs& c, bool hi_set, uint32_t mk) {
    const uint32_t* x = hi_set ? c.b : c.a;
    return as_f16x8(x[0] & mk, x[1] & mk, x[2] & mk, x[3] & mk);
}
__device__ __forceinline__ f16x8 code_slice2(const CodeRegs& c, int u) {
    return code_slice_set(c, u >= 2, code_mask2(u));
}
// 4-bit nibble nib (0: low, 1: high) of every byte, field 6..9
__device__ __forceinline__ f16x8 code_slice4(const CodeRegs& c, int nib) {
    return code_slice_set(c, nib != 0, 0x03C003C0u);
}
__device__ __forceinline__ float code_unscale2(int u) { return __builtin_ldexpf(1.0f, 18 - 2 * (u & 1)); }
__device__ __forceinline__ float code_unscale4() { return __builtin_ldexpf(1.0f, 18); }

// ---- trailing tokens [ntiles*64, T) on the VALU: partial key block and the
// fp16 residual keys, one token per lane for the logits, two channels per
// lane for the values.  Runs on one wave; qf holds HG*D floats, pl HG*PSTR.

// tokens [ntiles * 64, T) of sequence b, nblk of its key blocks quantized
// (an empty range writes an empty partial: m = -inf, l = 0, acc = 0).  Run
// by both waves of the workgroup; it is a chain of dependent round trips
// that a launch can end on, so every phase issues all of its loads before
// using any:
//  - wave 0, lane j = token j: the query (one 16-byte load per lane) and
//    the token's whole fp16 residual key row (16 loads), or for a quantized
//    token (G = 32 only) its codes and side values 16 channels at a time;
//    logits in channel order, softmax, weights to LDS;
//  - both waves, lane = channel (wave w: channels 64w ..): values 16
//    tokens at a time, accumulated in token order.
// The tail spans at most two key blocks, whose rows are looked up once.
template <int HG, class Blocks, int BITS = 2>
__device__ void tail_split(const MfmaParams& p, const Blocks& blocks, int b, int kvh, int s, float* qf, float* pl,
                           int64_t T, int64_t nblk, int ntiles) {
    constexpr int PER = 32 / BITS;              // codes per word
    constexpr uint32_t LMASK = (1u << BITS) - 1u;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hq0 = kvh * HG;
    const int64_t t0 = int64_t(ntiles) * 64;
    const int n_tail = int(T - t0);
    const int64_t Tq = nblk * p.G;
    const int64_t jb = t0 / p.G;   // first key block of the tail
    const int64_t row0 = n_tail > 0 ? blocks(p, b, kvh, jb) : 0;
    const int64_t row1 = n_tail > 0 && (T - 1) / p.G > jb ? blocks(p, b, kvh, jb + 1) : row0;
    float m[HG], l[HG];
    if (wave == 0) {
        // the query: HG * D fp16, 8 per lane
        uint4 qv = make_uint4(0u, 0u, 0u, 0u);
        if (lane < HG * D / 8) qv = *reinterpret_cast<const uint4*>(p.q + (int64_t(b) * p.Hq + hq0) * D + 8 * lane);
        const int64_t t = t0 + lane;
        const bool valid = lane < n_tail;
        const bool resid = t >= Tq;
        // a residual key row: all 16 loads at once
        uint4 kr[16];
        const uint16_t* krow = p.kr + ((int64_t(b) * p.Hkv + kvh) * p.G + (valid && resid ? t - Tq : 0)) * D;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            kr[i] = valid && resid ? *reinterpret_cast<const uint4*>(krow + 8 * i) : make_uint4(0u, 0u, 0u, 0u);
        if (lane < HG * D / 8) {
            const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qf[8 * lane + 2 * e] = lo_h(w[e]);
                qf[8 * lane + 2 * e + 1] = hi_h(w[e]);
            }
        }
        wave_sync();
        float sc[HG];
#pragma unroll
        for (int h = 0; h < HG; ++h) sc[h] = 0.0f;
        if (valid && resid) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t w[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float kh = (e & 1) ? hi_h(w[e >> 1]) : lo_h(w[e >> 1]);
#pragma unroll
                    for (int h = 0; h < HG; ++h) sc[h] = fmaf(qf[h * D + 8 * i + e], kh, sc[h]);
                }
            }
        }
        // (a separate pass, so that the residual row's registers are free)
        if (valid && !resid) {
            // token i of quantized block jb or jb + 1 (the tail starts at
            // block jb's first token)
            const int jt = int(t - t0);
            const int64_t rowq = jt < p.G ? row0 : row1;
            const int i = jt < p.G ? jt : jt - p.G;
            for (int c0 = 0; c0 < D; c0 += 16) {
                const int64_t side = rowq * D + c0;
                uint32_t wd[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) wd[e] = p.kc[(side + e) * (p.G / PER) + i / PER];
                uint32_t sw[8], zw[8];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const uint4 sv = *reinterpret_cast<const uint4*>(p.ks + side + 8 * e);
                    const uint4 zv = *reinterpret_cast<const uint4*>(p.kz + side + 8 * e);
                    sw[4 * e] = sv.x; sw[4 * e + 1] = sv.y; sw[4 * e + 2] = sv.z; sw[4 * e + 3] = sv.w;
                    zw[4 * e] = zv.x; zw[4 * e + 1] = zv.y; zw[4 * e + 2] = zv.z; zw[4 * e + 3] = zv.w;
                }
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float se = (e & 1) ? hi_h(sw[e >> 1]) : lo_h(sw[e >> 1]);
                    const float ze = (e & 1) ? hi_h(zw[e >> 1]) : lo_h(zw[e >> 1]);
                    const float kh = fmaf(float((wd[e] >> (BITS * (i % PER))) & LMASK), se, ze);
#pragma unroll
                    for (int h = 0; h < HG; ++h) sc[h] = fmaf(qf[h * D + c0 + e], kh, sc[h]);
                }
            }
        }
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
    }
    __syncthreads();
    // PV: this lane's channel, 16 tokens per round of loads
    const int c = 64 * wave + lane;
    float acc[HG];
#pragma unroll
    for (int h = 0; h < HG; ++h) acc[h] = 0.0f;
    for (int j0 = 0; j0 < n_tail; j0 += 16) {
        uint32_t w[16];
        uint16_t sv[16], zv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            // past the tail: reload its last token (in bounds, unused).  The
            // tail starts on a block boundary (t0 = jb * G), so token j of it
            // is in block jb + (j >= G)
            const int j = j0 + e < n_tail ? j0 + e : n_tail - 1;
            const int64_t row = j < p.G ? row0 * p.G + j : row1 * p.G + (j - p.G);
            w[e] = p.vc[row * (D / PER) + c / PER];
            sv[e] = p.vs[row * 4 + c / 32];
            zv[e] = p.vz[row * 4 + c / 32];
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            if (j0 + e < n_tail) {
                const float vh = fmaf(float((w[e] >> (BITS * (c % PER))) & LMASK), h2f(sv[e]), h2f(zv[e]));
#pragma unroll
                for (int h = 0; h < HG; ++h) acc[h] = fmaf(pl[h * PSTR + j0 + e], vh, acc[h]);
            }
        }
    }
#pragma unroll
    for (int h = 0; h < HG; ++h) p.ws_acc[((int64_t(b) * p.Hq + hq0 + h) * p.S + s) * D + c] = acc[h];
    if (wave == 0) {
#pragma unroll
        for (int h = 0; h < HG; ++h) {
            if (lane == h) {
                const int64_t slot = (int64_t(b) * p.Hq + hq0 + h) * p.S + s;
                p.ws_ml[slot * 2] = m[h];
                p.ws_ml[slot * 2 + 1] = l[h];
            }
        }
    }
}

// The decode step's append, done by the tail workgroup (both waves call
// it; wave 0's lanes do the work) before it attends: the new token T - 1 completes no key block, so its key is
// residual row T - 1 - nblk * G and its value row is quantized by the same
// device code as the append kernels (bit-identical).  No other workgroup
// reads these rows: the main splits end at the last whole tile, and the
// tail covers everything after it.
template <int BITS>
__device__ void fused_append(const MfmaParams& p, int b, int kvh, int lane) {
    const int64_t bh = int64_t(b) * p.Hkv + kvh;
    const int64_t t = p.T - 1;
    constexpr int TPR = D / 8;   // threads per row: 8 channels each
    if (threadIdx.x >= 64) {
        // wave 1 only waits for wave 0's stores
    } else if (lane < TPR) {
        // one value row: whole 4-lane groups (lanes 0 .. 15)
        qdev::ValueArgs va;
        va.vin = p.v_new;
        va.n_in = 1;
        va.row0 = 0;
        va.n_tok = 1;
        va.vd = D;
        va.BH = 0;   // unused by the row routine
        va.codes = p.vc_w;
        va.scale = p.vs_w;
        va.zero = p.vz_w;
        const qdev::ContigRows rows{p.cap, t, 1};
        qdev::quant_values_thread<BITS>(va, rows, bh * TPR + lane);
    } else if (lane < 2 * TPR) {
        const int v = lane - TPR;
        const int64_t r = t - p.nblk * p.G;
        *reinterpret_cast<uint4*>(p.kr_w + (bh * p.G + r) * D + v * 8) =
            *reinterpret_cast<const uint4*>(p.k_new + bh * D + v * 8);
    }
    // the stores complete before either wave reads these rows back
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __syncthreads();
}

// The paged decode step's append of token L of sequence b, done by the tail
// workgroup (both waves) before it attends: the value row is quantized into
// its page; the key goes into residual row L mod G, or, when it is the
// block's last, the block (G - 1 residual rows and the new key) is
// quantized per channel into its page.  The same device code as the append
// kernels (bit-identical).  Main splits read only tiles complete before the
// step, so no other workgroup reads these rows.
template <int G, int BITS>
__device__ void fused_append_paged(const MfmaParams& p, int b, int kvh, int64_t L) {
    const int tid = threadIdx.x;
    const int64_t bh = int64_t(b) * p.Hkv + kvh;
    constexpr int TPR = D / 8;
    const PagedSeq ps{p.table, p.lens, p.n_new, p.maxb, p.npages};
    if (tid < TPR) {
        qdev::ValueArgs va;
        va.vin = p.v_new;
        va.n_in = 1;
        va.row0 = 0;
        va.n_tok = 1;
        va.vd = D;
        va.BH = 0;
        va.codes = p.vc_w;
        va.scale = p.vs_w;
        va.zero = p.vz_w;
        const qdev::PagedRows rows{ps, p.Hkv, G, 1};
        qdev::quant_values_thread<BITS>(va, rows, bh * TPR + tid);
    }
    if (L % G == G - 1) {
        const int64_t fb = L / G;
        const int64_t dst = qdev::paged_block_row(ps, b, kvh, p.Hkv, fb);
        if (dst >= 0) {
            const qdev::KeyJob j{p.k_new + bh * D, p.kr + bh * G * D, fb * G, L, fb * G, dst};
            // a multiple of 64 when a channel pair spans several waves' lanes
            const int64_t nk = qdev::key_threads_per_block<G, BITS>(D);
            for (int64_t base = 0; base < nk; base += blockDim.x) {
                const int64_t idx = base + tid;
                if (idx < nk) {
                    int64_t unit;
                    int cp, sp;
                    qdev::key_thread_coords<G, BITS>(idx, D, unit, cp, sp);
                    qdev::quant_key_pair<G, BITS>(j, D, cp, sp, p.kc_w, p.ks_w, p.kz_w);
                }
            }
        }
    } else if (tid >= 64 && tid < 64 + TPR) {
        const int v = tid - 64;
        *reinterpret_cast<uint4*>(p.kr_w + (bh * G + L % G) * D + v * 8) =
            *reinterpret_cast<const uint4*>(p.k_new + bh * D + v * 8);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __syncthreads();
}

// Tokens and appended rows of sequence b in a paged call.  Without the fused
// append: the clamped length, none appended.  With it: the length before the
// step and 1 when the step appends to b (lens[b] >= 0, n_new[b] in {0, 1},
// within capacity and max_len), else the clamped length and 0.
__device__ __forceinline__ void paged_step_len(const MfmaParams& p, int b, int G, int& L, int& n_app) {
    L = seq_len(p, b);
    n_app = 0;
    if (p.fuse) {
        const int raw = p.lens[b];
        const int nn = p.n_new ? p.n_new[b] : 1;
        const int64_t lim = int64_t(p.maxb) * G < p.max_len ? int64_t(p.maxb) * G : p.max_len;
        if (raw >= 0 && (nn == 0 || nn == 1) && int64_t(raw) + nn <= lim) {
            L = raw;
            n_app = nn;
        }
    }
}

// the contiguous cache's tail: its counters are in the parameters
template <int HG, int BITS = 2>
__device__ void tail_split(const MfmaParams& p, int b, int kvh, int s, float* qf, float* pl) {
    if (p.fuse) fused_append<BITS>(p, b, kvh, threadIdx.x & 63);
    tail_split<HG, ContigBlocks, BITS>(p, ContigBlocks{}, b, kvh, s, qf, pl, p.T, p.nblk, p.ntiles);
}

// The tail workgroup (partial tile and residual keys, a chain of dependent
// loads on one wave) is block x = 0 of its (sequence, KV head), so that it
// starts with the first wave of workgroups instead of the last; it still
// writes partial slot S_main.  Returns the partial slot of this workgroup.
// Block coordinates: (sequence b, KV head kvh, partial slot s, tail).  The
// split-major grid (KV heads, batch, slots) makes consecutive workgroups take
// the same split of different (sequence, KV head) pairs; the GQA kernels
// launch it over contiguous caches (32K pass-1 -2% at 2 bits, -3.5% at 4 bits,
// interleaved on one box).  The slot-major grid (slots, KV heads, batch) is
// kept by the MHA kernels (+1.5% with the other order) and by paged caches
// (+13% on the ragged workload).  Slot 0 of the grid is the tail split,
// which writes partial slot S_main.
template <bool SPLIT_MAJOR>
__device__ __forceinline__ int block_coords(const MfmaParams& p, int& b, int& kvh, bool& tail) {
    const int x = SPLIT_MAJOR ? int(blockIdx.z) : int(blockIdx.x);
    kvh = SPLIT_MAJOR ? int(blockIdx.x) : int(blockIdx.y);
    b = SPLIT_MAJOR ? int(blockIdx.y) : int(blockIdx.z);
    const bool has_tail = p.S > p.S_main;
    tail = has_tail && x == 0;
    return tail ? p.S_main : x - (has_tail ? 1 : 0);
}
template <bool SPLIT_MAJOR>
inline dim3 decode_grid(int S, int Hkv, int B) { return SPLIT_MAJOR ? dim3(Hkv, B, S) : dim3(S, Hkv, B); }

// a main split with no tiles (a sequence shorter than the split's range)
template <int HG>
__device__ void empty_partial(const MfmaParams& p, int b, int kvh, int s) {
    const int hq0 = kvh * HG;
    for (int i = threadIdx.x; i < HG * D; i += blockDim.x)
        p.ws_acc[((int64_t(b) * p.Hq + hq0 + i / D) * p.S + s) * D + i % D] = 0.0f;
    if (threadIdx.x < HG) {
        const int64_t slot = (int64_t(b) * p.Hq + hq0 + threadIdx.x) * p.S + s;
        p.ws_ml[slot * 2] = -INFINITY;
        p.ws_ml[slot * 2 + 1] = 0.0f;
    }
}

}  // namespace
}  // namespace kvq
