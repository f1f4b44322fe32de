// kvq_prefill.hip -- causal prefill attention over the prompt's fp16 keys and
// values on the matrix cores, fused with the bulk quantization of those keys
// and values into an empty cache.
//
// Method ("Makale Bülteni -- KIVI", section "Kod ve Entegrasyon Haritası"): in
// the prefill phase KIVI runs ordinary attention over the full-precision
// prompt (a FlashAttention kernel there) and the cache is quantized from the
// same fp16 tensors (section "İddia ve Gerçeklik: KIVI": keys per channel in
// G-token blocks with the unfilled block kept in fp16, values per token).
// This kernel does both in one pass over the prompt in HBM.
//
// Work split: one eight-wave workgroup per (128 query rows, query head,
// sequence); wave w owns rows 16w .. 16w + 15.  The grid is one dimension
// with the query block slowest, so the longest causal windows of every head
// start first and the shortest fill the end.  A workgroup walks the 64-token
// key / value tiles of its causal window, staging each tile in LDS row-major
// (keys and values alike) for all eight waves, in two buffers so that one
// barrier per tile suffices; on the two diagonal tiles a wave masks the tile
// that crosses its rows and skips one that lies wholly after them.
//   S^T = K Q^T  (A = key rows from LDS, B = the query rows, in registers)
//   O^T = V^T P^T (A = value columns, read from the value rows with the
//                 transposing ds_read_b64_tr_b16; B = the weights, in registers)
// With these orientations each lane holds one query row in both results: the
// weights of S^T's accumulator feed O^T's B operand without leaving the lane,
// and the softmax rescale and the final 1/l stay lane-local.  Softmax in
// log2 units with the running maximum moved only when a logit exceeds it by
// more than 2^8 (weights stay <= 256 in fp16).  The weights enter the second
// product as fp16 pairs hi = fp16(p), lo = fp16(p - hi) (two products into
// one accumulator), so they keep ~22 bits where FlashAttention's single fp16
// weight keeps 11: with unrounded sums l the output is then within the fp16
// rounding of the result, not within 2^-11 max|v| of it.
//
// Fused quantize: the workgroups of query block i quantize its tiles 2i and
// 2i + 1 (values of their rows, the key blocks they complete, the unfilled
// block's rows into the residual) from the copies still staged in the two LDS
// buffers after the loop, split over the KV head's query heads, with the
// append kernels' device code: the cache equals kv_quantize_append's bit for
// bit and the prompt is read from HBM once.
#include "kvq_quant_dev.h"

namespace kvq {
namespace {

constexpr int PD = 128;     // head dim of q, k and v
constexpr int PNW = 8;      // waves per workgroup, 16 query rows each
constexpr int PBM = 16 * PNW;
// dwords per staged key and value row (128 fp16 + 16 pad).  A row stride of
// 8 banks (mod 64) suits both the 16-byte key reads and the transposed value
// reads: the LDS bank-conflict counter reads a third of what a 4-bank stride
// gives for either array (measured over whole launches)
constexpr int PKS = 72;
constexpr int PVR = 72;
constexpr float PTAU = 8.0f;

template <bool B>
struct Diag {
    static constexpr bool value = B;
};

typedef _Float16 pf16x8 __attribute__((ext_vector_type(8)));
typedef float pf32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ pf16x8 as_pf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(pf16x8, u4v{a, b, c, d});
}
typedef _Float16 f16x2p __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, h2{_Float16(a), _Float16(b)});
}

struct PrefillBuf {
    __attribute__((aligned(16))) uint32_t kl[64 * PKS];    // key rows of the tile
    __attribute__((aligned(16))) uint32_t vl[64 * PVR];    // value rows of the tile
};
// tile j is staged in buffer j & 1, so the block's two diagonal tiles are both
// still staged after the loop (70 KB: two eight-wave workgroups per CU)
struct PrefillLds {
    PrefillBuf buf[2];
};

// One 64-token tile in registers: thread t holds key and value row t >> 3,
// channels 16 (t & 7) .. + 15
struct PTile {
    uint4 k[2], v[2];
};

typedef short ps4 __attribute__((ext_vector_type(4)));
// ds_read_b64_tr_b16: within each group of 16 lanes, lane j receives 16-bit
// element j & 3 of the 8-byte rows named by lanes (j >> 2) + 4e, e = 0..3
// (read off an in-bounds probe on gfx950)
__device__ __forceinline__ uint2 ld_tr16(const uint32_t* p) {
    const ps4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) ps4*)(p));
    return __builtin_bit_cast(uint2, r);
}

// staged tiles as the quantizers' inputs: tile row tok - t0
struct LdsValueSrc {
    const uint32_t* vl;
    __device__ uint4 row8(int64_t, int64_t tok, int sub) const {
        return *reinterpret_cast<const uint4*>(vl + tok * PVR + 4 * sub);
    }
};
struct LdsKeySrc {
    const uint32_t* kl;
    int64_t t0;
    __device__ uint32_t pair(int64_t tok, int cp) const { return kl[(tok - t0) * PKS + cp]; }
};

// buffer resource over the n_rows rows of one (sequence, head) slice: rows
// past the prompt read as zeros (the range check), without a branch
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const uint16_t* base, int n_rows) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, n_rows * PD * 2, 0x00020000);
}
__device__ __forceinline__ uint4 ldr(__amdgpu_buffer_rsrc_t r, int byte_off) {
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
    const u4v v = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void load_rows(__amdgpu_buffer_rsrc_t rs, int t0, int tid, uint4* r) {
    const int off = (t0 + (tid >> 3)) * (PD * 2) + 32 * (tid & 7);
#pragma unroll
    for (int e = 0; e < 2; ++e) r[e] = ldr(rs, off + 16 * e);
}

__device__ __forceinline__ void stage_ptile(const PTile& r, PrefillBuf& L, int tid) {
    uint32_t* kd = L.kl + (tid >> 3) * PKS + 8 * (tid & 7);
    uint32_t* vd = L.vl + (tid >> 3) * PVR + 8 * (tid & 7);
#pragma unroll
    for (int e = 0; e < 2; ++e) *reinterpret_cast<uint4*>(kd + 4 * e) = r.k[e];
#pragma unroll
    for (int e = 0; e < 2; ++e) *reinterpret_cast<uint4*>(vd + 4 * e) = r.v[e];
}

// The block's share of the cache: for each of its tiles (2qb and, inside
// the prompt, 2qb + 1), the values of its rows, the key blocks inside it that
// the prompt fills, and the residual rows of the unfilled block, read from
// the staged tile (the append kernels' device functions, so the same bits).
// Per tile the work is six one-wave units, spread over the grp workgroups of
// the KV head's query heads (workgroup r takes units r, r + grp, ..., the
// k-th of them on wave k mod 8):
//   units 0, 1: key channel pairs 32u .. 32u + 31 of the 64-token block
//               (G = 64) or key block u (G = 32), then (unit 0) the residual;
//   units 2..5: value rows 16 (u - 2) .. + 15.
template <int G, int KB, int VB>
__device__ void quantize_unit(const PrefillArgs& a, const PrefillBuf& L, int64_t bh, int t0, int u, int lane) {
    const int n = a.T - t0 < 64 ? a.T - t0 : 64;
    const int nfull = a.T / G;   // key blocks the prompt fills
    if (u < 2) {
        // one wave of the key threads of the tile's block(s): 64 per block for
        // G = 32; for G = 64 a block takes two waves (row halves 32 lanes apart)
        int64_t unit;
        int cp, sp;
        qdev::key_thread_coords<G, KB>(64 * u + lane, PD, unit, cp, sp);
        const int64_t blk = t0 / G + unit;
        if (blk < nfull) {
            const qdev::KeyJob j{a.k + bh * int64_t(a.T) * PD, a.kr + bh * G * PD, blk * G, 0, 0,
                                 bh * a.nblk_cap + blk};
            qdev::quant_key_pair<G, KB>(j, PD, cp, sp, a.kc, a.ks, a.kz, LdsKeySrc{L.kl, t0});
        }
        if (u == 0) {
            // residual: rows nfull * G .. T - 1 that lie in this tile
            const int r0 = nfull * G > t0 ? nfull * G : t0;
            for (int i = lane; i < (t0 + n - r0) * (PD / 8); i += 64) {
                const int t = r0 + i / (PD / 8), c = 8 * (i % (PD / 8));
                *reinterpret_cast<uint4*>(a.kr + (bh * G + (t - nfull * G)) * PD + c) =
                    *reinterpret_cast<const uint4*>(L.kl + (t - t0) * PKS + c / 2);
            }
        }
        return;
    }
    const int v0 = 16 * (u - 2);
    const int nv = n - v0 < 16 ? n - v0 : 16;
    if (nv <= 0) return;
    qdev::ValueArgs va;
    va.vin = nullptr;   // rows come from the staged tile
    va.n_in = a.T;
    va.row0 = t0 + v0;
    va.n_tok = nv;
    va.vd = PD;
    va.BH = 1;
    va.codes = a.vc;
    va.scale = a.vs;
    va.zero = a.vz;
    const qdev::ContigRows rows{a.cap, bh * a.cap + t0 + v0, nv};
    // 4 rows x 8 channels per thread, whole 4-lane groups: lanes past the
    // count would index the next (sequence, head)
    if (lane < qdev::value_threads(1, nv, PD))
        qdev::quant_values_thread<VB>(va, rows, lane, LdsValueSrc{L.vl + v0 * PVR});
}

template <int G, int KB, int VB>
__device__ void quantize_block(const PrefillArgs& a, const PrefillLds& L, int64_t bh, int qb, int ntile, int r,
                               int grp, int wave, int lane) {
    for (int u = r + grp * wave; u < 12; u += PNW * grp) {
        const int tile = 2 * qb + u / 6;
        if (tile < ntile) quantize_unit<G, KB, VB>(a, L.buf[tile & 1], bh, 64 * tile, u % 6, lane);
    }
}

template <int G, int KB, int VB>
__global__ __launch_bounds__(64 * PNW) void k_prefill(PrefillArgs a) {
    __shared__ PrefillLds L;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, kg = lane >> 4;
    // one grid dimension, query block slowest: the longest causal windows of
    // every (head, sequence) start first, the shortest fill the end
    const int nqb = (a.T + PBM - 1) / PBM, units = a.Hq * a.B;
    const int qb = nqb - 1 - int(blockIdx.x) / units;
    const int hq = int(blockIdx.x) % units % a.Hq, b = int(blockIdx.x) % units / a.Hq;
    const int grp = a.Hq / a.Hkv, kvh = hq / grp;
    const int64_t bh = int64_t(b) * a.Hkv + kvh;
    const __amdgpu_buffer_rsrc_t krs = slice_rsrc(a.k + bh * int64_t(a.T) * PD, a.T);
    const __amdgpu_buffer_rsrc_t vrs = slice_rsrc(a.v + bh * int64_t(a.T) * PD, a.T);

    // query row of this lane (the B operand of S^T): channels 32ks + 8kg .. + 7
    const int row0 = PBM * qb + 16 * wave;   // the wave's first row
    const int qrow = row0 + n;
    pf16x8 qb8[4];
    {
        const __amdgpu_buffer_rsrc_t qrs = slice_rsrc(a.q + (int64_t(b) * a.Hq + hq) * int64_t(a.T) * PD, a.T);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint4 w = ldr(qrs, qrow * (PD * 2) + 64 * ks + 16 * kg);
            qb8[ks] = as_pf16x8(w.x, w.y, w.z, w.w);
        }
    }
    pf32x4 O[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) O[c] = pf32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.0f;

    // tiles 0 .. ntile - 1: the causal window of the block's last row, within
    // the prompt; tiles 2qb and 2qb + 1 are the block's own (quantized here)
    const int last_tile = (a.T - 1) / 64;
    const int ntile = (2 * qb + 1 < last_tile ? 2 * qb + 1 : last_tile) + 1;
    // the next tile's rows: keys issued right after staging, values after
    // the softmax (not live across the first product)
    PTile cur;
    load_rows(krs, 0, tid, cur.k);
    load_rows(vrs, 0, tid, cur.v);
    auto step = [&](int j, auto diag) {
        constexpr bool DIAG = decltype(diag)::value;
        // buffer j & 1 held tile j - 2: every wave finished that tile before
        // the barrier after staging tile j - 1, so one barrier per tile
        PrefillBuf& B = L.buf[j & 1];
        stage_ptile(cur, B, tid);
        __syncthreads();
        if (j + 1 < ntile) load_rows(krs, 64 * (j + 1), tid, cur.k);
        // every row sees all of a tile before the block's own two; on those two
        // a wave's rows see none of the tile (skip), part of it (mask), or all
        const bool none = DIAG && 64 * j > row0 + 15;
        const bool part = DIAG && 64 * j + 63 > row0;
        uint32_t pw[8], pl[8];
        if (!none) {
            // ---- S^T = K Q^T: lane (n, kg) gets tokens 16cb + 4kg + i of row n
            pf32x4 S[4];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                S[cb] = pf32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const uint4 kw = *reinterpret_cast<const uint4*>(B.kl + (16 * cb + n) * PKS + 16 * ks + 4 * kg);
                    S[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_pf16x8(kw.x, kw.y, kw.z, kw.w), qb8[ks], S[cb],
                                                                   0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // ---- online softmax (log2 units), tokens after the row masked; the
            // logits stay unscaled, sigma2 enters the maximum and the exponent's FMA
            float s[16];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i) s[4 * cb + i] = S[cb][i];
            if (part) {
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (64 * j + 16 * cb + 4 * kg + i > qrow) s[4 * cb + i] = -INFINITY;
            }
            float mx = s[0];
#pragma unroll
            for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
            mx *= a.sigma2;
            if (__builtin_amdgcn_ballot_w64(mx > m + PTAU) != 0) {
                // exact row maximum over the four lanes of the row (kg = 0..3)
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float mn = fmaxf(m, mx);
                const float alpha = __builtin_amdgcn_exp2f(m - mn);
                m = mn;
                l *= alpha;
#pragma unroll
                for (int c = 0; c < 8; ++c)
#pragma unroll
                    for (int i = 0; i < 4; ++i) O[c][i] *= alpha;
            }
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[e], a.sigma2, -m));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[e + 1], a.sigma2, -m));
                l += p0 + p1;
                pw[e / 2] = pack_h2(p0, p1);
                // p - hi is exact in fp32 (hi is p rounded to 11 bits)
                const f16x2p h = __builtin_bit_cast(f16x2p, pw[e / 2]);
                pl[e / 2] = pack_h2(p0 - float(h[0]), p1 - float(h[1]));
            }
        }
        if (j + 1 < ntile) load_rows(vrs, 64 * (j + 1), tid, cur.v);
        if (!none) {
            // ---- O^T += V^T P^T over 2 K-steps of 32 tokens: K order of lane
            // group kg = tokens 32ks + 4kg + 0..3, then 32ks + 16 + 4kg + 0..3
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const pf16x8 P = as_pf16x8(pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]);
                const pf16x8 Pl = as_pf16x8(pl[4 * ks], pl[4 * ks + 1], pl[4 * ks + 2], pl[4 * ks + 3]);
                // lane n names value row 32ks + 4kg + (n >> 2) (and + 16), channels
                // 16c + 4 (n & 3) .. + 3; it receives channel 16c + n of the four
                // rows 32ks + 4kg + e (then + 16), e = 0..3
                const uint32_t* vr = B.vl + (32 * ks + 4 * kg + (n >> 2)) * PVR + 2 * (n & 3);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const uint2 lo = ld_tr16(vr + 8 * c);
                    const uint2 hi = ld_tr16(vr + 16 * PVR + 8 * c);
                    const pf16x8 Vt = as_pf16x8(lo.x, lo.y, hi.x, hi.y);
                    O[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Vt, P, O[c], 0, 0, 0);
                    O[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Vt, Pl, O[c], 0, 0, 0);
                    if (c & 1) __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };
    // tiles before the block's own two need no causal mask
    const int nfull = 2 * qb < ntile ? 2 * qb : ntile;
    int j = 0;
    for (; j < nfull; ++j) step(j, Diag<false>{});
    for (; j < ntile; ++j) step(j, Diag<true>{});
    // ---- l over the row's four lanes, O / l, fp16 rows to out
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (qrow < a.T) {
        const float inv = 1.0f / l;
        uint16_t* op = a.out + ((int64_t(b) * a.Hq + hq) * a.T + qrow) * PD + 4 * kg;
#pragma unroll
        for (int c = 0; c < 8; ++c)
            *reinterpret_cast<uint2*>(op + 16 * c) = make_uint2(pack_h2(O[c][0] * inv, O[c][1] * inv),
                                                                pack_h2(O[c][2] * inv, O[c][3] * inv));
    }
    // ---- the block's tiles, both still staged, into the cache (after the
    // output, when the accumulators are dead)
    if (a.quant) quantize_block<G, KB, VB>(a, L, bh, qb, ntile, hq % grp, grp, wave, lane);
}

}  // namespace

bool prefill_supported(const kvq_cache_cfg& c) {
    return c.key.dim == PD && c.value.dim == PD && (c.key.group == 32 || c.key.group == 64) &&
           (c.key.bits == 2 || c.key.bits == 4) && (c.value.bits == 2 || c.value.bits == 4) && c.value.group == 32;
}

hipError_t launch_prefill(const PrefillArgs& a, const kvq_cache_cfg& c, hipStream_t st) {
    const dim3 grid(unsigned((a.T + PBM - 1) / PBM) * unsigned(a.Hq * a.B));
#define KVQ_PF(GG, KK, VV)                                                                  \
    if (c.key.group == GG && c.key.bits == KK && c.value.bits == VV) {                      \
        hipLaunchKernelGGL((k_prefill<GG, KK, VV>), grid, dim3(64 * PNW), 0, st, a);         \
        return hipGetLastError();                                                           \
    }
    KVQ_PF(64, 2, 2)
    KVQ_PF(32, 2, 2)
    KVQ_PF(64, 4, 4)
    KVQ_PF(32, 4, 4)
    KVQ_PF(64, 2, 4)
    KVQ_PF(32, 2, 4)
    KVQ_PF(64, 4, 2)
    KVQ_PF(32, 4, 2)
#undef KVQ_PF
    return hipErrorInvalidValue;
}

}  // namespace kvq
