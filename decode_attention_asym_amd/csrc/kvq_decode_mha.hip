// kvq_decode_mha.hip -- split-K decode attention on MFMA for multi-head
// caches (one query head per KV head), head dim 128, 2-bit or 4-bit keys
// (G = 32 or 64) and values in 32-channel groups.
//
// Method ("Makale Bülteni -- KIVI", section "İddia ve Gerçeklik: KIVI"):
// logits over the per-channel-quantized keys and the fp16 residual keys,
// softmax, weighted sum of the per-token-quantized values, with the codes
// unpacked and dequantized inside this loop.
//
// With a single query head both contractions are matrix-vector products, yet
// the matrix cores still take them more cheaply than the VALU: the 2-bit
// codes enter v_mfma_f32_16x16x32_f16 exactly as fp16 subnormals (a shift
// per register of two code bytes and one AND per register of two codes, as
// in the GQA kernel),
// and the hi/lo halves of the folded scales ride along as extra rows of the
// A operand at no cost.  The VALU is left with the unpacking, the online
// softmax and the scale folding.
//  * keys: q' = q * s_k per (block, channel) as rows hi, lo; the zero term
//    sum_c q_c z_c is a per-block bias.  The other 14 rows repeat them.
//  * values: p' = p * s_v per (token, group) as rows (group, hi/lo); of the
//    16 rows, the 4 of the column's channel half are used.
//  * online softmax in log2 units with a lazily moved maximum (TAU).
// Work split and pipelining follow the GQA kernel: one two-wave workgroup
// per run of 64-token tiles (wave 0 keys + softmax, wave 1 values one tile
// behind, one workgroup barrier per tile), plus one VALU workgroup for the
// trailing partial tile and the residual keys.
#include "kvq_mfma_tiles.h"

namespace kvq {
namespace {

struct LdsK {
    __attribute__((aligned(16))) uint32_t kl[KTILE_DW];      // key codes, cache layout
    __attribute__((aligned(16))) uint32_t qa[2 * 2 * QSTR];  // q' rows [block][hi, lo]
    __attribute__((aligned(16))) uint32_t ksl[2 * 2 * 64];   // key [scale|zero][block][128 fp16], quad order
};

struct LdsV {
    __attribute__((aligned(16))) uint32_t vl[VTILE_DW];  // value codes, cache layout
    __attribute__((aligned(16))) uint32_t pa[8 * ASTR];   // p' rows [group][hi, lo]
    // value [scale|zero][group][token pair], then a row of fp16 ones and a row of zeros
    __attribute__((aligned(16))) uint32_t vsl[2 * 128 + 2 * 32];
};

// softmax weights p as fp16 hi + lo pairs: dword 2k + j holds tokens
// 4k + j, 4k + j + 2 (the quad order of the K dimension)
struct Handoff {
    __attribute__((aligned(16))) uint32_t ph[32];
    __attribute__((aligned(16))) uint32_t pq[32];
    float alpha;   // rescale of earlier accumulations
};

struct Lds {
    LdsK k;
    LdsV v;
    Handoff hb[2];
    float misc[4];
};

// Key side of one tile: produces p and alpha in `hb`.  m_run is the running
// maximum (log2 units, wave-uniform); qw holds query channels
// 4(lane >> 1) + (lane & 1) and that + 2 (fp16, quad order).
template <int G, class Run>
__device__ __forceinline__ void key_tile(const MfmaParams& p, KTile& cur, float& m_run, LdsK& L,
                                         Handoff& hb, uint32_t qw, int lane,
                                         int64_t bh, int nxt, const Run& run) {
    constexpr int NBT = 64 / G;
    const int n = lane & 15, kg = lane >> 4;

    // ---- stage key codes and side values, then prefetch tile i + 2
    stage_keys<G>(cur, L.kl, L.ksl, lane);
    // unconditional (past the run it reads nothing) so that every path has
    // the same loads in flight and the wait before staging covers only the
    // older tile
    load_ktile<G>(p, run, bh, nxt, lane, cur);
    wave_sync();

    // ---- q' = q * s_k as fp16 rows hi, lo; sigma2 * sum_c q z_k per block
    float bias[NBT];
#pragma unroll
    for (int be = 0; be < NBT; ++be) {
        const uint32_t sw = L.ksl[be * 64 + lane], zw = L.ksl[128 + be * 64 + lane];
        uint32_t hi, lo;
        split_prod_h(qw, sw, hi, lo);
        L.qa[(2 * be) * QSTR + lane] = hi;
        L.qa[(2 * be + 1) * QSTR + lane] = lo;
        bias[be] = wave_sum(dot2h(qw, zw, 0.0f)) * p.sigma2;
    }
    wave_sync();

    // ---- S = q' . codes: 4 MFMA tiles of 16 tokens x 4 K-steps of 32 channels
    f32x4 S[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) S[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ksx = 0; ksx < 4; ++ksx) {
#pragma unroll
        for (int be = 0; be < NBT; ++be) {
            const uint4 a = *reinterpret_cast<const uint4*>(L.qa + (2 * be + (n & 1)) * QSTR + 16 * ksx + 4 * kg);
            const f16x8 A = as_f16x8(a.x, a.y, a.z, a.w);
            const CodeRegs c = code_operands(ld_tr8(L.kl + key_row_dw<G>(ksx, be, kg, n)));
            if (G == 64) {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    S[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, code_slice2(c, u), S[u], 0, 0, 0);
            } else {
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const uint32_t mk = code_mask2(n >> 3);   // position 2v + (n >> 3)
                    S[2 * be + v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, code_slice_set(c, v != 0, mk), S[2 * be + v], 0, 0, 0);
                }
            }
        }
    }

    // ---- softmax.  Result rows 4kg + j hold the hi (j even) and lo (j odd)
    // partial logits, the same in every lane group kg; lane n has column n of
    // each of the 4 MFMA tiles.  G = 64: tile u, column n is token 4n + u.
    // G = 32: tile 2be + v, column n is token
    // 32be + 16((n & 7) >> 2) + 4(n & 3) + 2v + (n >> 3).
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int up = G == 64 ? i : 2 * (i & 1) + (n >> 3);   // code position in the byte
        const float f = p.sigma2 * code_unscale2(up);
        x[i] = fmaf(S[i][0] + S[i][1], f, bias[G == 64 ? 0 : (i >> 1)]);
    }
    const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    float alpha = 1.0f;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + TAU) != 0) {
        const float mnew = fmaxf(m_run, readlane_f(row_max16(mx), 0));
        alpha = fast_exp2(m_run - mnew);
        m_run = mnew;
    }
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(x[i] - m_run);
    // weights as fp16 hi + lo pairs (tokens 4k + j, 4k + j + 2)
    if (kg == 0) {
        uint32_t h0, l0, h1, l1;
        if (G == 64) {
            // tokens 4n + u: pairs (u = 0, 2) and (1, 3) of quad n
            split_f32(pv[0], pv[2], p.neg1, h0, l0);
            split_f32(pv[1], pv[3], p.neg1, h1, l1);
            *reinterpret_cast<uint2*>(hb.ph + 2 * n) = make_uint2(h0, h1);
            *reinterpret_cast<uint2*>(hb.pq + 2 * n) = make_uint2(l0, l1);
        } else {
            // tiles 2be + v: pair (v = 0, 1) of quad k = 8be + 4((n & 7) >> 2) + (n & 3), j = n >> 3
            split_f32(pv[0], pv[1], p.neg1, h0, l0);
            split_f32(pv[2], pv[3], p.neg1, h1, l1);
            const int dw = 2 * (4 * ((n & 7) >> 2) + (n & 3)) + (n >> 3);
            hb.ph[dw] = h0;
            hb.pq[dw] = l0;
            hb.ph[dw + 16] = h1;
            hb.pq[dw + 16] = l1;
        }
    }
    if (lane == 0) hb.alpha = alpha;
}

struct VState {
    f32x4 O[2][4];   // PV accumulators [channel half][code position]
    // sum_t p z_v per group and l = sum_t p on MFMA: even rows hi, odd rows
    // lo; column g < 4 the zero-point sum of group g, column 4 the weight sum
    f32x4 Z;
};

// Value side of one tile, reading p and alpha from `hb`.
template <int G, class Run>
__device__ __forceinline__ void value_tile(const MfmaParams& p, VTile& cur, VState& st, LdsV& L,
                                           const Handoff& hb, int lane, int64_t bh,
                                           int nxt, const Run& run) {
    const int n = lane & 15, kg = lane >> 4;
    // ---- stage value codes and side values, then prefetch tile i + 2
    stage_values(cur, L.vl, L.vsl, lane);
    load_vtile<G>(p, run, bh, nxt, lane, cur);

    // ---- rescale what was accumulated with the previous maximum
    const float alpha = hb.alpha;
    if (alpha < 1.0f) {
#pragma unroll
        for (int P = 0; P < 2; ++P)
#pragma unroll
            for (int u = 0; u < 4; ++u) st.O[P][u] *= alpha;
        st.Z *= alpha;
    }
    wave_sync();

    // ---- p' = p * s_v as fp16 rows (group, hi/lo); sum_t p, sum_t p z_v.
    // Lane (tp, gp): token pair tp (tokens 4(tp >> 1) + (tp & 1) and that + 2,
    // quad order) and groups 2gp, 2gp + 1.
    {
        const int tp = lane & 31, gp = lane >> 5;
        const uint32_t ph = hb.ph[tp], pq = hb.pq[tp];
        const uint32_t s0 = L.vsl[(2 * gp) * 32 + tp], s1 = L.vsl[(2 * gp + 1) * 32 + tp];
        uint32_t h, l;
        split_prod_hl(ph, pq, s0, h, l);
        L.pa[(4 * gp) * ASTR + tp] = h;
        L.pa[(4 * gp + 1) * ASTR + tp] = l;
        split_prod_hl(ph, pq, s1, h, l);
        L.pa[(4 * gp + 2) * ASTR + tp] = h;
        L.pa[(4 * gp + 3) * ASTR + tp] = l;
    }
    // ---- sum_t p z_v and sum_t p: A = the weights' hi (even rows) and lo
    // (odd rows), B column n = the zero-points of group n (n < 4), ones
    // (n = 4) or zeros, over the tile's 64 tokens in quad order
    {
        const uint32_t* arow = ((n & 1) ? hb.pq : hb.ph) + 4 * kg;
        const uint32_t* brow = L.vsl + 128 + (n < 5 ? n : 5) * 32 + 4 * kg;
#pragma unroll
        for (int ksx = 0; ksx < 2; ++ksx) {
            const uint4 a = *reinterpret_cast<const uint4*>(arow + 16 * ksx);
            const uint4 z = *reinterpret_cast<const uint4*>(brow + 16 * ksx);
            st.Z = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a.x, a.y, a.z, a.w), as_f16x8(z.x, z.y, z.z, z.w),
                                                          st.Z, 0, 0, 0);
        }
    }
    wave_sync();

    // ---- O += p' . codes: 2 channel halves x 4 code positions x 2 K-steps of
    // 32 tokens.  A row n holds group 2P + ((n >> 1) & 1), hi (n even) / lo.
#pragma unroll
    for (int P = 0; P < 2; ++P) {
        const int row = 4 * P + (n & 3);
#pragma unroll
        for (int ksx = 0; ksx < 2; ++ksx) {
            const uint4 a = *reinterpret_cast<const uint4*>(L.pa + row * ASTR + 16 * ksx + 4 * kg);
            const f16x8 A = as_f16x8(a.x, a.y, a.z, a.w);
            const CodeRegs c = code_operands(ld_tr8(L.vl + value_row_dw(ksx, P, kg, n)));
#pragma unroll
            for (int u = 0; u < 4; ++u)
                st.O[P][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, code_slice2(c, u),
                                                                    st.O[P][u], 0, 0, 0);
        }
    }
}

template <int G, bool PAGED>
__global__ __launch_bounds__(128) void k_decode_mha(MfmaParams p) {
    __shared__ Lds L;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = lane & 15, kg = lane >> 4;
    int b, kvh;
    bool tail;
    const int s = block_coords<false>(p, b, kvh, tail);
    const int64_t bh = int64_t(b) * p.Hkv + kvh;
    const int64_t slot = (int64_t(b) * p.Hq + kvh) * p.S + s;
    // paged: the sequence's own length, fixed-size splits (as in the GQA kernel)
    int t_lo, t_hi;
    [[maybe_unused]] PagedRun prun;
    if constexpr (PAGED) {
        // the step's fused append (if any) adds token len0; main splits cover the
        // tiles complete before it, the tail everything after them
        int len0, n_app;
        paged_step_len(p, b, G, len0, n_app);
        const int ntiles = len0 / G * G / 64;
        if (tail) {
            if (n_app) fused_append_paged<G, 2>(p, b, kvh, len0);
            const int T1 = len0 + n_app;
            tail_split<1>(p, PagedBlocks{}, b, kvh, s, reinterpret_cast<float*>(L.k.qa),
                               reinterpret_cast<float*>(L.v.pa), T1, T1 / G, ntiles);
            return;
        }
        t_lo = s * p.chunk;
        prun = paged_run<G>(p, b, kvh, t_lo, lane);
        t_hi = t_lo + p.chunk < ntiles ? t_lo + p.chunk : ntiles;
        if (t_lo >= t_hi) {
            empty_partial<1>(p, b, kvh, s);
            return;
        }
        prun.t_last = t_hi - 1;
    } else {
        if (tail) {
            tail_split<1>(p, b, kvh, s, reinterpret_cast<float*>(L.k.qa), reinterpret_cast<float*>(L.v.pa));
            return;
        }
        t_lo = int(int64_t(s) * p.ntiles / p.S_main);
        t_hi = int(int64_t(s + 1) * p.ntiles / p.S_main);
    }
    const int ntl = t_hi - t_lo;

    if (wave == 0) {
        // query channel pair of this lane in quad order
        const uint2 qq = reinterpret_cast<const uint2*>(p.q + (int64_t(b) * p.Hq + kvh) * D)[lane >> 1];
        const uint32_t qw = (lane & 1) ? pair_hi(qq.x, qq.y) : pair_lo(qq.x, qq.y);
        float m_run = -INFINITY;
        KTile ta, tb;
        const auto run = pick_run<G, PAGED>(p, prun, bh, t_lo, t_hi);
        load_ktile<G>(p, run, bh, t_lo, lane, ta);
        load_ktile<G>(p, run, bh, t_lo + 1, lane, tb);
        // keep these loads ahead of (not interleaved with) the prefetch of tile 2
        __builtin_amdgcn_sched_barrier(0);
        // two register tiles in flight: tile j is staged from set j & 1,
        // which then receives tile j + 2, and hands over through hb[j & 1].
        // The loop body always processes two tiles, so every path has the
        // same loads in flight and the wait before staging covers only the
        // older tile.
        key_tile<G>(p, ta, m_run, L.k, L.hb[0], qw, lane, bh, t_lo + 2, run);
        __syncthreads();
        int j = 1;
        for (; j + 1 < ntl; j += 2) {
            key_tile<G>(p, tb, m_run, L.k, L.hb[1], qw, lane, bh, t_lo + j + 2, run);
            __syncthreads();
            key_tile<G>(p, ta, m_run, L.k, L.hb[0], qw, lane, bh, t_lo + j + 3, run);
            __syncthreads();
        }
        if (j < ntl) {
            key_tile<G>(p, tb, m_run, L.k, L.hb[1], qw, lane, bh, t_lo + j + 2, run);
            __syncthreads();
        }
        if (lane == 0) L.misc[0] = m_run;
        __syncthreads();
    } else {
        VState st;
        st.Z = f32x4{0.f, 0.f, 0.f, 0.f};
        // the ones and zeros rows after the side values (B operand of the sums)
        L.v.vsl[256 + lane] = lane < 32 ? 0x3c003c00u : 0u;
#pragma unroll
        for (int P = 0; P < 2; ++P)
#pragma unroll
            for (int u = 0; u < 4; ++u) st.O[P][u] = f32x4{0.f, 0.f, 0.f, 0.f};
        // value work trails the key work by one tile: tile j after barrier j
        VTile ta, tb;
        const auto run = pick_run<G, PAGED>(p, prun, bh, t_lo, t_hi);
        load_vtile<G>(p, run, bh, t_lo, lane, ta);
        load_vtile<G>(p, run, bh, t_lo + 1, lane, tb);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        value_tile<G>(p, ta, st, L.v, L.hb[0], lane, bh, t_lo + 2, run);
        __syncthreads();
        int j = 1;
        for (; j + 1 < ntl; j += 2) {
            value_tile<G>(p, tb, st, L.v, L.hb[1], lane, bh, t_lo + j + 2, run);
            __syncthreads();
            value_tile<G>(p, ta, st, L.v, L.hb[0], lane, bh, t_lo + j + 3, run);
            __syncthreads();
        }
        if (j < ntl) {
            value_tile<G>(p, tb, st, L.v, L.hb[1], lane, bh, t_lo + j + 2, run);
            __syncthreads();
        }
        // ---- epilogue: l and the value-zero sums (hi + lo rows; lanes 0..3
        // hold groups 0..3, lane 4 the weight sum)
        const float zsum = st.Z[0] + st.Z[1];
        const float vz0 = readlane_f(zsum, 0), vz1 = readlane_f(zsum, 1);
        const float vz2 = readlane_f(zsum, 2), vz3 = readlane_f(zsum, 3);
        const float lsum = readlane_f(zsum, 4);
        if (kg == 0) {
            const bool up = (n >> 3) != 0;   // the column's group within the channel half
            // (scalar selects: an indexed array here would be lowered to scratch)
            const float zb0 = up ? vz1 : vz0, zb1 = up ? vz3 : vz2;
#pragma unroll
            for (int P = 0; P < 2; ++P)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int c = 64 * P + 32 * (n >> 3) + 4 * (n & 7) + u;
                    const float hi = up ? st.O[P][u][2] : st.O[P][u][0];
                    const float lo = up ? st.O[P][u][3] : st.O[P][u][1];
                    p.ws_acc[slot * D + c] = fmaf(hi + lo, code_unscale2(u), P ? zb1 : zb0);
                }
        }
        if (lane == 0) {
            p.ws_ml[slot * 2] = L.misc[0];
            p.ws_ml[slot * 2 + 1] = lsum;
        }
    }
}

// ---------------------------------------------------------------------------
// 4-bit keys and values (the 4 KB tiles of kvq_mfma_tiles.h): per K-step two
// transposed key reads of two nibbles each, four value passes of one group
// each; the A rows are the 2-bit kernel's hi/lo rows.

struct LdsK4 {
    __attribute__((aligned(16))) uint32_t kl[KTILE4_DW];
    __attribute__((aligned(16))) uint32_t qa[2 * 2 * QSTR];
    __attribute__((aligned(16))) uint32_t ksl[2 * 2 * 64];
};
struct LdsV4 {
    __attribute__((aligned(16))) uint32_t vl[VTILE4_DW];
    __attribute__((aligned(16))) uint32_t pa[8 * ASTR];   // p' rows [group][hi, lo]
    __attribute__((aligned(16))) uint32_t vsl[2 * 128 + 2 * 32];
};
struct Lds4 {
    LdsK4 k;
    LdsV4 v;
    Handoff hb[2];
    float misc[4];
};

template <int G, class Run>
__device__ __forceinline__ void key_tile4(const MfmaParams& p, KTile4& cur, float& m_run, LdsK4& L, Handoff& hb,
                                          uint32_t qw, int lane, int64_t bh, int nxt, const Run& run) {
    constexpr int NBT = 64 / G;
    const int n = lane & 15, kg = lane >> 4;
    stage_keys4<G>(cur, L.kl, L.ksl, lane);
    load_ktile4<G>(p, run, bh, nxt, lane, cur);
    wave_sync();

    float bias[NBT];
#pragma unroll
    for (int be = 0; be < NBT; ++be) {
        const uint32_t sw = L.ksl[be * 64 + lane], zw = L.ksl[128 + be * 64 + lane];
        uint32_t hi, lo;
        split_prod_h(qw, sw, hi, lo);
        L.qa[(2 * be) * QSTR + lane] = hi;
        L.qa[(2 * be + 1) * QSTR + lane] = lo;
        bias[be] = wave_sum(dot2h(qw, zw, 0.0f)) * p.sigma2;
    }
    wave_sync();

    // ---- S[2r + nib], column n = token 32r + 2n + nib
    f32x4 S[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) S[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ksx = 0; ksx < 4; ++ksx) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int be = G == 64 ? 0 : r;
            const uint4 a = *reinterpret_cast<const uint4*>(L.qa + (2 * be + (n & 1)) * QSTR + 16 * ksx + 4 * kg);
            const f16x8 A = as_f16x8(a.x, a.y, a.z, a.w);
            const CodeRegs c = code_operands(ld_tr8(L.kl + key_row_dw4<G>(ksx, r, kg, n)));
#pragma unroll
            for (int nib = 0; nib < 2; ++nib)
                S[2 * r + nib] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, code_slice4(c, nib),
                                                                       S[2 * r + nib], 0, 0, 0);
        }
    }
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float f = p.sigma2 * code_unscale4();
        x[i] = fmaf(S[i][0] + S[i][1], f, bias[G == 64 ? 0 : (i >> 1)]);
    }
    const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    float alpha = 1.0f;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + TAU) != 0) {
        const float mnew = fmaxf(m_run, readlane_f(row_max16(mx), 0));
        alpha = fast_exp2(m_run - mnew);
        m_run = mnew;
    }
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(x[i] - m_run);
    // ---- weights as fp16 hi + lo pairs (tokens 4k + j, 4k + j + 2): for each
    // half r, the even lane pairs its low-nibble token with the odd
    // neighbour's, the odd lane its high-nibble token (dword 16r + n)
    const bool nodd = (n & 1) != 0;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const float o = dpp<0xb1>(nodd ? pv[2 * r] : pv[2 * r + 1]);
        uint32_t h, l;
        split_f32(nodd ? o : pv[2 * r], nodd ? pv[2 * r + 1] : o, p.neg1, h, l);
        if (kg == 0) {
            hb.ph[16 * r + n] = h;
            hb.pq[16 * r + n] = l;
        }
    }
    if (lane == 0) hb.alpha = alpha;
}

struct VState4 {
    f32x4 O[4][2];   // PV accumulators [pass = value group][nibble]
    f32x4 Z;
};

template <int G, class Run>
__device__ __forceinline__ void value_tile4(const MfmaParams& p, VTile4& cur, VState4& st, LdsV4& L, const Handoff& hb,
                                            int lane, int64_t bh, int nxt, const Run& run) {
    const int n = lane & 15, kg = lane >> 4;
    stage_values4(cur, L.vl, L.vsl, lane);
    load_vtile4<G>(p, run, bh, nxt, lane, cur);
    const float alpha = hb.alpha;
    if (alpha < 1.0f) {
#pragma unroll
        for (int P = 0; P < 4; ++P)
#pragma unroll
            for (int u = 0; u < 2; ++u) st.O[P][u] *= alpha;
        st.Z *= alpha;
    }
    wave_sync();
    // ---- p' = p * s_v as fp16 rows (group, hi/lo), as for 2 bits
    {
        const int tp = lane & 31, gp = lane >> 5;
        const uint32_t ph = hb.ph[tp], pq = hb.pq[tp];
        const uint32_t s0 = L.vsl[(2 * gp) * 32 + tp], s1 = L.vsl[(2 * gp + 1) * 32 + tp];
        uint32_t h, l;
        split_prod_hl(ph, pq, s0, h, l);
        L.pa[(4 * gp) * ASTR + tp] = h;
        L.pa[(4 * gp + 1) * ASTR + tp] = l;
        split_prod_hl(ph, pq, s1, h, l);
        L.pa[(4 * gp + 2) * ASTR + tp] = h;
        L.pa[(4 * gp + 3) * ASTR + tp] = l;
    }
    {
        const uint32_t* arow = ((n & 1) ? hb.pq : hb.ph) + 4 * kg;
        const uint32_t* brow = L.vsl + 128 + (n < 5 ? n : 5) * 32 + 4 * kg;
#pragma unroll
        for (int ksx = 0; ksx < 2; ++ksx) {
            const uint4 a = *reinterpret_cast<const uint4*>(arow + 16 * ksx);
            const uint4 z = *reinterpret_cast<const uint4*>(brow + 16 * ksx);
            st.Z = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a.x, a.y, a.z, a.w), as_f16x8(z.x, z.y, z.z, z.w),
                                                          st.Z, 0, 0, 0);
        }
    }
    wave_sync();
    // ---- O += p' . codes: pass P = value group P, A rows (P, hi/lo) repeated
#pragma unroll
    for (int P = 0; P < 4; ++P) {
        const int row = 2 * P + (n & 1);
#pragma unroll
        for (int ksx = 0; ksx < 2; ++ksx) {
            const uint4 a = *reinterpret_cast<const uint4*>(L.pa + row * ASTR + 16 * ksx + 4 * kg);
            const f16x8 A = as_f16x8(a.x, a.y, a.z, a.w);
            const CodeRegs c = code_operands(ld_tr8(L.vl + value_row_dw4(ksx, P, kg, n)));
#pragma unroll
            for (int nib = 0; nib < 2; ++nib)
                st.O[P][nib] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, code_slice4(c, nib),
                                                                      st.O[P][nib], 0, 0, 0);
        }
    }
}

template <int G, bool PAGED>
__global__ __launch_bounds__(128) void k_decode_mha4(MfmaParams p) {
    __shared__ Lds4 L;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = lane & 15, kg = lane >> 4;
    int b, kvh;
    bool tail;
    const int s = block_coords<false>(p, b, kvh, tail);
    const int64_t bh = int64_t(b) * p.Hkv + kvh;
    const int64_t slot = (int64_t(b) * p.Hq + kvh) * p.S + s;
    int t_lo, t_hi;
    [[maybe_unused]] PagedRun prun;
    if constexpr (PAGED) {
        // the step's fused append (if any) adds token len0; main splits cover the
        // tiles complete before it, the tail everything after them
        int len0, n_app;
        paged_step_len(p, b, G, len0, n_app);
        const int ntiles = len0 / G * G / 64;
        if (tail) {
            if (n_app) fused_append_paged<G, 4>(p, b, kvh, len0);
            const int T1 = len0 + n_app;
            tail_split<1, PagedBlocks, 4>(p, PagedBlocks{}, b, kvh, s, reinterpret_cast<float*>(L.k.qa),
                               reinterpret_cast<float*>(L.v.pa), T1, T1 / G, ntiles);
            return;
        }
        t_lo = s * p.chunk;
        prun = paged_run<G>(p, b, kvh, t_lo, lane);
        t_hi = t_lo + p.chunk < ntiles ? t_lo + p.chunk : ntiles;
        if (t_lo >= t_hi) {
            empty_partial<1>(p, b, kvh, s);
            return;
        }
        prun.t_last = t_hi - 1;
    } else {
        if (tail) {
            tail_split<1, 4>(p, b, kvh, s, reinterpret_cast<float*>(L.k.qa), reinterpret_cast<float*>(L.v.pa));
            return;
        }
        t_lo = int(int64_t(s) * p.ntiles / p.S_main);
        t_hi = int(int64_t(s + 1) * p.ntiles / p.S_main);
    }
    const int ntl = t_hi - t_lo;

    if (wave == 0) {
        const uint2 qq = reinterpret_cast<const uint2*>(p.q + (int64_t(b) * p.Hq + kvh) * D)[lane >> 1];
        const uint32_t qw = (lane & 1) ? pair_hi(qq.x, qq.y) : pair_lo(qq.x, qq.y);
        float m_run = -INFINITY;
        KTile4 ta, tb;
        const auto run = pick_run4<G, PAGED>(p, prun, bh, t_lo, t_hi);
        load_ktile4<G>(p, run, bh, t_lo, lane, ta);
        load_ktile4<G>(p, run, bh, t_lo + 1, lane, tb);
        __builtin_amdgcn_sched_barrier(0);
        key_tile4<G>(p, ta, m_run, L.k, L.hb[0], qw, lane, bh, t_lo + 2, run);
        __syncthreads();
        int j = 1;
        for (; j + 1 < ntl; j += 2) {
            key_tile4<G>(p, tb, m_run, L.k, L.hb[1], qw, lane, bh, t_lo + j + 2, run);
            __syncthreads();
            key_tile4<G>(p, ta, m_run, L.k, L.hb[0], qw, lane, bh, t_lo + j + 3, run);
            __syncthreads();
        }
        if (j < ntl) {
            key_tile4<G>(p, tb, m_run, L.k, L.hb[1], qw, lane, bh, t_lo + j + 2, run);
            __syncthreads();
        }
        if (lane == 0) L.misc[0] = m_run;
        __syncthreads();
    } else {
        VState4 st;
        st.Z = f32x4{0.f, 0.f, 0.f, 0.f};
        L.v.vsl[256 + lane] = lane < 32 ? 0x3c003c00u : 0u;
#pragma unroll
        for (int P = 0; P < 4; ++P)
#pragma unroll
            for (int u = 0; u < 2; ++u) st.O[P][u] = f32x4{0.f, 0.f, 0.f, 0.f};
        VTile4 ta, tb;
        const auto run = pick_run4<G, PAGED>(p, prun, bh, t_lo, t_hi);
        load_vtile4<G>(p, run, bh, t_lo, lane, ta);
        load_vtile4<G>(p, run, bh, t_lo + 1, lane, tb);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        value_tile4<G>(p, ta, st, L.v, L.hb[0], lane, bh, t_lo + 2, run);
        __syncthreads();
        int j = 1;
        for (; j + 1 < ntl; j += 2) {
            value_tile4<G>(p, tb, st, L.v, L.hb[1], lane, bh, t_lo + j + 2, run);
            __syncthreads();
            value_tile4<G>(p, ta, st, L.v, L.hb[0], lane, bh, t_lo + j + 3, run);
            __syncthreads();
        }
        if (j < ntl) {
            value_tile4<G>(p, tb, st, L.v, L.hb[1], lane, bh, t_lo + j + 2, run);
            __syncthreads();
        }
        const float zsum = st.Z[0] + st.Z[1];
        const float vz0 = readlane_f(zsum, 0), vz1 = readlane_f(zsum, 1);
        const float vz2 = readlane_f(zsum, 2), vz3 = readlane_f(zsum, 3);
        const float lsum = readlane_f(zsum, 4);
        if (kg == 0) {
#pragma unroll
            for (int P = 0; P < 4; ++P)
#pragma unroll
                for (int nib = 0; nib < 2; ++nib) {
                    const int c = 32 * P + 8 * (n >> 2) + 2 * (n & 3) + nib;
                    const float zb = sel4(P, vz0, vz1, vz2, vz3);
                    p.ws_acc[slot * D + c] = fmaf(st.O[P][nib][0] + st.O[P][nib][1],
                                                  code_unscale4(), zb);
                }
        }
        if (lane == 0) {
            p.ws_ml[slot * 2] = L.misc[0];
            p.ws_ml[slot * 2 + 1] = lsum;
        }
    }
}

}  // namespace

bool mha_supported(const kvq_cache& c, int Hq) {
    return (mfma_shape_ok(c) || mfma_cfg_ok4(c.cfg)) && Hq == c.cfg.n_kv_heads;
}

hipError_t launch_decode_mha(const DecodeArgs& a, hipStream_t st) {
    const MfmaParams p = mfma_params(a);
    const dim3 grid = decode_grid<false>(a.S, a.g.Hkv, a.g.B);
    if (a.g.kbits == 4) {
        if (a.g.kG == 64)
            hipExtLaunchKernelGGL((k_decode_mha4<64, false>), grid, dim3(128), 0, st, a.ev_start, a.ev_stop, 0, p);
        else
            hipExtLaunchKernelGGL((k_decode_mha4<32, false>), grid, dim3(128), 0, st, a.ev_start, a.ev_stop, 0, p);
        return hipGetLastError();
    }
    if (a.g.kG == 64)
        hipExtLaunchKernelGGL((k_decode_mha<64, false>), grid, dim3(128), 0, st, a.ev_start, a.ev_stop, 0, p);
    else
        hipExtLaunchKernelGGL((k_decode_mha<32, false>), grid, dim3(128), 0, st, a.ev_start, a.ev_stop, 0, p);
    return hipGetLastError();
}

bool mha_cfg_supported(const kvq_cache_cfg& c, int Hq) { return (mfma_cfg_ok(c) || mfma_cfg_ok4(c)) && Hq == c.n_kv_heads; }

hipError_t launch_decode_mha_paged(const DecodeArgs& a, hipStream_t st) {
    const MfmaParams p = mfma_params(a);
    const dim3 grid = decode_grid<false>(a.S, a.g.Hkv, a.g.B);
    if (a.g.kbits == 4) {
        if (a.g.kG == 64)
            hipExtLaunchKernelGGL((k_decode_mha4<64, true>), grid, dim3(128), 0, st, a.ev_start, a.ev_stop, 0, p);
        else
            hipExtLaunchKernelGGL((k_decode_mha4<32, true>), grid, dim3(128), 0, st, a.ev_start, a.ev_stop, 0, p);
        return hipGetLastError();
    }
    if (a.g.kG == 64)
        hipExtLaunchKernelGGL((k_decode_mha<64, true>), grid, dim3(128), 0, st, a.ev_start, a.ev_stop, 0, p);
    else
        hipExtLaunchKernelGGL((k_decode_mha<32, true>), grid, dim3(128), 0, st, a.ev_start, a.ev_stop, 0, p);
    return hipGetLastError();
}

}  // namespace kvq
