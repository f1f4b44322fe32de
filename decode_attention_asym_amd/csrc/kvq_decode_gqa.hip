// kvq_decode_gqa.hip -- split-K decode attention on MFMA for GQA caches:
// 4 query heads per KV head, head dim 128, 2-bit keys (G = 32 or 64) and
// 2-bit values (32-channel groups); k_decode_gqa4 takes 4-bit keys and
// values.
//
// Method ("Makale Bülteni -- KIVI", section "İddia ve Gerçeklik: KIVI"):
// logits over the per-channel-quantized keys and the fp16 residual keys,
// softmax, weighted sum of the per-token-quantized values; the codes are
// unpacked and dequantized inside this loop, never written back as fp16.
// GQA: four query heads share each KV head (section "Kod ve Entegrasyon
// Haritası"), which makes QK^T and PV dense enough for the matrix cores.
//
// How the contractions reach v_mfma_f32_16x16x32_f16 exactly:
//  * a 2-bit code c alone in bits [f, f+1] of an fp16 lane (all other bits
//    zero) is the exact subnormal c * 2^(f - 24).  The transposed LDS read
//    hands each lane the code bytes of its MFMA column; one shift per
//    register of two bytes puts them at bit 6 or bit 2 of the fp16 halves,
//    and one AND per code position then leaves one code in bits 6..7 or
//    8..9 of each half (fields high in the mantissa keep the matrix cores'
//    sums accurate; kvq_mfma_tiles.h, code_operands).  The power-of-two
//    factors are undone on the fp32 results.
//  * keys: khat = code * s + z with s, z per (block, channel).  The scale is
//    folded into the query (q' = q * s, exact in fp32) which is fed as two
//    fp16 rows hi + lo (q' - hi), so logits keep ~22 bits; the zero term
//    sum_c q_c z_c is a per-(head, block) bias computed on the VALU.
//  * values: vhat = code * s + z with s, z per (token, 32-channel group).
//    The scale is folded into the softmax weights (p' = p * s) as hi/lo
//    rows; sum_t p_t z_t per (head, group) and sum_t p_t come from two more
//    MFMAs per tile over the weights' hi/lo rows.
//  * online softmax in log2 units; the running maximum only moves when a
//    tile exceeds it by more than 2^8 (weights stay <= 256, fp16-safe).
// One two-wave workgroup handles one contiguous run of 64-token tiles of one
// (sequence, KV head); the global loads of later tiles overlap the current
// tile.  The keys of a trailing partial tile and the residual are
// handled by one extra workgroup per (sequence, KV head) on the VALU.  Over a
// contiguous cache the grid is split-major (block_coords in
// kvq_mfma_tiles.h).
#include "kvq_mfma_tiles.h"

namespace kvq {
namespace {

constexpr int HG = 4;  // query heads per KV head

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
    __attribute__((aligned(16))) uint32_t kl[KTILE_DW];      // key codes, cache layout
    __attribute__((aligned(16))) uint32_t qa[2 * 8 * QSTR];  // q' rows (fp16) per key block
    __attribute__((aligned(16))) uint32_t ksl[2 * 2 * 64];   // key [scale|zero][block][128 fp16], quad order
    float bias[8];                                          // sigma2 * sum_c q z_k per (block, head)
};

struct LdsV {
    __attribute__((aligned(16))) uint32_t vl[VTILE_DW];      // value codes, cache layout
    __attribute__((aligned(16))) uint32_t pa[2 * 16 * ASTR];  // p' rows (fp16) per pass
    // value [scale|zero][group][token pair], then a row of fp16 ones and a row of zeros
    __attribute__((aligned(16))) uint32_t vsl[2 * 128 + 2 * 32];
};

// softmax weights p as fp16 hi + lo pairs: [head][token pair], dword 2k + j
// holding tokens 4k + j, 4k + j + 2; 48-dword rows keep the key wave's
// writes free of bank conflicts
constexpr int PHS = 48;
struct Handoff {
    // 8 dwords between the arrays: the value wave reads hi rows of ph and lo
    // rows of pq in one instruction, and rows of both then start on distinct
    // multiples of 8 banks (fewer LDS bank-conflict cycles, measured)
    __attribute__((aligned(16))) uint32_t ph[HG * PHS + 8];
    __attribute__((aligned(16))) uint32_t pq[HG * PHS];
    float alpha[HG];   // rescale of earlier accumulations
};

struct Lds {
    LdsK k;
    LdsV v;
    Handoff hb[2];
    float misc[64];
};

struct KState {
    float m0, m1, m2, m3;   // running maxima per head (log2 units, wave-uniform)
};

// Key side of one tile: produces p and alpha in `hb`.  qw holds this lane's
// query channels 8 chunk .. 8 chunk + 7 as fp16 pairs in quad order.
template <int G, class Run>
__device__ __forceinline__ void key_tile(const MfmaParams& p, KTile& cur, KState& st, LdsK& L,
                                         Handoff& hb, const uint32_t* qw, int lane,
                                         int64_t bh, int nxt, const Run& run) {
    constexpr int NBT = 64 / G;
    const int n = lane & 15, kg = lane >> 4;
    const int hh = lane >> 4, chunk = lane & 15;

    // ---- stage key codes and side values, then prefetch tile i + 2
    stage_keys<G>(cur, L.kl, L.ksl, lane);
    // unconditional (past the run it reads nothing) so that every path has
    // the same loads in flight and the wait before staging covers only the
    // older tile
    load_ktile<G>(p, run, bh, nxt, lane, cur);
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
            split_prod_h(qw[i], sw[i], hi[i], lo[i]);
            bias = dot2h(qw[i], zw[i], bias);
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
            // byte n & 3 of word row n >> 2 (G = 64; (n >> 2) & 1 of block be
            // for G = 32) of channels 32ksx + 8kg + 0..7
            const CodeRegs c = code_operands(ld_tr8(L.kl + key_row_dw<G>(ksx, be, kg, n)));
            if (G == 64) {
                // A rows 0..7 = q' with rows 8..15 zero (token positions 0, 2)
                // and the reverse (1, 3), from q' rows n and n ^ 8 (rows 8..15
                // of the buffer are zero for G = 64): tokens 4n + 2v land in
                // rows 0..7 and 4n + 2v + 1 in rows 8..15 of accumulator v
                const uint4 ae = *reinterpret_cast<const uint4*>(L.qa + n * QSTR + 16 * ksx + 4 * kg);
                const uint4 ao = *reinterpret_cast<const uint4*>(L.qa + (n ^ 8) * QSTR + 16 * ksx + 4 * kg);
                const f16x8 Ae = as_f16x8(ae.x, ae.y, ae.z, ae.w), Ao = as_f16x8(ao.x, ao.y, ao.z, ao.w);
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    S[v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ae, code_slice2(c, 2 * v), S[v], 0, 0, 0);
                    S[v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ao, code_slice2(c, 2 * v + 1), S[v], 0, 0, 0);
                }
            } else {
                const uint4 a = *reinterpret_cast<const uint4*>(L.qa + (be * 8 + (n & 7)) * QSTR + 16 * ksx + 4 * kg);
                const f16x8 A = as_f16x8(a.x, a.y, a.z, a.w);
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const uint32_t mk = code_mask2(n >> 3);   // position 2v + (n >> 3)
                    S[2 * be + v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, code_slice_set(c, v != 0, mk), S[2 * be + v], 0, 0, 0);
                }
            }
        }
    }

    // ---- softmax.  Lane (n, kg) holds rows 4kg..4kg+3; lanes kg and kg+2
    // see heads 2(kg&1), 2(kg&1)+1 (hi/lo row pairs) and split the columns'
    // tokens so that each lane ends up with a token pair 4k + j, 4k + j + 2:
    //   G = 64: accumulator v, column n holds token 4n + 2v in rows 0..7
    //           (lanes kg < 2) and 4n + 2v + 1 in rows 8..15 (k = n,
    //           j = kg >> 1);
    //   G = 32: A rows 8..15 repeat rows 0..7; tile 2be + v, column n is
    //           token 32be + 16((n & 7) >> 2) + 4(n & 3) + 2v + (n >> 3);
    //           lanes kg < 2 take block 0 and kg >= 2 block 1 (j = n >> 3).
    const bool odd = (kg & 1) != 0;
    [[maybe_unused]] const bool up2 = (kg >> 1) != 0;
    float sA[2], sB[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
        // element-wise selects keep the accumulators in registers
        float Sv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            Sv[e] = G == 64 ? S[v][e] : (up2 ? S[2 + v][e] : S[v][e]);
        const int up = G == 64 ? 2 * v + (kg >> 1) : 2 * v + (n >> 3);
        const int be = G == 64 ? 0 : (kg >> 1);
        const float f = p.sigma2 * code_unscale2(up);
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
    // ---- weights as fp16 hi + lo pairs (tokens 4k + j, 4k + j + 2)
    const int hA = 2 * (kg & 1), hB = hA + 1;
    const int dw = G == 64 ? 2 * n + (kg >> 1)
                           : 2 * (8 * (kg >> 1) + 4 * ((n & 7) >> 2) + (n & 3)) + (n >> 3);
    uint32_t h, l;
    split_f32(sA[0], sA[1], p.neg1, h, l);
    hb.ph[hA * PHS + dw] = h;
    hb.pq[hA * PHS + dw] = l;
    split_f32(sB[0], sB[1], p.neg1, h, l);
    hb.ph[hB * PHS + dw] = h;
    hb.pq[hB * PHS + dw] = l;
    if (lane < HG) hb.alpha[lane] = sel4(lane, a0, a1, a2, a3);
}

struct VState {
    f32x4 O[2][4];   // PV accumulators [pass][channel tile]
    // sum_t p z_v per (head, group) and l = sum_t p on MFMA: rows 2h (hi),
    // 2h + 1 (lo) of head h (rows 8..15 repeat them), column g < 4 the
    // zero-point sum of group g, column 4 the weight sum
    f32x4 Z;
};

// Value side of one tile, reading p and alpha from `hb`.
template <int G, class Run>
__device__ __forceinline__ void value_tile(const MfmaParams& p, VTile& cur, VState& st, LdsV& L,
                                           const Handoff& hb, int lane, int64_t bh,
                                           int nxt, const Run& run) {
    const int n = lane & 15, kg = lane >> 4;
    const int hh = lane >> 4, chunk = lane & 15;
    // ---- stage value codes and side values, then prefetch tile i + 2
    stage_values(cur, L.vl, L.vsl, lane);
    load_vtile<G>(p, run, bh, nxt, lane, cur);

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
        st.Z[0] *= aA;
        st.Z[1] *= aA;
        st.Z[2] *= aB;
        st.Z[3] *= aB;
    }
    wave_sync();

    // ---- p' = p * s_v as fp16 hi/lo rows per value group.  Lane (hh, chunk):
    // tokens 4 chunk .. 4 chunk + 3 of head hh, as the pairs (t0, t2),
    // (t1, t3) that the rows hold in quad order.
    {
        const uint2 ph = *reinterpret_cast<const uint2*>(hb.ph + hh * PHS + 2 * chunk);
        const uint2 pq = *reinterpret_cast<const uint2*>(hb.pq + hh * PHS + 2 * chunk);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint2 sv = *reinterpret_cast<const uint2*>(L.vsl + g * 32 + 2 * chunk);
            uint32_t h0, l0, h1, l1;
            split_prod_hl(ph.x, pq.x, sv.x, h0, l0);
            split_prod_hl(ph.y, pq.y, sv.y, h1, l1);
            // row ((pass*2 + gsel)*4 + head)*2 + hl; 64 tokens = 32 dwords per row
            uint32_t* rowp = L.pa + ((((g >> 1) * 2 + (g & 1)) * 4 + hh) * 2) * ASTR + 2 * chunk;
            *reinterpret_cast<uint2*>(rowp) = make_uint2(h0, h1);
            *reinterpret_cast<uint2*>(rowp + ASTR) = make_uint2(l0, l1);
        }
    }
    // ---- sum_t p z_v and sum_t p: A = the weights' hi/lo rows (row n & 7 =
    // head (n & 7) >> 1, hi or lo), B column n = the zero-points of group n
    // (n < 4), ones (n = 4) or zeros, over the tile's 64 tokens in quad order
    {
        const int r = n & 7;
        const uint32_t* arow = ((r & 1) ? hb.pq : hb.ph) + (r >> 1) * PHS + 4 * kg;
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

    // ---- O += p' . codes: 2 passes x 4 channel tiles x 2 K-steps of 32 tokens
#pragma unroll
    for (int P = 0; P < 2; ++P) {
#pragma unroll
        for (int ksx = 0; ksx < 2; ++ksx) {
            const uint4 a = *reinterpret_cast<const uint4*>(L.pa + (P * 16 + n) * ASTR + 16 * ksx + 4 * kg);
            const f16x8 A = as_f16x8(a.x, a.y, a.z, a.w);
            // byte n & 3 of word 4P + (n >> 2) of tokens 32ksx + 8kg + 0..7
            const CodeRegs c = code_operands(ld_tr8(L.vl + value_row_dw(ksx, P, kg, n)));
#pragma unroll
            for (int u = 0; u < 4; ++u)
                st.O[P][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, code_slice2(c, u),
                                                                    st.O[P][u], 0, 0, 0);
        }
    }
}


template <int G, bool PAGED>
__global__ __launch_bounds__(128) void k_decode_gqa(MfmaParams p) {
    __shared__ Lds L;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = lane & 15, kg = lane >> 4;
    const int hh = lane >> 4, chunk = lane & 15;
    int b, kvh;
    bool tail;
    const int s = block_coords<!PAGED>(p, b, kvh, tail);
    const int64_t bh = int64_t(b) * p.Hkv + kvh;
    const int hq0 = kvh * HG;
    // a paged sequence has its own length; main split s takes tiles
    // [s * chunk, (s + 1) * chunk) of it, so the splits past a shorter
    // sequence's tiles are empty, and the page numbers of a split are known
    // before its length is
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
            tail_split<HG>(p, PagedBlocks{}, b, kvh, s, reinterpret_cast<float*>(L.k.qa),
                               reinterpret_cast<float*>(L.v.pa), T1, T1 / G, ntiles);
            return;
        }
        t_lo = s * p.chunk;
        prun = paged_run<G>(p, b, kvh, t_lo, lane);
        t_hi = t_lo + p.chunk < ntiles ? t_lo + p.chunk : ntiles;
        if (t_lo >= t_hi) {
            empty_partial<HG>(p, b, kvh, s);
            return;
        }
        prun.t_last = t_hi - 1;
    } else {
        if (tail) {
            tail_split<HG>(p, b, kvh, s, reinterpret_cast<float*>(L.k.qa), reinterpret_cast<float*>(L.v.pa));
            return;
        }
        t_lo = int(int64_t(s) * p.ntiles / p.S_main);
        t_hi = int(int64_t(s + 1) * p.ntiles / p.S_main);
    }
    const int ntl = t_hi - t_lo;

    if (wave == 0) {
        // G = 64 uses q' rows 0..7; rows 8..15 are the zero rows of the
        // split A operands
        if (G == 64)
            for (int i = lane; i < 8 * QSTR; i += 64) L.k.qa[8 * QSTR + i] = 0u;
        // query channels 8 chunk .. 8 chunk + 7 of head hh, in quad order
        const uint4 raw = *reinterpret_cast<const uint4*>(p.q + ((int64_t(b) * p.Hq + hq0 + hh) * D + 8 * chunk));
        const uint32_t qv[4] = {pair_lo(raw.x, raw.y), pair_hi(raw.x, raw.y), pair_lo(raw.z, raw.w),
                                pair_hi(raw.z, raw.w)};
        KState st;
        st.m0 = st.m1 = st.m2 = st.m3 = -INFINITY;
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
        key_tile<G>(p, ta, st, L.k, L.hb[0], qv, lane, bh, t_lo + 2, run);
        __syncthreads();
        int j = 1;
        for (; j + 1 < ntl; j += 2) {
            key_tile<G>(p, tb, st, L.k, L.hb[1], qv, lane, bh, t_lo + j + 2, run);
            __syncthreads();
            key_tile<G>(p, ta, st, L.k, L.hb[0], qv, lane, bh, t_lo + j + 3, run);
            __syncthreads();
        }
        if (j < ntl) {
            key_tile<G>(p, tb, st, L.k, L.hb[1], qv, lane, bh, t_lo + j + 2, run);
            __syncthreads();
        }
        if (lane < HG) L.misc[lane] = sel4(lane, st.m0, st.m1, st.m2, st.m3);
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
        // ---- epilogue: l and the value-zero sums, hi + lo rows of each head
        if (kg < 2 && n < 5) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int h = 2 * kg + j;
                const float v = st.Z[2 * j] + st.Z[2 * j + 1];
                L.misc[n < 4 ? 32 + h * 4 + n : 16 + h] = v;
            }
        }
        wave_sync();
        if ((kg >> 1) == (n >> 3)) {
#pragma unroll
            for (int P = 0; P < 2; ++P)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int c = 64 * P + 32 * (n >> 3) + 4 * (n & 7) + u;
                    const int g = 2 * P + (n >> 3);
                    const float f = code_unscale2(u);
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

// ---------------------------------------------------------------------------
// 4-bit keys and values: the same two-wave pipeline over the 4 KB tiles of
// kvq_mfma_tiles.h.  A code byte holds two tokens (keys) or two channels
// (values), taken by one mask each from the copies of the bytes shifted to
// put the low or the high nibble at bits 6..9 of the fp16 halves.

struct LdsK4 {
    __attribute__((aligned(16))) uint32_t kl[KTILE4_DW];
    __attribute__((aligned(16))) uint32_t qz[QSTR];   // a zero row (the idle half of split A operands)
    __attribute__((aligned(16))) uint32_t qa[2 * 8 * QSTR];
    __attribute__((aligned(16))) uint32_t ksl[2 * 2 * 64];
    float bias[8];
};
struct LdsV4 {
    __attribute__((aligned(16))) uint32_t vl[VTILE4_DW];
    __attribute__((aligned(16))) uint32_t pa[2 * 16 * ASTR];   // p' rows: pass P (= value group), head, hi/lo
    __attribute__((aligned(16))) uint32_t vsl[2 * 128 + 2 * 32];
};
struct Lds4 {
    LdsK4 k;
    LdsV4 v;
    Handoff hb[2];
    float misc[64];
};

template <int G, class Run>
__device__ __forceinline__ void key_tile4(const MfmaParams& p, KTile4& cur, KState& st, LdsK4& L, Handoff& hb,
                                          const uint32_t* qw, int lane, int64_t bh, int nxt, const Run& run) {
    constexpr int NBT = 64 / G;
    const int n = lane & 15, kg = lane >> 4;
    const int hh = lane >> 4, chunk = lane & 15;

    stage_keys4<G>(cur, L.kl, L.ksl, lane);
    load_ktile4<G>(p, run, bh, nxt, lane, cur);
    wave_sync();

    // ---- q' = q * s_k as fp16 hi/lo rows, sigma2 * sum_c q z_k per (block, head): as for 2 bits
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
            split_prod_h(qw[i], sw[i], hi[i], lo[i]);
            bias = dot2h(qw[i], zw[i], bias);
        }
        uint32_t* row = L.qa + (be * 8 + 2 * hh) * QSTR + 4 * chunk;
        *reinterpret_cast<uint4*>(row) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *reinterpret_cast<uint4*>(row + QSTR) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        bias = row_sum16(bias);
        if (chunk == 0) L.bias[be * 4 + hh] = bias * p.sigma2;
    }
    wave_sync();

    // ---- S = q' . codes: per K-step of 32 channels, two transposed reads
    // (tile tokens 0..31 and 32..63; for G = 32 the two blocks) of two
    // nibbles each.  S[2r + nib], column n = token 32r + 2n + nib.
    f32x4 S[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) S[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ksx = 0; ksx < 4; ++ksx) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int be = G == 64 ? 0 : r;
            // q' in A rows 8r .. 8r + 7, the other half zero: half r of the
            // tile lands in rows 8r .. 8r + 7 of the accumulators
            const uint32_t* arow = (n >> 3) == r ? L.qa + (be * 8 + (n & 7)) * QSTR : L.qz;
            const uint4 a = *reinterpret_cast<const uint4*>(arow + 16 * ksx + 4 * kg);
            const f16x8 A = as_f16x8(a.x, a.y, a.z, a.w);
            const CodeRegs c = code_operands(ld_tr8(L.kl + key_row_dw4<G>(ksx, r, kg, n)));
#pragma unroll
            for (int nib = 0; nib < 2; ++nib)
                S[nib] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, code_slice4(c, nib), S[nib],
                                                               0, 0, 0);
        }
    }

    // ---- softmax: lanes kg and kg + 2 see heads 2(kg&1), 2(kg&1)+1; lanes
    // kg < 2 hold the first half of the tile (r = 0, rows 0..7), kg >= 2 the
    // second (rows 8..15), so a lane holds tokens 32r + 2n, + 1
    const bool odd = (kg & 1) != 0;
    const int beh = G == 64 ? 0 : (kg >> 1);
    float sA[2], sB[2];
#pragma unroll
    for (int nib = 0; nib < 2; ++nib) {
        float Sv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) Sv[e] = S[nib][e];
        const float f = p.sigma2 * code_unscale4();
        sA[nib] = fmaf(Sv[0] + Sv[1], f, L.bias[beh * 4 + 2 * (kg & 1)]);
        sB[nib] = fmaf(Sv[2] + Sv[3], f, L.bias[beh * 4 + 2 * (kg & 1) + 1]);
    }
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
    for (int nib = 0; nib < 2; ++nib) {
        sA[nib] = fast_exp2(sA[nib] - mrA);
        sB[nib] = fast_exp2(sB[nib] - mrB);
    }
    // ---- weights as fp16 hi + lo pairs (tokens 4k + j, 4k + j + 2): lane n
    // holds 4k + 2(n & 1) + nib with k = 8r + (n >> 1), so an even lane pairs
    // its low-nibble token with its odd neighbour's and the odd lane its
    // high-nibble token with the even neighbour's (dword 16r + n)
    const int hA = 2 * (kg & 1), hB = hA + 1;
    const int dw = 16 * (kg >> 1) + n;
    const bool nodd = (n & 1) != 0;
    const float oA = dpp<0xb1>(nodd ? sA[0] : sA[1]);
    const float oB = dpp<0xb1>(nodd ? sB[0] : sB[1]);
    uint32_t h, l;
    split_f32(nodd ? oA : sA[0], nodd ? sA[1] : oA, p.neg1, h, l);
    hb.ph[hA * PHS + dw] = h;
    hb.pq[hA * PHS + dw] = l;
    split_f32(nodd ? oB : sB[0], nodd ? sB[1] : oB, p.neg1, h, l);
    hb.ph[hB * PHS + dw] = h;
    hb.pq[hB * PHS + dw] = l;
    if (lane < HG) hb.alpha[lane] = sel4(lane, a0, a1, a2, a3);
}

struct VState4 {
    f32x4 O[4][2];   // PV accumulators [pass = value group][nibble]
    f32x4 Z;         // as VState::Z
};

template <int G, class Run>
__device__ __forceinline__ void value_tile4(const MfmaParams& p, VTile4& cur, VState4& st, LdsV4& L, const Handoff& hb,
                                            int lane, int64_t bh, int nxt, const Run& run) {
    const int n = lane & 15, kg = lane >> 4;
    const int hh = lane >> 4, chunk = lane & 15;
    stage_values4(cur, L.vl, L.vsl, lane);
    load_vtile4<G>(p, run, bh, nxt, lane, cur);

    const float a0 = hb.alpha[0], a1 = hb.alpha[1], a2 = hb.alpha[2], a3 = hb.alpha[3];
    if (fminf(fminf(a0, a1), fminf(a2, a3)) < 1.0f) {
        const bool odd = (kg & 1) != 0;
        const float aA = odd ? a2 : a0, aB = odd ? a3 : a1;
#pragma unroll
        for (int P = 0; P < 4; ++P)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                st.O[P][u][0] *= aA;
                st.O[P][u][1] *= aA;
                st.O[P][u][2] *= aB;
                st.O[P][u][3] *= aB;
            }
        st.Z[0] *= aA;
        st.Z[1] *= aA;
        st.Z[2] *= aB;
        st.Z[3] *= aB;
    }
    wave_sync();

    // ---- p' = p * s_v as fp16 hi/lo rows per value group g: rows (g * 4 +
    // head) * 2 + hl, the same rows as for 2 bits (there pass g >> 1, half g & 1)
    {
        const uint2 ph = *reinterpret_cast<const uint2*>(hb.ph + hh * PHS + 2 * chunk);
        const uint2 pq = *reinterpret_cast<const uint2*>(hb.pq + hh * PHS + 2 * chunk);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint2 sv = *reinterpret_cast<const uint2*>(L.vsl + g * 32 + 2 * chunk);
            uint32_t h0, l0, h1, l1;
            split_prod_hl(ph.x, pq.x, sv.x, h0, l0);
            split_prod_hl(ph.y, pq.y, sv.y, h1, l1);
            uint32_t* rowp = L.pa + ((g * 4 + hh) * 2) * ASTR + 2 * chunk;
            *reinterpret_cast<uint2*>(rowp) = make_uint2(h0, h1);
            *reinterpret_cast<uint2*>(rowp + ASTR) = make_uint2(l0, l1);
        }
    }
    // ---- sum_t p z_v and sum_t p on the matrix cores, as for 2 bits
    {
        const int r = n & 7;
        const uint32_t* arow = ((r & 1) ? hb.pq : hb.ph) + (r >> 1) * PHS + 4 * kg;
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

    // ---- O += p' . codes: 4 passes (one value group each) x 2 K-steps of
    // 32 tokens x 2 nibbles; A rows 8..15 repeat rows 0..7
#pragma unroll
    for (int P = 0; P < 4; ++P) {
#pragma unroll
        for (int ksx = 0; ksx < 2; ++ksx) {
            const uint4 a = *reinterpret_cast<const uint4*>(L.pa + (P * 8 + (n & 7)) * ASTR + 16 * ksx + 4 * kg);
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
__global__ __launch_bounds__(128) void k_decode_gqa4(MfmaParams p) {
    __shared__ Lds4 L;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = lane & 15, kg = lane >> 4;
    const int hh = lane >> 4, chunk = lane & 15;
    int b, kvh;
    bool tail;
    const int s = block_coords<!PAGED>(p, b, kvh, tail);
    const int64_t bh = int64_t(b) * p.Hkv + kvh;
    const int hq0 = kvh * HG;
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
            tail_split<HG, PagedBlocks, 4>(p, PagedBlocks{}, b, kvh, s, reinterpret_cast<float*>(L.k.qa),
                               reinterpret_cast<float*>(L.v.pa), T1, T1 / G, ntiles);
            return;
        }
        t_lo = s * p.chunk;
        prun = paged_run<G>(p, b, kvh, t_lo, lane);
        t_hi = t_lo + p.chunk < ntiles ? t_lo + p.chunk : ntiles;
        if (t_lo >= t_hi) {
            empty_partial<HG>(p, b, kvh, s);
            return;
        }
        prun.t_last = t_hi - 1;
    } else {
        if (tail) {
            tail_split<HG, 4>(p, b, kvh, s, reinterpret_cast<float*>(L.k.qa), reinterpret_cast<float*>(L.v.pa));
            return;
        }
        t_lo = int(int64_t(s) * p.ntiles / p.S_main);
        t_hi = int(int64_t(s + 1) * p.ntiles / p.S_main);
    }
    const int ntl = t_hi - t_lo;

    if (wave == 0) {
        for (int i = lane; i < QSTR; i += 64) L.k.qz[i] = 0u;   // the zero row of the split A operands
        const uint4 raw = *reinterpret_cast<const uint4*>(p.q + ((int64_t(b) * p.Hq + hq0 + hh) * D + 8 * chunk));
        const uint32_t qv[4] = {pair_lo(raw.x, raw.y), pair_hi(raw.x, raw.y), pair_lo(raw.z, raw.w),
                                pair_hi(raw.z, raw.w)};
        KState st;
        st.m0 = st.m1 = st.m2 = st.m3 = -INFINITY;
        KTile4 ta, tb;
        const auto run = pick_run4<G, PAGED>(p, prun, bh, t_lo, t_hi);
        load_ktile4<G>(p, run, bh, t_lo, lane, ta);
        load_ktile4<G>(p, run, bh, t_lo + 1, lane, tb);
        __builtin_amdgcn_sched_barrier(0);
        key_tile4<G>(p, ta, st, L.k, L.hb[0], qv, lane, bh, t_lo + 2, run);
        __syncthreads();
        int j = 1;
        for (; j + 1 < ntl; j += 2) {
            key_tile4<G>(p, tb, st, L.k, L.hb[1], qv, lane, bh, t_lo + j + 2, run);
            __syncthreads();
            key_tile4<G>(p, ta, st, L.k, L.hb[0], qv, lane, bh, t_lo + j + 3, run);
            __syncthreads();
        }
        if (j < ntl) {
            key_tile4<G>(p, tb, st, L.k, L.hb[1], qv, lane, bh, t_lo + j + 2, run);
            __syncthreads();
        }
        if (lane < HG) L.misc[lane] = sel4(lane, st.m0, st.m1, st.m2, st.m3);
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
        // ---- epilogue: l and the value-zero sums, as for 2 bits
        if (kg < 2 && n < 5) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int h = 2 * kg + j;
                const float v = st.Z[2 * j] + st.Z[2 * j + 1];
                L.misc[n < 4 ? 32 + h * 4 + n : 16 + h] = v;
            }
        }
        wave_sync();
        // rows 0..7 (head 2kg + j, hi/lo); rows 8..15 repeat them
        if (kg < 2) {
#pragma unroll
            for (int P = 0; P < 4; ++P)
#pragma unroll
                for (int nib = 0; nib < 2; ++nib) {
                    const int c = 32 * P + 8 * (n >> 2) + 2 * (n & 3) + nib;
                    const float f = code_unscale4();
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int h = 2 * kg + j;
                        const float acc = fmaf(st.O[P][nib][2 * j] + st.O[P][nib][2 * j + 1], f, L.misc[32 + h * 4 + P]);
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
    return (mfma_cfg_ok(c.cfg) || mfma_cfg_ok4(c.cfg)) && Hq == HG * c.cfg.n_kv_heads;
}

bool gqa_cfg_supported(const kvq_cache_cfg& c, int Hq) {
    return (mfma_cfg_ok(c) || mfma_cfg_ok4(c)) && Hq == HG * c.n_kv_heads;
}

hipError_t launch_decode_gqa(const DecodeArgs& a, hipStream_t st) {
    const MfmaParams p = mfma_params(a);
    const dim3 grid = decode_grid<true>(a.S, a.g.Hkv, a.g.B);
    if (a.g.kbits == 4) {
        if (a.g.kG == 64)
            hipExtLaunchKernelGGL((k_decode_gqa4<64, false>), grid, dim3(128), 0, st, a.ev_start, a.ev_stop, 0, p);
        else
            hipExtLaunchKernelGGL((k_decode_gqa4<32, false>), grid, dim3(128), 0, st, a.ev_start, a.ev_stop, 0, p);
        return hipGetLastError();
    }
    if (a.g.kG == 64)
        hipExtLaunchKernelGGL((k_decode_gqa<64, false>), grid, dim3(128), 0, st, a.ev_start, a.ev_stop, 0, p);
    else
        hipExtLaunchKernelGGL((k_decode_gqa<32, false>), grid, dim3(128), 0, st, a.ev_start, a.ev_stop, 0, p);
    return hipGetLastError();
}

hipError_t launch_decode_gqa_paged(const DecodeArgs& a, hipStream_t st) {
    const MfmaParams p = mfma_params(a);
    const dim3 grid = decode_grid<false>(a.S, a.g.Hkv, a.g.B);
    if (a.g.kbits == 4) {
        if (a.g.kG == 64)
            hipExtLaunchKernelGGL((k_decode_gqa4<64, true>), grid, dim3(128), 0, st, a.ev_start, a.ev_stop, 0, p);
        else
            hipExtLaunchKernelGGL((k_decode_gqa4<32, true>), grid, dim3(128), 0, st, a.ev_start, a.ev_stop, 0, p);
        return hipGetLastError();
    }
    if (a.g.kG == 64)
        hipExtLaunchKernelGGL((k_decode_gqa<64, true>), grid, dim3(128), 0, st, a.ev_start, a.ev_stop, 0, p);
    else
        hipExtLaunchKernelGGL((k_decode_gqa<32, true>), grid, dim3(128), 0, st, a.ev_start, a.ev_stop, 0, p);
    return hipGetLastError();
}

}  // namespace kvq
