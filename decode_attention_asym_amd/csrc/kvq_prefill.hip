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
// Work split: one four-wave workgroup per (64 query rows, query head,
// sequence); wave w owns rows 16w .. 16w + 15.  It walks the 64-token key /
// value tiles 0 .. i of its causal window (the diagonal tile last, with the
// mask), staging each tile in LDS: keys row-major, values transposed
// (channel-major), so that both products read 16-byte or 8-byte rows.
//   S^T = K Q^T  (A = key rows from LDS, B = the query rows, in registers)
//   O^T = V^T P^T (A = value columns from LDS, B = the weights, in registers)
// With these orientations each lane holds one query row in both results: the
// weights of S^T's accumulator feed O^T's B operand without leaving the lane,
// and the softmax rescale and the final 1/l stay lane-local.  Softmax in
// log2 units with the running maximum moved only when a logit exceeds it by
// more than 2^8 (weights stay <= 256 in fp16); weights are rounded to fp16
// for the second product, l sums them in fp32.
//
// Fused quantize: the workgroup of the first query head of each KV head and
// query block i also quantizes tile i (values of its rows, the key blocks it
// completes, the unfilled block's rows into the residual) with the append
// kernels' device code, so the cache equals kv_quantize_append's bit for bit.
#include "kvq_quant_dev.h"

namespace kvq {
namespace {

constexpr int PD = 128;     // head dim of q, k and v
constexpr int PKS = 68;     // dwords per staged key row (128 fp16 + 8 pad)
constexpr int PVS = 36;     // dwords per staged value column (64 fp16 + 8 pad)
constexpr float PTAU = 8.0f;

typedef _Float16 pf16x8 __attribute__((ext_vector_type(8)));
typedef float pf32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ pf16x8 as_pf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(pf16x8, u4v{a, b, c, d});
}
__device__ __forceinline__ uint32_t plo(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x05040100u); }
__device__ __forceinline__ uint32_t phi(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x07060302u); }
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, h2{_Float16(a), _Float16(b)});
}
__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

struct PrefillLds {
    __attribute__((aligned(16))) uint32_t kl[64 * PKS];    // key rows of the tile
    __attribute__((aligned(16))) uint32_t vt[PD * PVS];    // value columns of the tile
};

// One 64-token tile in registers: thread t holds key row t >> 2, channels
// 32 (t & 3) .. + 31, and value rows 2 (t & 31), + 1, channels 16 (t >> 5) .. + 15
struct PTile {
    uint4 k[4];
    uint4 va[2], vb[2];
};

__device__ __forceinline__ void load_ptile(const PrefillArgs& a, const uint16_t* kbase, const uint16_t* vbase,
                                           int t0, int tid, PTile& r) {
    const int kr = t0 + (tid >> 2), kq = tid & 3;
    const bool kin = kr < a.T;
    const uint16_t* kp = kbase + int64_t(kin ? kr : 0) * PD + 32 * kq;
#pragma unroll
    for (int e = 0; e < 4; ++e) r.k[e] = kin ? ld16(kp + 8 * e) : make_uint4(0u, 0u, 0u, 0u);
    const int vr = t0 + 2 * (tid & 31), vc = 16 * (tid >> 5);
    const bool va = vr < a.T, vb = vr + 1 < a.T;
    const uint16_t* vp = vbase + int64_t(va ? vr : 0) * PD + vc;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        r.va[e] = va ? ld16(vp + 8 * e) : make_uint4(0u, 0u, 0u, 0u);
        r.vb[e] = vb ? ld16(vp + PD + 8 * e) : make_uint4(0u, 0u, 0u, 0u);
    }
}

__device__ __forceinline__ void stage_ptile(const PTile& r, PrefillLds& L, int tid) {
    uint32_t* kd = L.kl + (tid >> 2) * PKS + 16 * (tid & 3);
#pragma unroll
    for (int e = 0; e < 4; ++e) *reinterpret_cast<uint4*>(kd + 4 * e) = r.k[e];
    // value column c, dword tp: tokens 2tp, 2tp + 1
    const int tp = tid & 31, c0 = 16 * (tid >> 5);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const uint32_t a[4] = {r.va[e].x, r.va[e].y, r.va[e].z, r.va[e].w};
        const uint32_t b[4] = {r.vb[e].x, r.vb[e].y, r.vb[e].z, r.vb[e].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int c = c0 + 8 * e + 2 * w;
            L.vt[c * PVS + tp] = plo(a[w], b[w]);
            L.vt[(c + 1) * PVS + tp] = phi(a[w], b[w]);
        }
    }
}

// The tile's share of the cache: values of rows t0 .. t0 + n - 1, the key
// blocks inside them that the prompt fills, and the residual rows of the
// unfilled block (the same device functions as the append kernels).
template <int G, int KB, int VB>
__device__ void quantize_tile(const PrefillArgs& a, int64_t bh, int t0, int tid) {
    const int n = a.T - t0 < 64 ? a.T - t0 : 64;
    {
        qdev::ValueArgs va;
        va.vin = a.v + bh * int64_t(a.T) * PD;
        va.n_in = a.T;
        va.row0 = t0;
        va.n_tok = n;
        va.vd = PD;
        va.BH = 1;
        va.codes = a.vc;
        va.scale = a.vs;
        va.zero = a.vz;
        const qdev::ContigRows rows{a.cap, bh * a.cap + t0, n};
        if (tid < qdev::value_threads(1, n, PD)) qdev::quant_values_thread<VB>(va, rows, tid);
    }
    constexpr int NB = 64 / G;
    const int64_t per = qdev::key_threads_per_block<G, KB>(PD);   // whole waves when a pair spans lanes
    const int nfull = a.T / G;                                    // blocks the prompt fills
    if (tid < NB * per) {
        int64_t unit;
        int cp, sp;
        qdev::key_thread_coords<G, KB>(tid, PD, unit, cp, sp);
        const int64_t blk = t0 / G + unit;
        if (blk < nfull) {
            const qdev::KeyJob j{a.k + bh * int64_t(a.T) * PD, a.kr + bh * G * PD, blk * G, 0, 0,
                                 bh * a.nblk_cap + blk};
            qdev::quant_key_pair<G, KB>(j, PD, cp, sp, a.kc, a.ks, a.kz);
        }
    }
    // residual: rows nfull * G .. T - 1 that lie in this tile
    const int r0 = nfull * G > t0 ? nfull * G : t0;
    for (int i = tid; i < (t0 + n - r0) * (PD / 8); i += 256) {
        const int t = r0 + i / (PD / 8), c = 8 * (i % (PD / 8));
        *reinterpret_cast<uint4*>(a.kr + (bh * G + (t - nfull * G)) * PD + c) =
            ld16(a.k + (bh * int64_t(a.T) + t) * PD + c);
    }
}

template <int G, int KB, int VB>
__global__ __launch_bounds__(256) void k_prefill(PrefillArgs a) {
    __shared__ PrefillLds L;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, kg = lane >> 4;
    // the longest causal windows start first
    const int qb = int(gridDim.x) - 1 - int(blockIdx.x);
    const int hq = blockIdx.y, b = blockIdx.z;
    const int grp = a.Hq / a.Hkv, kvh = hq / grp;
    const int64_t bh = int64_t(b) * a.Hkv + kvh;
    const uint16_t* kbase = a.k + bh * int64_t(a.T) * PD;
    const uint16_t* vbase = a.v + bh * int64_t(a.T) * PD;

    // query row of this lane (the B operand of S^T): channels 32ks + 8kg .. + 7
    const int qrow = 64 * qb + 16 * wave + n;
    pf16x8 qb8[4];
    {
        const bool in = qrow < a.T;
        const uint16_t* qp = a.q + ((int64_t(b) * a.Hq + hq) * a.T + (in ? qrow : 0)) * PD + 8 * kg;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint4 w = in ? ld16(qp + 32 * ks) : make_uint4(0u, 0u, 0u, 0u);
            qb8[ks] = as_pf16x8(w.x, w.y, w.z, w.w);
        }
    }
    pf32x4 O[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) O[c] = pf32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.0f;

    PTile cur;
    load_ptile(a, kbase, vbase, 0, tid, cur);
    for (int j = 0; j <= qb; ++j) {
        __syncthreads();   // every wave is done with tile j - 1
        stage_ptile(cur, L, tid);
        __syncthreads();
        if (j < qb) load_ptile(a, kbase, vbase, 64 * (j + 1), tid, cur);

        // ---- S^T = K Q^T: lane (n, kg) gets tokens 16cb + 4kg + i of row n
        pf32x4 S[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            S[cb] = pf32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const uint4 kw = *reinterpret_cast<const uint4*>(L.kl + (16 * cb + n) * PKS + 16 * ks + 4 * kg);
                S[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_pf16x8(kw.x, kw.y, kw.z, kw.w), qb8[ks], S[cb], 0, 0, 0);
            }
        }
        // ---- online softmax (log2 units), the diagonal tile masked
        float s[16];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) s[4 * cb + i] = S[cb][i] * a.sigma2;
        if (j == qb) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * cb + 4 * kg + i > 16 * wave + n) s[4 * cb + i] = -INFINITY;
        }
        float mx = s[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
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
        uint32_t pw[8];
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const float p0 = __builtin_amdgcn_exp2f(s[e] - m), p1 = __builtin_amdgcn_exp2f(s[e + 1] - m);
            l += p0 + p1;
            pw[e / 2] = pack_h2(p0, p1);
        }
        // ---- O^T += V^T P^T over 2 K-steps of 32 tokens: K order of lane
        // group kg = tokens 32ks + 4kg + 0..3, then 32ks + 16 + 4kg + 0..3
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const pf16x8 P = as_pf16x8(pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t* vr = L.vt + (16 * c + n) * PVS + 16 * ks + 2 * kg;
                const uint2 lo = *reinterpret_cast<const uint2*>(vr);
                const uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
                O[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_pf16x8(lo.x, lo.y, hi.x, hi.y), P, O[c], 0, 0, 0);
            }
        }
    }
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
    if (a.quant && hq % grp == 0) quantize_tile<G, KB, VB>(a, bh, 64 * qb, tid);
}

}  // namespace

bool prefill_supported(const kvq_cache_cfg& c) {
    return c.key.dim == PD && c.value.dim == PD && (c.key.group == 32 || c.key.group == 64) &&
           (c.key.bits == 2 || c.key.bits == 4) && (c.value.bits == 2 || c.value.bits == 4) && c.value.group == 32;
}

hipError_t launch_prefill(const PrefillArgs& a, const kvq_cache_cfg& c, hipStream_t st) {
    const dim3 grid((a.T + 63) / 64, a.Hq, a.B);
#define KVQ_PF(GG, KK, VV)                                                                  \
    if (c.key.group == GG && c.key.bits == KK && c.value.bits == VV) {                      \
        hipLaunchKernelGGL((k_prefill<GG, KK, VV>), grid, dim3(256), 0, st, a);             \
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
