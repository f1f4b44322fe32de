// kvq_decode_generic.hip -- plain split-K decode attention over the 2-bit
// cache (any supported bits / dims / kind) plus the pass-2 merge.
//
// Serves shapes the specialised kernels do not cover and gives every shape a
// straightforward GPU path: one workgroup per (split, query head, sequence),
// one token per thread for the logits (codes unpacked and dequantized in
// registers), an online softmax over 256-token chunks, then each thread
// accumulates p * vhat for its channels.  Logits: sigma * q . khat_t over the
// quantized blocks and the fp16 residual keys ("Makale Bülteni -- KIVI",
// section "İddia ve Gerçeklik: KIVI"); MLA adds the content and RoPE paths
// ("QuantMLA ...", section "Giriş ve Problem Analizi").
#include <hip/hip_fp16.h>
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

struct GenParams {
    const uint32_t* kc;
    const uint16_t *ks, *kz, *kr;
    const uint32_t* vc;
    const uint16_t *vs, *vz;
    const uint16_t* q;
    float *ws_acc, *ws_ml;
    int Hq, Hkv, S, U;
    int64_t T, nblk, cap, nblk_cap;
    int kd, kG, kbits, kW, vd, vbits, vWT, vNG;
    float sigma2;   // softmax scale * log2(e): logits and maxima in log2 units
    // paged caches: block table [B][maxb], lengths [B] (clamped to
    // [0, max_len]), pool size, key blocks per split
    const int32_t *table, *lens;
    int maxb, npages, chunk, max_len;
};

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// block row of key block j of (b, kvh): key codes at row * kd * kW words,
// key side values at row * kd, value rows row * kG + i.  Contiguous:
// (b * Hkv + kvh) * nblk_cap + j; paged: page * Hkv + kvh (the table entry
// clamped into the pool, so a bad entry never reads outside the arrays).
template <bool PAGED>
__device__ __forceinline__ int64_t block_row(const GenParams& p, int b, int kvh, int64_t j) {
    if (PAGED) {
        int pg = p.table[int64_t(b) * p.maxb + j];
        pg = pg < 0 ? 0 : (pg >= p.npages ? p.npages - 1 : pg);
        return int64_t(pg) * p.Hkv + kvh;
    }
    return (int64_t(b) * p.Hkv + kvh) * p.nblk_cap + j;
}

template <bool PAGED>
__device__ __forceinline__ float key_hat(const GenParams& p, int b, int kvh, int64_t nblk, int64_t t, int c) {
    const int64_t Tq = nblk * p.kG;
    if (t >= Tq) return h2f(p.kr[((int64_t(b) * p.Hkv + kvh) * p.kG + (t - Tq)) * p.kd + c]);
    const int per = 32 / p.kbits;
    const int64_t blk = t / p.kG;
    const int i = int(t - blk * p.kG);
    const int64_t side = block_row<PAGED>(p, b, kvh, blk) * p.kd + c;
    const uint32_t w = p.kc[side * p.kW + i / per];
    const uint32_t code = (w >> (p.kbits * (i % per))) & ((1u << p.kbits) - 1u);
    return fmaf(float(code), h2f(p.ks[side]), h2f(p.kz[side]));
}

template <bool PAGED>
__device__ __forceinline__ float value_hat(const GenParams& p, int b, int kvh, int64_t t, int c) {
    const int per = 32 / p.vbits;
    const int64_t blk = t / p.kG;
    const int64_t row = block_row<PAGED>(p, b, kvh, blk) * p.kG + (t - blk * p.kG);
    const uint32_t w = p.vc[row * p.vWT + c / per];
    const uint32_t code = (w >> (p.vbits * (c % per))) & ((1u << p.vbits) - 1u);
    const int64_t side = row * p.vNG + c / 32;
    return fmaf(float(code), h2f(p.vs[side]), h2f(p.vz[side]));
}

__device__ __forceinline__ float wave_max(float x) {
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <bool MLA, bool PAGED>
__global__ __launch_bounds__(256) void k_decode_generic(GenParams p) {
    __shared__ float qs[1024];
    __shared__ float ps[256];
    __shared__ float red[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int s = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
    const int kvh = hq / (p.Hq / p.Hkv);
    const int qd = MLA ? p.vd + p.kd : p.kd;
    for (int i = tid; i < qd; i += 256) qs[i] = h2f(p.q[(int64_t(b) * p.Hq + hq) * qd + i]);
    // work units: key blocks, the residual counting as one more.  Contiguous:
    // the splits share the units evenly; paged: each sequence has its own
    // length and split s takes units [s * chunk, (s + 1) * chunk)
    int64_t T = p.T, nblk = p.nblk, u0, u1;
    if (PAGED) {
        const int l = p.lens[b];
        T = l < 0 ? 0 : (l > p.max_len ? p.max_len : l);
        nblk = T / p.kG;
        const int64_t U = nblk + (T > nblk * p.kG ? 1 : 0);
        u0 = int64_t(s) * p.chunk;
        u1 = u0 + p.chunk < U ? u0 + p.chunk : U;
    } else {
        u0 = int64_t(s) * p.U / p.S;
        u1 = int64_t(s + 1) * p.U / p.S;
    }
    const int64_t t0 = u0 * p.kG;
    const int64_t t1 = u1 * p.kG < T ? u1 * p.kG : T;
    float m = -INFINITY, l = 0.0f, acc0 = 0.0f, acc1 = 0.0f;
    __syncthreads();
    for (int64_t base = t0; base < t1; base += 256) {
        const int64_t t = base + tid;
        float sc = -INFINITY;
        if (t < t1) {
            float dot = 0.0f;
            if (MLA) {
                for (int c = 0; c < p.vd; ++c) dot = fmaf(qs[c], value_hat<PAGED>(p, b, kvh, t, c), dot);
                for (int c = 0; c < p.kd; ++c) dot = fmaf(qs[p.vd + c], key_hat<PAGED>(p, b, kvh, nblk, t, c), dot);
            } else {
                for (int c = 0; c < p.kd; ++c) dot = fmaf(qs[c], key_hat<PAGED>(p, b, kvh, nblk, t, c), dot);
            }
            sc = p.sigma2 * dot;
        }
        float wm = wave_max(sc);
        if (lane == 0) red[0][wv] = wm;
        __syncthreads();
        const float cm = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
        const float mnew = fmaxf(m, cm);
        const float pt = t < t1 ? exp2f(sc - mnew) : 0.0f;
        const float alpha = exp2f(m - mnew);
        const float ws = wave_sum(pt);
        if (lane == 0) red[1][wv] = ws;
        ps[tid] = pt;
        __syncthreads();
        l = l * alpha + ((red[1][0] + red[1][1]) + (red[1][2] + red[1][3]));
        acc0 *= alpha;
        acc1 *= alpha;
        const int n = int(t1 - base < 256 ? t1 - base : 256);
        for (int j = 0; j < n; ++j) {
            const float pj = ps[j];
            if (tid < p.vd) acc0 = fmaf(pj, value_hat<PAGED>(p, b, kvh, base + j, tid), acc0);
            if (tid + 256 < p.vd) acc1 = fmaf(pj, value_hat<PAGED>(p, b, kvh, base + j, tid + 256), acc1);
        }
        m = mnew;
        __syncthreads();
    }
    const int64_t slot = (int64_t(b) * p.Hq + hq) * p.S + s;
    if (tid < p.vd) p.ws_acc[slot * p.vd + tid] = acc0;
    if (tid + 256 < p.vd) p.ws_acc[slot * p.vd + tid + 256] = acc1;
    if (tid == 0) {
        p.ws_ml[slot * 2] = m;
        p.ws_ml[slot * 2 + 1] = l;
    }
}

// Pass 2 (maxima in log2 units): m = max_s m_s, L = sum_s l_s 2^{m_s - m},
// o = sum_s acc_s 2^{m_s - m} / L.  Empty slots (m_s = -inf, l_s = 0, from
// splits past a short paged sequence) weigh 0; a sequence with no tokens
// gets o = 0.
// The paged decode step's length advance, after every pass-1 workgroup has
// read the lengths: sequence b gains the row the step appended to it (the
// validity rule of the kernels' paged_step_len).
struct MergeAdvance {
    int32_t* lens;             // null: nothing to advance
    const int32_t* n_new;      // rows per sequence (0 or 1), null = 1
    int Hq;
    int64_t lim;               // min(capacity, max_len)
};

__global__ __launch_bounds__(256) void k_merge(const float* __restrict__ ws_acc,
                                               const float* __restrict__ ws_ml, int S, int vd,
                                               uint16_t* __restrict__ out, MergeAdvance adv) {
    __shared__ float wsh[KVQ_MAX_SPLITS];
    __shared__ float red[4];
    __shared__ float tot[2];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t pair = blockIdx.x;
    if (adv.lens && tid == 0 && pair % adv.Hq == 0) {
        const int64_t b = pair / adv.Hq;
        const int raw = adv.lens[b];
        const int nn = adv.n_new ? adv.n_new[b] : 1;
        if (raw >= 0 && (nn == 0 || nn == 1) && int64_t(raw) + nn <= adv.lim) adv.lens[b] = raw + nn;
    }
    const float* ml = ws_ml + pair * S * 2;
    const float mi = tid < S ? ml[tid * 2] : -INFINITY;
    const float wm = wave_max(mi);
    if (lane == 0) red[wv] = wm;
    __syncthreads();
    if (tid == 0) tot[0] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    const float M = tot[0];
    const float w = tid < S && mi > -INFINITY ? exp2f(mi - M) : 0.0f;
    if (tid < S) wsh[tid] = w;
    const float lsum = wave_sum(tid < S ? ml[tid * 2 + 1] * w : 0.0f);
    __syncthreads();
    if (lane == 0) red[wv] = lsum;
    __syncthreads();
    if (tid == 0) tot[1] = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    const float inv = tot[1] > 0.0f ? 1.0f / tot[1] : 0.0f;
    const float* acc = ws_acc + pair * S * vd;
    // P threads per channel (P = 256 / vd for vd <= 128) sum interleaved
    // slots s = part, part + P, ..., 8 loads in flight per round; the parts
    // add up in LDS (part order)
    const int P = vd >= 256 ? 1 : 256 / vd;
    const int cw = 256 / P;   // channels per pass
    __shared__ float part_sum[256];
    for (int c0 = 0; c0 < vd; c0 += cw) {
        const int c = c0 + tid % cw, part = tid / cw;
        float o = 0.0f;
        if (c < vd) {
            for (int s0 = part; s0 < S; s0 += 8 * P) {
                float a[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int sl = s0 + e * P;
                    a[e] = sl < S ? acc[int64_t(sl) * vd + c] : 0.0f;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int sl = s0 + e * P;
                    if (sl < S) o = fmaf(a[e], wsh[sl], o);
                }
            }
        }
        if (P > 1) {
            __syncthreads();
            part_sum[tid] = o;
            __syncthreads();
            if (part == 0 && c < vd) {
                for (int q = 1; q < P; ++q) o += part_sum[q * cw + tid];
            }
        }
        if (part == 0 && c < vd) out[pair * vd + c] = __half_as_ushort(__float2half_rn(o * inv));
    }
}

}  // namespace

namespace {
GenParams gen_params(const DecodeArgs& a) {
    const kvq_cache_buffers& buf = a.pc ? a.pc->buf : a.c->buf;
    GenParams p;
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
    p.U = a.U;
    p.T = a.T;
    p.nblk = a.nblk;
    p.cap = a.g.cap;
    p.nblk_cap = a.g.nblk_cap;
    p.kd = a.g.kd;
    p.kG = a.g.kG;
    p.kbits = a.g.kbits;
    p.kW = a.g.kW;
    p.vd = a.g.vd;
    p.vbits = a.g.vbits;
    p.vWT = a.g.vWT;
    p.vNG = a.g.vNG;
    p.sigma2 = a.sigma * 1.4426950408889634f;
    p.table = a.ps.table;
    p.lens = a.ps.lens;
    p.maxb = a.ps.maxb;
    p.npages = a.ps.n_pages;
    p.chunk = a.chunk;
    p.max_len = a.max_len;
    return p;
}
}  // namespace

hipError_t launch_decode_generic(const DecodeArgs& a, hipStream_t st) {
    const GenParams p = gen_params(a);
    const dim3 grid(a.S, a.Hq, a.g.B);
    if (a.c->cfg.kind == KVQ_KIND_MLA)
        hipExtLaunchKernelGGL((k_decode_generic<true, false>), grid, dim3(256), 0, st, a.ev_start, a.ev_stop, 0, p);
    else
        hipExtLaunchKernelGGL((k_decode_generic<false, false>), grid, dim3(256), 0, st, a.ev_start, a.ev_stop, 0, p);
    return hipGetLastError();
}

hipError_t launch_decode_generic_paged(const DecodeArgs& a, hipStream_t st) {
    const GenParams p = gen_params(a);
    const dim3 grid(a.S, a.Hq, a.g.B);
    if (a.pc->cfg.kind == KVQ_KIND_MLA)
        hipExtLaunchKernelGGL((k_decode_generic<true, true>), grid, dim3(256), 0, st, a.ev_start, a.ev_stop, 0, p);
    else
        hipExtLaunchKernelGGL((k_decode_generic<false, true>), grid, dim3(256), 0, st, a.ev_start, a.ev_stop, 0, p);
    return hipGetLastError();
}

hipError_t launch_merge(const DecodeArgs& a, hipStream_t st) {
    MergeAdvance adv;
    adv.lens = a.lens_adv;
    adv.n_new = a.ps.n_new;
    adv.Hq = a.Hq;
    const int64_t cap = int64_t(a.ps.maxb) * a.g.kG;
    adv.lim = cap < a.max_len ? cap : a.max_len;
    hipLaunchKernelGGL(k_merge, dim3(a.g.B * a.Hq), dim3(256), 0, st, a.ws_acc, a.ws_ml, a.S,
                       a.g.vd, static_cast<uint16_t*>(a.out), adv);
    return hipGetLastError();
}

}  // namespace kvq
