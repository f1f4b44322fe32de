// kvq_quant.hip -- quantize / pack kernels of the KIVI-style cache on gfx950.
//
// "Makale Bülteni -- KIVI", section "İddia ve Gerçeklik: KIVI": values are
// quantized per token, keys per channel over blocks of G tokens, both as
// asymmetric 2-bit codes (zero = group minimum, scale = range / 3); the
// unfilled key block stays fp16 in the residual.  "QuantMLA ...", section
// "QuantMLA Mimarisi ve Temel Bileşenleri": the same per-token rule serves the
// INT2 content latent and the per-channel rule the INT4 RoPE key.
//
//
// The value quantizer and the row policies live in kvq_quant_dev.h (shared
// with the decode kernels' fused append).
#include <hip/hip_fp16.h>

#include "kvq_internal.h"
#include "kvq_quant_dev.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

using namespace qdev;

template <int BITS>
__global__ __launch_bounds__(256) void k_quant_values(ValueArgs a, ContigRows rows) {
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= value_threads(a.BH, a.n_tok, a.vd)) return;   // whole 4-lane groups leave together
    quant_values_thread<BITS>(a, rows, idx);
}

// The key quantizer (KeyShape, KeyJob, quant_key_pair) lives in kvq_quant_dev.h.

// Contiguous cache: blocks blk0 .. blk0 + nb - 1 of every (sequence, KV head)
struct KeyArgs {
    const uint16_t* kin;     // [BH][n_in][kd]
    const uint16_t* resid;   // [BH][G][kd]
    int64_t n_in, in_tok0, res_tok0, blk0, nblk_cap;
    int nb, kd, BH;
    uint32_t* codes;
    uint16_t *scale, *zero;
};

// CPT channels per thread: 4 (8-byte loads of each row) where the channel
// quads fill whole waves, else 2.  Measured on MI355X, bulk prefill of the
// 32K and 128K GQA caches (D = 128): +3..8% with 4; the 64-channel MLA RoPE
// key at G = 64 would leave half of each wave idle with 4.
template <int G, int BITS, int CPT>
__global__ __launch_bounds__(256) void k_quant_keys(KeyArgs a) {
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    // whole waves leave together: the per-block count is a multiple of 64 when SPL > 1
    if (idx >= int64_t(a.BH) * a.nb * key_threads_per_block<G, BITS, CPT>(a.kd)) return;
    int64_t unit;
    int cp, sp;
    key_thread_coords<G, BITS, CPT>(idx, a.kd, unit, cp, sp);
    const int64_t blk = a.blk0 + unit % a.nb, bh = unit / a.nb;
    const KeyJob j{a.kin + bh * a.n_in * a.kd, a.resid + bh * G * a.kd, blk * G, a.in_tok0, a.res_tok0,
                   bh * a.nblk_cap + blk};
    quant_key_pair<G, BITS, CPT>(j, a.kd, cp, sp, a.codes, a.scale, a.zero);
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
__global__ __launch_bounds__(256) void k_append_rows(ValueArgs va, ContigRows rows, ResidArgs ka) {
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t nv = value_threads(va.BH, va.n_tok, va.vd);
    if (idx < nv)
        quant_values_thread<BITS>(va, rows, idx);
    else if (idx - nv < resid_threads(ka))
        resid_copy_thread(ka, idx - nv);
}

// ------------------------------------------------------------ paged append
// Pages hold one G-token key block and the values of the same tokens; the
// residual keeps one block per sequence slot.  Sequence b appends rows at
// tokens lens[b] ..; inputs are [BH][n_max][d].

struct PagedKeyArgs {
    const uint16_t* kin;     // [BH][n_max][kd]
    uint16_t* resid;         // [BH][G][kd]
    PagedSeq ps;
    int n_max, kd, Hkv, BH, J;   // J: block slots per sequence that may complete
    uint32_t* codes;
    uint16_t *scale, *zero;
};

// Every block that the append completes, quantized into its page: slot j of
// sequence b is block lens[b] / G + j.  Units (sequence, KV head, slot) map
// to whole waves when SPL > 1, and every exit below is per unit.
template <int G, int BITS>
__global__ __launch_bounds__(256) void k_paged_keys(PagedKeyArgs a) {
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= int64_t(a.BH) * a.J * key_threads_per_block<G, BITS>(a.kd)) return;
    int64_t unit;
    int cp, sp;
    key_thread_coords<G, BITS>(idx, a.kd, unit, cp, sp);
    const int js = int(unit % a.J);
    const int64_t bh = unit / a.J;
    const int b = int(bh / a.Hkv), kvh = int(bh % a.Hkv);
    const int n = seq_rows(a.ps, b, a.n_max, G);
    if (n == 0) return;
    const int64_t pos = a.ps.lens[b];
    const int64_t fb = pos / G, blk = fb + js;
    if ((blk + 1) * G > pos + n) return;   // not completed by this append
    const int64_t dst = paged_block_row(a.ps, b, kvh, a.Hkv, blk);
    if (dst < 0) return;
    const KeyJob j{a.kin + bh * a.n_max * a.kd, a.resid + bh * G * a.kd, blk * G, pos, fb * G, dst};
    quant_key_pair<G, BITS>(j, a.kd, cp, sp, a.codes, a.scale, a.zero);
}

// Value rows into their pages, and the key rows of the block left unfilled
// into the residual (rows t mod G).  Runs after k_paged_keys, which reads
// the residual rows it replaces.  Only the last G input rows of a sequence
// can stay in the residual, so the copy threads cover (sequence, KV head,
// one of those G rows, 8 channels).
template <int BITS>
__global__ __launch_bounds__(256) void k_paged_rows(ValueArgs va, PagedRows rows, const uint16_t* __restrict__ kin,
                                                    uint16_t* __restrict__ resid, int kd) {
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t nv = value_threads(va.BH, va.n_tok, va.vd);
    if (idx < nv) {
        quant_values_thread<BITS>(va, rows, idx);
        return;
    }
    const int vpr = kd / 8;
    const int G = rows.G;
    const int64_t i = idx - nv;
    if (i >= int64_t(va.BH) * G * vpr) return;
    const int v = int(i % vpr);
    const int r = int((i / vpr) % G);
    const int64_t bh = i / vpr / G;
    const int64_t n = rows.count(bh);
    const int64_t tok = n - G + r;   // the last G rows of this sequence's input
    if (tok < 0) return;
    const int64_t pos = rows.ps.lens[bh / rows.Hkv], t = pos + tok;
    if (t < (pos + n) / G * G) return;   // in a block this append completed
    *reinterpret_cast<uint4*>(resid + (bh * G + t % G) * kd + v * 8) =
        *reinterpret_cast<const uint4*>(kin + (bh * va.n_tok + tok) * kd + v * 8);
}

// One row per sequence (the decode step) in one launch: a workgroup per
// (sequence, KV head) quantizes the value row into its page and either puts
// the key into the residual or, when it is the block's last key, quantizes
// the block (G - 1 residual rows and the new key) into its page.
template <int G, int KBITS, int VBITS>
__global__ __launch_bounds__(256) void k_paged_token(ValueArgs va, PagedRows rows, PagedKeyArgs ka) {
    const int64_t bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int b = int(bh / ka.Hkv), kvh = int(bh % ka.Hkv);
    if (seq_rows(ka.ps, b, 1, G) == 0) return;   // the whole workgroup
    const int tpt = va.vd / 8;
    if (tid < tpt) quant_values_thread<VBITS>(va, rows, bh * tpt + tid);   // whole 4-lane groups
    const int64_t pos = ka.ps.lens[b];
    const int kd = ka.kd;
    if (pos % G == G - 1) {
        const int64_t fb = pos / G;
        const int64_t dst = paged_block_row(ka.ps, b, kvh, ka.Hkv, fb);
        if (dst < 0) return;
        const KeyJob j{ka.kin + bh * kd, ka.resid + bh * G * kd, fb * G, pos, fb * G, dst};
        const int64_t nk = key_threads_per_block<G, KBITS>(kd);   // a multiple of 64 when SPL > 1
        for (int64_t base = 0; base < nk; base += 256) {
            const int64_t idx = base + tid;
            if (idx >= nk) break;
            int64_t unit;
            int cp, sp;
            key_thread_coords<G, KBITS>(idx, kd, unit, cp, sp);
            quant_key_pair<G, KBITS>(j, kd, cp, sp, ka.codes, ka.scale, ka.zero);
        }
    } else if (tid < kd / 8) {
        *reinterpret_cast<uint4*>(ka.resid + (bh * G + pos % G) * kd + tid * 8) =
            *reinterpret_cast<const uint4*>(ka.kin + bh * kd + tid * 8);
    }
}

inline unsigned grid_of(int64_t threads) { return unsigned((threads + 255) / 256); }

template <int G, int BITS>
hipError_t launch_keys_t(const kvq_cache& c, const Geom& g, const void* k_in, int64_t n_in,
                         int64_t in_tok0, int64_t res_tok0, int64_t blk0, int64_t nb,
                         hipStream_t st) {
    KeyArgs a;
    a.kin = static_cast<const uint16_t*>(k_in);
    a.resid = static_cast<const uint16_t*>(c.buf.k_resid);
    a.n_in = n_in;
    a.in_tok0 = in_tok0;
    a.res_tok0 = res_tok0;
    a.blk0 = blk0;
    a.nblk_cap = g.nblk_cap;
    a.nb = int(nb);
    a.kd = g.kd;
    a.BH = g.B * g.Hkv;
    a.codes = static_cast<uint32_t*>(c.buf.k_codes);
    a.scale = static_cast<uint16_t*>(c.buf.k_scale);
    a.zero = static_cast<uint16_t*>(c.buf.k_zero);
    using S = KeyShape<G, BITS>;
    if (S::SPL == 1 || (g.kd / 4) % S::CPW == 0) {
        const int64_t threads = int64_t(a.BH) * nb * key_threads_per_block<G, BITS, 4>(g.kd);
        hipLaunchKernelGGL((k_quant_keys<G, BITS, 4>), dim3(grid_of(threads)), dim3(256), 0, st, a);
    } else {
        const int64_t threads = int64_t(a.BH) * nb * key_threads_per_block<G, BITS, 2>(g.kd);
        hipLaunchKernelGGL((k_quant_keys<G, BITS, 2>), dim3(grid_of(threads)), dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace

namespace {
ValueArgs value_args(const kvq_cache_buffers& buf, const Geom& g, const void* v_in, int64_t n_in, int64_t row0,
                     int64_t n_tok) {
    ValueArgs a;
    a.vin = static_cast<const uint16_t*>(v_in);
    a.n_in = n_in;
    a.row0 = row0;
    a.n_tok = n_tok;
    a.vd = g.vd;
    a.BH = g.B * g.Hkv;
    a.codes = static_cast<uint32_t*>(buf.v_codes);
    a.scale = static_cast<uint16_t*>(buf.v_scale);
    a.zero = static_cast<uint16_t*>(buf.v_zero);
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
    const ValueArgs a = value_args(c.buf, g, v_in, n_in, row0, n_tok);
    const ContigRows rows{g.cap, t_dst0, n_tok};
    const unsigned grid = grid_of(value_threads(a.BH, n_tok, a.vd));
    if (g.vbits == 2)
        hipLaunchKernelGGL(k_quant_values<2>, dim3(grid), dim3(256), 0, st, a, rows);
    else
        hipLaunchKernelGGL(k_quant_values<4>, dim3(grid), dim3(256), 0, st, a, rows);
    return hipGetLastError();
}

hipError_t launch_append_rows(const kvq_cache& c, const Geom& g, const void* k_in, const void* v_in,
                              int64_t n, int64_t R, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const ValueArgs va = value_args(c.buf, g, v_in, n, 0, n);
    const ContigRows rows{g.cap, c.T, n};
    const ResidArgs ka = resid_args(c, g, k_in, n, 0, R, n);
    const unsigned grid = grid_of(value_threads(va.BH, n, va.vd) + resid_threads(ka));
    if (g.vbits == 2)
        hipLaunchKernelGGL(k_append_rows<2>, dim3(grid), dim3(256), 0, st, va, rows, ka);
    else
        hipLaunchKernelGGL(k_append_rows<4>, dim3(grid), dim3(256), 0, st, va, rows, ka);
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

namespace {
template <int G, int KB>
hipError_t launch_paged_t(const kvq_paged& c, const Geom& g, const void* k_in, const void* v_in, int n_max,
                          const PagedSeq& ps, hipStream_t st) {
    const ValueArgs va = value_args(c.buf, g, v_in, n_max, 0, n_max);
    const PagedRows rows{ps, g.Hkv, G, n_max};
    PagedKeyArgs ka;
    ka.kin = static_cast<const uint16_t*>(k_in);
    ka.resid = static_cast<uint16_t*>(c.buf.k_resid);
    ka.ps = ps;
    ka.n_max = n_max;
    ka.kd = g.kd;
    ka.Hkv = g.Hkv;
    ka.BH = g.B * g.Hkv;
    // blocks one append can complete: (R + n) / G with R <= G - 1
    ka.J = (n_max + G - 1) / G;
    ka.codes = static_cast<uint32_t*>(c.buf.k_codes);
    ka.scale = static_cast<uint16_t*>(c.buf.k_scale);
    ka.zero = static_cast<uint16_t*>(c.buf.k_zero);
    if (n_max == 1) {
        if (g.vbits == 2)
            hipLaunchKernelGGL((k_paged_token<G, KB, 2>), dim3(ka.BH), dim3(256), 0, st, va, rows, ka);
        else
            hipLaunchKernelGGL((k_paged_token<G, KB, 4>), dim3(ka.BH), dim3(256), 0, st, va, rows, ka);
        return hipGetLastError();
    }
    const int64_t kthreads = int64_t(ka.BH) * ka.J * key_threads_per_block<G, KB>(g.kd);
    hipLaunchKernelGGL((k_paged_keys<G, KB>), dim3(grid_of(kthreads)), dim3(256), 0, st, ka);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rthreads = value_threads(va.BH, n_max, g.vd) + int64_t(va.BH) * G * (g.kd / 8);
    uint16_t* resid = static_cast<uint16_t*>(c.buf.k_resid);
    if (g.vbits == 2)
        hipLaunchKernelGGL(k_paged_rows<2>, dim3(grid_of(rthreads)), dim3(256), 0, st, va, rows, ka.kin, resid, g.kd);
    else
        hipLaunchKernelGGL(k_paged_rows<4>, dim3(grid_of(rthreads)), dim3(256), 0, st, va, rows, ka.kin, resid, g.kd);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_paged_append(const kvq_paged& c, const Geom& g, const void* k_in, const void* v_in, int n_max,
                               const PagedSeq& ps, hipStream_t st) {
    if (n_max <= 0) return hipSuccess;
#define KVQ_PAGED(GG, BB) \
    if (g.kG == GG && g.kbits == BB) return launch_paged_t<GG, BB>(c, g, k_in, v_in, n_max, ps, st);
    KVQ_PAGED(16, 2)
    KVQ_PAGED(32, 2)
    KVQ_PAGED(64, 2)
    KVQ_PAGED(128, 2)
    KVQ_PAGED(16, 4)
    KVQ_PAGED(32, 4)
    KVQ_PAGED(64, 4)
#undef KVQ_PAGED
    return hipErrorInvalidValue;
}

}  // namespace kvq
