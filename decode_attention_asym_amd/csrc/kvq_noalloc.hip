// kvq_noalloc.hip -- kv_decode_attention_noalloc: decode attention whose
// split partials live in a library-owned static device array instead of a
// caller-supplied workspace, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  Same kernels, same split plan, same bits as
// kv_decode_attention.
#include <mutex>

#include "kvq_internal.h"

namespace {

// The partials of one call: [B][Hq][S][vd] accumulators then [B][Hq][S][2]
// (m, l).  Every slot a call's merge reads is written by that call's
// pass-1, so nothing here needs clearing between calls.  Each GPU holds its
// own copy until the process ends.
static __device__ __align__(256) unsigned char scratch[KVQ_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch` per device

// Device address of this device's scratch array, looked up once per device
// with that device current (the host-side name `scratch` is only a handle
// for the lookup, never an address to hand to a kernel).
kvq_status scratch_ptr(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KVQ_E_HIP;
    if (dev >= kMaxDevices) return KVQ_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_E_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return KVQ_OK;
}

}  // namespace

extern "C" kvq_status kv_decode_attention_noalloc(const kvq_cache* c, const void* q, int32_t Hq, float sigma,
                                                  int32_t n_splits, void* out, void* stream) {
    // the checks kv_decode_attention makes, plus the scratch limit, before
    // any HIP call
    if (!c || !q || !out) return KVQ_E_NULL;
    if (Hq < 1 || Hq % c->cfg.n_kv_heads != 0) return KVQ_E_SHAPE;
    if (n_splits < 0 || n_splits > KVQ_MAX_SPLITS) return KVQ_E_SHAPE;
    if ((reinterpret_cast<uintptr_t>(q) & 15u) || (reinterpret_cast<uintptr_t>(out) & 15u)) return KVQ_E_ALIGN;
    if (c->T <= 0) return KVQ_E_STATE;
    uint64_t need = 0;
    const kvq_status st = kvq::decode_workspace_now(*c, Hq, n_splits, &need);
    if (st != KVQ_OK) return st;
    if (need > KVQ_SCRATCH_BYTES) return KVQ_E_SCRATCH;
    void* ws = nullptr;
    const kvq_status sp = scratch_ptr(&ws);
    if (sp != KVQ_OK) return sp;
    return kv_decode_attention(c, q, Hq, sigma, n_splits, out, ws, KVQ_SCRATCH_BYTES, stream);
}
