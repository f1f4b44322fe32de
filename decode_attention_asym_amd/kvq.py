"""ctypes binding of libkvq.so (C ABI in include/kvq.h).

Functions keep the C names and only marshal arguments; every step of the path
runs in the library's HIP kernels.  ``DeviceCache`` is a convenience holder
that allocates the caller-owned device arrays with PyTorch (device memory and
streams are all PyTorch is used for).  Loading fails loudly when the library
has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIB selects another build of the library (e.g. an instrumented one)
LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(HERE, "libkvq.so")

KVQ_KIND_KIVI, KVQ_KIND_MLA = 0, 1
KVQ_AXIS_PER_CHANNEL, KVQ_AXIS_PER_TOKEN = 0, 1
KVQ_APPEND_NO_AUTOFLUSH = 1
KVQ_STEP_ADVANCE_LENGTHS = 1
KVQ_PREFILL_ATTENTION_ONLY = 1
KVQ_MAX_SPLITS = 256
KVQ_SCRATCH_BYTES = 32 << 20
STATUS = {0: "KVQ_OK", -1: "KVQ_E_NULL", -2: "KVQ_E_SHAPE", -3: "KVQ_E_ALIGN",
          -4: "KVQ_E_CAPACITY", -5: "KVQ_E_UNSUPPORTED", -6: "KVQ_E_WORKSPACE",
          -7: "KVQ_E_HIP", -8: "KVQ_E_STATE", -9: "KVQ_E_SCRATCH"}
EXPORTS = ["kv_cache_buffer_bytes", "kv_cache_init", "kv_cache_destroy", "kv_cache_reset",
           "kv_cache_state", "kv_quantize_append", "kv_flush_residual",
           "kv_decode_workspace_bytes", "kv_decode_attention", "kv_set_timing_events",
           "kv_decode_variant", "kvq_status_str",
           "kv_paged_buffer_bytes", "kv_paged_init", "kv_paged_destroy", "kv_paged_append",
           "kv_paged_workspace_bytes", "kv_paged_decode", "kv_paged_variant", "kv_decode_step",
           "kv_paged_decode_step", "kv_prefill_attention", "kv_decode_attention_noalloc"]


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({kvq_status_str(status)})")


class StreamCfg(C.Structure):
    _fields_ = [("bits", C.c_int32), ("axis", C.c_int32), ("dim", C.c_int32), ("group", C.c_int32)]


class CacheCfg(C.Structure):
    _fields_ = [("kind", C.c_int32), ("batch", C.c_int32), ("n_kv_heads", C.c_int32),
                ("reserved", C.c_int32), ("max_tokens", C.c_int64),
                ("key", StreamCfg), ("value", StreamCfg)]


BUFFER_NAMES = ["k_codes", "k_scale", "k_zero", "k_resid", "v_codes", "v_scale", "v_zero"]


class BufferSizes(C.Structure):
    _fields_ = [(n, C.c_uint64) for n in BUFFER_NAMES]


class CacheBuffers(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in BUFFER_NAMES]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(there is no fallback implementation)")
        L = C.CDLL(LIB_PATH)
        p, i32, i64, u32, u64 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32, C.c_uint64
        sig = {
            "kv_cache_buffer_bytes": (C.c_int, [C.POINTER(CacheCfg), C.POINTER(BufferSizes)]),
            "kv_cache_init": (C.c_int, [C.POINTER(CacheCfg), C.POINTER(CacheBuffers), C.POINTER(p)]),
            "kv_cache_destroy": (None, [p]),
            "kv_cache_reset": (C.c_int, [p]),
            "kv_cache_state": (C.c_int, [p, C.POINTER(i64), C.POINTER(i32)]),
            "kv_quantize_append": (C.c_int, [p, p, p, i64, u32, p]),
            "kv_flush_residual": (C.c_int, [p, p, C.POINTER(i32)]),
            "kv_decode_workspace_bytes": (C.c_int, [p, i32, i32, C.POINTER(u64)]),
            "kv_decode_attention": (C.c_int, [p, p, i32, C.c_float, i32, p, p, u64, p]),
            "kv_set_timing_events": (C.c_int, [p, p]),
            "kv_decode_variant": (C.c_char_p, [p, i32]),
            "kvq_status_str": (C.c_char_p, [C.c_int]),
            "kv_paged_buffer_bytes": (C.c_int, [C.POINTER(CacheCfg), i32, C.POINTER(BufferSizes)]),
            "kv_paged_init": (C.c_int, [C.POINTER(CacheCfg), i32, C.POINTER(CacheBuffers), C.POINTER(p)]),
            "kv_paged_destroy": (None, [p]),
            "kv_paged_append": (C.c_int, [p, p, p, i32, p, p, p, p]),
            "kv_paged_workspace_bytes": (C.c_int, [p, i32, i32, i32, C.POINTER(u64)]),
            "kv_paged_decode": (C.c_int, [p, p, i32, C.c_float, p, p, i32, i32, p, p, u64, p]),
            "kv_paged_variant": (C.c_char_p, [p, i32, i32]),
            "kv_decode_step": (C.c_int, [p, p, p, p, i32, C.c_float, i32, p, p, u64, p]),
            "kv_decode_attention_noalloc": (C.c_int, [p, p, i32, C.c_float, i32, p, p]),
            "kv_paged_decode_step": (C.c_int, [p, p, p, p, i32, C.c_float, p, p, p, i32, i32, u32, p, p, u64, p]),
            "kv_prefill_attention": (C.c_int, [p, p, p, p, i64, i32, C.c_float, u32, p, p]),
        }
        for name, (res, args) in sig.items():
            try:
                f = getattr(L, name)
            except AttributeError:
                # only an override build (KVQ_LIB, e.g. an older revision)
                # may lack an entry point; calling it then fails
                if not os.environ.get("KVQ_LIB"):
                    raise
                continue
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        raise KvqError(status, what)


# ------------------------------------------------------------- C entry points

def kvq_status_str(status: int) -> str:
    return lib().kvq_status_str(status).decode()


def kv_cache_buffer_bytes(cfg: CacheCfg) -> BufferSizes:
    out = BufferSizes()
    _check(lib().kv_cache_buffer_bytes(C.byref(cfg), C.byref(out)), "kv_cache_buffer_bytes")
    return out


def kv_cache_init(cfg: CacheCfg, bufs: CacheBuffers) -> int:
    h = C.c_void_p()
    _check(lib().kv_cache_init(C.byref(cfg), C.byref(bufs), C.byref(h)), "kv_cache_init")
    return h.value


def kv_cache_destroy(handle) -> None:
    lib().kv_cache_destroy(handle)


def kv_cache_reset(handle) -> None:
    _check(lib().kv_cache_reset(handle), "kv_cache_reset")


def kv_cache_state(handle):
    t, r = C.c_int64(), C.c_int32()
    _check(lib().kv_cache_state(handle, C.byref(t), C.byref(r)), "kv_cache_state")
    return t.value, r.value


def kv_quantize_append(handle, k_ptr, v_ptr, n_tokens: int, flags: int = 0, stream=None) -> None:
    _check(lib().kv_quantize_append(handle, k_ptr, v_ptr, n_tokens, flags, stream),
           "kv_quantize_append")


def kv_flush_residual(handle, stream=None) -> int:
    n = C.c_int32()
    _check(lib().kv_flush_residual(handle, stream, C.byref(n)), "kv_flush_residual")
    return n.value


def kv_decode_workspace_bytes(handle, n_q_heads: int, n_splits: int = 0) -> int:
    b = C.c_uint64()
    _check(lib().kv_decode_workspace_bytes(handle, n_q_heads, n_splits, C.byref(b)),
           "kv_decode_workspace_bytes")
    return b.value


def kv_decode_attention(handle, q_ptr, n_q_heads: int, softmax_scale: float, n_splits: int,
                        out_ptr, ws_ptr, ws_bytes: int, stream=None) -> None:
    _check(lib().kv_decode_attention(handle, q_ptr, n_q_heads, C.c_float(softmax_scale), n_splits,
                                     out_ptr, ws_ptr, ws_bytes, stream), "kv_decode_attention")


def kv_decode_attention_noalloc(handle, q_ptr, n_q_heads: int, softmax_scale: float, n_splits: int, out_ptr,
                                stream=None) -> None:
    _check(lib().kv_decode_attention_noalloc(handle, q_ptr, n_q_heads, C.c_float(softmax_scale), n_splits, out_ptr,
                                             stream), "kv_decode_attention_noalloc")


def kv_decode_step(handle, k_ptr, v_ptr, q_ptr, n_q_heads: int, softmax_scale: float, n_splits: int,
                   out_ptr, ws_ptr, ws_bytes: int, stream=None) -> None:
    _check(lib().kv_decode_step(handle, k_ptr, v_ptr, q_ptr, n_q_heads, C.c_float(softmax_scale), n_splits,
                                out_ptr, ws_ptr, ws_bytes, stream), "kv_decode_step")


def kv_prefill_attention(handle, q_ptr, k_ptr, v_ptr, n: int, n_q_heads: int, softmax_scale: float, flags: int,
                         out_ptr, stream=None) -> None:
    _check(lib().kv_prefill_attention(handle, q_ptr, k_ptr, v_ptr, n, n_q_heads, C.c_float(softmax_scale), flags,
                                      out_ptr, stream), "kv_prefill_attention")


def kv_set_timing_events(ev_before, ev_after) -> None:
    _check(lib().kv_set_timing_events(ev_before, ev_after), "kv_set_timing_events")


def kv_decode_variant(handle, n_q_heads: int) -> str:
    return lib().kv_decode_variant(handle, n_q_heads).decode()


def kv_paged_buffer_bytes(cfg: CacheCfg, n_pages: int) -> BufferSizes:
    out = BufferSizes()
    _check(lib().kv_paged_buffer_bytes(C.byref(cfg), n_pages, C.byref(out)), "kv_paged_buffer_bytes")
    return out


def kv_paged_init(cfg: CacheCfg, n_pages: int, bufs: CacheBuffers) -> int:
    h = C.c_void_p()
    _check(lib().kv_paged_init(C.byref(cfg), n_pages, C.byref(bufs), C.byref(h)), "kv_paged_init")
    return h.value


def kv_paged_destroy(handle) -> None:
    lib().kv_paged_destroy(handle)


def kv_paged_append(handle, k_ptr, v_ptr, n_max: int, n_new_ptr, seq_lens_ptr, table_ptr, stream=None) -> None:
    _check(lib().kv_paged_append(handle, k_ptr, v_ptr, n_max, n_new_ptr, seq_lens_ptr, table_ptr, stream),
           "kv_paged_append")


def kv_paged_workspace_bytes(handle, n_q_heads: int, max_len: int, n_splits: int = 0) -> int:
    b = C.c_uint64()
    _check(lib().kv_paged_workspace_bytes(handle, n_q_heads, max_len, n_splits, C.byref(b)),
           "kv_paged_workspace_bytes")
    return b.value


def kv_paged_decode(handle, q_ptr, n_q_heads: int, softmax_scale: float, seq_lens_ptr, table_ptr,
                    max_len: int, n_splits: int, out_ptr, ws_ptr, ws_bytes: int, stream=None) -> None:
    _check(lib().kv_paged_decode(handle, q_ptr, n_q_heads, C.c_float(softmax_scale), seq_lens_ptr, table_ptr,
                                 max_len, n_splits, out_ptr, ws_ptr, ws_bytes, stream), "kv_paged_decode")


def kv_paged_decode_step(handle, k_ptr, v_ptr, q_ptr, n_q_heads: int, softmax_scale: float, n_new_ptr,
                         seq_lens_ptr, table_ptr, max_len: int, n_splits: int, flags: int, out_ptr, ws_ptr,
                         ws_bytes: int, stream=None) -> None:
    _check(lib().kv_paged_decode_step(handle, k_ptr, v_ptr, q_ptr, n_q_heads, C.c_float(softmax_scale), n_new_ptr,
                                      seq_lens_ptr, table_ptr, max_len, n_splits, flags, out_ptr, ws_ptr, ws_bytes,
                                      stream), "kv_paged_decode_step")


def kv_paged_variant(handle, n_q_heads: int, max_len: int) -> str:
    return lib().kv_paged_variant(handle, n_q_heads, max_len).decode()


# ------------------------------------------------------------- config helpers

def cache_cfg(kind, batch, n_kv_heads, max_tokens, kd, kG, kbits, vd, vG=32, vbits=2) -> CacheCfg:
    return CacheCfg(kind, batch, n_kv_heads, 0, max_tokens,
                    StreamCfg(kbits, KVQ_AXIS_PER_CHANNEL, kd, kG),
                    StreamCfg(vbits, KVQ_AXIS_PER_TOKEN, vd, vG))


def cfg_for(w, max_tokens: int) -> CacheCfg:
    """CacheCfg of a configs.Workload."""
    kind = KVQ_KIND_KIVI if w.kind == "kivi" else KVQ_KIND_MLA
    return cache_cfg(kind, w.batch, w.n_kv_heads, max_tokens, w.kd, w.kG, w.kbits, w.vd, w.vG, w.vbits)


class DeviceCache:
    """Caller-owned device arrays (allocated with torch) plus a kvq_cache handle."""

    def __init__(self, cfg: CacheCfg, device="cuda"):
        import torch

        self.torch = torch
        self.cfg = cfg
        self.device = torch.device(device)
        sizes = kv_cache_buffer_bytes(cfg)
        self.arrays = {}
        for n in BUFFER_NAMES:
            nbytes = max(16, int(getattr(sizes, n)))
            self.arrays[n] = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.bufs = CacheBuffers(*[self.arrays[n].data_ptr() for n in BUFFER_NAMES])
        self.handle = kv_cache_init(cfg, self.bufs)
        self.sizes = sizes

    def close(self):
        if self.handle:
            kv_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def stream(self):
        return self.torch.cuda.current_stream(self.device).cuda_stream

    def append(self, k, v, flags: int = 0):
        n = k.shape[-2]
        kv_quantize_append(self.handle, k.data_ptr(), v.data_ptr(), n, flags, self.stream())

    def flush(self) -> int:
        return kv_flush_residual(self.handle, self.stream())

    def state(self):
        return kv_cache_state(self.handle)

    def workspace(self, n_q_heads: int, n_splits: int = 0):
        nbytes = kv_decode_workspace_bytes(self.handle, n_q_heads, n_splits)
        return self.torch.empty(max(16, nbytes), dtype=self.torch.uint8, device=self.device)

    def decode(self, q, softmax_scale: float, n_splits: int = 0, out=None, ws=None):
        torch = self.torch
        B, Hq = q.shape[0], q.shape[1]
        vd = self.cfg.value.dim
        if out is None:
            out = torch.empty((B, Hq, vd), dtype=torch.float16, device=self.device)
        if ws is None:
            ws = self.workspace(Hq, n_splits)
        kv_decode_attention(self.handle, q.data_ptr(), Hq, softmax_scale, n_splits,
                            out.data_ptr(), ws.data_ptr(), ws.numel(), self.stream())
        return out

    def decode_noalloc(self, q, softmax_scale: float, n_splits: int = 0, out=None):
        """kv_decode_attention_noalloc: partials in the library's static scratch."""
        torch = self.torch
        B, Hq = q.shape[0], q.shape[1]
        if out is None:
            out = torch.empty((B, Hq, self.cfg.value.dim), dtype=torch.float16, device=self.device)
        kv_decode_attention_noalloc(self.handle, q.data_ptr(), Hq, softmax_scale, n_splits, out.data_ptr(),
                                    self.stream())
        return out

    def variant(self, n_q_heads: int) -> str:
        return kv_decode_variant(self.handle, n_q_heads)

    def prefill(self, q, k, v, softmax_scale: float, flags: int = 0, out=None):
        """Causal attention of the prompt (q [B][Hq][n][d], k / v [B][Hkv][n][d]) and,
        unless KVQ_PREFILL_ATTENTION_ONLY, its append to this empty cache
        (kv_prefill_attention).  Returns out [B][Hq][n][d]."""
        if out is None:
            out = self.torch.empty(q.shape, dtype=self.torch.float16, device=self.device)
        kv_prefill_attention(self.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), q.shape[2], q.shape[1],
                             softmax_scale, flags, out.data_ptr(), self.stream())
        return out

    def step(self, k, v, q, softmax_scale: float, n_splits: int = 0, out=None, ws=None):
        """Append one token per sequence (k, v: [B][Hkv][1][d]) and attend (kv_decode_step)."""
        torch = self.torch
        B, Hq = q.shape[0], q.shape[1]
        if out is None:
            out = torch.empty((B, Hq, self.cfg.value.dim), dtype=torch.float16, device=self.device)
        if ws is None:
            ws = self.workspace(Hq, n_splits)
        kv_decode_step(self.handle, k.data_ptr(), v.data_ptr(), q.data_ptr(), Hq, softmax_scale, n_splits,
                       out.data_ptr(), ws.data_ptr(), ws.numel(), self.stream())
        return out

    # typed views of the device arrays in the documented layouts
    def views(self):
        torch = self.torch
        c = self.cfg
        B, H, cap = c.batch, c.n_kv_heads, c.max_tokens
        kd, G, kb, vd, vG, vb = c.key.dim, c.key.group, c.key.bits, c.value.dim, c.value.group, c.value.bits
        nb = cap // G
        a = self.arrays

        def v(name, dtype, shape):
            n = 1
            for s in shape:
                n *= s
            return a[name].view(dtype)[:n].view(*shape)

        return {
            "k_codes": v("k_codes", torch.int32, (B, H, nb, kd, G * kb // 32)),
            "k_scale": v("k_scale", torch.int16, (B, H, nb, kd)),
            "k_zero": v("k_zero", torch.int16, (B, H, nb, kd)),
            "k_resid": v("k_resid", torch.int16, (B, H, G, kd)),
            "v_codes": v("v_codes", torch.int32, (B, H, cap, vd * vb // 32)),
            "v_scale": v("v_scale", torch.int16, (B, H, cap, vd // vG)),
            "v_zero": v("v_zero", torch.int16, (B, H, cap, vd // vG)),
        }


class PagedCache:
    """Caller-owned page pools and residual (allocated with torch) plus a
    kvq_paged handle.  Block tables and lengths are the caller's int32 device
    tensors, passed to each call."""

    def __init__(self, cfg: CacheCfg, n_pages: int, device="cuda"):
        import torch

        self.torch = torch
        self.cfg = cfg
        self.n_pages = n_pages
        self.device = torch.device(device)
        sizes = kv_paged_buffer_bytes(cfg, n_pages)
        self.arrays = {}
        for n in BUFFER_NAMES:
            nbytes = max(16, int(getattr(sizes, n)))
            self.arrays[n] = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.bufs = CacheBuffers(*[self.arrays[n].data_ptr() for n in BUFFER_NAMES])
        self.handle = kv_paged_init(cfg, n_pages, self.bufs)
        self.sizes = sizes

    def close(self):
        if self.handle:
            kv_paged_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def stream(self):
        return self.torch.cuda.current_stream(self.device).cuda_stream

    def append(self, k, v, seq_lens, block_table, n_new=None):
        """k, v: [B][Hkv][n_max][d] fp16; seq_lens, block_table, n_new: int32 device tensors."""
        n_max = k.shape[-2]
        kv_paged_append(self.handle, k.data_ptr(), v.data_ptr(), n_max,
                        None if n_new is None else n_new.data_ptr(), seq_lens.data_ptr(),
                        block_table.data_ptr(), self.stream())

    def workspace(self, n_q_heads: int, max_len: int, n_splits: int = 0):
        nbytes = kv_paged_workspace_bytes(self.handle, n_q_heads, max_len, n_splits)
        return self.torch.empty(max(16, nbytes), dtype=self.torch.uint8, device=self.device)

    def decode(self, q, softmax_scale: float, seq_lens, block_table, max_len: int, n_splits: int = 0,
               out=None, ws=None):
        torch = self.torch
        B, Hq = q.shape[0], q.shape[1]
        if out is None:
            out = torch.empty((B, Hq, self.cfg.value.dim), dtype=torch.float16, device=self.device)
        if ws is None:
            ws = self.workspace(Hq, max_len, n_splits)
        kv_paged_decode(self.handle, q.data_ptr(), Hq, softmax_scale, seq_lens.data_ptr(),
                        block_table.data_ptr(), max_len, n_splits, out.data_ptr(), ws.data_ptr(),
                        ws.numel(), self.stream())
        return out

    def variant(self, n_q_heads: int, max_len: int) -> str:
        return kv_paged_variant(self.handle, n_q_heads, max_len)

    def step(self, k, v, q, softmax_scale: float, seq_lens, block_table, max_len: int, n_new=None,
             advance: bool = True, n_splits: int = 0, out=None, ws=None):
        """One paged decode step (kv_paged_decode_step): k, v [B][Hkv][1][d]."""
        torch = self.torch
        B, Hq = q.shape[0], q.shape[1]
        if out is None:
            out = torch.empty((B, Hq, self.cfg.value.dim), dtype=torch.float16, device=self.device)
        if ws is None:
            ws = self.workspace(Hq, max_len, n_splits)
        kv_paged_decode_step(self.handle, k.data_ptr(), v.data_ptr(), q.data_ptr(), Hq, softmax_scale,
                             None if n_new is None else n_new.data_ptr(), seq_lens.data_ptr(),
                             block_table.data_ptr(), max_len, n_splits,
                             KVQ_STEP_ADVANCE_LENGTHS if advance else 0, out.data_ptr(), ws.data_ptr(),
                             ws.numel(), self.stream())
        return out

    def views(self):
        """Typed views of the page pools and the residual in the documented layouts."""
        torch = self.torch
        c = self.cfg
        B, H, P = c.batch, c.n_kv_heads, self.n_pages
        kd, G, kb, vd, vG, vb = c.key.dim, c.key.group, c.key.bits, c.value.dim, c.value.group, c.value.bits
        a = self.arrays

        def v(name, dtype, shape):
            n = 1
            for s in shape:
                n *= s
            return a[name].view(dtype)[:n].view(*shape)

        return {
            "k_codes": v("k_codes", torch.int32, (P, H, kd, G * kb // 32)),
            "k_scale": v("k_scale", torch.int16, (P, H, kd)),
            "k_zero": v("k_zero", torch.int16, (P, H, kd)),
            "k_resid": v("k_resid", torch.int16, (B, H, G, kd)),
            "v_codes": v("v_codes", torch.int32, (P, H, G, vd * vb // 32)),
            "v_scale": v("v_scale", torch.int16, (P, H, G, vd // vG)),
            "v_zero": v("v_zero", torch.int16, (P, H, G, vd // vG)),
        }
