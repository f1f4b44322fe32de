"""CPU oracle for KIVI-style asymmetric low-bit KV-cache quantization and
decode attention (plain C in ``kvq_oracle.c``, loaded with ctypes).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``decode_attention_asym_amd``) never imports it and shares no code with it.

Each wrapper below takes and returns numpy arrays; fp16 data travels as its
raw binary16 bit pattern (``numpy.uint16``) so that nothing here rounds.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
# KVQ_ORACLE_LIB selects another build (the sanitizer build below)
_LIB = os.environ.get("KVQ_ORACLE_LIB") or os.path.join(_HERE, "libkvq_oracle.so")
_CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-pthread"]
SAN_LIB = os.path.join(_HERE, "libkvq_oracle_san.so")


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    lib_path = os.path.join(_HERE, "libkvq_oracle.so")
    tmp = lib_path + ".tmp"
    cmd = ["gcc", *_CFLAGS, _SRC, "-lm", "-o", tmp]
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(tmp, lib_path)
    return lib_path


def build_sanitized(clang: str) -> str:
    """The oracle under AddressSanitizer and UndefinedBehaviorSanitizer, built
    with `clang` (the one whose ASan runtime gets preloaded)."""
    tmp = SAN_LIB + ".tmp"
    cmd = [clang, *[f for f in _CFLAGS if f != "-O2"], "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan", _SRC, "-lm", "-o", tmp]
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


_lib = None


class OrcCache(C.Structure):
    _fields_ = [("B", C.c_int64), ("H", C.c_int64), ("T", C.c_int64),
                ("kq_blocks", C.c_int64), ("nblk_cap", C.c_int64), ("tok_cap", C.c_int64),
                ("kd", C.c_int32), ("kG", C.c_int32), ("kbits", C.c_int32),
                ("vd", C.c_int32), ("vG", C.c_int32), ("vbits", C.c_int32),
                ("k_codes", C.c_void_p), ("k_scale", C.c_void_p),
                ("k_zero", C.c_void_p), ("k_resid", C.c_void_p),
                ("v_codes", C.c_void_p), ("v_scale", C.c_void_p),
                ("v_zero", C.c_void_p)]


def default_threads() -> int:
    """Worker threads for the oracle: the CPUs this process may run on, at
    most 16 (a GPU host's share per GPU, whatever the machine's count)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def lib():
    """Load the oracle library.  It is compiled by build() only (never here:
    a process that has initialised a GPU must not start a compiler)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} is not built; run __graft_entry__.build() or oracle.build()")
        L = C.CDLL(_LIB)
        p, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
        L.orc_half_to_float.restype = C.c_float
        L.orc_half_to_float.argtypes = [C.c_uint16]
        L.orc_float_to_half.restype = C.c_uint16
        L.orc_float_to_half.argtypes = [C.c_float]
        L.orc_half_to_float_n.argtypes = [p, p, i64]
        L.orc_float_to_half_n.argtypes = [p, p, i64]
        L.orc_quant_group.restype = C.c_int
        L.orc_quant_group.argtypes = [p, i64, i64, C.c_int, p, p, p, p]
        L.orc_pack.argtypes = [p, i64, C.c_int, p]
        L.orc_unpack.argtypes = [p, i64, C.c_int, p]
        L.orc_quantize_keys.restype = i64
        L.orc_quantize_keys.argtypes = [p, i64, i64, i64, i64, C.c_int, C.c_int, i64, p, p, p, p]
        L.orc_quantize_values.restype = C.c_int
        L.orc_quantize_values.argtypes = [p, i64, i64, i64, i64, C.c_int, C.c_int, i64, p, p, p]
        for f in (L.orc_dequant_keys, L.orc_dequant_values):
            f.restype = C.c_int
            f.argtypes = [C.POINTER(OrcCache), i64, i64, p]
        for f in (L.orc_attention_kivi, L.orc_attention_mla):
            f.restype = C.c_int
            f.argtypes = [C.POINTER(OrcCache), p, i32, C.c_float, p, i64, p, C.c_int]
        L.orc_prefill_attention.restype = C.c_int
        L.orc_prefill_attention.argtypes = [p, p, p, i64, i64, i64, i64, i32, i32, C.c_double, p, i64, p, C.c_int]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


# ----------------------------------------------------------------- fp16

def half_to_float(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_half_to_float_n(_ptr(h), _ptr(out), h.size)
    return out


def float_to_half(f) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().orc_float_to_half_n(_ptr(f), _ptr(out), f.size)
    return out


# ------------------------------------------------------------- quantizer

def quant_group(x_bits, bits: int):
    """One group -> (codes uint8[n], scale_h, zero_h, scale32)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16).ravel()
    codes = np.empty(x.size, np.uint8)
    s = C.c_uint16()
    z = C.c_uint16()
    s32 = C.c_float()
    rc = lib().orc_quant_group(_ptr(x), x.size, 1, bits, _ptr(codes),
                               C.byref(s), C.byref(z), C.byref(s32))
    if rc != 0:
        raise ValueError("oracle quant_group rejected its input")
    return codes, int(s.value), int(z.value), float(s32.value)


def pack(codes, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8).ravel()
    per = 32 // bits
    assert codes.size % per == 0
    words = np.empty(codes.size // per, np.uint32)
    lib().orc_pack(_ptr(codes), codes.size, bits, _ptr(words))
    return words


def unpack(words, n: int, bits: int) -> np.ndarray:
    words = np.ascontiguousarray(words, dtype=np.uint32).ravel()
    codes = np.empty(n, np.uint8)
    lib().orc_unpack(_ptr(words), n, bits, _ptr(codes))
    return codes


def _per_sequence(fn, B: int, threads: int | None) -> None:
    """Run fn(b) for every sequence b, on up to `threads` threads (the C
    calls release the GIL; each writes a disjoint slice)."""
    threads = default_threads() if threads is None else max(1, threads)
    if threads == 1 or B == 1:
        for b in range(B):
            fn(b)
        return
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(max_workers=min(threads, B)) as ex:
        list(ex.map(fn, range(B)))


def quantize_keys(k_bits, G: int, bits: int, nblk_cap: int | None = None, threads: int | None = 1):
    """k_bits: uint16 [B][H][T][D] -> dict(k_codes, k_scale, k_zero, k_resid, R).
    threads > 1 (None = default_threads()) quantizes the sequences in
    parallel, one oracle call each; the result is the same."""
    k = np.ascontiguousarray(k_bits, dtype=np.uint16)
    B, H, T, D = k.shape
    if nblk_cap is None:
        nblk_cap = max(1, T // G)
    W = G * bits // 32
    codes = np.zeros((B, H, nblk_cap, D, W), np.uint32)
    scale = np.zeros((B, H, nblk_cap, D), np.uint16)
    zero = np.zeros((B, H, nblk_cap, D), np.uint16)
    resid = np.zeros((B, H, G, D), np.uint16)
    rs = [0] * B

    def one(b):
        rs[b] = lib().orc_quantize_keys(_ptr(k[b]), 1, H, T, D, G, bits, nblk_cap, _ptr(codes[b]), _ptr(scale[b]),
                                        _ptr(zero[b]), _ptr(resid[b]))

    _per_sequence(one, B, threads)
    if min(rs) < 0:
        raise ValueError("oracle quantize_keys rejected its input")
    return dict(k_codes=codes, k_scale=scale, k_zero=zero, k_resid=resid, R=int(rs[0]))


def quantize_values(v_bits, Gv: int, bits: int, tok_cap: int | None = None, threads: int | None = 1):
    """v_bits: uint16 [B][H][T][D] -> dict(v_codes, v_scale, v_zero); threads
    as for quantize_keys."""
    v = np.ascontiguousarray(v_bits, dtype=np.uint16)
    B, H, T, D = v.shape
    if tok_cap is None:
        tok_cap = max(1, T)
    codes = np.zeros((B, H, tok_cap, D * bits // 32), np.uint32)
    scale = np.zeros((B, H, tok_cap, D // Gv), np.uint16)
    zero = np.zeros((B, H, tok_cap, D // Gv), np.uint16)
    rcs = [0] * B

    def one(b):
        rcs[b] = lib().orc_quantize_values(_ptr(v[b]), 1, H, T, D, Gv, bits, tok_cap, _ptr(codes[b]), _ptr(scale[b]),
                                           _ptr(zero[b]))

    _per_sequence(one, B, threads)
    if min(rcs) != 0:
        raise ValueError("oracle quantize_values rejected its input")
    return dict(v_codes=codes, v_scale=scale, v_zero=zero)


class Cache:
    """A quantized cache held in numpy arrays, in the oracle's layouts."""

    def __init__(self, T, kG, kbits, vG, vbits, keys: dict, values: dict, kq_blocks: int = -1):
        self.k = keys
        self.v = values
        B, H, nblk_cap, kd, _ = keys["k_codes"].shape
        _, _, tok_cap, _ = values["v_codes"].shape
        vd = values["v_scale"].shape[3] * vG
        self.s = OrcCache(B, H, T, kq_blocks, nblk_cap, tok_cap, kd, kG, kbits, vd, vG, vbits,
                          _ptr(keys["k_codes"]).value, _ptr(keys["k_scale"]).value,
                          _ptr(keys["k_zero"]).value, _ptr(keys["k_resid"]).value,
                          _ptr(values["v_codes"]).value, _ptr(values["v_scale"]).value,
                          _ptr(values["v_zero"]).value)

    @property
    def dims(self):
        return self.s.B, self.s.H, self.s.T, self.s.kd, self.s.vd


def build_cache(k_bits, v_bits, kG, kbits, vG, vbits, nblk_cap=None, tok_cap=None,
                kq_blocks: int | None = None, threads: int | None = 1) -> Cache:
    """Oracle cache of T tokens.  kq_blocks (default floor(T/kG)) quantized
    key blocks; the remaining T - kq_blocks*kG (<= kG) keys stay fp16.
    threads: as for quantize_keys."""
    T = k_bits.shape[2]
    assert v_bits.shape[2] == T
    if kq_blocks is None:
        keys = quantize_keys(k_bits, kG, kbits, nblk_cap, threads=threads)
        kq = -1
    else:
        Tq = kq_blocks * kG
        assert 0 <= T - Tq <= kG
        keys = quantize_keys(np.ascontiguousarray(k_bits[:, :, :Tq]), kG, kbits,
                             nblk_cap if nblk_cap is not None else max(1, kq_blocks), threads=threads)
        keys["k_resid"][:, :, :T - Tq] = k_bits[:, :, Tq:]
        keys["R"] = T - Tq
        kq = kq_blocks
    values = quantize_values(v_bits, vG, vbits, tok_cap, threads=threads)
    return Cache(T, kG, kbits, vG, vbits, keys, values, kq)


def dequant_keys(cache: Cache, b: int, h: int) -> np.ndarray:
    out = np.empty((cache.s.T, cache.s.kd), np.float64)
    if lib().orc_dequant_keys(C.byref(cache.s), b, h, _ptr(out)) != 0:
        raise ValueError("bad cache")
    return out


def dequant_values(cache: Cache, b: int, h: int) -> np.ndarray:
    out = np.empty((cache.s.T, cache.s.vd), np.float64)
    if lib().orc_dequant_values(C.byref(cache.s), b, h, _ptr(out)) != 0:
        raise ValueError("bad cache")
    return out


def _attention(fn, cache: Cache, q_bits, sigma, pairs, nthreads):
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    Hq = q.shape[1]
    if pairs is None:
        out = np.empty((cache.s.B, Hq, cache.s.vd), np.float64)
        pp, n = None, 0
    else:
        pa = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
        out = np.empty((pa.shape[0], cache.s.vd), np.float64)
        pp, n = _ptr(pa), pa.shape[0]
    if nthreads is None:
        nthreads = default_threads()
    rc = fn(C.byref(cache.s), _ptr(q), Hq, C.c_float(sigma), pp, n, _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle attention rejected its input")
    return out


def attention_kivi(cache: Cache, q_bits, sigma: float, pairs=None, nthreads=None):
    """q_bits: uint16 [B][Hq][D] -> fp64 [B][Hq][D] (or [npairs][D])."""
    return _attention(lib().orc_attention_kivi, cache, q_bits, sigma, pairs, nthreads)


def attention_mla(cache: Cache, q_bits, sigma: float, pairs=None, nthreads=None):
    """q_bits: uint16 [B][Hq][vd + kd] -> fp64 [B][Hq][vd] (or [npairs][vd])."""
    return _attention(lib().orc_attention_mla, cache, q_bits, sigma, pairs, nthreads)


def prefill_attention(q_bits, k_bits, v_bits, sigma: float, rows=None, nthreads=None):
    """Causal prefill attention (fp64): q uint16 [B][Hq][T][d], k / v uint16
    [B][Hkv][T][d|dv]; rows: (b, h, i) triples, default every row.  Returns
    fp64 [nrows][dv] (or [B][Hq][T][dv] when rows is None)."""
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    k = np.ascontiguousarray(k_bits, dtype=np.uint16)
    v = np.ascontiguousarray(v_bits, dtype=np.uint16)
    B, Hq, T, d = q.shape
    Hkv, dv = k.shape[1], v.shape[3]
    full = rows is None
    if full:
        bb, hh, ii = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(T), indexing="ij")
        rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
    rr = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.empty((rr.shape[0], dv), np.float64)
    if nthreads is None:
        nthreads = default_threads()
    L = lib()
    rc = L.orc_prefill_attention(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, T, d, dv, C.c_double(sigma), _ptr(rr),
                                 rr.shape[0], _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle prefill attention rejected its input")
    return out.reshape(B, Hq, T, dv) if full else out

