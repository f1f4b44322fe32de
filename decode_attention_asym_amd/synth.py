"""Seeded synthetic inputs (fp16 K, V, Q) for the workloads in ``configs``.

This module only draws random numbers; it holds none of the method's
arithmetic.  Both the HIP path and the CPU oracle consume exactly these bits.

Recipe (the pages give the distribution qualitatively: about 1% of key
channels carry large outliers that stay fixed along the whole sequence, values
show no such pattern -- "Makale Bülteni -- KIVI", section "İddia ve
Gerçeklik: KIVI"):
  * every (tensor, batch, kv-head) slice has its own numpy PCG64 stream,
    seeded with SeedSequence([0x4B495649 + workload.index, tensor, b, h]);
  * draw N(0, 1) in float32, row-major [T][dim];
  * keys: the outlier channels (max(1, ceil(1% of n_kv_heads * key_dim))
    channels of the flattened (kv head, channel) index, drawn once per
    workload without replacement) are multiplied by ``outlier_scale`` in
    float32;
  * cast to fp16 with round-to-nearest-even; returned as uint16 bit patterns.
A prefix of a longer draw equals the shorter draw, so caches of different
lengths built from one workload agree on their common tokens.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

from .configs import Workload

SEED_BASE = 0x4B495649
T_KEY, T_VALUE, T_QUERY, T_OUTLIER, T_LENS, T_PAGES, T_PROMPT_Q = 0, 1, 2, 3, 4, 5, 6


def _rng(w: Workload, *words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_BASE + w.index, *words])))


def outlier_channels(w: Workload) -> np.ndarray:
    """Sorted flat indices kvh * key_dim + channel of the outlier key channels."""
    n = w.n_kv_heads * w.kd
    return np.sort(_rng(w, T_OUTLIER).choice(n, size=w.n_outlier, replace=False))


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def key_slice(w: Workload, b: int, h: int, T: int | None = None, outliers: bool = True) -> np.ndarray:
    T = w.T if T is None else T
    x = _normal(_rng(w, T_KEY, b, h), (T, w.kd))
    if outliers:
        flat = outlier_channels(w)
        ch = flat[flat // w.kd == h] % w.kd
        if ch.size:
            x[:, ch] *= np.float32(w.outlier_scale)
    return x.astype(np.float16).view(np.uint16)


def value_slice(w: Workload, b: int, h: int, T: int | None = None) -> np.ndarray:
    T = w.T if T is None else T
    return _normal(_rng(w, T_VALUE, b, h), (T, w.vd)).astype(np.float16).view(np.uint16)


def query(w: Workload) -> np.ndarray:
    """uint16 [B][Hq][qd]."""
    x = _normal(_rng(w, T_QUERY), (w.batch, w.n_q_heads, w.qd))
    return x.astype(np.float16).view(np.uint16)


def prompt_queries(w: Workload, T: int | None = None, threads=None) -> np.ndarray:
    """uint16 [B][Hq][T][qd]: the query rows of a prompt (prefill), N(0, 1),
    one stream per (sequence, query head)."""
    T = w.T if T is None else T
    out = np.empty((w.batch, w.n_q_heads, T, w.qd), np.uint16)

    def job(bh):
        b, h = divmod(bh, w.n_q_heads)
        out[b, h] = _normal(_rng(w, T_PROMPT_Q, b, h), (T, w.qd)).astype(np.float16).view(np.uint16)

    n = threads or min(16, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(job, range(w.batch * w.n_q_heads)))
    return out


def _fill(fn, w: Workload, T: int, dim: int, out: np.ndarray | None, threads: int | None):
    B, H = w.batch, w.n_kv_heads
    if out is None:
        out = np.empty((B, H, T, dim), np.uint16)
    assert out.shape == (B, H, T, dim) and out.dtype == np.uint16

    def job(bh):
        b, h = divmod(bh, H)
        out[b, h] = fn(w, b, h, T)

    n = threads or min(16, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(job, range(B * H)))
    return out


def keys(w: Workload, T: int | None = None, out=None, threads=None) -> np.ndarray:
    """uint16 [B][Hkv][T][kd]."""
    return _fill(key_slice, w, w.T if T is None else T, w.kd, out, threads)


def values(w: Workload, T: int | None = None, out=None, threads=None) -> np.ndarray:
    """uint16 [B][Hkv][T][vd]."""
    return _fill(value_slice, w, w.T if T is None else T, w.vd, out, threads)


# ---------------------------------------------------------------- paged caches
# Serving-style inputs: sequences of different lengths whose key blocks sit
# in pages scattered over one pool.  Lengths: uniform integers in
# [lo_frac * T, T], the last sequence exactly T (so the longest equals the
# fixed-length workload); pages: a seeded random permutation of the pool,
# handed out block by block, with `spare` pages never used.

def ragged_lengths(w: Workload, lo_frac: float = 0.5) -> np.ndarray:
    """int32 [B] sequence lengths."""
    lo = int(lo_frac * w.T)
    lens = _rng(w, T_LENS).integers(lo, w.T + 1, size=w.batch).astype(np.int32)
    lens[-1] = w.T
    return lens


def page_table(w: Workload, blocks: np.ndarray, maxb: int, spare: int = 3, seed_word: int = 0):
    """(table int32 [B][maxb], n_pages): sequence b gets blocks[b] pages from a
    shuffled pool of sum(blocks) + spare pages; unused entries are -1."""
    n_pages = int(np.sum(blocks)) + spare
    perm = _rng(w, T_PAGES, seed_word).permutation(n_pages).astype(np.int32)
    table = np.full((w.batch, maxb), -1, np.int32)
    k = 0
    for b in range(w.batch):
        nb = int(blocks[b])
        table[b, :nb] = perm[k:k + nb]
        k += nb
    return table, n_pages
