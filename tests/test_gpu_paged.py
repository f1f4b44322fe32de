"""GPU parity of the paged cache through the C ABI.

Ragged sequences append in three phases (a multi-row prefill, single-row
decode steps in which some sequences sit out, a multi-row burst that crosses
block boundaries from the residual), with their blocks in shuffled pages of
one pool.  The pages the kernels fill (gathered through the block table) and
every residual must equal the oracle's per-sequence cache bit for bit, and
decode attention must sit within 2e-3 (max-abs) of the oracle's fp64 result
for every sequence; a sequence of length 0 must read exactly 0.
"""
import dataclasses

import numpy as np
import pytest

from gpu_util import (MEAN_EXCESS_TOL, TOL, assert_slices_equal, configs, dev_f16, host_u16, kvq, log,
                      mean_excess, oracle_attention, oracle_cache_full, oracle_slice, synth, torch)

pytestmark = pytest.mark.gpu


def _workload(shape, T):
    if shape == "mla":
        return configs.Workload("paged_mla", 520, "mla", 3, 16, 1, T, 64, 64, 4, 512, 32, 2, 20.0)
    if shape == "mla_int4":   # INT4 content latent and INT4 RoPE key
        return configs.Workload("paged_mla4", 521, "mla", 3, 16, 1, T, 64, 64, 4, 512, 32, 4, 20.0)
    d = {
        "gqa4_g64": (6, 8, 2, 128, 64, 2, 2),
        "gqa4_g32": (6, 8, 2, 128, 32, 2, 2),
        "mha_d64": (5, 2, 2, 64, 32, 2, 2),
        "mha_d128": (4, 2, 2, 128, 64, 2, 2),
        "mha_d128_g32": (4, 2, 2, 128, 32, 2, 2),
        "gqa4_4bit_g64": (6, 8, 2, 128, 64, 4, 4),
        "gqa4_4bit_g32": (6, 8, 2, 128, 32, 4, 4),
        "mha_d128_4bit": (4, 2, 2, 128, 64, 4, 4),
        "kv4bit": (4, 4, 2, 64, 32, 4, 4),
        "d32_g64": (3, 2, 2, 32, 64, 2, 2),
    }[shape]
    B, Hq, Hkv, D, G, kb, vb = d
    return configs.Workload("paged_" + shape, 510, "kivi", B, Hq, Hkv, T, D, G, kb, D, 32, vb, 50.0)


def _final_lengths(w):
    G = w.kG
    pick = [0, 1, G - 1, G, G + 1, 2 * G + 5, w.T, 3 * G]
    return np.array([min(pick[i % len(pick)], w.T) for i in range(w.batch)], np.int32)


class Paged:
    """A paged cache plus its host-side lengths and block table."""

    def __init__(self, w, final, spare=3, seed_word=0):
        t = torch()
        self.w = w
        G = w.kG
        self.cap = max(G, -(-int(final.max()) // G) * G)
        self.maxb = self.cap // G
        blocks = -(-final // G)   # the partial block holds values, so it needs its page
        self.table, self.n_pages = synth.page_table(w, blocks, self.maxb, spare, seed_word)
        self.pc = kvq.PagedCache(kvq.cfg_for(w, self.cap), self.n_pages)
        for a in self.pc.arrays.values():
            a.fill_(0x5A)   # a sentinel, so rows the kernels skip stay recognisable
        self.lens = np.zeros(w.batch, np.int32)
        self.table_dev = t.from_numpy(self.table).cuda()

    def append(self, k_full, v_full, n_new):
        """Rows lens[b] .. lens[b] + n_new[b] of the full draws."""
        t = torch()
        w = self.w
        n_max = int(n_new.max())
        if n_max == 0:
            return
        k = np.zeros((w.batch, w.n_kv_heads, n_max, w.kd), np.uint16)
        v = np.zeros((w.batch, w.n_kv_heads, n_max, w.vd), np.uint16)
        for b in range(w.batch):
            s, n = int(self.lens[b]), int(n_new[b])
            k[b, :, :n] = k_full[b, :, s:s + n]
            v[b, :, :n] = v_full[b, :, s:s + n]
        lens_dev = t.from_numpy(self.lens.copy()).cuda()
        nn_dev = t.from_numpy(n_new.astype(np.int32)).cuda()
        self.pc.append(dev_f16(k), dev_f16(v), lens_dev, self.table_dev, nn_dev)
        t.cuda.synchronize()
        self.lens = self.lens + n_new.astype(np.int32)

    def gather(self, b, h):
        """The (b, h) cache as the oracle lays it out, through the block table."""
        t = torch()
        t.cuda.synchronize()
        w, G, F = self.w, self.w.kG, int(self.lens[b])
        nb, R = F // G, F % G
        pages = self.table[b, :-(-F // G)]
        vw = self.pc.views()
        tok = np.arange(F)
        vp = t.from_numpy(pages[tok // G].astype(np.int64)).cuda()
        vs = t.from_numpy((tok % G).astype(np.int64)).cuda()
        kp = t.from_numpy(pages[:nb].astype(np.int64)).cuda()
        out = {
            "k_codes": vw["k_codes"][kp, h], "k_scale": vw["k_scale"][kp, h], "k_zero": vw["k_zero"][kp, h],
            "k_resid": vw["k_resid"][b, h, :R],
            "v_codes": vw["v_codes"][vp, h, vs], "v_scale": vw["v_scale"][vp, h, vs],
            "v_zero": vw["v_zero"][vp, h, vs],
        }
        res = {}
        for name, a in out.items():
            a = a.cpu().numpy()
            res[name] = a.view(np.uint32) if a.dtype == np.int32 else a.view(np.uint16)
        return res

    def decode(self, q_u16, max_len=None, n_splits=0):
        t = torch()
        lens_dev = t.from_numpy(self.lens.copy()).cuda()
        max_len = int(self.lens.max()) if max_len is None else max_len
        out = self.pc.decode(dev_f16(q_u16), self.w.sigma, lens_dev, self.table_dev, max_len, n_splits)
        t.cuda.synchronize()
        return host_u16(out).view(np.float16).astype(np.float64)


def _three_phases(pg, k_full, v_full, final):
    """prefill two thirds, up to 5 single-row steps, then the rest in one burst"""
    A = final * 2 // 3
    D = np.minimum(final - A, 5)
    pg.append(k_full, v_full, A)
    for i in range(5):
        pg.append(k_full, v_full, (D > i).astype(np.int32))
    pg.append(k_full, v_full, final - A - D)
    assert np.array_equal(pg.lens, final)


def _check_cache(orc, pg, k_full, v_full):
    w = pg.w
    for b in range(w.batch):
        F = int(pg.lens[b])
        if F == 0:
            continue
        for h in range(w.n_kv_heads):
            ref = oracle_slice(orc, w, k_full[b, h, :F], v_full[b, h, :F], pg.cap // w.kG, pg.cap)
            assert_slices_equal(pg.gather(b, h), ref, f"{w.name} b{b} h{h} T{F}")


def _check_decode(orc, pg, k_full, v_full, q, got, seqs=None):
    w = pg.w
    worst, gots, refs = 0.0, [], []
    for b in (range(w.batch) if seqs is None else seqs):
        F = int(pg.lens[b])
        if F == 0:
            assert np.all(got[b] == 0.0), (w.name, b)
            continue
        sub = dataclasses.replace(w, batch=1, T=F)
        cache = oracle_cache_full(orc, sub, k_full[b:b + 1, :, :F], v_full[b:b + 1, :, :F], pg.cap)
        ref = oracle_attention(orc, sub, cache, np.ascontiguousarray(q[b:b + 1]))[0]
        worst = max(worst, float(np.abs(got[b] - ref).max()))
        gots.append(got[b].ravel())
        refs.append(ref.ravel())
    excess = mean_excess(np.concatenate(gots), np.concatenate(refs))
    assert worst <= TOL, (w.name, worst)
    assert excess <= MEAN_EXCESS_TOL, (w.name, excess)
    return worst, excess


@pytest.mark.parametrize("shape", ["gqa4_g64", "gqa4_g32", "mha_d64", "mha_d128", "mha_d128_g32", "kv4bit", "mla", "mla_int4",
                                   "d32_g64", "gqa4_4bit_g64", "gqa4_4bit_g32", "mha_d128_4bit"])
def test_paged_ragged_append_and_decode(orc, shape):
    w = _workload(shape, 700)
    final = _final_lengths(w)
    log(f"[paged {shape}] lengths {final.tolist()}")
    k_full, v_full, q = synth.keys(w), synth.values(w), synth.query(w)
    pg = Paged(w, final)
    log(f"[paged {shape}] variant {pg.pc.variant(w.n_q_heads, int(final.max()))} pages {pg.n_pages}")
    _three_phases(pg, k_full, v_full, final)
    _check_cache(orc, pg, k_full, v_full)
    # the bound at the longest sequence, a looser bound (empty splits), and
    # explicit split counts
    for max_len, ns in ((None, 0), (pg.cap, 0), (None, 1), (None, 3)):
        got = pg.decode(q, max_len, ns)
        worst, excess = _check_decode(orc, pg, k_full, v_full, q, got)
        log(f"[paged {shape}] max_len {max_len} splits {ns}: max|err| {worst:.3e} mean excess {excess:.2e}")


def test_paged_decode_steps_match_oracle(orc):
    """Single-row appends that fill a block from the residual, decoding after
    each step (the serving loop), GQA shape with G = 64."""
    w = _workload("gqa4_g64", 3 * 64 + 3)
    final = np.array([64 - 3, 2 * 64 - 2, 3 * 64 + 3, 5, 64, 130], np.int32)
    k_full, v_full, q = synth.keys(w), synth.values(w), synth.query(w)
    pg = Paged(w, final)
    pg.append(k_full, v_full, np.maximum(final - 6, 0))
    for step in range(6):
        pg.append(k_full, v_full, (pg.lens < final).astype(np.int32))
        got = pg.decode(q)
        _check_decode(orc, pg, k_full, v_full, q, got)
    assert np.array_equal(pg.lens, final)
    _check_cache(orc, pg, k_full, v_full)


def test_paged_skips_out_of_range_entries(orc):
    """The kernels' own range checks: a negative length, a row count above
    n_max and a page number outside the pool make the append skip those
    sequences / rows (their memory keeps the sentinel), the other sequences
    are unaffected, and decode reads a clamped length as 0 tokens."""
    t = torch()
    w = _workload("gqa4_g64", 200)
    final = np.array([130, 100, 150, 70, 64, 199], np.int32)
    k_full, v_full, q = synth.keys(w), synth.values(w), synth.query(w)
    pg = Paged(w, final)
    bad_table = pg.table.copy()
    bad_table[2, 1] = pg.n_pages + 7           # block 1 of sequence 2: outside the pool
    lens = np.zeros(w.batch, np.int32)
    lens[0] = -3                                # sequence 0: bad length
    n_new = final.copy()
    n_new[1] = int(final.max()) + 1             # sequence 1: more rows than n_max
    n_max = int(final.max())
    k = np.ascontiguousarray(k_full[:, :, :n_max])
    v = np.ascontiguousarray(v_full[:, :, :n_max])
    before = {n: a.clone() for n, a in pg.pc.arrays.items()}
    pg.pc.append(dev_f16(k), dev_f16(v), t.from_numpy(lens).cuda(), t.from_numpy(bad_table).cuda(),
                 t.from_numpy(n_new).cuda())
    t.cuda.synchronize()
    vw = pg.pc.views()
    vb = kvq.PagedCache.views(_Snap(pg.pc, before))
    # sequences 0 and 1: their residual rows are untouched
    for b in (0, 1):
        assert t.equal(vw["k_resid"][b], vb["k_resid"][b])
    # sequence 2, block 1: its page received nothing
    p_bad = int(pg.table[2, 1])
    for n in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero"):
        assert t.equal(vw[n][p_bad], vb[n][p_bad]), n
    # the valid sequences match the oracle
    pg.lens = np.where(np.arange(w.batch) < 3, 0, final).astype(np.int32)
    for b in range(3, w.batch):
        for h in range(w.n_kv_heads):
            F = int(final[b])
            ref = oracle_slice(orc, w, k_full[b, h, :F], v_full[b, h, :F], pg.cap // w.kG, pg.cap)
            assert_slices_equal(pg.gather(b, h), ref, f"b{b} h{h}")
    # decode: a negative length reads as 0 tokens
    dl = pg.lens.copy()
    dl[0] = -5
    out = pg.pc.decode(dev_f16(q), w.sigma, t.from_numpy(dl).cuda(), pg.table_dev, int(final.max()))
    t.cuda.synchronize()
    got = host_u16(out).view(np.float16).astype(np.float64)
    assert np.all(got[0] == 0.0)
    _check_decode(orc, pg, k_full, v_full, q, got, seqs=range(3, w.batch))


class _Snap:
    """views() over a saved copy of a paged cache's arrays"""

    def __init__(self, pc, arrays):
        self.torch, self.cfg, self.n_pages, self.arrays = pc.torch, pc.cfg, pc.n_pages, arrays


@pytest.mark.parametrize("T,G", [(4096 + 37, 64), (4096 + 21, 32)])
def test_paged_gqa_ragged_4k(orc, T, G):
    """32 query / 8 KV heads, D = 128, ragged lengths in [T/2, T], shuffled
    pages: the MFMA kernel across many tiles per split; sampled sequences
    against the oracle."""
    w = configs.Workload("paged_gqa_4k", 530, "kivi", 8, 32, 8, T, 128, G, 2, 128, 32, 2, 50.0)
    final = synth.ragged_lengths(w)
    k_full, v_full, q = synth.keys(w), synth.values(w), synth.query(w)
    pg = Paged(w, final, spare=11)
    assert pg.pc.variant(w.n_q_heads, T) == "gqa_mfma_paged"
    pg.append(k_full, v_full, final)
    got = pg.decode(q, T)
    worst, excess = _check_decode(orc, pg, k_full, v_full, q, got, seqs=[0, 3, w.batch - 1])
    for b in (0, w.batch - 1):
        for h in (0, w.n_kv_heads - 1):
            F = int(final[b])
            ref = oracle_slice(orc, w, k_full[b, h, :F], v_full[b, h, :F], pg.cap // w.kG, pg.cap)
            assert_slices_equal(pg.gather(b, h), ref, f"b{b} h{h}")
    log(f"[paged gqa 4k G{G}] max|err| {worst:.3e} mean excess {excess:.2e}")


def _rows_at(w, k_full, v_full, lens, n_new):
    """[B][Hkv][1][d] inputs: row lens[b] of each sequence that appends."""
    k = np.zeros((w.batch, w.n_kv_heads, 1, w.kd), np.uint16)
    v = np.zeros((w.batch, w.n_kv_heads, 1, w.vd), np.uint16)
    for b in range(w.batch):
        if n_new[b]:
            k[b, :, 0] = k_full[b, :, lens[b]]
            v[b, :, 0] = v_full[b, :, lens[b]]
    return k, v


@pytest.mark.parametrize("shape", ["gqa4_g64", "gqa4_g32", "mha_d128", "gqa4_4bit_g64", "gqa4_4bit_g32",
                                   "mha_d128_4bit", "mha_d128_g32"])
def test_paged_decode_step(orc, shape):
    """kv_paged_decode_step (append fused into the attention launch, lengths
    advanced on the device) against kv_paged_append + kv_paged_decode over
    G + 2 steps in which some sequences sit out: caches bit-identical after
    every step, outputs bit-identical for every sequence whose block did not
    complete in the step, all within 2e-3 of the oracle."""
    t = torch()
    G = 32 if shape in ("gqa4_g32", "gqa4_4bit_g32", "mha_d128_g32") else 64
    w = _workload(shape, 5 * G)
    lens0 = np.array([G - 1, G - 2, 0, 5, 2 * G - 1, 3 * G - 3][:w.batch], np.int32)
    steps = G + 2
    nn_all = np.array([[0 if (j + b) % 5 == 0 else 1 for b in range(w.batch)] for j in range(steps)], np.int32)
    final = lens0 + nn_all.sum(0).astype(np.int32)
    assert final.max() <= w.T
    k_full, v_full, q = synth.keys(w), synth.values(w), synth.query(w)
    a, ref = Paged(w, final), Paged(w, final)
    for pg in (a, ref):
        pg.append(k_full, v_full, lens0)
    assert a.pc.variant(w.n_q_heads, a.cap) in ("gqa_mfma_paged", "mha_mfma_paged")
    lens_dev = t.from_numpy(lens0.copy()).cuda()
    qd = dev_f16(q)
    ws = a.pc.workspace(w.n_q_heads, a.cap)
    for j in range(steps):
        nn = nn_all[j]
        kn, vn = _rows_at(w, k_full, v_full, ref.lens, nn)
        completes = (ref.lens % G == G - 1) & (nn == 1)
        out = a.pc.step(dev_f16(kn), dev_f16(vn), qd, w.sigma, lens_dev, a.table_dev, a.cap,
                        n_new=t.from_numpy(nn.copy()).cuda(), ws=ws)
        t.cuda.synchronize()
        got = host_u16(out).view(np.float16).astype(np.float64)
        ref.append(k_full, v_full, nn)
        want = ref.decode(q, a.cap)
        assert np.array_equal(lens_dev.cpu().numpy(), ref.lens), j
        same = ~completes
        assert np.array_equal(got[same], want[same]), (shape, j)
        a.lens = ref.lens.copy()
        if j % 7 == 0 or completes.any():
            _check_decode(orc, a, k_full, v_full, q, got)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            assert_slices_equal(a.gather(b, h), ref.gather(b, h), f"{shape} b{b} h{h}")
    _check_cache(orc, a, k_full, v_full)


def test_paged_decode_step_graph(orc):
    """The paged decode step with its device-side length advance, captured
    once in a HIP graph and replayed: after every replay (with eager input
    updates and synchronisation in between) the output and the lengths equal
    an eager step on a twin cache, and the cache matches the oracle."""
    t = torch()
    w = _workload("gqa4_g64", 2 * 64 + 20)
    lens0 = np.array([60, 62, 1, 64, 100, 127], np.int32)
    R = 6
    final = lens0 + R
    k_full, v_full, q = synth.keys(w), synth.values(w), synth.query(w)
    g_pg, e_pg = Paged(w, final), Paged(w, final)
    for pg in (g_pg, e_pg):
        pg.append(k_full, v_full, lens0)
    qd = dev_f16(q)
    kn_s = t.zeros((w.batch, w.n_kv_heads, 1, w.kd), dtype=t.float16, device="cuda")
    vn_s = t.zeros((w.batch, w.n_kv_heads, 1, w.vd), dtype=t.float16, device="cuda")
    out_s = t.empty((w.batch, w.n_q_heads, w.vd), dtype=t.float16, device="cuda")
    ws_s = g_pg.pc.workspace(w.n_q_heads, g_pg.cap)
    lens_g = t.from_numpy(lens0.copy()).cuda()
    lens_e = t.from_numpy(lens0.copy()).cuda()
    t.cuda.synchronize()
    graph = t.cuda.CUDAGraph()
    with t.cuda.graph(graph):
        g_pg.pc.step(kn_s, vn_s, qd, w.sigma, lens_g, g_pg.table_dev, g_pg.cap, out=out_s, ws=ws_s)
    t.cuda.synchronize()
    assert np.array_equal(lens_g.cpu().numpy(), lens0)   # capture runs nothing
    host = lens0.copy()
    for r in range(R):
        kn, vn = _rows_at(w, k_full, v_full, host, np.ones(w.batch, np.int32))
        kn_s.copy_(dev_f16(kn))
        vn_s.copy_(dev_f16(vn))
        t.cuda.synchronize()
        graph.replay()
        t.cuda.synchronize()
        got = host_u16(out_s).view(np.float16)
        want = host_u16(e_pg.pc.step(dev_f16(kn), dev_f16(vn), qd, w.sigma, lens_e, e_pg.table_dev, e_pg.cap))
        t.cuda.synchronize()
        host = host + 1
        assert np.array_equal(lens_g.cpu().numpy(), host), r
        assert np.array_equal(lens_e.cpu().numpy(), host), r
        assert np.array_equal(got.view(np.uint16), want), r
        log(f"[graph] replay {r}: output and lengths equal the eager step")
    g_pg.lens = host.copy()
    _check_cache(orc, g_pg, k_full, v_full)
    _check_decode(orc, g_pg, k_full, v_full, q, host_u16(out_s).view(np.float16).astype(np.float64))
