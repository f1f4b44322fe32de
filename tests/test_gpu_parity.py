"""GPU parity through the C ABI: the cache the HIP kernels build must equal the
oracle's bit for bit (codes, packed words, fp16 scales and zeros, residual),
and decode attention must sit within 2e-3 (max-abs) of the oracle's fp64
result, on all five workloads and on edge cases."""
import numpy as np
import pytest

from gpu_util import (MEAN_EXCESS_TOL, TOL, assert_slices_equal, mean_excess, configs, dev_f16, host_u16, kvq, log, new_cache,
                      oracle_attention, oracle_cache_full, oracle_slice, sample_pairs, slice_of,
                      synth, torch)

pytestmark = pytest.mark.gpu

FULL = [w.name for w in configs.WORKLOADS]


def _decode(dc, w, q_u16, n_splits=0):
    t = torch()
    out = dc.decode(dev_f16(q_u16), w.sigma, n_splits)
    t.cuda.synchronize()
    return host_u16(out).view(np.float16).astype(np.float64)


def _host_arrays(dc):
    """The device cache's seven arrays on the host, in their layouts."""
    t = torch()
    t.cuda.synchronize()
    out = {}
    for name, arr in dc.views().items():
        a = arr.cpu().numpy()
        out[name] = a.view(np.uint32) if a.dtype == np.int32 else a.view(np.uint16)
    return out


def assert_cache_equal(got, cache, T, nblk, what=""):
    """Every slice of a device cache (host copy) equals the oracle's cache
    bit for bit over the valid region: nblk key blocks, T - nblk * G
    residual keys, T value rows."""
    R = T - nblk * cache.s.kG
    ref = {"k_codes": cache.k["k_codes"][:, :, :nblk], "k_scale": cache.k["k_scale"][:, :, :nblk],
           "k_zero": cache.k["k_zero"][:, :, :nblk], "k_resid": cache.k["k_resid"][:, :, :R],
           "v_codes": cache.v["v_codes"][:, :, :T], "v_scale": cache.v["v_scale"][:, :, :T],
           "v_zero": cache.v["v_zero"][:, :, :T]}
    lim = {"k_codes": nblk, "k_scale": nblk, "k_zero": nblk, "k_resid": R}
    for name, r in ref.items():
        g = got[name][:, :, :lim.get(name, T)]
        assert g.shape == r.shape, (what, name, g.shape, r.shape)
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError(f"{what} {name}: {len(bad)} mismatches, first at {bad[0].tolist()}: "
                                 f"gpu {g[tuple(bad[0])]:#x} oracle {r[tuple(bad[0])]:#x}")


# MLA: all 128 heads of 8 sequences spread over the batch (the oracle takes
# ~1 s per sequence on 16 cores; the cache is compared on every sequence)
MLA_SEQS = 8


@pytest.mark.parametrize("name", FULL)
def test_workload_parity(orc, name):
    """Full-size workload: bulk prefill quantize, then decode attention.
    The whole cache (every (sequence, KV head) slice: codes, packed words,
    fp16 scales and zeros, residual) must equal the oracle's bit for bit;
    attention is compared on every (sequence, query head) pair (MLA: every
    head of 8 sequences).  About 30 s for the 32K GQA workload on 16 host
    cores, most of it the oracle."""
    w = configs.BY_NAME[name]
    cap = w.capacity(64)
    log(f"[{name}] inputs B={w.batch} Hkv={w.n_kv_heads} T={w.T}")
    k = synth.keys(w)
    v = synth.values(w)
    q = synth.query(w)
    dc = new_cache(w, cap)
    dc.append(dev_f16(k), dev_f16(v))
    assert dc.state() == (w.T, w.R)
    log(f"[{name}] variant {dc.variant(w.n_q_heads)}")
    got = _decode(dc, w, q)
    host = _host_arrays(dc)
    dc.close()
    del dc
    cache = orc.build_cache(k, v, w.kG, w.kbits, w.vG, w.vbits, nblk_cap=cap // w.kG, tok_cap=cap, threads=None)
    del k, v
    assert_cache_equal(host, cache, w.T, w.n_blocks, name)
    del host
    log(f"[{name}] cache bit-exact on all {w.batch * w.n_kv_heads} slices")
    if w.kind == "mla":
        seqs = sorted({int(round(i * (w.batch - 1) / (MLA_SEQS - 1))) for i in range(MLA_SEQS)})
        pairs = [(b, h) for b in seqs for h in range(w.n_q_heads)]
        ref = oracle_attention(orc, w, cache, q, pairs=pairs)
        gv = np.stack([got[b, h] for b, h in pairs])
    else:
        ref = oracle_attention(orc, w, cache, q).reshape(-1, w.vd)
        gv = got.reshape(-1, w.vd)
        pairs = range(len(gv))
    worst = float(np.abs(gv - ref).max())
    excess = mean_excess(gv.ravel(), ref.ravel())
    log(f"[{name}] pairs {len(pairs)} max|err| {worst:.3e} mean excess {excess:.2e} max|o| {np.abs(ref).max():.3f}")
    assert worst <= TOL
    assert excess <= MEAN_EXCESS_TOL


def _tiny(T, Hq=4, Hkv=2, D=64, G=32, kbits=2, vbits=2, B=2, idx=200):
    return configs.Workload("tiny", idx, "kivi", B, Hq, Hkv, T, D, G, kbits, D, 32, vbits, 50.0)


def _mla_tiny(T, Hq=16, B=2, idx=300, vbits=2):
    return configs.Workload("mla_tiny", idx, "mla", B, Hq, 1, T, 64, 64, 4, 512, 32, vbits, 20.0)


def _check_decode(orc, w, dc, k, v, n_splits=0, kq_blocks=None):
    cap = dc.cfg.max_tokens
    q = synth.query(w)
    got = _decode(dc, w, q, n_splits)
    cache = orc.build_cache(k, v, w.kG, w.kbits, w.vG, w.vbits, nblk_cap=cap // w.kG,
                            tok_cap=cap, kq_blocks=kq_blocks)
    ref = oracle_attention(orc, w, cache, q)
    err = np.abs(got - ref).max()
    assert err <= TOL, (w, n_splits, err)
    excess = mean_excess(got, ref)
    assert excess <= MEAN_EXCESS_TOL, (w, n_splits, excess)
    return got


def _shape(shape, T):
    """Small caches that reach each decode kernel: generic (D = 64, 8-way
    GQA, MLA), the MHA and GQA MFMA kernels (D = 128) with both G."""
    if shape == "mha":
        return _tiny(T, Hq=2, Hkv=2)
    if shape == "mha128_g32":
        return _tiny(T, Hq=2, Hkv=2, D=128, G=32)
    if shape == "mha128_g64":
        return _tiny(T, Hq=2, Hkv=2, D=128, G=64)
    if shape == "gqa4_g64":
        return _tiny(T, Hq=8, Hkv=2, D=128, G=64)
    if shape == "gqa4":
        return _tiny(T, Hq=8, Hkv=2, D=128)
    if shape == "mha128_4bit_g64":
        return _tiny(T, Hq=2, Hkv=2, D=128, G=64, kbits=4, vbits=4)
    if shape == "mha128_4bit_g32":
        return _tiny(T, Hq=2, Hkv=2, D=128, G=32, kbits=4, vbits=4)
    if shape == "gqa4_4bit_g64":
        return _tiny(T, Hq=8, Hkv=2, D=128, G=64, kbits=4, vbits=4)
    if shape == "gqa4_4bit_g32":
        return _tiny(T, Hq=8, Hkv=2, D=128, G=32, kbits=4, vbits=4)
    if shape == "mla64":
        return _mla_tiny(T, Hq=64)
    if shape == "mla128":
        return _mla_tiny(T, Hq=128, B=1)
    # QuantMLA's INT4 content latent (RoPE key INT4 as always)
    if shape == "mla4":
        return _mla_tiny(T, vbits=4, idx=310)
    if shape == "mla4_64":
        return _mla_tiny(T, Hq=64, vbits=4, idx=311)
    if shape == "mla4_128":
        return _mla_tiny(T, Hq=128, B=1, vbits=4, idx=312)
    raise KeyError(shape)


@pytest.mark.parametrize("T", [1, 15, 31, 32, 33, 101, 3 * 64 + 5, 700])
@pytest.mark.parametrize("shape", ["mha", "mha128_g32", "mha128_g64", "gqa4", "gqa8_g64", "mla", "mla64",
                                   "mla128", "gqa4_4bit_g64", "gqa4_4bit_g32", "mha128_4bit_g64",
                                   "mha128_4bit_g32", "mla4", "mla4_64", "mla4_128"])
def test_edge_lengths(orc, T, shape):
    if shape in ("mha", "mha128_g32", "mha128_g64", "mla64", "mla128", "gqa4_4bit_g64", "gqa4_4bit_g32",
                 "mha128_4bit_g64", "mha128_4bit_g32", "mla4", "mla4_64", "mla4_128"):
        w = _shape(shape, T)
    elif shape == "gqa4":
        w = _tiny(T, Hq=8, Hkv=2, D=128)
    elif shape == "gqa8_g64":
        w = _tiny(T, Hq=8, Hkv=1, D=128, G=64)
    else:
        w = _mla_tiny(T)
    cap = w.capacity(16)
    k, v = synth.keys(w), synth.values(w)
    dc = new_cache(w, cap)
    dc.append(dev_f16(k), dev_f16(v))
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            assert_slices_equal(slice_of(dc, b, h, T, T // w.kG),
                                oracle_slice(orc, w, k[b, h], v[b, h], cap // w.kG, cap), f"T{T}")
    _check_decode(orc, w, dc, k, v)


@pytest.mark.parametrize("n_splits", [1, 2, 3, 7, 64, 256])
@pytest.mark.parametrize("shape", ["gqa4", "mha128_g32", "mla64", "gqa4_4bit_g64", "gqa4_4bit_g32", "mha128_4bit_g32",
                                   "mla4_64", "mla4"])
def test_split_counts(orc, n_splits, shape):
    w = _tiny(1000, Hq=8, Hkv=2, D=128, G=32) if shape == "gqa4" else _shape(shape, 1000)
    cap = w.capacity()
    k, v = synth.keys(w), synth.values(w)
    dc = new_cache(w, cap)
    dc.append(dev_f16(k), dev_f16(v))
    _check_decode(orc, w, dc, k, v, n_splits=n_splits)


@pytest.mark.parametrize("D,G,kbits", [(96, 64, 2), (160, 64, 2), (256, 64, 2), (256, 32, 4), (96, 32, 2),
                                        (96, 128, 2), (192, 128, 2), (64, 16, 4)])
def test_key_widths(orc, D, G, kbits):
    """Key dimensions whose channel quads fill whole waves (256 at G = 64,
    192 at G = 128, any at G <= 32) take the four-channel key quantizer
    threads, the others (96 and 160 at G = 64, 96 at G = 128) the
    two-channel ones: every cache slice matches the oracle bit for bit and
    the attention stays within the bar."""
    w = _tiny(3 * G + 11, Hq=4, Hkv=2, D=D, G=G, kbits=kbits)
    cap = w.capacity(16)
    k, v = synth.keys(w), synth.values(w)
    dc = new_cache(w, cap)
    dc.append(dev_f16(k), dev_f16(v))
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            assert_slices_equal(slice_of(dc, b, h, w.T, w.T // w.kG),
                                oracle_slice(orc, w, k[b, h], v[b, h], cap // w.kG, cap), f"D{D} G{G}")
    _check_decode(orc, w, dc, k, v)


def _cache_arrays(dc, T, nblk):
    B, H = dc.cfg.batch, dc.cfg.n_kv_heads
    return [slice_of(dc, b, h, T, nblk) for b in range(B) for h in range(H)]


@pytest.mark.parametrize("mode", ["auto_single", "manual_flush", "chunks"])
def test_streaming_equals_bulk(orc, mode):
    """Appending token by token (auto-flush, or explicit flushes) or in
    ragged chunks builds the same cache, bit for bit, as one bulk append."""
    w = _tiny(250, Hq=4, Hkv=2, D=64, G=32)
    cap = w.capacity()
    k, v = synth.keys(w), synth.values(w)
    kd, vd = dev_f16(k), dev_f16(v)
    bulk = new_cache(w, cap)
    bulk.append(kd, vd)
    ref = _cache_arrays(bulk, w.T, w.n_blocks)
    st = new_cache(w, cap)
    t = 0
    rng = np.random.default_rng(5)
    while t < w.T:
        n = 1 if mode != "chunks" else int(min(w.T - t, rng.integers(1, 80)))
        ks = kd[:, :, t:t + n].contiguous()
        vs = vd[:, :, t:t + n].contiguous()
        if mode == "manual_flush":
            st.append(ks, vs, kvq.KVQ_APPEND_NO_AUTOFLUSH)
            T_, R_ = st.state()
            assert st.flush() == (1 if R_ == w.kG else 0)
        else:
            st.append(ks, vs)
        t += n
    assert st.state() == (w.T, w.R)
    got = _cache_arrays(st, w.T, w.n_blocks)
    for a, b in zip(got, ref):
        assert_slices_equal(a, b, mode)
    q = dev_f16(synth.query(w))
    o1 = host_u16(bulk.decode(q, w.sigma))
    o2 = host_u16(st.decode(q, w.sigma))
    assert np.array_equal(o1, o2)


def test_unflushed_full_residual(orc):
    """With no auto-flush a residual can hold all G keys; decode reads them
    as fp16 keys, and a flush then quantizes them as the next block."""
    w = _tiny(96, Hq=4, Hkv=2, D=64, G=32)
    cap = w.capacity(32)
    k, v = synth.keys(w), synth.values(w)
    dc = new_cache(w, cap)
    dc.append(dev_f16(k[:, :, :64]), dev_f16(v[:, :, :64]))
    dc.append(dev_f16(k[:, :, 64:]), dev_f16(v[:, :, 64:]), kvq.KVQ_APPEND_NO_AUTOFLUSH)
    assert dc.state() == (96, 32)
    _check_decode(orc, w, dc, k, v, kq_blocks=2)
    with pytest.raises(kvq.KvqError):
        dc.append(dev_f16(k[:, :, :1]), dev_f16(v[:, :, :1]), kvq.KVQ_APPEND_NO_AUTOFLUSH)
    assert dc.flush() == 1 and dc.state() == (96, 0)
    _check_decode(orc, w, dc, k, v)


@pytest.mark.parametrize("shape", ["gqa4_g32", "mha128_g32", "gqa4_g64", "mha128_g64", "mla64", "mla4_64"])
def test_unflushed_full_residual_mfma(orc, shape):
    """MFMA kernels: the KIVI tail then holds the longest it can, a whole
    quantized block plus a full residual (G = 32), or a full residual of 64
    keys (G = 64); the MLA kernel reads a full 64-key RoPE residual."""
    G = 32 if shape.endswith("g32") else 64
    nq = 3 * 32 if G == 32 else 2 * 64          # quantized tokens, odd block count for G = 32
    T = nq + G
    w = _tiny(T, Hq=8, Hkv=2, D=128, G=G) if shape.startswith("gqa4") else _shape(shape, T)
    assert w.kG == G
    cap = w.capacity(G)
    k, v = synth.keys(w), synth.values(w)
    dc = new_cache(w, cap)
    dc.append(dev_f16(k[:, :, :nq]), dev_f16(v[:, :, :nq]))
    dc.append(dev_f16(k[:, :, nq:]), dev_f16(v[:, :, nq:]), kvq.KVQ_APPEND_NO_AUTOFLUSH)
    assert dc.state() == (T, G)
    log(f"[{shape}] variant {dc.variant(w.n_q_heads)}")
    _check_decode(orc, w, dc, k, v, kq_blocks=nq // G)


@pytest.mark.parametrize("G,kbits", [(64, 2), (128, 2), (64, 4)])
def test_head_dim_32(orc, G, kbits):
    """kd = 32: fewer channel pairs than a wave's share when a block spans
    several row ranges (G > 32), bulk and single-token appends."""
    w = _tiny(3 * G + 7, Hq=2, Hkv=2, D=32, G=G, kbits=kbits)
    cap = w.capacity(8)
    k, v = synth.keys(w), synth.values(w)
    dc = new_cache(w, cap)
    n0 = w.T - 5
    dc.append(dev_f16(np.ascontiguousarray(k[:, :, :n0])), dev_f16(np.ascontiguousarray(v[:, :, :n0])))
    for t in range(n0, w.T):
        dc.append(dev_f16(np.ascontiguousarray(k[:, :, t:t + 1])), dev_f16(np.ascontiguousarray(v[:, :, t:t + 1])))
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            assert_slices_equal(slice_of(dc, b, h, w.T, w.n_blocks),
                                oracle_slice(orc, w, k[b, h], v[b, h], cap // w.kG, cap))
    _check_decode(orc, w, dc, k, v)


@pytest.mark.parametrize("kbits,vbits,G", [(4, 4, 32), (4, 2, 64), (2, 4, 16), (2, 2, 128), (4, 4, 16)])
def test_bit_widths_and_groups(orc, kbits, vbits, G):
    w = _tiny(3 * G + 7, Hq=4, Hkv=2, D=64, G=G, kbits=kbits, vbits=vbits)
    cap = w.capacity()
    k, v = synth.keys(w), synth.values(w)
    dc = new_cache(w, cap)
    dc.append(dev_f16(k), dev_f16(v))
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            assert_slices_equal(slice_of(dc, b, h, w.T, w.n_blocks),
                                oracle_slice(orc, w, k[b, h], v[b, h], cap // w.kG, cap))
    _check_decode(orc, w, dc, k, v)


def _adversarial_rows(n_rows, D, rng):
    """fp16 rows built to hit exact ties, near ties, constant and tiny-range
    groups, signed zeros and the extremes of the fp16 range."""
    rows = []
    for r in range(n_rows):
        kind = r % 6
        if kind == 0:      # exact ties: members (j + 1/2) * 2^e over [0, 3 * 2^e]
            e = int(rng.integers(-12, 10))
            vals = np.array([0, 3] + list(rng.integers(0, 7, D - 2) * 0.5), np.float64) * 2.0 ** e
        elif kind == 1:    # random finite bit patterns (wide dynamic range)
            bits = rng.integers(0, 0x7c00, D).astype(np.uint16) | (rng.integers(0, 2, D).astype(np.uint16) << 15)
            rows.append(bits)
            continue
        elif kind == 2:    # constant groups and signed zeros
            vals = np.full(D, float(rng.choice([0.0, -0.0, 1.5, -7.25])))
            vals[::3] = -0.0 if vals[0] == 0 else vals[0]
        elif kind == 3:    # tiny ranges: fp16 subnormal scales
            vals = rng.integers(0, 4, D) * 2.0 ** -24
        elif kind == 4:    # extremes
            vals = rng.choice([65504.0, -65504.0, 0.0, 1.0], D)
        else:              # dense small integers: many ties at scale 1
            vals = rng.integers(-3, 4, D).astype(np.float64)
        rows.append(vals.astype(np.float16).view(np.uint16))
    return np.stack(rows)


@pytest.mark.parametrize("G,bits", [(64, 2), (32, 2), (64, 4), (32, 4)])
def test_adversarial_quantization(orc, G, bits):
    """Bit-exact codes / scales / zeros on rows built to stress rounding, for
    both key groups and both code widths (keys and values)."""
    D, T = 128, 64 * 9
    rng = np.random.default_rng(11 + G + bits)
    w = configs.Workload("adv", 400, "kivi", 1, 2, 2, T, D, G, bits, D, 32, bits, 1.0)
    k = np.stack([_adversarial_rows(T, D, rng) for _ in range(2)])[None]
    v = np.stack([_adversarial_rows(T, D, rng) for _ in range(2)])[None]
    # keys are grouped down the token axis: also transpose-built blocks
    k[0, 1] = _adversarial_rows(D, T, rng).T
    cap = w.capacity()
    dc = new_cache(w, cap)
    dc.append(dev_f16(k), dev_f16(v))
    for h in range(2):
        assert_slices_equal(slice_of(dc, 0, h, T, T // G),
                            oracle_slice(orc, w, k[0, h], v[0, h], cap // G, cap), f"adv G{G} b{bits} h{h}")


def _near_tie_rows(T, D, bits, rng, glen=32):
    """fp16 groups of glen consecutive elements whose members sit at and
    within two fp16 ulps of the half-integer multiples of the group's scale,
    for random ranges and minima: the codes the reciprocal path cannot
    decide alone"""
    L = (1 << bits) - 1
    n = T * D // glen
    span = rng.integers(0x2000, 0x7800, n).astype(np.uint16).view(np.float16).astype(np.float32)
    mn = np.where(rng.random(n) < 0.5, 0.0, rng.standard_normal(n)).astype(np.float16).astype(np.float32)
    mx = (mn + span).astype(np.float16).astype(np.float32)
    mx = np.where(np.isfinite(mx) & (mx > mn), mx, mn + 1).astype(np.float16).astype(np.float32)
    scale = ((mx - mn) / np.float32(L)).astype(np.float32)
    k = rng.integers(0, L, (n, glen - 2))
    x = (mn[:, None] + (k + 0.5) * scale[:, None]).astype(np.float16)
    step = rng.integers(-2, 3, (n, glen - 2))
    for toward, cnt in ((np.float16(np.inf), 1), (np.float16(-np.inf), -1)):
        for _ in range(2):
            x = np.where(step * cnt > 0, np.nextafter(x, toward), x)
            step = step - np.where(step * cnt > 0, cnt, 0)
    x = np.clip(x.astype(np.float32), mn[:, None], mx[:, None]).astype(np.float16)
    grp = np.concatenate([mn[:, None].astype(np.float16), mx[:, None].astype(np.float16), x], axis=1)
    grp = grp[:, rng.permutation(glen)]
    return grp.reshape(T, D).view(np.uint16)


@pytest.mark.parametrize("G,bits", [(32, 2), (64, 2), (32, 4), (64, 4)])
def test_random_bit_pattern_fuzz(orc, G, bits):
    """Millions of codes from random finite fp16 patterns and from groups
    built around ties: the fast quotient path must agree with the IEEE
    division everywhere, for both key groups and both code widths."""
    D, T = 128, 8192
    rng = np.random.default_rng(12 + G + bits)
    w = configs.Workload("fuzz", 401, "kivi", 1, 2, 2, T, D, G, bits, D, 32, bits, 1.0)
    mag = rng.integers(0, 0x7c00, (1, 1, T, D)).astype(np.uint16)
    sign = (rng.integers(0, 2, (1, 1, T, D)).astype(np.uint16) << 15)
    # head 0: random patterns (keys) / narrow-exponent patterns, which make
    # near-ties between neighbouring values common (values); head 1: groups
    # built around ties, along the channel axis for values and, transposed,
    # along the token axis for keys
    k = np.concatenate([mag | sign, _near_tie_rows(D, T, bits, rng, G).T[None, None]], axis=1)
    v = np.concatenate([rng.integers(0x3800, 0x4400, (1, 1, T, D)).astype(np.uint16),
                        _near_tie_rows(T, D, bits, rng)[None, None]], axis=1)
    k, v = np.ascontiguousarray(k), np.ascontiguousarray(v)
    cap = w.capacity()
    dc = new_cache(w, cap)
    dc.append(dev_f16(k), dev_f16(v))
    for h in range(2):
        assert_slices_equal(slice_of(dc, 0, h, T, T // G),
                            oracle_slice(orc, w, k[0, h], v[0, h], cap // G, cap), f"fuzz G{G} b{bits} h{h}")


@pytest.mark.parametrize("shape", ["gqa4_g64", "gqa4", "mha128_g32", "mha128_g64", "mha", "mla64", "mla4_64",
                                   "gqa4_4bit_g64",
                                   "gqa4_4bit_g32", "mha128_4bit_g64", "mha128_4bit_g32"])
def test_decode_step_matches_separate_calls(orc, shape):
    """kv_decode_step (append fused into the attention launch for the GQA and
    MHA kernels while no block completes) against kv_quantize_append +
    kv_decode_attention: caches and outputs bit-identical over steps that
    cross key-block boundaries, starting from an empty cache."""
    G = 64 if shape in ("gqa4_g64", "mha128_g64", "mla64", "mla4_64", "gqa4_4bit_g64", "mha128_4bit_g64") else 32
    n0 = 2 * G - 3
    steps = G + 6
    w = _shape(shape, n0 + steps)
    cap = w.capacity(8)
    k, v, q = synth.keys(w), synth.values(w), synth.query(w)
    a, b = new_cache(w, cap), new_cache(w, cap)
    qd = dev_f16(q)
    t = torch()
    for dc in (a, b):
        dc.append(dev_f16(np.ascontiguousarray(k[:, :, :n0])), dev_f16(np.ascontiguousarray(v[:, :, :n0])))
    ws = a.workspace(w.n_q_heads)
    fused = 0
    for j in range(steps):
        tok = n0 + j
        kn = dev_f16(np.ascontiguousarray(k[:, :, tok:tok + 1]))
        vn = dev_f16(np.ascontiguousarray(v[:, :, tok:tok + 1]))
        fused += (tok % G) != G - 1
        oa = a.step(kn, vn, qd, w.sigma, ws=ws)
        b.append(kn, vn)
        ob = b.decode(qd, w.sigma)
        t.cuda.synchronize()
        assert a.state() == b.state() == (tok + 1, (tok + 1) % G)
        ga, gb = host_u16(oa), host_u16(ob)
        assert np.array_equal(ga, gb), (shape, tok, int(np.sum(ga != gb)))
    for bb in range(w.batch):
        for h in range(w.n_kv_heads):
            sa = slice_of(a, bb, h, w.T, w.n_blocks)
            assert_slices_equal(sa, slice_of(b, bb, h, w.T, w.n_blocks), f"{shape} b{bb} h{h}")
    _check_decode(orc, w, a, k, v)
    log(f"[step {shape}] variant {a.variant(w.n_q_heads)}, {steps} steps, {fused} with the append fused")


@pytest.mark.parametrize("G", [64, 32])
def test_gqa_4bit_full_size(orc, G):
    """The 32K-token, 32q/8kv, D = 128 GQA workload with 4-bit keys and
    values (4 KB tiles on the matrix cores), at batch 4: the whole cache
    bit-exact and attention within 2e-3 on every (sequence, query head)."""
    import dataclasses
    base = configs.BY_NAME["mistral_7b_gqa_t32805"]
    w = dataclasses.replace(base, name=f"gqa_4bit_g{G}", kG=G, kbits=4, vbits=4, batch=4)
    cap = w.capacity(64)
    k, v, q = synth.keys(w), synth.values(w), synth.query(w)
    dc = new_cache(w, cap)
    dc.append(dev_f16(k), dev_f16(v))
    assert dc.variant(w.n_q_heads) == "gqa_mfma"
    got = _decode(dc, w, q)
    host = _host_arrays(dc)
    dc.close()
    cache = orc.build_cache(k, v, w.kG, w.kbits, w.vG, w.vbits, nblk_cap=cap // w.kG, tok_cap=cap, threads=None)
    assert_cache_equal(host, cache, w.T, w.n_blocks, f"4-bit G{G}")
    ref = oracle_attention(orc, w, cache, q)
    worst = float(np.abs(got - ref).max())
    excess = mean_excess(got.ravel(), ref.ravel())
    log(f"[4-bit G{G}] max|err| {worst:.3e} mean excess {excess:.2e}")
    assert worst <= TOL
    assert excess <= MEAN_EXCESS_TOL


def test_mla_int4_full_size(orc):
    """QuantMLA's INT4/INT4 cache (content latent and RoPE key both 4-bit) at
    the MLA workload's shape, 8 sequences of 16384 tokens, 128 heads: the
    whole cache bit-exact and every (sequence, head) within 2e-3."""
    import dataclasses
    base = configs.BY_NAME["mla_absorbed_b64_t16384"]
    w = dataclasses.replace(base, name="mla_int4_b8", vbits=4, batch=8)
    cap = w.capacity(64)
    k, v, q = synth.keys(w), synth.values(w), synth.query(w)
    dc = new_cache(w, cap)
    dc.append(dev_f16(k), dev_f16(v))
    assert dc.variant(w.n_q_heads) == "mla_mfma"
    got = _decode(dc, w, q)
    host = _host_arrays(dc)
    dc.close()
    cache = orc.build_cache(k, v, w.kG, w.kbits, w.vG, w.vbits, nblk_cap=cap // w.kG, tok_cap=cap, threads=None)
    assert_cache_equal(host, cache, w.T, w.n_blocks, "mla int4")
    ref = oracle_attention(orc, w, cache, q)
    worst = float(np.abs(got - ref).max())
    excess = mean_excess(got.ravel(), ref.ravel())
    log(f"[mla int4] max|err| {worst:.3e} mean excess {excess:.2e} max|o| {np.abs(ref).max():.3f}")
    assert worst <= TOL
    assert excess <= MEAN_EXCESS_TOL


def _rising_keys(w, k_u16, q_u16, rate):
    """Keys whose logits climb by about `rate` (natural units) per token for
    the mean query of each KV head's group, so that the kernels' running
    maxima move over and over after the first tile (and the accumulators get
    rescaled mid-run); the values are untouched."""
    k = k_u16.view(np.float16).astype(np.float64)
    q = q_u16.view(np.float16).astype(np.float64)
    g = w.n_q_heads // w.n_kv_heads
    qk = q[..., -w.kd:]   # the part of q that meets the keys: all of it (KIVI), q_r (MLA)
    ramp = np.arange(k.shape[2], dtype=np.float64)[:, None]
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            rows = qk[b, h * g:(h + 1) * g]
            d = rows.mean(axis=0)
            d /= np.linalg.norm(d)
            a = rate / (w.sigma * np.abs(rows @ d).mean())
            k[b, h] += a * ramp * d[None, :]
    return k.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("n_splits", [0, 1])
@pytest.mark.parametrize("shape", ["mha128_g32", "mha128_g64", "gqa4_g64", "gqa4", "gqa4_4bit_g64", "mla64",
                                   "mla128", "mla4_128"])
def test_rising_logits(orc, shape, n_splits):
    """Maxima that keep moving: every lazy rescale path against the oracle."""
    T = 700
    w = _tiny(T, Hq=8, Hkv=2, D=128) if shape == "gqa4" else _shape(shape, T)
    cap = w.capacity(16)
    k = _rising_keys(w, synth.keys(w), synth.query(w), 0.5)
    v = synth.values(w)
    dc = new_cache(w, cap)
    dc.append(dev_f16(k), dev_f16(v))
    log(f"[rising {shape}] variant {dc.variant(w.n_q_heads)}, splits {n_splits}")
    _check_decode(orc, w, dc, k, v, n_splits=n_splits)
