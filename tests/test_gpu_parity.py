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


@pytest.mark.parametrize("name", FULL)
def test_workload_parity(orc, name):
    """Full-size workload: bulk prefill quantize, then decode attention.  The
    cache is compared on every (b, kv head) slice for the two small
    workloads and on sampled slices for the large ones; attention on every
    query head of the sampled slices."""
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
    BH = w.batch * w.n_kv_heads
    group = w.n_q_heads // w.n_kv_heads
    if BH * w.T <= (1 << 20) + 1:
        slices = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
        slices = slices[::8] + [slices[-1]] if len(slices) > 32 else slices
    else:
        slices = sorted({(b, hq // group) for b, hq in sample_pairs(w, 4, seed=w.index)})
    worst, omax, gots, refs = 0.0, 0.0, [], []
    for b, h in slices:
        ref = oracle_slice(orc, w, k[b, h], v[b, h], cap // w.kG, cap)
        assert_slices_equal(slice_of(dc, b, h, w.T, w.n_blocks), ref, f"{name} b{b} h{h}")
        heads = range(h * group, (h + 1) * group)
        if w.kind == "mla":
            heads = list(range(0, w.n_q_heads, 16)) + [w.n_q_heads - 1]
        cache = oracle_cache_full(orc, w, k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], cap)
        qs = q[b:b + 1, list(heads)]
        if w.kind == "kivi":
            qs = np.ascontiguousarray(qs)
            # a one-head cache: every query head of the slice maps onto it
            sub = configs.Workload(w.name, w.index, "kivi", 1, len(heads), 1, w.T, w.kd, w.kG,
                                   w.kbits, w.vd, w.vG, w.vbits, w.outlier_scale)
        else:
            qs = np.ascontiguousarray(qs)
            sub = configs.Workload(w.name, w.index, "mla", 1, len(heads), 1, w.T, w.kd, w.kG,
                                   w.kbits, w.vd, w.vG, w.vbits, w.outlier_scale)
        ref_o = oracle_attention(orc, sub, cache, qs)[0]
        gots.append(got[b, list(heads)].ravel())
        refs.append(ref_o.ravel())
        worst = max(worst, np.abs(gots[-1] - refs[-1]).max())
        omax = max(omax, np.abs(ref_o).max())
    excess = mean_excess(np.concatenate(gots), np.concatenate(refs))
    log(f"[{name}] slices {len(slices)} max|err| {worst:.3e} mean excess {excess:.2e} max|o| {omax:.3f}")
    assert worst <= TOL
    assert excess <= MEAN_EXCESS_TOL


def _tiny(T, Hq=4, Hkv=2, D=64, G=32, kbits=2, vbits=2, B=2, idx=200):
    return configs.Workload("tiny", idx, "kivi", B, Hq, Hkv, T, D, G, kbits, D, 32, vbits, 50.0)


def _mla_tiny(T, Hq=16, B=2, idx=300):
    return configs.Workload("mla_tiny", idx, "mla", B, Hq, 1, T, 64, 64, 4, 512, 32, 2, 20.0)


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
    raise KeyError(shape)


@pytest.mark.parametrize("T", [1, 15, 31, 32, 33, 101, 3 * 64 + 5, 700])
@pytest.mark.parametrize("shape", ["mha", "mha128_g32", "mha128_g64", "gqa4", "gqa8_g64", "mla", "mla64",
                                   "mla128", "gqa4_4bit_g64", "gqa4_4bit_g32", "mha128_4bit_g64",
                                   "mha128_4bit_g32"])
def test_edge_lengths(orc, T, shape):
    if shape in ("mha", "mha128_g32", "mha128_g64", "mla64", "mla128", "gqa4_4bit_g64", "gqa4_4bit_g32",
                 "mha128_4bit_g64", "mha128_4bit_g32"):
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
@pytest.mark.parametrize("shape", ["gqa4", "mha128_g32", "mla64", "gqa4_4bit_g64", "gqa4_4bit_g32", "mha128_4bit_g32"])
def test_split_counts(orc, n_splits, shape):
    w = _tiny(1000, Hq=8, Hkv=2, D=128, G=32) if shape == "gqa4" else _shape(shape, 1000)
    cap = w.capacity()
    k, v = synth.keys(w), synth.values(w)
    dc = new_cache(w, cap)
    dc.append(dev_f16(k), dev_f16(v))
    _check_decode(orc, w, dc, k, v, n_splits=n_splits)


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


@pytest.mark.parametrize("shape", ["gqa4_g32", "mha128_g32", "gqa4_g64", "mha128_g64", "mla64"])
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


def test_adversarial_quantization(orc):
    """Bit-exact codes / scales / zeros on rows built to stress rounding."""
    D, T = 128, 64 * 9
    rng = np.random.default_rng(11)
    w = configs.Workload("adv", 400, "kivi", 1, 2, 2, T, D, 64, 2, D, 32, 2, 1.0)
    k = np.stack([_adversarial_rows(T, D, rng) for _ in range(2)])[None]
    v = np.stack([_adversarial_rows(T, D, rng) for _ in range(2)])[None]
    # keys are grouped down the token axis: also transpose-built blocks
    k[0, 1] = _adversarial_rows(D, T, rng).T
    cap = w.capacity()
    dc = new_cache(w, cap)
    dc.append(dev_f16(k), dev_f16(v))
    for h in range(2):
        assert_slices_equal(slice_of(dc, 0, h, T, T // 64),
                            oracle_slice(orc, w, k[0, h], v[0, h], cap // 64, cap), f"adv h{h}")


def test_random_bit_pattern_fuzz(orc):
    """Millions of codes from random finite fp16 patterns: the fast quotient
    path must agree with the IEEE division everywhere."""
    D, T = 128, 8192
    rng = np.random.default_rng(12)
    w = configs.Workload("fuzz", 401, "kivi", 1, 1, 1, T, D, 32, 2, D, 32, 2, 1.0)
    mag = rng.integers(0, 0x7c00, (1, 1, T, D)).astype(np.uint16)
    sign = (rng.integers(0, 2, (1, 1, T, D)).astype(np.uint16) << 15)
    k = mag | sign
    # narrow-exponent patterns make near-ties between neighbouring values common
    v = (rng.integers(0x3800, 0x4400, (1, 1, T, D)).astype(np.uint16))
    cap = w.capacity()
    dc = new_cache(w, cap)
    dc.append(dev_f16(k), dev_f16(v))
    assert_slices_equal(slice_of(dc, 0, 0, T, T // 32),
                        oracle_slice(orc, w, k[0, 0], v[0, 0], cap // 32, cap), "fuzz")


@pytest.mark.parametrize("shape", ["gqa4_g64", "gqa4", "mha128_g32", "mha128_g64", "mha", "mla64", "gqa4_4bit_g64",
                                   "gqa4_4bit_g32", "mha128_4bit_g64", "mha128_4bit_g32"])
def test_decode_step_matches_separate_calls(orc, shape):
    """kv_decode_step (append fused into the attention launch for the GQA and
    MHA kernels while no block completes) against kv_quantize_append +
    kv_decode_attention: caches and outputs bit-identical over steps that
    cross key-block boundaries, starting from an empty cache."""
    G = 64 if shape in ("gqa4_g64", "mha128_g64", "mla64", "gqa4_4bit_g64", "mha128_4bit_g64") else 32
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
    values (4 KB tiles on the matrix cores): cache bit-exact and attention
    within 2e-3 on sampled (sequence, KV head) slices."""
    import dataclasses
    base = configs.BY_NAME["mistral_7b_gqa_t32805"]
    w = dataclasses.replace(base, name=f"gqa_4bit_g{G}", kG=G, kbits=4, vbits=4, batch=4)
    cap = w.capacity(64)
    k, v, q = synth.keys(w), synth.values(w), synth.query(w)
    dc = new_cache(w, cap)
    dc.append(dev_f16(k), dev_f16(v))
    assert dc.variant(w.n_q_heads) == "gqa_mfma"
    got = _decode(dc, w, q)
    group = w.n_q_heads // w.n_kv_heads
    worst, gots, refs = 0.0, [], []
    for b, h in [(0, 0), (1, 5), (3, 7)]:
        ref = oracle_slice(orc, w, k[b, h], v[b, h], cap // w.kG, cap)
        assert_slices_equal(slice_of(dc, b, h, w.T, w.n_blocks), ref, f"4-bit G{G} b{b} h{h}")
        heads = list(range(h * group, (h + 1) * group))
        cache = oracle_cache_full(orc, w, k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], cap)
        sub = configs.Workload(w.name, w.index, "kivi", 1, group, 1, w.T, w.kd, w.kG, w.kbits, w.vd, w.vG, w.vbits,
                               w.outlier_scale)
        ref_o = oracle_attention(orc, sub, cache, np.ascontiguousarray(q[b:b + 1, heads]))[0]
        gots.append(got[b, heads].ravel())
        refs.append(ref_o.ravel())
        worst = max(worst, float(np.abs(gots[-1] - refs[-1]).max()))
    excess = mean_excess(np.concatenate(gots), np.concatenate(refs))
    log(f"[4-bit G{G}] max|err| {worst:.3e} mean excess {excess:.2e}")
    assert worst <= TOL
    assert excess <= MEAN_EXCESS_TOL
