"""Pins for the CPU oracle (no GPU): the oracle is checked against things other
than itself -- numpy's binary16 conversion, worked values fixed by exact
rational arithmetic, closed forms, invariants of the quantizer the pages
describe ("Makale Bülteni -- KIVI", section "İddia ve Gerçeklik: KIVI"), and
an independent numpy fp64 brute force over the documented cache layout.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from decode_attention_asym_amd import configs, synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quant_worked_values.json")))
CASES = {c["id"]: c for c in GOLD["cases"]}


def h(x):
    return int(x, 16)


# ------------------------------------------------------------ helpers (numpy)

def f32_of_fraction(x: Fraction) -> float:
    """Exact rational -> nearest binary32 (ties to even), normal range only."""
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    m = x / Fraction(2) ** (e - 23)          # in [2^23, 2^24)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(Fraction(fl) * Fraction(2) ** (e - 23))


def f32_bits(x: float) -> int:
    return int(np.array(x, np.float32).view(np.uint32))


def np_unpack(words: np.ndarray, bits: int) -> np.ndarray:
    """Codes of u32 words, LSB first: [..., W] -> [..., W * 32/bits]."""
    per = 32 // bits
    sh = (np.arange(per, dtype=np.uint32) * bits).astype(np.uint32)
    c = (words[..., None] >> sh) & np.uint32((1 << bits) - 1)
    return c.reshape(*words.shape[:-1], words.shape[-1] * per).astype(np.int64)


def f16(bits_arr) -> np.ndarray:
    return np.asarray(bits_arr, np.uint16).view(np.float16).astype(np.float64)


def np_dequant_keys(cache, b, h_):
    """Key rows [T][kd] from the documented layout: codes [blk][c][words],
    word j of channel c holding tokens (32/bits)*j.. of the block."""
    k = cache.k
    T, G, bits = cache.s.T, cache.s.kG, cache.s.kbits
    nb, R = T // G, T % G
    codes = np_unpack(k["k_codes"][b, h_, :nb], bits)          # [nb][kd][G]
    khat = codes * f16(k["k_scale"][b, h_, :nb])[..., None] + f16(k["k_zero"][b, h_, :nb])[..., None]
    khat = khat.transpose(0, 2, 1).reshape(nb * G, cache.s.kd)   # [nb*G][kd]
    resid = f16(k["k_resid"][b, h_, :R])
    return np.concatenate([khat, resid], 0)


def np_dequant_values(cache, b, h_):
    v = cache.v
    T, Gv, bits = cache.s.T, cache.s.vG, cache.s.vbits
    codes = np_unpack(v["v_codes"][b, h_, :T], bits)            # [T][vd]
    sc = np.repeat(f16(v["v_scale"][b, h_, :T]), Gv, axis=1)
    ze = np.repeat(f16(v["v_zero"][b, h_, :T]), Gv, axis=1)
    return codes * sc + ze


def np_softmax_attend(s, vhat):
    s = s - s.max()
    p = np.exp(s)
    return (p[:, None] * vhat).sum(0) / p.sum()


# ---------------------------------------------------------------- fp16 pins

def test_half_to_float_all_patterns(orc):
    allh = np.arange(65536, dtype=np.uint16)
    got = orc.half_to_float(allh)
    ref = allh.view(np.float16).astype(np.float32)
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_float_to_half_matches_numpy(orc):
    r = np.random.default_rng(1)
    f = np.concatenate([
        r.standard_normal(1 << 18).astype(np.float32) * np.float32(300),
        (r.random(1 << 18) * 1e-4).astype(np.float32),                      # subnormal fp16 range
        r.integers(0, 2**32, 1 << 18, dtype=np.uint64).astype(np.uint32).view(np.float32),
        # exact ties between neighbouring fp16 values, both parities
        ((np.arange(2048, dtype=np.float32) + np.float32(0.5)) * np.float32(2.0 ** -24)),
        ((np.arange(1024, 2048, dtype=np.float32) + np.float32(0.5)) * np.float32(2.0 ** -10)),
        np.array([65504, 65519.99, 65520, 65536, -65520, 6.0e-8, 2.0 ** -25, 2.0 ** -26], np.float32),
    ])
    f = f[np.isfinite(f)]
    with np.errstate(over="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    assert (orc.float_to_half(f) == ref).all()


# ------------------------------------------------------------ worked values

@pytest.mark.parametrize("cid", sorted(CASES))
def test_worked_values(orc, cid):
    c = CASES[cid]
    x = np.array([h(v) for v in c["x_f16"]], np.uint16)
    codes, sh, zh, s32 = orc.quant_group(x, c["bits"])
    assert codes.tolist() == c["codes"]
    assert sh == h(c["scale_h"]) and zh == h(c["zero_h"])
    assert f32_bits(s32) == h(c["scale32"])
    if "words" in c:
        assert [int(w) for w in orc.pack(codes, c["bits"])] == [h(w) for w in c["words"]]


def test_worked_values_fp32_facts():
    """The fixture's binary32 facts, from exact rationals (independent of the oracle)."""
    third = f32_of_fraction(Fraction(1, 3))
    assert f32_bits(third) == 0x3EAAAAAB
    q = Fraction(1, 2) / Fraction(third)
    assert q < Fraction(3, 2) and f32_of_fraction(q) == 1.5          # W3: rounds up to the tie
    mn, mx, x = (Fraction(float(np.uint16(v).view(np.float16))) for v in (0x3C26, 0x40EE, 0x3F01))
    rng = f32_of_fraction(mx - mn)
    s = f32_of_fraction(Fraction(rng) / 3)
    assert f32_bits(s) == 0x3EF3AAAB
    d = f32_of_fraction(x - mn)
    assert f32_of_fraction(Fraction(d) / Fraction(s)) == 1.5         # W4 true quotient -> code 2
    rcp = f32_of_fraction(1 / Fraction(s))
    assert f32_of_fraction(Fraction(d) * Fraction(rcp)) < 1.5        # W4 reciprocal -> code 1
    assert int(np.float16(s).view(np.uint16)) == 0x379D


# --------------------------------------------------------------- invariants

def _random_groups(rng, n_groups, n, kind):
    if kind == "normal":
        x = rng.standard_normal((n_groups, n)).astype(np.float32)
    elif kind == "outlier":
        x = rng.standard_normal((n_groups, n)).astype(np.float32) * np.float32(50)
    elif kind == "shifted":
        x = (rng.standard_normal((n_groups, n)) * 0.01 + 700).astype(np.float32)
    else:  # few distinct values -> many exact ties
        x = rng.integers(-4, 5, (n_groups, n)).astype(np.float32) * np.float32(0.5)
    return x.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("kind", ["normal", "outlier", "shifted", "ties"])
def test_error_bound_and_extremes(orc, bits, kind):
    rng = np.random.default_rng(bits * 10 + len(kind))
    L = (1 << bits) - 1
    for grp in _random_groups(rng, 300, 32, kind):
        codes, sh, zh, s32 = orc.quant_group(grp, bits)
        x = f16(grp)
        mn, mx = x.min(), x.max()
        if mx == mn:
            assert (codes == 0).all()
            continue
        # I3: the extremes map to 0 and L
        assert codes[x.argmin()] == 0 and codes[x.argmax()] == L
        # I2 with the fp32 scale and with the stored fp16 side values
        err32 = np.abs(x - (codes * s32 + mn))
        assert (err32 <= s32 / 2 + 2.0 ** -22 * (mx - mn)).all()
        err16 = np.abs(x - (codes * f16(sh) + f16(zh)))
        assert (err16 <= s32 * (0.5 + 3 * 2.0 ** -11 * L / 3) + 2.0 ** -22 * (mx - mn) + 1e-12).all()
        assert f16(zh) == mn


def test_constant_group_exact(orc):
    for v in [0.0, -0.0, 1.0, -3.5, 65504.0, 6.0e-8]:
        grp = np.full(32, v, np.float16).view(np.uint16)
        codes, sh, zh, s32 = orc.quant_group(grp, 2)
        assert (codes == 0).all() and sh == 0 and s32 == 0.0
        assert zh == np.float16(v + 0.0).view(np.uint16)  # -0 canonicalised to +0
    mixed = np.array([0x8000, 0x0000] * 8, np.uint16)
    assert orc.quant_group(mixed, 2)[2] == 0x0000


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_roundtrip(orc, bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, 32 * 64).astype(np.uint8)
    words = orc.pack(codes, bits)
    assert (np_unpack(words, bits) == codes).all()
    assert (orc.unpack(words, codes.size, bits) == codes).all()


@pytest.mark.parametrize("G,kbits,vbits", [(32, 2, 2), (64, 2, 2), (64, 4, 4), (32, 4, 4), (64, 4, 2), (16, 2, 4)])
def test_layout_dequant_tracks_input(orc, G, kbits, vbits):
    """Dequantized keys/values, read through the documented layout by numpy,
    sit within the I2 bound of the input at the same (token, channel), for
    both key groups of the workloads (32, 64) and both code widths (the MLA
    RoPE key is a 4-bit, G = 64 key stream).  A transposed, mis-indexed or
    mis-packed store fails this at any of these settings."""
    import dataclasses
    w = dataclasses.replace(configs.WORKLOADS[0], kG=G, kbits=kbits, vbits=vbits)
    Lk, Lv = (1 << kbits) - 1, (1 << vbits) - 1
    for b, hh in [(0, 0), (0, 1)]:
        k = synth.key_slice(w, b, hh)[None, None]
        v = synth.value_slice(w, b, hh)[None, None]
        cache = orc.build_cache(k, v, w.kG, w.kbits, w.vG, w.vbits)
        kh, vh = np_dequant_keys(cache, 0, 0), np_dequant_values(cache, 0, 0)
        assert np.array_equal(kh, orc.dequant_keys(cache, 0, 0))
        assert np.array_equal(vh, orc.dequant_values(cache, 0, 0))
        kx, vx = f16(k[0, 0]), f16(v[0, 0])
        nb = w.T // w.kG
        assert nb >= 3
        for blk in range(nb):
            sl = slice(blk * w.kG, (blk + 1) * w.kG)
            rngk = kx[sl].max(0) - kx[sl].min(0)
            bound = rngk / Lk * (0.5 + Lk * 2.0 ** -11) * (1 + 1e-6) + 1e-9
            assert (np.abs(kh[sl] - kx[sl]) <= bound).all()
            # a tighter bound than a neighbouring token's value would meet
            assert np.abs(kh[sl] - kx[sl]).max() < np.abs(np.diff(kx[sl], axis=0)).max()
        assert np.array_equal(kh[nb * w.kG:], kx[nb * w.kG:])  # residual kept exactly
        for g in range(w.vd // w.vG):
            sl = slice(g * w.vG, (g + 1) * w.vG)
            rngv = vx[:, sl].max(1, keepdims=True) - vx[:, sl].min(1, keepdims=True)
            bound = rngv / Lv * (0.5 + Lv * 2.0 ** -11) * (1 + 1e-6) + 1e-9
            assert (np.abs(vh[:, sl] - vx[:, sl]) <= bound).all()


def test_outlier_confinement(orc):
    """I5: scaling the outlier key channels leaves every other channel's codes,
    scales and zeros bit-identical ("İddia ve Gerçeklik: KIVI": per-channel
    grouping keeps outlier error inside its channel)."""
    w = configs.WORKLOADS[0]
    flat = synth.outlier_channels(w)
    assert flat.size == 2
    for hh in range(w.n_kv_heads):
        out_ch = set((flat[flat // w.kd == hh] % w.kd).tolist())
        a = orc.quantize_keys(synth.key_slice(w, 0, hh)[None, None], w.kG, w.kbits)
        b = orc.quantize_keys(synth.key_slice(w, 0, hh, outliers=False)[None, None], w.kG, w.kbits)
        for c in range(w.kd):
            same = all(np.array_equal(a[n][0, 0, :, c], b[n][0, 0, :, c])
                       for n in ("k_codes", "k_scale", "k_zero"))
            assert same == (c not in out_ch)


def test_per_token_keys_collapse_contrast(orc):
    """The pages' contrast: quantizing keys per token lets an outlier channel
    set every group's scale, wrecking the normal channels; per channel does not."""
    w = configs.WORKLOADS[0]
    k = synth.key_slice(w, 0, 0)
    flat = synth.outlier_channels(w)
    normal = np.setdiff1d(np.arange(w.kd), flat[flat // w.kd == 0] % w.kd)
    x = f16(k)
    per_channel = orc.quantize_keys(k[None, None], w.kG, 2)
    cache = orc.Cache(w.T, w.kG, 2, w.vG, 2, per_channel,
                      orc.quantize_values(synth.value_slice(w, 0, 0)[None, None], w.vG, 2))
    err_pc = np.abs(orc.dequant_keys(cache, 0, 0) - x)[:, normal].mean()
    tok = orc.quantize_values(k[None, None], w.kd, 2)  # one group = all channels of a token
    codes = np_unpack(tok["v_codes"][0, 0], 2)
    deq = codes * f16(tok["v_scale"][0, 0]) + f16(tok["v_zero"][0, 0])
    err_pt = np.abs(deq - x)[:, normal].mean()
    if flat[flat // w.kd == 0].size:
        assert err_pt > 5 * err_pc


# ---------------------------------------------------------------- attention

def _tiny_kivi(T, B=1, Hq=2, Hkv=2, D=64, G=32, seed=7):
    return configs.Workload("t", 100 + seed, "kivi", B, Hq, Hkv, T, D, G, 2, D, 32, 2, 50.0)


def _cache_for(orc, w, T=None):
    T = w.T if T is None else T
    k = synth.keys(w, T)
    v = synth.values(w, T)
    return orc.build_cache(k, v, w.kG, w.kbits, w.vG, w.vbits), k, v


def _np_attention_kivi(cache, q_bits, sigma):
    B, H, T, kd, vd = cache.dims
    Hq = q_bits.shape[1]
    out = np.zeros((B, Hq, vd))
    q = f16(q_bits)
    for b in range(B):
        for hq in range(Hq):
            kvh = hq // (Hq // H)
            kh, vh = np_dequant_keys(cache, b, kvh), np_dequant_values(cache, b, kvh)
            out[b, hq] = np_softmax_attend(float(np.float32(sigma)) * (kh @ q[b, hq]), vh)
    return out


def _np_attention_mla(cache, q_bits, sigma):
    B, H, T, kd, vd = cache.dims
    Hq = q_bits.shape[1]
    out = np.zeros((B, Hq, vd))
    q = f16(q_bits)
    for b in range(B):
        ch, kr = np_dequant_values(cache, b, 0), np_dequant_keys(cache, b, 0)
        for hq in range(Hq):
            s = float(np.float32(sigma)) * (ch @ q[b, hq, :vd] + kr @ q[b, hq, vd:])
            out[b, hq] = np_softmax_attend(s, ch)
    return out


@pytest.mark.parametrize("T", [1, 31, 32, 33, 101, 250])
@pytest.mark.parametrize("heads", [(2, 2), (4, 2), (4, 1)])
def test_attention_bruteforce_kivi(orc, T, heads):
    """I9: independent numpy fp64 attention over numpy-dequantized K/V."""
    Hq, Hkv = heads
    w = _tiny_kivi(T, B=2, Hq=Hq, Hkv=Hkv)
    cache, _, _ = _cache_for(orc, w)
    q = synth.query(w)
    got = orc.attention_kivi(cache, q, w.sigma, nthreads=4)
    ref = _np_attention_kivi(cache, q, w.sigma)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_attention_bruteforce_workload0(orc):
    w = configs.WORKLOADS[0]
    cache, _, _ = _cache_for(orc, w)
    q = synth.query(w)
    got = orc.attention_kivi(cache, q, w.sigma)
    ref = _np_attention_kivi(cache, q, w.sigma)
    assert np.abs(got - ref).max() <= 1e-12


@pytest.mark.parametrize("vbits", [2, 4])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_attention_bruteforce_mla(orc, T, vbits):
    """MLA with the content latent at INT2 or INT4 (QuantMLA's two content
    widths) and the RoPE key at INT4, against numpy over the documented
    layouts."""
    w = configs.Workload("m", 150, "mla", 2, 8, 1, T, 64, 64, 4, 128, 32, vbits, 20.0)
    cache, _, _ = _cache_for(orc, w)
    q = synth.query(w)
    got = orc.attention_mla(cache, q, w.sigma, nthreads=2)
    ref = _np_attention_mla(cache, q, w.sigma)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_attention_pairs_subset(orc):
    w = _tiny_kivi(77, B=3, Hq=4, Hkv=2)
    cache, _, _ = _cache_for(orc, w)
    q = synth.query(w)
    full = orc.attention_kivi(cache, q, w.sigma)
    pairs = [(2, 3), (0, 1), (1, 0)]
    sub = orc.attention_kivi(cache, q, w.sigma, pairs=pairs)
    for i, (b, hq) in enumerate(pairs):
        assert np.array_equal(sub[i], full[b, hq])


def test_attention_closed_forms(orc):
    """I7: q = 0 gives the mean of the dequantized values; a dominating logit
    selects its token; T < G is plain attention over the fp16 keys; GQA with
    identical heads equals MHA."""
    w = _tiny_kivi(100)
    cache, k, v = _cache_for(orc, w)
    q0 = np.zeros((1, 2, 64), np.uint16)
    o = orc.attention_kivi(cache, q0, w.sigma)
    for hh in range(2):
        assert np.allclose(o[0, hh], np_dequant_values(cache, 0, hh).mean(0), rtol=0, atol=1e-12)
    # dominating logit: a query along one token's key with a huge scale
    kh = np_dequant_keys(cache, 0, 0)
    qv = np.float16(kh[57] / np.linalg.norm(kh[57]))
    qbits = np.stack([qv, qv])[None].view(np.uint16)
    s = kh @ qv.astype(np.float64)
    tstar = int(np.argmax(s))
    sigma = float(60.0 / (s[tstar] - np.partition(s, -2)[-2]))
    o = orc.attention_kivi(cache, qbits, sigma)
    assert np.allclose(o[0, 0], np_dequant_values(cache, 0, 0)[tstar], atol=1e-9)
    # T < G: every key is a residual key
    ws = _tiny_kivi(20)
    cs, ks, vs = _cache_for(orc, ws)
    qs = synth.query(ws)
    o = orc.attention_kivi(cs, qs, ws.sigma)
    for hh in range(2):
        s = float(np.float32(ws.sigma)) * (f16(ks[0, hh]) @ f16(qs[0, hh]))
        assert np.allclose(o[0, hh], np_softmax_attend(s, np_dequant_values(cs, 0, hh)), atol=1e-12)
    # GQA with identical query heads inside each group == MHA on one head per group
    wg = _tiny_kivi(90, Hq=4, Hkv=2)
    cg, _, _ = _cache_for(orc, wg)
    qg = synth.query(wg)
    qg[0, 1], qg[0, 3] = qg[0, 0], qg[0, 2]
    og = orc.attention_kivi(cg, qg, wg.sigma)
    om = orc.attention_kivi(cg, qg[:, [0, 2]], wg.sigma)
    assert np.array_equal(og[0, 0], om[0, 0]) and np.array_equal(og[0, 1], om[0, 0])
    assert np.array_equal(og[0, 2], om[0, 1]) and np.array_equal(og[0, 3], om[0, 1])


def test_synth_prefix_property():
    w = configs.WORKLOADS[0]
    a = synth.key_slice(w, 0, 1, T=40)
    b = synth.key_slice(w, 0, 1, T=250)
    assert np.array_equal(a, b[:40])
    assert synth.outlier_channels(configs.WORKLOADS[2]).size == 11
    assert synth.outlier_channels(configs.WORKLOADS[1]).size == 41
    assert synth.outlier_channels(configs.WORKLOADS[4]).size == 1


def test_attention_unflushed_full_residual(orc):
    """A residual that reached G keys without a flush keeps them in fp16."""
    w = _tiny_kivi(96, Hq=4, Hkv=2)          # 3 blocks of 32; the last stays fp16
    k, v = synth.keys(w), synth.values(w)
    cache = orc.build_cache(k, v, w.kG, w.kbits, w.vG, w.vbits, kq_blocks=2)
    q = synth.query(w)
    got = orc.attention_kivi(cache, q, w.sigma)
    flushed = orc.build_cache(k[:, :, :64], v[:, :, :64], w.kG, w.kbits, w.vG, w.vbits)
    for hq in range(4):
        kvh = hq // 2
        kh = np.concatenate([np_dequant_keys(flushed, 0, kvh), f16(k[0, kvh, 64:])], 0)
        vh = np_dequant_values(cache, 0, kvh)
        s = float(np.float32(w.sigma)) * (kh @ f16(q[0, hq]))
        assert np.abs(got[0, hq] - np_softmax_attend(s, vh)).max() <= 1e-12
