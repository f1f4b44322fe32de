"""GPU parity of kv_prefill_attention (causal prompt attention on the matrix
cores, fused with the bulk quantize of the prompt) through the C ABI.

Outputs are compared with the oracle's fp64 causal attention over the same
fp16 bits, at the decode path's bar: max-abs 2e-3 (fp16 output against the
unrounded fp64 result) plus the mean-excess bound.  From the arithmetic: the
weights enter the PV product as fp16 hi + lo pairs (relative error ~2^-22)
against an unrounded l, the logits are fp32 sums of exact fp16 products, and
the fp16 output adds at most half an ulp (9.8e-4 for |o| < 4, 1.95e-3 below
8), so the kernel's own error is orders below the bar.  The cache must
equal, bit for bit, both a twin cache filled by kv_quantize_append from the
same tensors and the oracle's quantizer.
"""
import dataclasses

import numpy as np
import pytest

from gpu_util import (MEAN_EXCESS_TOL, TOL, assert_slices_equal, configs, dev_f16, host_u16, kvq, log, mean_excess,
                      new_cache, oracle_slice, slice_of, synth, torch)

pytestmark = pytest.mark.gpu

SHAPES = {  # B, Hq, Hkv, G, key bits, value bits
    "gqa4_g64": (2, 8, 2, 64, 2, 2),
    "gqa4_g32": (2, 8, 2, 32, 2, 2),
    "mha_g32": (1, 3, 3, 32, 2, 2),
    "gqa8_g64": (1, 16, 2, 64, 2, 2),
    "gqa4_4bit": (2, 8, 2, 64, 4, 4),
    "gqa4_k2v4_g32": (1, 4, 1, 32, 2, 4),
}
MEAN_TOL = MEAN_EXCESS_TOL


def _workload(shape, T):
    B, Hq, Hkv, G, kb, vb = SHAPES[shape]
    return configs.Workload("prefill_" + shape, 530 + list(SHAPES).index(shape), "kivi", B, Hq, Hkv, T, 128, G, kb,
                            128, 32, vb, 50.0)


def _inputs(w):
    return synth.prompt_queries(w), synth.keys(w), synth.values(w)


def _tol(v):
    return TOL


def _cap(w):
    return -(-w.T // w.kG) * w.kG + w.kG


def _check_out(orc, w, q, k, v, got, rows=None):
    ref = orc.prefill_attention(q, k, v, w.sigma, rows=rows)
    if rows is not None:
        got = np.stack([got[b, h, i] for b, h, i in rows])
    err = np.abs(got - ref)
    tol = _tol(v)
    worst = float(err.max())
    excess = mean_excess(got, ref)
    assert worst <= tol, (w.name, w.T, worst, tol, np.unravel_index(int(err.argmax()), err.shape))
    assert excess <= MEAN_TOL, (w.name, w.T, excess)
    return worst, excess


def _check_cache(orc, w, dc, twin, k, v):
    st, st2 = dc.state(), twin.state()
    assert st == st2, (st, st2)
    T, nblk = w.T, w.T // w.kG
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            got = slice_of(dc, b, h, T, nblk)
            assert_slices_equal(got, slice_of(twin, b, h, T, nblk), f"{w.name} b{b} h{h} vs append")
            assert_slices_equal(got, oracle_slice(orc, w, k[b, h], v[b, h], dc.cfg.max_tokens // w.kG,
                                                  dc.cfg.max_tokens), f"{w.name} b{b} h{h} vs oracle")


@pytest.mark.parametrize("shape,T", [("gqa4_g64", 1), ("gqa4_g64", 63), ("gqa4_g64", 64), ("gqa4_g64", 65),
                                     ("gqa4_g64", 200), ("gqa4_g32", 200), ("gqa4_g32", 97), ("mha_g32", 130),
                                     ("gqa8_g64", 150), ("gqa4_4bit", 200), ("gqa4_k2v4_g32", 75)])
def test_prefill_matches_oracle(orc, shape, T):
    t = torch()
    w = _workload(shape, T)
    q, k, v = _inputs(w)
    dc, twin = new_cache(w, _cap(w)), new_cache(w, _cap(w))
    log(f"[prefill {shape} T{T}] launch")
    out = dc.prefill(dev_f16(q), dev_f16(k), dev_f16(v), w.sigma)
    twin.append(dev_f16(k), dev_f16(v))
    t.cuda.synchronize()
    got = host_u16(out).view(np.float16).astype(np.float64)
    worst, excess = _check_out(orc, w, q, k, v, got)
    log(f"[prefill {shape} T{T}] max|err| {worst:.3e} (tol {_tol(v):.3e}) mean excess {excess:.2e}")
    _check_cache(orc, w, dc, twin, k, v)
    dc.close()
    twin.close()


def test_prefill_attention_only_leaves_cache_alone(orc):
    t = torch()
    w = _workload("gqa4_g32", 150)
    q, k, v = _inputs(w)
    dc, ref = new_cache(w, _cap(w)), new_cache(w, _cap(w))
    for a in dc.arrays.values():
        a.fill_(0x5A)
    before = {n: a.clone() for n, a in dc.arrays.items()}
    o1 = dc.prefill(dev_f16(q), dev_f16(k), dev_f16(v), w.sigma, flags=kvq.KVQ_PREFILL_ATTENTION_ONLY)
    o2 = ref.prefill(dev_f16(q), dev_f16(k), dev_f16(v), w.sigma)
    t.cuda.synchronize()
    assert dc.state() == (0, 0)
    for n, a in dc.arrays.items():
        assert t.equal(a, before[n]), n
    assert np.array_equal(host_u16(o1), host_u16(o2))
    # attention only also runs on a cache that already holds tokens
    o3 = ref.prefill(dev_f16(q), dev_f16(k), dev_f16(v), w.sigma, flags=kvq.KVQ_PREFILL_ATTENTION_ONLY)
    t.cuda.synchronize()
    assert np.array_equal(host_u16(o3), host_u16(o2))
    dc.close()
    ref.close()


def test_prefill_needs_an_empty_cache():
    w = _workload("gqa4_g64", 70)
    q, k, v = _inputs(w)
    dc = new_cache(w, _cap(w))
    dc.append(dev_f16(k[:, :, :3].copy()), dev_f16(v[:, :, :3].copy()))
    with pytest.raises(kvq.KvqError) as e:
        dc.prefill(dev_f16(q), dev_f16(k), dev_f16(v), w.sigma)
    assert e.value.status == -8
    small = new_cache(w, 64)
    with pytest.raises(kvq.KvqError) as e:
        small.prefill(dev_f16(q), dev_f16(k), dev_f16(v), w.sigma)
    assert e.value.status == -4
    dc.close()
    small.close()


def test_decode_after_prefill_equals_decode_after_append(orc):
    t = torch()
    w = _workload("gqa4_g64", 333)
    q, k, v = _inputs(w)
    dc, twin = new_cache(w, _cap(w)), new_cache(w, _cap(w))
    dc.prefill(dev_f16(q), dev_f16(k), dev_f16(v), w.sigma)
    twin.append(dev_f16(k), dev_f16(v))
    qd = dev_f16(synth.query(w))
    a = dc.decode(qd, w.sigma)
    b = twin.decode(qd, w.sigma)
    t.cuda.synchronize()
    assert np.array_equal(host_u16(a), host_u16(b))
    dc.close()
    twin.close()


def test_prefill_full_size_every_row(orc):
    """The Mistral-7B-shaped prompt (32 query / 8 KV heads, D 128, G 64) at
    4096 tokens, one sequence: every output row against the oracle (about
    137 GFLOP of fp64 work, ~10 s on 16 host cores), the whole cache against
    kv_quantize_append."""
    t = torch()
    w = dataclasses.replace(configs.BY_NAME["mistral_7b_gqa_prefill_b4_t4096"], batch=1)
    q, k, v = _inputs(w)
    dc, twin = new_cache(w, w.T), new_cache(w, w.T)
    out = dc.prefill(dev_f16(q), dev_f16(k), dev_f16(v), w.sigma)
    twin.append(dev_f16(k), dev_f16(v))
    t.cuda.synchronize()
    got = host_u16(out).view(np.float16).astype(np.float64)
    worst, excess = _check_out(orc, w, q, k, v, got)
    log(f"[prefill full] {w.n_q_heads * w.T} rows: max|err| {worst:.3e} mean excess {excess:.2e}")
    for name, a in dc.arrays.items():
        assert t.equal(a, twin.arrays[name]) or name == "k_resid", name
    assert dc.state() == twin.state()
    dc.close()
    twin.close()
