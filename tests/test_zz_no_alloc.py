"""kv_decode_attention_noalloc (split partials in the library's static
scratch array, no device allocation) against kv_decode_attention with a
caller workspace: outputs identical bit for bit, on two calls in a row, the
second over a smaller input, then a call after both on a third shape; and
the scratch limit refused with KVQ_E_SCRATCH."""
import numpy as np
import pytest

from gpu_util import configs, dev_f16, host_u16, kvq, log, new_cache, synth, torch

pytestmark = pytest.mark.gpu


def _pair(w, n_splits=0):
    """both entry points on one cache; returns (workspace out, no-alloc out)"""
    t = torch()
    cap = w.capacity(64)
    dc = new_cache(w, cap)
    dc.append(dev_f16(synth.keys(w)), dev_f16(synth.values(w)))
    q = dev_f16(synth.query(w))
    ref = dc.decode(q, w.sigma, n_splits)
    # stale contents from an earlier call must not matter: poison the output
    out = t.full_like(ref, float("nan"))
    dc.decode_noalloc(q, w.sigma, n_splits, out=out)
    t.cuda.synchronize()
    log(f"[noalloc {w.name}] variant {dc.variant(w.n_q_heads)} splits {n_splits}")
    a, b = host_u16(ref), host_u16(out)
    dc.close()
    return a, b


def test_noalloc_matches_workspace_entry_point():
    big = configs.Workload("noalloc_gqa", 501, "kivi", 4, 32, 8, 4096 + 37, 128, 64, 2, 128, 32, 2, 50.0)
    small = configs.Workload("noalloc_gqa_small", 502, "kivi", 2, 8, 2, 300, 128, 64, 2, 128, 32, 2, 50.0)
    mla = configs.Workload("noalloc_mla", 503, "mla", 2, 128, 1, 1000, 64, 64, 4, 512, 32, 2, 20.0)
    for w, ns in ((big, 0), (small, 0), (mla, 3), (small, 5)):
        a, b = _pair(w, ns)
        assert np.array_equal(a, b), (w.name, int(np.sum(a != b)))


def test_noalloc_rejects_partials_beyond_scratch():
    # MLA, 64 sequences x 128 heads x 4 slots x (512 + 2) x 4 B = 67 MB > 32 MiB
    w = configs.Workload("noalloc_mla_big", 504, "mla", 64, 128, 1, 64, 64, 64, 4, 512, 32, 2, 20.0)
    dc = new_cache(w, w.capacity(64))
    dc.append(dev_f16(synth.keys(w)), dev_f16(synth.values(w)))
    q = dev_f16(synth.query(w))
    with pytest.raises(kvq.KvqError) as e:
        dc.decode_noalloc(q, w.sigma, 4)
    assert e.value.status == -9
    torch().cuda.synchronize()
    dc.close()
