"""C-ABI checks that need no GPU: libkvq.so loads, exports every function
include/kvq.h declares, sizes its arrays per the documented layouts, and
rejects bad arguments on the host before any HIP call."""
import ctypes as C
import os
import re

import pytest

from decode_attention_asym_amd import configs, kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

# fake, 16-byte aligned device addresses: only reached by calls that must
# fail (or finish) on the host without touching HIP
FAKE = [0x10000 * (i + 1) for i in range(7)]


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq?_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = C.CDLL(kvq.LIB_PATH)
    names = header_functions()
    assert set(names) == set(kvq.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def kivi_cfg(**kw):
    d = dict(kind=kvq.KVQ_KIND_KIVI, batch=2, n_kv_heads=4, max_tokens=256, kd=128, kG=32,
             kbits=2, vd=128, vG=32, vbits=2)
    d.update(kw)
    return kvq.cache_cfg(**d)


def test_buffer_sizes_follow_layout():
    for w in configs.WORKLOADS:
        cap = w.capacity(64)
        s = kvq.kv_cache_buffer_bytes(kvq.cfg_for(w, cap))
        bh = w.batch * w.n_kv_heads
        nb = cap // w.kG
        assert s.k_codes == bh * nb * w.kd * (w.kG * w.kbits // 32) * 4
        assert s.k_scale == s.k_zero == bh * nb * w.kd * 2
        assert s.k_resid == bh * w.kG * w.kd * 2
        assert s.v_codes == bh * cap * w.vd * w.vbits // 8
        assert s.v_scale == s.v_zero == bh * cap * (w.vd // 32) * 2


@pytest.mark.parametrize("kw,status", [
    (dict(kind=7), -2), (dict(batch=0), -2), (dict(n_kv_heads=0), -2),
    (dict(kbits=3), -2), (dict(vbits=8), -2), (dict(kd=100, vd=100), -2),
    (dict(kd=64), -2), (dict(kG=48), -2), (dict(kG=128, kbits=4), -5),
    (dict(vG=64), -5), (dict(max_tokens=250), -2), (dict(max_tokens=16), -2),
    (dict(kind=kvq.KVQ_KIND_MLA, n_kv_heads=2), -2), (dict(kd=1024, vd=1024), -2),
])
def test_bad_configs(kw, status):
    with pytest.raises(kvq.KvqError) as e:
        kvq.kv_cache_buffer_bytes(kivi_cfg(**kw))
    assert e.value.status == status


def test_bad_axis_and_reserved():
    cfg = kivi_cfg()
    cfg.key.axis = kvq.KVQ_AXIS_PER_TOKEN
    with pytest.raises(kvq.KvqError) as e:
        kvq.kv_cache_buffer_bytes(cfg)
    assert e.value.status == -5
    cfg = kivi_cfg()
    cfg.reserved = 1
    with pytest.raises(kvq.KvqError):
        kvq.kv_cache_buffer_bytes(cfg)


def test_null_arguments():
    L = kvq.lib()
    assert L.kv_cache_buffer_bytes(None, None) == -1
    assert L.kv_cache_init(C.byref(kivi_cfg()), None, None) == -1
    assert L.kv_quantize_append(None, None, None, 1, 0, None) == -1
    assert L.kv_flush_residual(None, None, None) == -1
    assert L.kv_decode_attention(None, None, 1, C.c_float(1.0), 0, None, None, 0, None) == -1
    assert L.kv_cache_state(None, None, None) == -1
    L.kv_cache_destroy(None)
    assert kvq.kv_decode_variant(None, 1) == "invalid"


def make_handle(**kw):
    bufs = kvq.CacheBuffers(*FAKE)
    return kvq.kv_cache_init(kivi_cfg(**kw), bufs)


def test_init_checks_pointers():
    cfg = kivi_cfg()
    bad = kvq.CacheBuffers(*FAKE)
    bad.v_zero = 0
    with pytest.raises(kvq.KvqError) as e:
        kvq.kv_cache_init(cfg, bad)
    assert e.value.status == -1
    bad = kvq.CacheBuffers(*FAKE)
    bad.k_scale = FAKE[1] + 2
    with pytest.raises(kvq.KvqError) as e:
        kvq.kv_cache_init(cfg, bad)
    assert e.value.status == -3


def test_append_validation_before_hip():
    h = make_handle()
    try:
        assert kvq.kv_cache_state(h) == (0, 0)
        kvq.kv_quantize_append(h, None, None, 0)        # n = 0: no-op, no HIP
        cases = [((0x1000, 0x2000, -1, 0), -2), ((0x1000, 0x2000, 1, 4), -2),
                 ((None, 0x2000, 1, 0), -1), ((0x1008, 0x2000, 1, 0), -3),
                 ((0x1000, 0x2000, 257, 0), -4),
                 ((0x1000, 0x2000, 33, kvq.KVQ_APPEND_NO_AUTOFLUSH), -4)]
        for (k, v, n, fl), st in cases:
            with pytest.raises(kvq.KvqError) as e:
                kvq.kv_quantize_append(h, k, v, n, fl)
            assert e.value.status == st
        assert kvq.kv_cache_state(h) == (0, 0)
        assert kvq.kv_flush_residual(h) == 0              # nothing to flush
    finally:
        kvq.kv_cache_destroy(h)


def test_decode_validation_before_hip():
    h = make_handle()
    try:
        ws = kvq.kv_decode_workspace_bytes(h, 8, 0)
        assert ws > 0 and ws % 4 == 0
        assert kvq.kv_decode_workspace_bytes(h, 8, 3) == 2 * 8 * 3 * (128 + 2) * 4
        for hq, s, st in [(6, 0, -2), (0, 0, -2), (8, -1, -2), (8, 257, -2)]:
            with pytest.raises(kvq.KvqError) as e:
                kvq.kv_decode_attention(h, 0x1000, hq, 1.0, s, 0x2000, 0x3000, ws)
            assert e.value.status == st
        with pytest.raises(kvq.KvqError) as e:
            kvq.kv_decode_attention(h, 0x1004, 8, 1.0, 0, 0x2000, 0x3000, ws)
        assert e.value.status == -3
        with pytest.raises(kvq.KvqError) as e:                # empty cache
            kvq.kv_decode_attention(h, 0x1000, 8, 1.0, 0, 0x2000, 0x3000, ws)
        assert e.value.status == -8
        assert kvq.kv_decode_variant(h, 8) in ("generic", "mha_mfma", "gqa_mfma", "mla_mfma")
    finally:
        kvq.kv_cache_destroy(h)


def test_status_strings():
    for s in kvq.STATUS:
        assert kvq.kvq_status_str(s) not in ("", "unknown status")
    assert kvq.kvq_status_str(-99) == "unknown status"


def test_timing_hook_arguments():
    with pytest.raises(kvq.KvqError):
        kvq.kv_set_timing_events(0x10, None)
    kvq.kv_set_timing_events(None, None)


@pytest.mark.parametrize("name,variant", [
    ("tiny_mha_d64_t250", "generic"),
    ("llama2_7b_layer_mha_t4096", "mha_mfma"),
    ("mistral_7b_gqa_t32805", "gqa_mfma"),
    ("longctx_gqa_t131072", "gqa_mfma"),
    ("mla_absorbed_b64_t16384", "mla_mfma"),
])
def test_variant_per_workload(name, variant):
    """Which decode kernel each workload reaches (host-side choice)."""
    from decode_attention_asym_amd import configs
    w = configs.BY_NAME[name]
    h = kvq.kv_cache_init(kvq.cfg_for(w, w.capacity()), kvq.CacheBuffers(*FAKE))
    try:
        assert kvq.kv_decode_variant(h, w.n_q_heads) == variant
    finally:
        kvq.kv_cache_destroy(h)
