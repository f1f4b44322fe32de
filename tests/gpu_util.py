"""Helpers shared by the GPU parity tests (the HIP path is called through the
C ABI via the ctypes binding; the oracle is called on the same seeded bits)."""
import sys

import numpy as np

from decode_attention_asym_amd import configs, kvq, synth

TOL = 2e-3   # max-abs, fp16 GPU output vs the oracle's unrounded fp64 result
# The max-abs bar is mostly the fp16 rounding of the output (half an ulp is
# 9.8e-4 for |o| in [2, 4)), so a small systematic error in the accumulated
# sums can hide under it.  Over many outputs the mean error beyond that
# rounding exposes it: correct kernels measure 0 .. 3e-5 on the shapes here
# (up to 32K tokens, both G, 1..12 splits), while weights p that were off by
# one part in 2^11 in the sums l and sum p z measured 7e-5 .. 2.2e-4 with one
# split per sequence.
MEAN_EXCESS_TOL = 5e-5


def mean_excess(got, ref):
    """mean |got - ref| minus the mean error of ref correctly rounded to fp16"""
    rounding = np.abs(ref.astype(np.float16).astype(np.float64) - ref)
    return float(np.abs(got - ref).mean() - rounding.mean())


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch():
    import torch as t
    return t


def dev_f16(arr_u16):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(arr_u16).view(np.int16)).view(t.float16).cuda()


def host_u16(tensor):
    return tensor.contiguous().cpu().view(torch().int16).numpy().view(np.uint16)


def new_cache(w, cap):
    return kvq.DeviceCache(kvq.cfg_for(w, cap))


def slice_of(dc, b, h, T, nblk):
    """The (b, h) slice of the device cache, valid region only, as numpy."""
    t = torch()
    t.cuda.synchronize()
    v = dc.views()
    R = T - nblk * dc.cfg.key.group
    out = {}
    for name, arr in v.items():
        a = arr[b, h]
        if name in ("k_codes", "k_scale", "k_zero"):
            a = a[:nblk]
        elif name == "k_resid":
            a = a[:R]
        else:
            a = a[:T]
        a = a.cpu().numpy()
        out[name] = a.view(np.uint32) if a.dtype == np.int32 else a.view(np.uint16)
    return out


def oracle_slice(orc, w, k_u16, v_u16, nblk_cap, cap):
    """Oracle cache for one (b, h): k_u16 [T][kd], v_u16 [T][vd]."""
    T = k_u16.shape[0]
    keys = orc.quantize_keys(k_u16[None, None], w.kG, w.kbits, nblk_cap)
    vals = orc.quantize_values(v_u16[None, None], w.vG, w.vbits, cap)
    nb, R = T // w.kG, T % w.kG
    return {
        "k_codes": keys["k_codes"][0, 0, :nb], "k_scale": keys["k_scale"][0, 0, :nb],
        "k_zero": keys["k_zero"][0, 0, :nb], "k_resid": keys["k_resid"][0, 0, :R],
        "v_codes": vals["v_codes"][0, 0, :T], "v_scale": vals["v_scale"][0, 0, :T],
        "v_zero": vals["v_zero"][0, 0, :T],
    }


def assert_slices_equal(got, ref, what=""):
    for name in ref:
        g, r = got[name], ref[name]
        assert g.shape == r.shape, (what, name, g.shape, r.shape)
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError(f"{what} {name}: {len(bad)} mismatches, first at {bad[0].tolist()}: "
                                 f"gpu {g[tuple(bad[0])]:#x} oracle {r[tuple(bad[0])]:#x}")


def oracle_cache_full(orc, w, k_u16, v_u16, cap):
    return orc.build_cache(k_u16, v_u16, w.kG, w.kbits, w.vG, w.vbits,
                           nblk_cap=cap // w.kG, tok_cap=cap)


def oracle_attention(orc, w, cache, q_u16, pairs=None):
    fn = orc.attention_kivi if w.kind == "kivi" else orc.attention_mla
    return fn(cache, q_u16, w.sigma, pairs=pairs)


def sample_pairs(w, n, seed=0):
    """(b, query head) pairs spread over the batch and the heads."""
    rng = np.random.default_rng(seed)
    pairs = {(0, 0), (w.batch - 1, w.n_q_heads - 1)}
    while len(pairs) < min(n, w.batch * w.n_q_heads):
        pairs.add((int(rng.integers(w.batch)), int(rng.integers(w.n_q_heads))))
    return sorted(pairs)


def workload(name):
    return configs.BY_NAME[name]


__all__ = ["configs", "synth", "kvq"]
