"""Benchmark: 2-bit decode attention over a KIVI-style cache on one MI355X.

One step = one decode token for every sequence of the workload in one
layer (kv_decode_step): append the new token (per-token value quantize, key
into the residual, per-channel key quantize of the block when it fills) and
split-K decode attention over the whole cache with the merge pass; while the
new key completes no block, the append runs inside the attention launch.  Steps rotate over
several layers, each with its own cache, at least 1 GB in total, so that a
cache smaller than the 256 MB Infinity Cache is still read from HBM.  Inputs
are seeded synthetic fp16 tensors already resident in HBM.  Prints ONE JSON
line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--layers L]
                  [--no-cpu-baseline] [--paged] [--separate-calls] [--prefill]

--prefill times the prompt instead: one step = kv_prefill_attention of the
whole prompt (causal attention on the matrix cores with the bulk quantize of
its keys and values fused in) into an empty cache.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak
DEFAULT_WORKLOAD = "mistral_7b_gqa_t32805"
PREFILL_WORKLOAD = "mistral_7b_gqa_prefill_b4_t4096"


class HipEvents:
    """hipEvent_t pairs through libamdhip64 (the pass-1 launch records its own
    start and stop timestamps into them)."""

    def __init__(self):
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self):
        e = C.c_void_p()
        assert self.hip.hipEventCreate(C.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b):
        ms = C.c_float()
        assert self.hip.hipEventElapsedTime(C.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-pairs", type=int, default=1024)
    ap.add_argument("--cpu-rows", type=int, default=100000, help="prefill: oracle rows timed for the CPU baseline")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--layers", type=int, default=0,
                    help="caches to rotate over (default: enough for 1 GB, at most 32)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--paged", action="store_true",
                    help="paged cache: ragged lengths in [T/2, T], blocks in shuffled pages")
    ap.add_argument("--batch", type=int, default=0,
                    help="sequences per step (default: the workload's); names the workload ..._b<N>")
    ap.add_argument("--bits", type=int, default=0, choices=[0, 2, 4],
                    help="key and value code width (default: the workload's; MLA: the content latent's, the RoPE key stays 4-bit)")
    ap.add_argument("--prefill", action="store_true",
                    help="prefill: causal prompt attention fused with the bulk quantize (kv_prefill_attention) "
                         "on the prefill workload")
    ap.add_argument("--separate-calls", action="store_true",
                    help="step as kv_quantize_append + kv_decode_attention instead of kv_decode_step")
    return ap.parse_args()


def profiled_traffic(variant: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 (FETCH_SIZE / WRITE_SIZE
    scaled by a plain-copy calibration, profiles/traffic.json), or None when
    no measurement exists or the kernel source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{variant}/{workload}")
    if not rec:
        return None
    srcs = rec["source"] if isinstance(rec["source"], list) else [rec["source"]]
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest()[:16] != rec["sha256_16"]:
        return None
    return int(rec["traffic_bytes"])


def profiled_counters(variant: str, workload: str):
    """The dominant kernel's rocprofv3 counters (MfmaUtil, VALUBusy, SALUBusy,
    LDSBankConflict in percent, profiles/counters.json), or None when no
    measurement exists or the kernel source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{variant}/{workload}")
    if not rec:
        return None
    h = hashlib.sha256()
    for f in rec["source"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest()[:16] != rec["sha256_16"]:
        return None
    return {k: rec[k] for k in ("MfmaUtil", "VALUBusy", "SALUBusy", "LDSBankConflict", "profile")}


def gpu_clock_state():
    """Current shader / memory / fabric clock levels of the first AMD GPU, as
    the driver's sysfs files mark them ('*'); plain file reads, so no child
    process starts from this GPU process.  None when the files are missing."""
    import glob
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        keep = []
        for name in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
            try:
                with open(os.path.join(dev, name)) as f:
                    keep += [f"{name[7:]} {ln.strip()}" for ln in f if ln.rstrip().endswith("*")]
            except OSError:
                continue
        if keep:
            return keep
    return None


def copy_probe():
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) of the decode kernel."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": n, "launches": 5}), flush=True)


def copy_ceiling_gbps():
    """Read + write rate of a plain 1 GiB device copy on this GPU (median of 5)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    ts = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    del src, dst
    return 2 * n / (float(np.median(ts)) * 1e-3) / 1e9


def cpu_baseline(w, k, v, q, cap, n_pairs, lens=None):
    """The oracle, as it stands, on a bounded sample of the same workload:
    decode attention of n_pairs (batch, query head) pairs over the full cache
    of their KV heads (sequence b's first lens[b] tokens when lengths are
    ragged), threaded over the pairs."""
    import oracle

    group = w.n_q_heads // w.n_kv_heads
    slices = []
    p = 0
    while len(slices) * group < n_pairs and p < w.batch * w.n_kv_heads:
        slices.append(divmod(p * 7 % (w.batch * w.n_kv_heads), w.n_kv_heads))
        p += 1
    caches, qs = [], []
    for b, h in slices:
        T = w.T if lens is None else int(lens[b])
        caches.append(oracle.build_cache(np.ascontiguousarray(k[b:b + 1, h:h + 1, :T]),
                                         np.ascontiguousarray(v[b:b + 1, h:h + 1, :T]), w.kG, w.kbits,
                                         w.vG, w.vbits, nblk_cap=cap // w.kG, tok_cap=cap))
        qs.append(np.ascontiguousarray(q[b:b + 1, h * group:(h + 1) * group]))
    # one oracle call per slice would serialise on `group` threads; run the
    # slices concurrently so that every host core has a pair
    import concurrent.futures as cf
    fn = oracle.attention_kivi if w.kind == "kivi" else oracle.attention_mla
    cores = min(os.cpu_count() or 1, len(slices) * group)
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=len(slices)) as ex:
        list(ex.map(lambda i: fn(caches[i], qs[i], w.sigma, nthreads=group), range(len(slices))))
    dt = time.perf_counter() - t0
    n_sl = len(slices)
    Ts = [w.T if lens is None else int(lens[b]) for b, _ in slices]
    sample_bytes = sum(w.cache_bytes(T) // (w.batch * w.n_kv_heads) for T in Ts) \
        + n_sl * group * (w.qd + w.vd) * 2
    span = f"T={w.T}" if lens is None else f"their lengths ({min(Ts)}..{max(Ts)})"
    return {"value": sample_bytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_sl} (batch, kv-head) slices x {group} query heads = {n_sl * group} "
                      f"decode pairs over {span} (of {w.batch * w.n_q_heads}); {dt:.2f} s wall",
            "tokens_per_s_attended": sum(Ts) / dt}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); "
              "sharding the decode step across GPUs is not implemented", file=sys.stderr)
        sys.exit(2)
    import torch

    from decode_attention_asym_amd import configs, kvq, synth

    if args.copy_probe:
        copy_probe()
        return
    if args.prefill and args.workload == DEFAULT_WORKLOAD:
        args.workload = PREFILL_WORKLOAD
    w = configs.BY_NAME[args.workload]
    if args.batch:
        import dataclasses
        w = dataclasses.replace(w, batch=args.batch, name=f"{w.name}_b{args.batch}")
    if args.bits and w.kind == "kivi" and args.bits != w.kbits:
        import dataclasses
        w = dataclasses.replace(w, kbits=args.bits, vbits=args.bits, name=f"{w.name}_{args.bits}bit")
    if args.bits and w.kind == "mla" and args.bits != w.vbits:
        # the content latent's width (the RoPE key is 4-bit either way)
        import dataclasses
        w = dataclasses.replace(w, vbits=args.bits, name=f"{w.name}_content{args.bits}bit")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.prefill:
        main_prefill(args, w, dev)
        return
    if args.paged:
        main_paged(args, w, dev)
        return
    n_steps = args.warmup + args.steps
    L = args.layers or min(32, max(1, -(-1_000_000_000 // w.cache_bytes())))
    n_new = -(-n_steps // L)              # new tokens each layer receives
    Tall = w.T + n_new
    cap = w.capacity(n_new + 1)
    t0 = time.time()
    k = synth.keys(w, Tall)
    v = synth.values(w, Tall)
    q = synth.query(w)
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def dev16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.float16).to(dev)

    kd = dev16(k[:, :, :w.T])
    vd = dev16(v[:, :, :w.T])
    # one contiguous [B][Hkv][1][d] tensor per decode step
    knew = dev16(np.ascontiguousarray(k[:, :, w.T:].transpose(2, 0, 1, 3))[:, :, :, None, :])
    vnew = dev16(np.ascontiguousarray(v[:, :, w.T:].transpose(2, 0, 1, 3))[:, :, :, None, :])
    qd = dev16(q)
    dcs = [kvq.DeviceCache(kvq.cfg_for(w, cap), device=dev) for _ in range(L)]
    dc = dcs[0]
    stream = torch.cuda.current_stream()

    # ---- bulk prefill quantize (the context): one untimed repetition (the
    # first touch of the cache's pages runs at about half speed), then the
    # median of five
    qt = []
    for rep in range(6):
        kvq.kv_cache_reset(dc.handle)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dc.append(kd, vd)
        b.record(stream)
        torch.cuda.synchronize()
        if rep > 0:
            qt.append(a.elapsed_time(b))
    q_ms = float(np.median(qt))
    q_bytes = 2 * w.batch * w.n_kv_heads * w.T * (w.kd + w.vd) + w.cache_bytes()
    for other in dcs[1:]:
        other.append(kd, vd)
    torch.cuda.synchronize()
    assert all(c.state() == (w.T, w.R) for c in dcs)
    del kd, vd

    out = torch.empty((w.batch, w.n_q_heads, w.vd), dtype=torch.float16, device=dev)
    ws = dc.workspace(w.n_q_heads, args.splits)
    hip = HipEvents()
    evs = [(hip.create(), hip.create()) for _ in range(args.steps)]

    # the step loop calls the C ABI with everything it needs precomputed, so
    # that host-side Python does not pace the small workloads
    lib = kvq.lib()
    c_append, c_decode, c_timing = lib.kv_quantize_append, lib.kv_decode_attention, lib.kv_set_timing_events
    c_step = None if args.separate_calls else lib.kv_decode_step
    handles = [c.handle for c in dcs]
    kptr = [knew[j].data_ptr() for j in range(knew.shape[0])]
    vptr = [vnew[j].data_ptr() for j in range(vnew.shape[0])]
    n_new = knew.shape[-2]
    sptr, qptr, optr, wptr, wbytes = stream.cuda_stream, qd.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel()

    def step(i, timed):
        # step i: layer i % L receives its token i // L
        h = handles[i % L]
        if timed:
            st = c_timing(*evs[i - args.warmup])
            assert st == 0, st
        if args.separate_calls:
            st = c_append(h, kptr[i // L], vptr[i // L], n_new, 0, sptr)
            assert st == 0, kvq.kvq_status_str(st)
            st = c_decode(h, qptr, w.n_q_heads, w.sigma, args.splits, optr, wptr, wbytes, sptr)
        else:
            st = c_step(h, kptr[i // L], vptr[i // L], qptr, w.n_q_heads, w.sigma, args.splits, optr, wptr,
                        wbytes, sptr)
        assert st == 0, kvq.kvq_status_str(st)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.warmup, n_steps):
        step(i, True)
    stop.record(stream)
    torch.cuda.synchronize()
    kvq.kv_set_timing_events(None, None)
    total_ms = start.elapsed_time(stop)
    pass1_ms = [hip.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)

    Ts = [w.T + i // L + 1 for i in range(args.warmup, n_steps)]
    alg_bytes = sum(w.decode_bytes(T) for T in Ts)
    value = alg_bytes / (total_ms * 1e-3) / 1e9
    p1_avg = float(np.mean(pass1_ms))
    p1_bytes = float(np.mean([w.cache_bytes(T) + w.batch * w.n_q_heads * w.qd * 2 for T in Ts]))
    achieved = p1_bytes / (p1_avg * 1e-3) / 1e9
    p1_flops = float(np.mean([w.decode_flops(T) for T in Ts]))
    tflops = p1_flops / (p1_avg * 1e-3) / 1e12
    ms_step = total_ms / args.steps
    p1_sorted = np.sort(pass1_ms)
    copy_gbps = copy_ceiling_gbps()

    variant = dc.variant(w.n_q_heads)
    if variant == "mla_mfma":
        # the absorbed MLA kernel is bound by the matrix cores: 2 flops per
        # multiply-add of q.c_hat, q_r.k_hat_r and p.c_hat
        roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                    "traffic": profiled_traffic(variant, w.name),
                    "counters": profiled_counters(variant, w.name),
                    "kernel": "decode pass-1 (" + variant + ")", "avg_us": round(p1_avg * 1e3, 2),
                    "alg_flops_per_launch": int(p1_flops), "alg_bytes_per_launch": int(p1_bytes),
                    "hbm_GBps": round(achieved, 2)}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": profiled_traffic(variant, w.name),
                    "counters": profiled_counters(variant, w.name),
                    "kernel": "decode pass-1 (" + variant + ")", "avg_us": round(p1_avg * 1e3, 2),
                    "alg_bytes_per_launch": int(p1_bytes)}
    res = {
        "metric": "2-bit decode attention KV bytes/s (tokens/s, % HBM peak; quantize GB/s)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.kd, "context": w.T, "G": w.kG,
                   "bits": w.kbits if w.kind == "kivi" else w.vbits, "value_group": w.vG, "layers": L,
                   "parallelism": "none (1 GPU)", **({"rope_bits": w.kbits} if w.kind == "mla" else {})},
        "roofline": roofline,
        "extra": {
            "decode_tokens_per_s": round(w.batch / (ms_step * 1e-3), 1),
            "attended_kv_tokens_per_s": round(w.batch * float(np.mean(Ts)) / (ms_step * 1e-3), 1),
            "hbm_frac_whole_step": round(value / HBM_PEAK_GBPS, 4),
            "pass1_us_p10_p50_p90": [round(float(np.percentile(p1_sorted, x)) * 1e3, 2) for x in (10, 50, 90)],
            "copy_ceiling_GBps": round(copy_gbps, 1),
            "gpu_clock_after_timed_steps": gpu_clock_state(),
            "pass1_frac_of_copy_ceiling": round(achieved / copy_gbps, 4),
            "quantize_GBps": round(q_bytes / (q_ms * 1e-3) / 1e9, 2),
            "quantize_ms": round(q_ms, 4),
            "quantize_bytes": int(q_bytes),
            "cache_bytes": int(w.cache_bytes()),
            "fp16_kv_equiv_bytes": int(w.fp16_kv_bytes()),
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, k[:, :, :w.T], v[:, :, :w.T], q, cap, args.cpu_pairs)
    print(json.dumps(res), flush=True)
    for c in dcs:
        c.close()


def main_paged(args, w, dev):
    """The same step on a paged cache: sequence b holds lens[b] tokens
    (uniform in [T/2, T], the longest exactly T), its key blocks in pages of
    a shuffled pool; each step appends one token to every sequence and
    attends over each sequence's own length: kv_paged_decode_step (the
    append inside the attention launch), or with --separate-calls
    kv_paged_append then kv_paged_decode."""
    import torch

    from decode_attention_asym_amd import kvq, synth

    n_steps = args.warmup + args.steps
    lens0 = synth.ragged_lengths(w)
    mean_bytes = float(np.mean([w.cache_bytes(int(T)) for T in lens0]))
    L = args.layers or min(32, max(1, -(-1_000_000_000 // int(mean_bytes))))
    n_new = -(-n_steps // L)
    cap = w.capacity(n_new + 1)
    maxb = cap // w.kG
    max_len = w.T + n_new
    t0 = time.time()
    k = synth.keys(w, w.T + n_new)
    v = synth.values(w, w.T + n_new)
    q = synth.query(w)
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def dev16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.float16).to(dev)

    def dev32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    blocks = -(-(lens0 + n_new) // w.kG)
    caches, tables = [], []
    for layer in range(L):
        table, n_pages = synth.page_table(w, blocks, maxb, spare=7, seed_word=layer)
        caches.append(kvq.PagedCache(kvq.cfg_for(w, cap), n_pages, device=dev))
        tables.append(dev32(table))
    stream = torch.cuda.current_stream()
    # prefill: every sequence's lens[b] tokens in one append
    kd, vd = dev16(k[:, :, :w.T]), dev16(v[:, :, :w.T])
    zeros, l0 = dev32(np.zeros(w.batch)), dev32(lens0)
    qt = []
    for layer in range(L):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        caches[layer].append(kd, vd, zeros, tables[layer], l0)
        b.record(stream)
        torch.cuda.synchronize()
        qt.append(a.elapsed_time(b))
    q_ms = float(np.median(qt))
    q_bytes = int(sum(2 * w.n_kv_heads * int(T) * (w.kd + w.vd) + w.cache_bytes(int(T)) // w.batch
                      for T in lens0))
    del kd, vd
    # the new token of step j for sequence b is its row lens0[b] + j
    rows = lens0[:, None] + np.arange(n_new)[None, :]                      # [B][n_new]
    kn = np.take_along_axis(k, rows[:, None, :, None], axis=2)              # [B][Hkv][n_new][kd]
    vn = np.take_along_axis(v, rows[:, None, :, None], axis=2)
    knew = dev16(np.ascontiguousarray(kn.transpose(2, 0, 1, 3))[:, :, :, None, :])
    vnew = dev16(np.ascontiguousarray(vn.transpose(2, 0, 1, 3))[:, :, :, None, :])
    lens_dev = [dev32(lens0 + j) for j in range(n_new + 1)]
    qd = dev16(q)
    out = torch.empty((w.batch, w.n_q_heads, w.vd), dtype=torch.float16, device=dev)
    ws = caches[0].workspace(w.n_q_heads, max_len, args.splits)
    hip = HipEvents()
    evs = [(hip.create(), hip.create()) for _ in range(args.steps)]

    lib = kvq.lib()
    c_append, c_decode, c_timing = lib.kv_paged_append, lib.kv_paged_decode, lib.kv_set_timing_events
    fused = not args.separate_calls and caches[0].variant(w.n_q_heads, max_len).endswith("mfma_paged")
    c_step = lib.kv_paged_decode_step if fused else None
    handles = [c.handle for c in caches]
    tptr = [t.data_ptr() for t in tables]
    lptr = [t.data_ptr() for t in lens_dev]
    kptr = [knew[j].data_ptr() for j in range(n_new)]
    vptr = [vnew[j].data_ptr() for j in range(n_new)]
    sptr, qptr, optr, wptr, wbytes = stream.cuda_stream, qd.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel()

    def step(i, timed):
        layer, j = i % L, i // L
        if timed:
            st = c_timing(*evs[i - args.warmup])
            assert st == 0, st
        if c_step is not None:
            # lengths before the step, not advanced: step j of every layer reads lens0 + j
            st = c_step(handles[layer], kptr[j], vptr[j], qptr, w.n_q_heads, w.sigma, None, lptr[j], tptr[layer],
                        max_len, args.splits, 0, optr, wptr, wbytes, sptr)
            assert st == 0, kvq.kvq_status_str(st)
            return
        st = c_append(handles[layer], kptr[j], vptr[j], 1, None, lptr[j], tptr[layer], sptr)
        assert st == 0, kvq.kvq_status_str(st)
        st = c_decode(handles[layer], qptr, w.n_q_heads, w.sigma, lptr[j + 1], tptr[layer], max_len, args.splits,
                      optr, wptr, wbytes, sptr)
        assert st == 0, kvq.kvq_status_str(st)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.warmup, n_steps):
        step(i, True)
    stop.record(stream)
    torch.cuda.synchronize()
    kvq.kv_set_timing_events(None, None)
    total_ms = start.elapsed_time(stop)
    pass1_ms = [hip.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)

    def step_bytes(j, qo):
        # every sequence after its append: lens0[b] + j + 1 tokens
        return sum(w.cache_bytes(int(T) + j + 1) // w.batch for T in lens0) + qo

    js = [i // L for i in range(args.warmup, n_steps)]
    alg_bytes = sum(step_bytes(j, w.qo_bytes()) for j in js)
    value = alg_bytes / (total_ms * 1e-3) / 1e9
    p1_avg = float(np.mean(pass1_ms))
    p1_bytes = float(np.mean([step_bytes(j, w.batch * w.n_q_heads * w.qd * 2) for j in js]))
    achieved = p1_bytes / (p1_avg * 1e-3) / 1e9
    ms_step = total_ms / args.steps
    p1_sorted = np.sort(pass1_ms)
    variant = caches[0].variant(w.n_q_heads, max_len)
    res = {
        "metric": "2-bit decode attention KV bytes/s (tokens/s, % HBM peak; quantize GB/s)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": w.name + "_paged_ragged", "batch": w.batch, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.kd, "context": f"{int(lens0.min())}..{w.T}",
                   "mean_context": round(float(lens0.mean()), 1), "G": w.kG, "bits": w.kbits,
                   "value_group": w.vG, "layers": L, "page_tokens": w.kG, "parallelism": "none (1 GPU)",
                   "step": "fused decode step" if fused else "append + decode"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": profiled_traffic(variant, w.name + "_paged_ragged"),
                     "counters": profiled_counters(variant, w.name + "_paged_ragged"),
                     "kernel": "decode pass-1 (" + variant + ")", "avg_us": round(p1_avg * 1e3, 2),
                     "alg_bytes_per_launch": int(p1_bytes)},
        "extra": {
            "decode_tokens_per_s": round(w.batch / (ms_step * 1e-3), 1),
            "attended_kv_tokens_per_s": round(float(np.mean([np.sum(lens0 + j + 1) for j in js])) / (ms_step * 1e-3), 1),
            "hbm_frac_whole_step": round(value / HBM_PEAK_GBPS, 4),
            "pass1_us_p10_p50_p90": [round(float(np.percentile(p1_sorted, x)) * 1e3, 2) for x in (10, 50, 90)],
            "prefill_quantize_GBps": round(q_bytes / (q_ms * 1e-3) / 1e9, 2),
            "prefill_quantize_ms": round(q_ms, 4),
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, k, v, q, cap, args.cpu_pairs, lens=lens0)
    print(json.dumps(res), flush=True)
    for c in caches:
        c.close()


def prefill_flops(w) -> int:
    """Algorithmic flops of causal attention over a T-token prompt: row i
    attends to i + 1 keys, 2 * d flops per key for q . k and 2 * d for p v,
    so sum_i (i + 1) * 2 (d_qk + d_v) = (d_qk + d_v) T (T + 1) per head."""
    return w.batch * w.n_q_heads * (w.qd + w.vd) * w.T * (w.T + 1)


def cpu_baseline_prefill(w, q, k, v, n_rows):
    """The oracle's prefill attention, as it stands, on n_rows rows spread
    over the prompt (every host core), scaled to flops/s by each row's own
    causal window."""
    import oracle

    rng = np.random.default_rng(0)
    rows = np.stack([rng.integers(0, w.batch, n_rows), rng.integers(0, w.n_q_heads, n_rows),
                     rng.integers(0, w.T, n_rows)], axis=1).astype(np.int64)
    cores = min(16, os.cpu_count() or 1)
    t0 = time.perf_counter()
    oracle.prefill_attention(q, k, v, w.sigma, rows=rows, nthreads=cores)
    dt = time.perf_counter() - t0
    flops = float(np.sum(2 * (w.qd + w.vd) * (rows[:, 2] + 1)))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": min(cores, n_rows), "kind": "oracle",
            "sample": f"{n_rows} random (sequence, head, row) outputs of the prompt, fp64; {dt:.2f} s wall"}


def main_prefill(args, w, dev):
    """One step = kv_prefill_attention of the whole prompt into an empty
    cache (the reset between steps is host-side only)."""
    import torch

    from decode_attention_asym_amd import kvq, synth

    t0 = time.time()
    q, k, v = synth.prompt_queries(w), synth.keys(w), synth.values(w)
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def dev16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.float16).to(dev)

    qd, kd, vd = dev16(q), dev16(k), dev16(v)
    cache = kvq.DeviceCache(kvq.cfg_for(w, -(-w.T // w.kG) * w.kG), device=dev)
    out = torch.empty((w.batch, w.n_q_heads, w.T, w.vd), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream()
    lib = kvq.lib()
    sptr = stream.cuda_stream

    def run(flags, n, append_first=False):
        for _ in range(n):
            lib.kv_cache_reset(cache.handle)
            if append_first:
                st = lib.kv_quantize_append(cache.handle, kd.data_ptr(), vd.data_ptr(), w.T, 0, sptr)
                assert st == 0, kvq.kvq_status_str(st)
            st = lib.kv_prefill_attention(cache.handle, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), w.T,
                                          w.n_q_heads, C.c_float(w.sigma), flags, out.data_ptr(), sptr)
            assert st == 0, kvq.kvq_status_str(st)

    def timed(flags, n, append_first=False):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run(flags, n, append_first)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    # the fused step (the reported figure) over all K steps; then, for
    # context, attention alone and append + attention alone, interleaved with
    # the fused step in three rounds so that clock drift shows in all three
    only = kvq.KVQ_PREFILL_ATTENTION_ONLY
    run(0, max(1, args.warmup))
    run(only, max(1, args.warmup))
    ms = timed(0, args.steps)
    n_ctx = max(1, args.steps // 3)
    rounds = [(timed(0, n_ctx), timed(only, n_ctx), timed(only, n_ctx, append_first=True)) for _ in range(3)]
    ms_fused_ctx, ms_attn, ms_sep = (float(np.mean([r[i] for r in rounds])) for i in range(3))
    flops = prefill_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    res = {
        "metric": "prefill attention TFLOP/s (causal, bulk quantize fused), prompt tokens/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.kd, "prompt_tokens": w.T, "G": w.kG, "bits": w.kbits, "value_group": w.vG,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": profiled_traffic("prefill", w.name), "counters": profiled_counters("prefill", w.name),
                     "kernel": "k_prefill (one launch per step)", "avg_us": round(ms * 1e3, 2),
                     "alg_flops_per_launch": int(flops)},
        "extra": {
            "prompt_tokens_per_s": round(w.batch * w.T / (ms * 1e-3), 1),
            "interleaved_rounds_ms": {"fused": round(ms_fused_ctx, 4), "attention_only": round(ms_attn, 4),
                                      "append_then_attention_only": round(ms_sep, 4)},
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(w, q, k, v, args.cpu_rows)
    print(json.dumps(res), flush=True)
    cache.close()


if __name__ == "__main__":
    main()
