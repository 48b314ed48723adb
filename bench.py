#!/usr/bin/env python3
"""Benchmark of the AirCache visual KV-cache compression pass on one MI355X.

One step is one whole pass (aircache_plan + aircache_compress: elite window,
cross-modal scores, statistics, budgets, top-k, compaction) over one batch of
synthetic, seeded inputs already resident in HBM. Inputs rotate over several
device copies (>= 1 GiB in total, four times the 256 MB Infinity Cache) so a
step cannot reuse the previous step's data from the last-level cache.

Prints one JSON line: visual KV token-layers compressed per second (L*B*N_v per
step), achieved HBM bandwidth of the pass and of its dominant kernel against
the 8 TB/s peak, and the single-threaded CPU oracle timed on the same inputs.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense, MI355X (fp32: the vector peak)
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "lvlm_kv_cache_amd", "csrc")
SOURCES = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith((".hip", ".h"))] + \
    [os.path.join(ROOT, "include", "aircache.h")]
METRIC = "visual KV tokens compressed/sec (all layers) + achieved HBM GB/s vs peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", "--iters", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", "--config", type=int, default=3, help="workload number 1-5 (3: the headline)")
    ap.add_argument("--seed", type=int, default=None)
    temp = ap.add_mutually_exclusive_group()
    temp.add_argument("--hot", action="store_true", help="no input rotation (cache-warm)")
    temp.add_argument("--cold", action="store_true",
                      help="inputs rotate over >= 1 GiB of copies so every step reads HBM (the default)")
    ap.add_argument("--base-scale", default=None, choices=["unit", "inv_sqrt_d"],
                    help="base distribution of the drawn Q/K/V (default: the workload's own; inv_sqrt_d on "
                         "workloads 3-5 is a stress run with many elite text tokens, not a headline figure)")
    ap.add_argument("--max-elite", type=int, default=64)
    ap.add_argument("--path", default="auto", choices=["auto", "small", "chunked", "tiled", "rows"])
    ap.add_argument("--select", default="shared", choices=["shared", "per_kv_head"],
                    help="one visual-token selection per (layer, sample), the method's, or one per KV head")
    ap.add_argument("--budget-mode", default="aircache", choices=["aircache", "uniform", "strength", "skewness", "pyramid"],
                    help="layer budget rule: the method's (default) or one of its allocation ablation's variants")
    ap.add_argument("--obs-window", type=int, default=0,
                    help="0: the elite observation window (default); k > 0: the last k text tokens instead; "
                         "-k: the last k visual tokens (the queries of every position are then drawn)")
    ap.add_argument("--skip-hot", action="store_true",
                    help="leave out the cache-warm loop (one input copy every step), so that every launch of the "
                         "run reads rotated inputs (profiles of the headline conditions)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-decode", action="store_true",
                    help="do not time decode attention and int8 quantisation over the compacted cache")
    ap.add_argument("--skip-prefill", action="store_true",
                    help="skip the prefill attention timing (aircache_prefill_layer / _attention)")
    ap.add_argument("--prefill-reps", type=int, default=7, help="timed calls of each prefill variant (interleaved)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run plain device-to-device copies of MIB MiB (the reference kernel that scales "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def source_digest():
    """sha256 over the HIP sources: a measured traffic figure is valid only for
    the kernels it was taken on."""
    h = hashlib.sha256()
    for f in SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's counts), or None when
    there is none or the sources changed since it was taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_digest():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(mib):
    """Plain copies of a known size with the hand-written copy kernel of
    libhbmprobe.so: their FETCH_SIZE / WRITE_SIZE per dispatch against mib MiB
    gives the scale of the counters. The three buffers rotate, so no copy
    finds its source in the last-level cache."""
    import ctypes as C
    import torch
    from lvlm_kv_cache_amd import build as lb
    lib = C.CDLL(lb.PROBE_OUT)
    lib.hbm_probe_grid.restype = C.c_int
    lib.hbm_probe_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int, C.c_void_p]
    n = mib << 20
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda").fill_(i + 1) for i in range(3)]
    grid = lib.hbm_probe_grid(8)
    sp = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i in range(5):
        a, b = bufs[i % 3], bufs[(i + 1) % 3]
        assert lib.hbm_probe_copy(C.c_void_p(a.data_ptr()), C.c_void_p(b.data_ptr()), n, grid, sp) == 0
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "dispatches": 5, "kernel": "copy_kernel"}))


def hbm_ceilings(mib=1024, reps=10):
    """What plain hand-written kernels reach on this device (libhbmprobe.so):
    a read-only stream and a copy of `mib` MiB (rotated over three buffers so
    none is in the last-level cache when it is read), in GB/s of bytes read
    plus written, and the interval between two back-to-back launches of an
    empty kernel on one stream, in microseconds."""
    import ctypes as C
    import torch
    from lvlm_kv_cache_amd import build as lb
    lib = C.CDLL(lb.PROBE_OUT)
    lib.hbm_probe_grid.restype = C.c_int
    lib.hbm_probe_sink_words.restype = C.c_size_t
    lib.hbm_probe_sink_words.argtypes = [C.c_int]
    lib.hbm_probe_read.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int, C.c_void_p]
    lib.hbm_probe_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int, C.c_void_p]
    lib.hbm_probe_empty.argtypes = [C.c_void_p]
    n = mib << 20
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda").fill_(i + 1) for i in range(3)]
    grid = lib.hbm_probe_grid(8)
    sink = torch.empty(int(lib.hbm_probe_sink_words(grid)), dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    sp = C.c_void_p(st.cuda_stream)

    def timed(fn, k):
        for i in range(2):
            fn(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for i in range(k):
            fn(i)
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / k

    def rd(i):
        assert lib.hbm_probe_read(C.c_void_p(bufs[i % 3].data_ptr()), n, C.c_void_p(sink.data_ptr()), grid, sp) == 0

    def cp(i):
        a, b = bufs[i % 3], bufs[(i + 1) % 3]
        assert lib.hbm_probe_copy(C.c_void_p(a.data_ptr()), C.c_void_p(b.data_ptr()), n, grid, sp) == 0

    def em(i):
        assert lib.hbm_probe_empty(sp) == 0

    t_read = timed(rd, reps)
    t_copy = timed(cp, reps)
    t_empty = timed(em, 200)
    del bufs, sink
    return {"read_gbps": n / t_read / 1e9, "copy_gbps": 2 * n / t_copy / 1e9, "empty_launch_us": t_empty * 1e6,
            "bytes_per_launch": n, "grid": grid}


def host_cpu():
    """The host CPU's model name and the logical CPUs this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count()
    return model, n


def algorithmic_bytes(w, n_elite, budget):
    """Bytes the method must move in one pass (reads and writes), from the
    measured elite counts and budgets. Dropped visual V rows are never read."""
    e, D = w.elem_bytes, w.D
    L, B = w.L, w.B
    ntk = n_elite.astype("int64")
    rhat = budget.astype("int64")
    k_scan = L * B * w.Hkv * (w.Nv + w.Nt) * D * e          # all keys, once
    q_rows = int((w.Hq * (ntk + 1)).sum()) * D * e          # last + elite text queries
    gather = 4 * int((w.Hkv * (rhat + w.Nt)).sum()) * D * e  # kept + text rows of K and V, read + write
    iv = 8 * L * B * w.Nv                                     # I_v written and read
    cross = L * B * w.Hkv * w.Nv * D * e + int((w.Hq * ntk).sum()) * D * e + int((w.Hkv * ntk).sum()) * D * e
    return dict(total=k_scan + q_rows + gather + iv, cross_score=cross, kv_gather=gather,
                elite_select=L * B * w.Hkv * w.Nt * D * e + L * B * w.Hq * D * e)


def algorithmic_flops(w, n_elite):
    """Multiply-adds x 2 the method needs in one pass: the last text query
    against every text key, and every elite query against the visual and
    elite text keys, for every query head."""
    ntk = n_elite.astype("int64")
    return int((2 * w.Hq * w.D * (w.Nt + ntk * (w.Nv + ntk))).sum())


def cpu_baseline(inp, target_s):
    import oracle
    w = inp.w
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.run(inp, threads=1, compact=True)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 30:
            break
    model, ncpu = host_cpu()
    return {"value": w.L * w.B * w.Nv * reps / el, "unit": "visual KV token-layers/s", "cores": 1,
            "kind": "oracle", "cpu_model": model, "nproc": ncpu,
            "sample": f"the full pass of workload {w.name} (all {w.L} layers, batch {w.B}) on the same "
                      f"inputs, {reps} repetition(s), {el:.1f} s, single-threaded C in double precision"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU: the pass runs on a single MI355X; --gpus {a.gpus} is not "
              "supported (the pass shards by sample, layer or KV head; that path is not built)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import workloads as wl
    from lvlm_kv_cache_amd import AirCache
    from lvlm_kv_cache_amd import _lib

    _lib.load()  # the HIP library must be built; there is no fallback
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if a.copy_calibration > 0:
        copy_calibration(a.copy_calibration)
        return
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = wl.CONFIGS[a.workload]
    if a.base_scale is not None and a.base_scale != w.base:
        w = dataclasses.replace(w, base=a.base_scale)
    seed = a.workload if a.seed is None else a.seed
    tdtype = torch.float32 if w.dtype == wl.F32 else torch.bfloat16

    def dev_layers(arr):
        out = []
        for l in range(w.L):
            t = torch.from_numpy(np.ascontiguousarray(arr[l]))
            if w.dtype == wl.BF16:
                t = t.view(torch.int16).view(tdtype)
            out.append(t.to(dev))
        return out

    # input copies, each drawn from its own seed (seed, seed + 1, ...), so
    # consecutive steps see different elite sets, budgets and schedules
    inp = wl.make_inputs(w, seed)
    def queries(ci):
        # a visual observation window reads every position's queries
        if a.obs_window < 0:
            return dev_layers(np.stack([wl.prefill_queries(ci, l) for l in range(w.L)]))
        return dev_layers(ci.q)

    copies = [(queries(inp), dev_layers(inp.k), dev_layers(inp.v))]
    per_copy = sum(t.numel() * t.element_size() for ts in copies[0] for t in ts)
    ncopy = 1 if a.hot else max(1, math.ceil((1 << 30) / per_copy))
    for i in range(1, ncopy):
        ci = wl.make_inputs(w, seed + i)
        copies.append((queries(ci), dev_layers(ci.k), dev_layers(ci.v)))
        del ci

    ac = AirCache(w.L, w.B, w.Hq, w.Hkv, w.D, w.Nv, w.Nt, dtype=tdtype, alpha=w.alpha, ratio=w.ratio,
                  max_elite=min(a.max_elite, w.Nt) if a.max_elite > 0 else 0, device=dev, path=a.path,
                  budget_mode=a.budget_mode, obs_window=a.obs_window, select=a.select)
    plan = ac.alloc_plan()
    k_out, v_out = ac.alloc_compacted()
    stream = torch.cuda.current_stream(dev)

    # one bound pass per input copy: argument checks and marshalling happen
    # here, outside the timed loops
    bound = [ac.bind(q, k, v, plan, k_out, v_out, stream=stream) for (q, k, v) in copies]
    fused = ac.run_launches == 1  # plan and compaction in one launch

    # every timed call writes its device status to a word of its own, all
    # checked after the loops (a call clears and sets only its own word)
    n_calls = 3 * a.steps
    status_words = torch.zeros(n_calls, dtype=torch.int32, device=dev)
    sbound = [bound[i % ncopy].with_status(status_words[i].data_ptr()) for i in range(n_calls)]

    def check_status(what, st):
        bad = torch.nonzero(st).flatten().tolist()
        if bad:
            raise RuntimeError(f"device status {int(st[bad[0]])} in {len(bad)} call(s) of the {what} loop "
                               "(raise --max-elite)")

    def step(i, pev=None, cev=None, bp=None):
        bp = bp if bp is not None else bound[i % ncopy]
        if pev is None and cev is None:
            bp.run()                   # aircache_run: the whole pass in one call
        else:
            bp.plan(events=pev)
            bp.compress(events=cev)

    # warm-up, then one call per input copy to read what each copy needs
    for i in range(a.warmup):
        step(i)
    n_elite, budget = [], []
    for i in range(ncopy):
        step(i)
        torch.cuda.synchronize()
        if int(plan.status.item()) != 0:
            raise RuntimeError(f"device status {int(plan.status.item())} on input copy {i} (raise --max-elite)")
        n_elite.append(plan.n_elite.cpu().numpy())
        budget.append(plan.budget.cpu().numpy())
    # algorithmic bytes and flops of a step: the mean over the copies the
    # steps rotate through (each copy is used equally often, up to one step)
    nb = [algorithmic_bytes(w, n, r) for n, r in zip(n_elite, budget)]
    nbytes = {k: sum(d[k] for d in nb) / ncopy for k in nb[0]}
    nflops = sum(algorithmic_flops(w, n) for n in n_elite) / ncopy
    n_elite_all = np.concatenate([n.ravel() for n in n_elite])
    budget_all = np.concatenate([r.ravel() for r in budget])
    dt = "bf16" if w.dtype == wl.BF16 else "f32"
    t_roof_us = max(nbytes["total"] / (PEAK_HBM_GBPS * 1e9), nflops / (PEAK_MFMA_TFLOPS[dt] * 1e12)) * 1e6

    # Headline: K whole passes between two events, no instrumentation inside.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(a.steps):
        step(i, bp=sbound[i])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    check_status("headline", status_words[:a.steps])

    # Per-kernel durations: the same K passes with events around each kernel
    # (the one launch of the whole pass where the chunked path compacts in it).
    if fused:
        names = _lib.RUN_KERNELS
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(a.steps)]
        for evs in ev:          # torch creates the underlying HIP event on first record
            for e in evs:
                e.record(stream)
        torch.cuda.synchronize()
        for i in range(a.steps):
            sbound[a.steps + i].run(events=ev[i])
        torch.cuda.synchronize()
        per_step = [1e3 * e[0].elapsed_time(e[1]) for e in ev]
        kern_us = {names[0]: sum(per_step) / a.steps}
        launch_pct = {q: float(np.percentile(per_step, q)) for q in (10, 50, 90)}
    else:
        names = _lib.PLAN_KERNELS + _lib.COMPRESS_KERNELS
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(_lib.PLAN_KERNELS) + 1)] +
              [torch.cuda.Event(enable_timing=True) for _ in range(len(_lib.COMPRESS_KERNELS) + 1)]
              for _ in range(a.steps)]
        np_ = len(_lib.PLAN_KERNELS) + 1
        for evs in ev:
            for e in evs:
                e.record(stream)
        torch.cuda.synchronize()
        for i in range(a.steps):
            step(i, pev=ev[i][:np_], cev=ev[i][np_:], bp=sbound[a.steps + i])
        torch.cuda.synchronize()
        kern = {n: 0.0 for n in names}
        for i in range(a.steps):
            p, c = ev[i][:np_], ev[i][np_:]
            for j, n in enumerate(_lib.PLAN_KERNELS):
                kern[n] += p[j].elapsed_time(p[j + 1])
            kern["kv_gather"] += c[0].elapsed_time(c[1])
        kern_us = {n: 1e3 * t / a.steps for n, t in kern.items()}
        launch_pct = None
    check_status("per-launch", status_words[a.steps:2 * a.steps])

    # Hot: the same steps on one input copy only (K partly cache-resident).
    ms_hot = None
    if not a.skip_hot:
        hot = [bound[0].with_status(status_words[2 * a.steps + i].data_ptr()) for i in range(a.steps)]
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(a.steps):
            step(0, bp=hot[i])
        e1.record(stream)
        torch.cuda.synchronize()
        ms_hot = e0.elapsed_time(e1) / a.steps
        check_status("hot", status_words[2 * a.steps:])
    # Decode attention over the compacted cache the last step wrote
    # (aircache_decode), new queries of the workload's dtype; K timed calls.
    dec = None
    if not a.skip_decode:
        torch.cuda.synchronize()
        budget_now = plan.budget.cpu().numpy()
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        qd = [(torch.randn(w.B, w.Hq, w.D, device=dev, generator=g) * (4.0 / math.sqrt(w.D))).to(tdtype)
              for _ in range(w.L)]
        od = [torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device=dev) for _ in range(w.L)]
        bdec = ac.bind_decode(qd, plan, k_out, v_out, od, stream=stream)
        for _ in range(3):
            bdec()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(a.steps):
            bdec()
        e1.record(stream)
        torch.cuda.synchronize()
        dec_us = 1e3 * e0.elapsed_time(e1) / a.steps
        esz = 2 if w.dtype == wl.BF16 else 4
        # K and V rows of every segment once, the new queries, the outputs
        dec_bytes = (2.0 * w.Hkv * w.D * esz * float((budget_now + w.Nt).sum()) +
                     w.L * w.B * w.Hq * w.D * (esz + 4))
        dec_gbps = dec_bytes / (dec_us * 1e-6) / 1e9
        dec = {"kernels": ["decode_partial_kernel or decode_wave_kernel", "decode_combine_kernel (none with one split)"], "us_per_call": dec_us,
               "algorithmic_bytes": dec_bytes, "achieved_gbps": dec_gbps, "peak_gbps": PEAK_HBM_GBPS,
               "frac": dec_gbps / PEAK_HBM_GBPS, "dense_cache_bytes": 2.0 * w.L * w.B * w.Hkv * w.S * w.D * esz,
               "retained_row_frac": float((budget_now + w.Nt).sum()) / (w.L * w.B * (w.Nv + w.Nt))}
    # int8 quantisation of the same compacted cache (aircache_quantize_i8);
    # K timed calls
    quant = None
    if not a.skip_decode:
        cap = k_out[0].numel()
        kq = [torch.empty(cap, dtype=torch.int8, device=dev) for _ in range(w.L)]
        vq = [torch.empty(cap, dtype=torch.int8, device=dev) for _ in range(w.L)]
        ks = torch.empty(w.L, w.B, w.Hkv, dtype=torch.float32, device=dev)
        vs = torch.empty(w.L, w.B, w.Hkv, dtype=torch.float32, device=dev)
        bq = ac.bind_quantize(plan, k_out, v_out, kq, vq, ks, vs, stream=stream)
        for _ in range(3):
            bq()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(a.steps):
            bq()
        e1.record(stream)
        torch.cuda.synchronize()
        q_us = 1e3 * e0.elapsed_time(e1) / a.steps
        esz = 2 if w.dtype == wl.BF16 else 4
        n_el = 2.0 * w.Hkv * w.D * float((budget_now + w.Nt).sum())  # K and V elements kept
        q_bytes = n_el * (esz + 1)  # each element read once, its code written
        quant = {"kernels": ["quantize_i8_kernel"], "us_per_call": q_us, "algorithmic_bytes": q_bytes,
                 "achieved_gbps": q_bytes / (q_us * 1e-6) / 1e9, "peak_gbps": PEAK_HBM_GBPS,
                 "frac": q_bytes / (q_us * 1e-6) / 1e9 / PEAK_HBM_GBPS}
        # decode attention over that int8 cache (aircache_decode_i8)
        bd8 = ac.bind_decode(qd, plan, kq, vq, od, stream=stream, scales=(ks, vs))
        for _ in range(3):
            bd8()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(a.steps):
            bd8()
        e1.record(stream)
        torch.cuda.synchronize()
        d8_us = 1e3 * e0.elapsed_time(e1) / a.steps
        d8_bytes = n_el * 1 + w.L * w.B * w.Hq * w.D * (esz + 4)  # every kept code once, queries, outputs
        dec["int8_cache"] = {"kernels": ["decode_partial_kernel or decode_wave_kernel (int8)", "decode_combine_kernel (none with one split)"],
                             "us_per_call": d8_us, "algorithmic_bytes": d8_bytes,
                             "achieved_gbps": d8_bytes / (d8_us * 1e-6) / 1e9,
                             "frac": d8_bytes / (d8_us * 1e-6) / 1e9 / PEAK_HBM_GBPS}
    # Prefill attention of every layer (bfloat16 workloads): alone
    # (aircache_prefill_attention), with the scores fused in
    # (aircache_prefill_layer) plus the compaction, and alone followed by the
    # separate pass (aircache_run); the first input copy, its visual queries
    # drawn by workloads.visual_queries.
    pf = None
    if not a.skip_prefill and w.dtype == wl.BF16 and a.obs_window >= 0:
        def dev_bits(arr):
            return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
        qa = [dev_bits(wl.prefill_queries(inp, l)) for l in range(w.L)]
        q0, k0, v0 = copies[0]
        po = [torch.empty_like(t) for t in qa]
        pplan = ac.alloc_plan()
        bp_plain = ac.bind_prefill(qa, k0, v0, po, None, stream=stream)
        bp_fused = ac.bind_prefill(qa, k0, v0, po, pplan, stream=stream)
        bcomp = ac.bind(q0, k0, v0, pplan, k_out, v_out, stream=stream)
        bpass = bound[0].with_status(status_words[0].data_ptr())

        variants = [bp_plain, lambda: (bp_fused(), bcomp.compress()), lambda: (bp_plain(), bpass.run())]
        for fn in variants:  # untimed first calls
            fn()
        torch.cuda.synchronize()
        # the variants interleaved, each call between its own events; medians
        evp = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(a.prefill_reps)] for _ in variants]
        for r in range(a.prefill_reps):
            for vi, fn in enumerate(variants):
                evp[vi][r][0].record(stream)
                fn()
                evp[vi][r][1].record(stream)
        torch.cuda.synchronize()
        us_plain, us_fused, us_sep = [1e3 * float(np.median([x.elapsed_time(y) for x, y in evs])) for evs in evp]
        if int(pplan.status.item()) != 0:
            raise RuntimeError(f"device status {int(pplan.status.item())} after the fused prefill")
        S = w.Nv + w.Nt
        flops = 4.0 * w.D * S * (S + 1) / 2 * w.B * w.Hq * w.L  # causal QK^T and PV, every layer
        tf = flops / (us_plain * 1e-6) / 1e12
        pf = {"kernels": ["prefill_kernel", "elite_select_kernel", "finalize_kernel", "topk_select_kernel",
                          "kv_gather_kernel"],
              "layers": w.L, "reps": a.prefill_reps, "statistic": "median of interleaved calls",
              "us_attention_only": us_plain,
              "us_fused_scores_and_compaction": us_fused,
              "us_attention_then_separate_pass": us_sep,
              "fused_overhead_frac": us_fused / us_plain - 1.0,
              "separate_overhead_frac": us_sep / us_plain - 1.0,
              "attention_flops": flops, "attention_tflops": tf, "peak_tflops": PEAK_MFMA_TFLOPS["bf16"],
              "attention_frac_of_mfma_peak": tf / PEAK_MFMA_TFLOPS["bf16"]}
        del qa, po
    ceil = hbm_ceilings()

    tokens = w.L * w.B * w.Nv
    value = tokens / (ms * 1e-3)
    gbps = nbytes["total"] / (ms * 1e-3) / 1e9
    path = ac.scoring_path
    if fused:  # the one kernel does the whole pass: its bytes are all the pass's bytes
        dom, dom_bytes = "aircache_pass", nbytes["total"]
    else:
        dom, dom_bytes = "cross_score", nbytes["cross_score"]
    dom_gbps = dom_bytes / (kern_us[dom] * 1e-6) / 1e9
    dom_kernel = {"rows": "cross_score_rows_kernel", "chunked": "aircache_pass_kernel",
                  "small": "aircache_small_kernel"}.get(path, "cross_score_kernel")
    # counters are taken on the workload as defined (its own base distribution)
    traffic = (measured_traffic(dom_kernel, w.name)
               if w.base == wl.CONFIGS[a.workload].base and a.budget_mode == "aircache" and a.obs_window == 0
               else None)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "visual KV token-layers/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == wl.BF16 else "f32",
        "data": "synthetic",
        "config": dict(w.describe(), base=w.base, budget_mode=a.budget_mode, obs_window=a.obs_window, select=a.select,
                       seed=seed, input_copies=ncopy, cache="hot" if a.hot else "rotated",
                       path=path, launches_per_step=ac.run_launches),
        "samples_per_s": w.B / (ms * 1e-3),
        "visual_tokens_per_s": w.B * w.Nv / (ms * 1e-3),  # B * N_v per step (all layers in it)
        # the pass's own bound: t_roof = max(bytes at the HBM peak, flops at the
        # MFMA peak of the dtype), and t_roof / t_step
        "t_roof_us": t_roof_us,
        "roof_frac": t_roof_us / (ms * 1e3),
        "hbm": {"algorithmic_bytes_per_step": nbytes["total"], "achieved_gbps": gbps,
                "peak_gbps": PEAK_HBM_GBPS, "frac_of_peak": gbps / PEAK_HBM_GBPS},
        "roofline": {"bound": "hbm", "kernel": dom_kernel, "achieved": dom_gbps, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": dom_gbps / PEAK_HBM_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": kern_us[dom]},
        "kernel_us": kern_us,
        "launch_us_p10_p50_p90": None if launch_pct is None else [launch_pct[10], launch_pct[50], launch_pct[90]],
        "hot_ms_per_step": ms_hot,
        # what plain hand-written kernels reach on the same device
        "ceilings": ceil,
        "pass_frac_of_copy_ceiling": gbps / ceil["copy_gbps"],
        "pass_frac_of_read_ceiling": gbps / ceil["read_gbps"],
        "elite_mean": float(n_elite_all.mean()),
        "elite_hist": {int(k): int(v) for k, v in zip(*np.unique(n_elite_all, return_counts=True))},
        "budget_sum_per_step": float(budget_all.sum() / ncopy),
        "budget_min_mean_max": [int(budget_all.min()), float(budget_all.mean()), int(budget_all.max())],
        # decode attention over the compacted cache (a consumer of the pass,
        # timed after the pass, not part of its step)
        "decode_attention": dec,
        "quantize_i8": quant,
        # prefill attention with the scores fused in, against the attention
        # alone and the attention followed by the separate pass
        "prefill": pf,
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, a.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
