#!/usr/bin/env python3
"""Benchmark of the compressed sparse KV attention hot path on one MI355X.

One step = the 1M-token layer pair: compress the raw bf16 KV [2^20, 512] at
m = 4 (262,144 entries) and m' = 128 (8,192 entries) into 576-wide entry
buffers in one fused pass over the raw rows, then CSA decode (indexer top-1024 + 128-token window) and HCA decode
(dense over all 8,192 entries) for 32 queries x 128 heads.  Inputs are seeded
synthetic tensors already resident in HBM; every kernel of the step runs in
the timed region.

Metric: compressed-KV entries attended per second, counted as (query,
compressed entry) pairs: 32 x 1024 (CSA) + 32 x 8192 (HCA) per step.

Prints one JSON line.  Per-kernel durations come from HIP events recorded on
the launch stream around each launch inside the timed steps; the roofline of
the dominant kernel divides its algorithmic bytes by its average duration.
The CPU baseline times the oracle on a bounded sample of the same step.
"""
import argparse
import functools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
D, R, E, I = 512, 64, 576, 64


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-chunk measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the tiny, CSA-decode and HCA-decode workload legs")
    return ap.parse_args()


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    from compressed_sparse_kv_overlapping_amd.profiling import source_digest
    entry = t.get("kernels", {}).get(kernel)
    if not entry or t.get("source_digest") != source_digest():
        return None
    return entry.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is described in DESIGN.md, not built.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import compressed_sparse_kv_overlapping_amd as cskv
    import workloads as wl
    from workloads.device import dev

    torch.cuda.set_device(0)
    cfg = wl.CONFIGS["layer_1m"]
    t_gen = time.time()
    inp = wl.make_inputs(cfg, seed=args.seed)
    T, B, H, k, W = cfg.T, cfg.B, cfg.H, cfg.k, cfg.W
    N4, N128 = T // cfg.m_csa, T // cfg.m_hca
    x, z = dev(inp["x"]), dev(inp["z"])
    b4, b128 = dev(inp["b4"]), dev(inp["b128"])
    ent4 = torch.empty((N4, E), dtype=torch.bfloat16, device="cuda")
    ent128 = torch.empty((N128, E), dtype=torch.bfloat16, device="cuda")
    ent4[:, D:] = dev(inp["rope4"])
    ent128[:, D:] = dev(inp["rope128"])
    win, q, q_hca = dev(inp["window"]), dev(inp["q"]), dev(inp["q_hca"])
    qI, kI = dev(inp["qI"]), dev(inp["kI"])
    out_csa = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    out_hca = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    lse_csa = torch.empty((B, H), dtype=torch.float32, device="cuda")
    lse_hca = torch.empty((B, H), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    ws_topk = torch.empty(cskv.index_topk_workspace_size(B, N4, k), dtype=torch.uint8, device="cuda")
    ws_csa = torch.empty(max(1, cskv.attend_workspace_size(B, H, k + W)), dtype=torch.uint8, device="cuda")
    ws_hca = torch.empty(max(1, cskv.hca_workspace_size(B, H, N128)), dtype=torch.uint8, device="cuda")
    ws_c = torch.empty(cskv.compress2_workspace_size(T, cfg.m_hca), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    gen_s = time.time() - t_gen

    parts = ["compress", "csa_topk", "csa_attend", "hca_attend"]

    def step(ev):
        ev[0].record()
        cskv.compress2(x, z, b4, cfg.m_csa, b128, cfg.m_hca, out_small=ent4, out_large=ent128,
                       workspace=ws_c)
        ev[1].record()
        cskv.index_topk(qI, kI, k, idx_out=idx, workspace=ws_topk)
        ev[2].record()
        cskv.sparse_attend(q, ent4, win, idx, out=out_csa, lse=lse_csa, workspace=ws_csa)
        ev[3].record()
        cskv.hca_attend(q_hca, ent128, out=out_hca, lse=lse_hca, workspace=ws_hca)
        ev[4].record()

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)]

    for _ in range(args.warmup):
        step(events())
    torch.cuda.synchronize()
    # warm cache (reported, labelled): the steps back to back, so what one
    # step leaves in the 256 MB last-level cache (the queries, keys and HCA
    # entries) is still there for the next
    wevs = [events() for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(wevs[i])
    stop.record()
    torch.cuda.synchronize()
    warm_ms = start.elapsed_time(stop) / args.steps
    warm_parts = {p: round(float(np.mean([e[j].elapsed_time(e[j + 1]) for e in wevs])), 4)
                  for j, p in enumerate(parts)}
    # cold cache (the headline): before every step, outside the step's
    # events, 1 GiB is written to a scratch buffer, which evicts the 256 MB
    # last-level cache, and then 512 MiB of another buffer are read, so that
    # the scratch lines the write left dirty are written back before the step
    # starts rather than during its first kernel; each step is timed by its
    # own events.  The same steps after the write alone ("dirty") are
    # reported beside it.
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    clean = torch.ones(1 << 26, dtype=torch.int64, device="cuda")
    acc = torch.zeros(1, dtype=torch.int64, device="cuda")

    def flush(i, writeback):
        scratch.fill_(i & 0xff)
        if writeback:
            acc.add_(clean.sum())

    def cold_steps(writeback):
        e_all = [events() for _ in range(args.steps)]
        torch.cuda.synchronize()
        t_0 = time.perf_counter()
        for i in range(args.steps):
            flush(i, writeback)
            step(e_all[i])
        torch.cuda.synchronize()
        return e_all, time.perf_counter() - t_0

    evs, wall = cold_steps(True)
    dirty_evs, _ = cold_steps(False)
    del scratch, clean
    dirty_ms = float(np.mean([e[0].elapsed_time(e[-1]) for e in dirty_evs]))
    dirty_parts = {p: round(float(np.mean([e[j].elapsed_time(e[j + 1]) for e in dirty_evs])), 4)
                   for j, p in enumerate(parts)}
    ms_step = float(np.mean([e[0].elapsed_time(e[-1]) for e in evs]))
    part_ms = {p: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs]))
               for j, p in enumerate(parts)}
    # per-step latency: first launch to last completion of each step
    lat = np.array([e[0].elapsed_time(e[-1]) for e in evs])
    latency = {"p50": round(float(np.percentile(lat, 50)), 4),
               "p95": round(float(np.percentile(lat, 95)), 4),
               "p99": round(float(np.percentile(lat, 99)), 4), "samples": int(len(lat)),
               "parts_p50": {p: round(float(np.percentile([e[j].elapsed_time(e[j + 1]) for e in evs], 50)), 4)
                             for j, p in enumerate(parts)}}

    pairs = B * k + B * N128
    value = pairs / (ms_step * 1e-3)

    # algorithmic bytes / flops per launch (inputs once, outputs once; the
    # selected entries are gathered per query, the shared window once)
    bx = 2 * T * D * 2
    alg = {
        "compress": {"bytes": bx + (N4 + N128) * D * 2},
        "csa_topk": {"bytes": N4 * I * 2 + B * I * 2 + B * k * 4, "flops": 2 * B * N4 * I},
        "csa_attend": {"bytes": B * k * E * 2 + W * E * 2 + B * H * E * 2 + B * H * D * 2,
                       "flops": 2 * B * H * (k + W) * (E + D)},
        "hca_attend": {"bytes": N128 * E * 2 + B * H * E * 2 + B * H * D * 2,
                       "flops": 2 * B * H * N128 * (E + D)},
    }
    detail = {}
    for p in parts:
        t = part_ms[p] * 1e-3
        d = {"ms": round(part_ms[p], 4), "GB/s": round(alg[p]["bytes"] / t / 1e9, 1),
             "hbm_frac": round(alg[p]["bytes"] / t / 1e9 / HBM_PEAK_GBS, 4)}
        if "flops" in alg[p]:
            d["TFLOP/s"] = round(alg[p]["flops"] / t / 1e12, 2)
            d["bf16_mfma_frac"] = round(alg[p]["flops"] / t / 1e12 / BF16_PEAK_TFLOPS, 4)
        detail[p] = d
    dom = max(parts, key=lambda p: part_ms[p])
    ach = alg[dom]["bytes"] / (part_ms[dom] * 1e-3) / 1e9
    traffic = measured_traffic(dom)
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "alg_bytes_per_launch": alg[dom]["bytes"]}

    comp_ms = part_ms["compress"]
    attn_ms = part_ms["csa_topk"] + part_ms["csa_attend"] + part_ms["hca_attend"]
    comp_bytes = alg["compress"]["bytes"]
    attn_bytes = alg["csa_topk"]["bytes"] + alg["csa_attend"]["bytes"] + alg["hca_attend"]["bytes"]

    result = {
        "metric": "compressed-KV entries attended/sec + % HBM peak, CSA/HCA decode at 1M ctx",
        "value": round(value, 1), "unit": "entries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "layer_1m", "raw_tokens": T, "entries_m4": N4, "entries_m128": N128,
                   "queries": B, "heads": H, "top_k": k, "window": W,
                   "pairs_per_step": pairs, "kv": "shared context"},
        "roofline": roofline,
        "cache": ("cold: before each step, outside its events, 1 GiB written to a scratch "
                  "buffer (evicting the 256 MB last-level cache), then 512 MiB of another "
                  "buffer read so that the write's dirty lines are written back before the "
                  "step; each step timed by its own events"),
        "cold_dirty_cache": {"ms_per_step": round(dirty_ms, 4), "parts_ms": dirty_parts,
                             "value": round(pairs / (dirty_ms * 1e-3), 1),
                             "note": ("the same steps after the 1 GiB write alone: the first "
                                      "kernel also writes back the scratch lines left dirty "
                                      "in the last-level cache")},
        "warm_cache": {"ms_per_step": round(warm_ms, 4), "parts_ms": warm_parts,
                       "value": round(pairs / (warm_ms * 1e-3), 1),
                       "note": "the same steps back to back (inputs left in the last-level cache)"},
        "latency_ms": latency,
        "cache_bytes": cache_accounting(T, W, k),
        "run": {"device": torch.cuda.get_device_name(0), "hip": torch.version.hip, "streams": 1,
                "queries": B, "context_tokens": T},
        "compressor_GBps": round(comp_bytes / (comp_ms * 1e-3) / 1e9, 1),
        "attention_GBps": round(attn_bytes / (attn_ms * 1e-3) / 1e9, 1),
        "decode_only_entries_per_s": round(pairs / (attn_ms * 1e-3), 1),
        "parts": detail,
        "wall_s_timed": round(wall, 3), "wall_note": "the timed steps with the cache flushes between them",
        "input_gen_s": round(gen_s, 1),
    }
    del x, z
    torch.cuda.empty_cache()
    if not args.no_prefill:
        result["prefill"] = bench_prefill(args, cskv, wl, dev, torch, np)
        torch.cuda.empty_cache()
        result["hca_prefill"] = bench_hca_prefill(args, cskv, wl, dev, torch, np)
        result["mxfp4_topk"] = bench_mxfp4_topk(args, cskv, wl, inp, cfg, torch, np,
                                                part_ms["csa_topk"])
        result["mxfp4_attend"] = bench_mxfp4_attend(args, cskv, inp, cfg, dev, torch, np,
                                                    part_ms)
        torch.cuda.empty_cache()
        result["per_sequence"] = bench_per_sequence(args, cskv, inp, cfg, dev, torch)
        torch.cuda.empty_cache()
    if not args.no_configs:
        result["configs"] = bench_configs(args, cskv, wl, dev, torch, np)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, inp, cfg, ms_step, np)
    print(json.dumps(result), flush=True)


def _time_eager(fn, outs, torch, iters=50):
    """Time a call sequence eagerly (events around back-to-back calls, inputs
    warm); returns the time and the outputs it left."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters * 1e3, ref


def _time_graph(fn, outs, ref, torch, iters=50):
    """Time one call sequence captured in a HIP graph and replayed.  Every
    checked replay starts from cleared outputs (eager work between replays)
    and must give the eager result bit for bit."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for _ in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            if not torch.equal(o, r):
                raise RuntimeError("a replayed graph differs from the eager result")
    e0.record()
    for _ in range(iters):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) / iters * 1e3
    del g
    return graph_us


def bench_configs(args, cskv, wl, dev, torch, np):
    """The three small workloads, each timed eagerly and as a replayed HIP
    graph (one call sequence captured; replays checked against the eager
    result): the tiny fp32 layer (both scales compressed from 4,096 raw
    tokens, CSA top-64 + 128 window rows and HCA over 32 entries, 1 query x 16
    heads), CSA decode (8 queries x 128 heads, top-1024 of 16,384 entries +
    128 window rows) and HCA decode (16 queries x 128 heads over 8,192
    entries), bf16."""
    res = {"note": "eager: events around 50 back-to-back calls (inputs warm), every leg timed "
                   "before any capture, so decode selections take the one-launch path where it "
                   "applies; graph: one call sequence captured in a HIP graph and replayed 50 "
                   "times (under capture the selection takes the multi-launch path)"}
    legs = {}
    f32, bf = torch.float32, torch.bfloat16
    # tiny
    cfg = wl.CONFIGS["tiny"]
    inp = wl.make_inputs(cfg, seed=args.seed)
    B, H, k, T = cfg.B, cfg.H, cfg.k, cfg.T
    x, z, b4, b128 = dev(inp["x"]), dev(inp["z"]), dev(inp["b4"]), dev(inp["b128"])
    e4 = torch.zeros((T // 4, E), dtype=f32, device="cuda")
    e128 = torch.zeros((T // 128, E), dtype=f32, device="cuda")
    e4[:, D:] = dev(inp["rope4"])
    e128[:, D:] = dev(inp["rope128"])
    q, qI, kI, win, qh = (dev(inp[n]) for n in ("q", "qI", "kI", "window", "q_hca"))
    o1 = torch.empty((B, H, D), dtype=f32, device="cuda")
    o2 = torch.empty((B, H, D), dtype=f32, device="cuda")
    l1 = torch.empty((B, H), dtype=f32, device="cuda")
    l2 = torch.empty((B, H), dtype=f32, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    wsc = torch.empty(cskv.compress2_workspace_size(T, 128), dtype=torch.uint8, device="cuda")
    wsa = torch.empty(cskv.csa_workspace_size(B, H, T // 4, cfg.W, k), dtype=torch.uint8, device="cuda")
    wsh = torch.empty(max(1, cskv.hca_workspace_size(B, H, T // 128)), dtype=torch.uint8, device="cuda")

    # (the arguments are bound now: the names are reused by the legs below)
    def tiny(x=x, z=z, b4=b4, b128=b128, e4=e4, e128=e128, q=q, qI=qI, kI=kI, win=win, k=k, o1=o1,
             l1=l1, idx=idx, wsc=wsc, wsa=wsa, qh=qh, o2=o2, l2=l2, wsh=wsh):
        cskv.compress2(x, z, b4, 4, b128, 128, out_small=e4, out_large=e128, workspace=wsc)
        cskv.csa_attend(q, qI, e4, kI, win, k, out=o1, lse=l1, idx_out=idx, workspace=wsa)
        cskv.hca_attend(qh, e128, out=o2, lse=l2, workspace=wsh)
    # the compressor writes columns [0, 512); the rope columns are inputs
    legs["tiny"] = (tiny, [e4[:, :D], e128[:, :D], o1, l1, o2, l2, idx])
    res["tiny"] = {"workload": "tiny", "dtype": "f32", "launches": "compress2 + csa_attend + hca_attend",
                   "pairs": B * k + B * (T // 128),
                   "bound": "launch latency (about 30 kB of inputs per step)"}
    # CSA decode
    cfg = wl.CONFIGS["csa_decode"]
    inp = wl.make_inputs(cfg, seed=args.seed)
    B, H, k, W, N = cfg.B, cfg.H, cfg.k, cfg.W, cfg.N_csa
    q, qI, kI, ent, win = (dev(inp[n]) for n in ("q", "qI", "kI", "entries", "window"))
    o = torch.empty((B, H, D), dtype=bf, device="cuda")
    l = torch.empty((B, H), dtype=f32, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    wsa = torch.empty(cskv.csa_workspace_size(B, H, N, W, k), dtype=torch.uint8, device="cuda")
    legs["csa_decode"] = (functools.partial(cskv.csa_attend, q, qI, ent, kI, win, k, out=o, lse=l,
                                            idx_out=idx, workspace=wsa), [o, l, idx])
    nbytes = N * I * 2 + B * I * 2 + B * k * E * 2 + W * E * 2 + B * H * E * 2 + B * H * D * 2
    res["csa_decode"] = {"workload": "csa_decode", "dtype": "bf16", "launches": "csa_attend",
                         "pairs": B * k, "alg_bytes": nbytes}
    # HCA decode
    cfg = wl.CONFIGS["hca_decode"]
    inp = wl.make_inputs(cfg, seed=args.seed)
    B, H, N = cfg.B, cfg.H, cfg.N_hca
    q, ent = dev(inp["q_hca"]), dev(inp["entries_hca"])
    o = torch.empty((B, H, D), dtype=bf, device="cuda")
    l = torch.empty((B, H), dtype=f32, device="cuda")
    wsh = torch.empty(max(1, cskv.hca_workspace_size(B, H, N)), dtype=torch.uint8, device="cuda")
    legs["hca_decode"] = (functools.partial(cskv.hca_attend, q, ent, out=o, lse=l, workspace=wsh), [o, l])
    res["hca_decode"] = {"workload": "hca_decode", "dtype": "bf16", "launches": "hca_attend",
                         "pairs": B * N, "flops": 2 * B * H * N * (E + D)}
    # every eager leg first: a capture runs on a side stream, after which the
    # library keeps decode selections on the multi-launch path
    refs = {}
    for name, (fn, outs) in legs.items():
        res[name]["eager_us"], refs[name] = _time_eager(fn, outs, torch)
    for name, (fn, outs) in legs.items():
        res[name]["graph_us"] = _time_graph(fn, outs, refs[name], torch)
    for name in legs:
        r = res[name]
        eu, gu = r["eager_us"], r["graph_us"]
        r["eager_us"], r["graph_us"] = round(eu, 2), round(gu, 2)
        r["entries_attended_per_s_eager"] = round(r["pairs"] / (eu * 1e-6), 1)
        r["entries_attended_per_s_graph"] = round(r.pop("pairs") / (gu * 1e-6), 1)
        best = min(eu, gu)
        if "alg_bytes" in r:
            nb = r.pop("alg_bytes")
            r["roofline"] = {"bound": "hbm", "achieved": round(nb / (best * 1e-6) / 1e9, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(nb / (best * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "alg_bytes": nb,
                             "timing": "eager" if eu <= gu else "graph"}
        if "flops" in r:
            fl = r.pop("flops")
            r["roofline"] = {"bound": "mfma", "achieved": round(fl / (best * 1e-6) / 1e12, 1),
                             "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(fl / (best * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                             "timing": "eager" if eu <= gu else "graph"}
    return res


def bench_per_sequence(args, cskv, inp, cfg, dev, torch):
    """The decode attention in per-sequence mode: each of the 32 queries has
    its own 1M-token caches (262,144 CSA entries and indexer keys, 8,192 HCA
    entries, its own window), the serving reading of a decode batch.  The
    caches are random bf16 drawn on the device (9.7 GB of CSA entries; the
    kernels' time does not depend on the values).  Each query scans its own
    keys and reads its own HCA entries, so this regime is HBM-bound."""
    B, H, k, W, N4, N128 = cfg.B, cfg.H, cfg.k, cfg.W, cfg.N_csa, cfg.N_hca
    g = torch.Generator(device="cuda").manual_seed(args.seed + 7)

    def rnd(*shape):
        t = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        for i in range(shape[0]):
            t[i] = torch.randn(shape[1:], generator=g, device="cuda").to(torch.bfloat16)
        return t
    ent4, keys, ent128, win = rnd(B, N4, E), rnd(B, N4, I), rnd(B, N128, E), rnd(B, W, E)
    qI, q, qh = dev(inp["qI"]), dev(inp["q"]), dev(inp["q_hca"])
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws_t = torch.empty(cskv.index_topk_workspace_size(B, N4, k, per_seq=True), dtype=torch.uint8,
                       device="cuda")
    ws_a = torch.empty(max(cskv.attend_workspace_size(B, H, k + W), cskv.hca_workspace_size(B, H, N128)),
                       dtype=torch.uint8, device="cuda")
    runs = {
        "csa_topk": lambda: cskv.index_topk(qI, keys, k, per_seq=True, idx_out=idx, workspace=ws_t),
        "csa_attend": lambda: cskv.sparse_attend(q, ent4, win, idx, per_seq=True, out=out, lse=lse,
                                                 workspace=ws_a),
        "hca_attend": lambda: cskv.hca_attend(qh, ent128, per_seq=True, out=out, lse=lse,
                                              workspace=ws_a),
    }
    alg = {"csa_topk": B * N4 * I * 2 + B * I * 2 + B * k * 4,
           "csa_attend": B * (k + W) * E * 2 + B * H * E * 2 + B * H * D * 2,
           "hca_attend": B * N128 * E * 2 + B * H * E * 2 + B * H * D * 2}
    res = {"workload": "layer_1m decode, per-sequence caches", "queries": B}
    for name, run in runs.items():
        for _ in range(3):
            run()
        steps = max(20, args.steps // 2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / steps
        gbs = alg[name] / (t * 1e-3) / 1e9
        res[name] = {"ms": round(t, 4), "alg_bytes": alg[name],
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    del ent4, keys, ent128, win
    return res


def cache_accounting(T, W, k):
    """Cache bytes of one layer by kind at T raw tokens, and their slope in
    bytes per raw token: the raw window is a constant, the compressed
    entries and indexer keys grow with T (bf16 storage, and MXFP4 with its
    scale bytes counted apart)."""
    n4, n128 = T // 4, T // 128
    bf16 = {"raw_window": W * E * 2, "csa_entries": n4 * E * 2, "hca_entries": n128 * E * 2,
            "indexer_keys": n4 * I * 2}
    mx = {"raw_window": W * E * 2, "csa_entries": n4 * E // 2, "hca_entries": n128 * E // 2,
          "indexer_keys": n4 * I // 2,
          "scales": n4 * E // 32 + n128 * E // 32 + n4 * I // 32}
    slope = lambda d: {kk: round((v - (W * E * 2 if kk == "raw_window" else 0)) / T, 4)
                       for kk, v in d.items()}
    return {"tokens": T, "selected_per_query": k,
            "bf16": {"bytes": bf16, "total": sum(bf16.values()), "per_token": slope(bf16)},
            "mxfp4": {"bytes": mx, "total": sum(mx.values()), "per_token": slope(mx)}}


def bench_prefill(args, cskv, wl, dev, torch, np):
    """The 4,096-query causal prefill chunk at positions 1,044,480..1,048,575
    over 262,144 entries (fp8 indexer, bf16 attention)."""
    cfg = wl.CONFIGS["csa_prefill"]
    inp = wl.make_inputs(cfg, seed=args.seed)
    B, H, k, W, N = cfg.B, cfg.H, cfg.k, cfg.W, cfg.N_csa
    q, ent, win = dev(inp["q"]), dev(inp["entries"]), dev(inp["window"])
    qI, kI = dev(inp["qI"]), dev(inp["kI"])
    scale = inp["qI"].scale * inp["kI"].scale
    qp = torch.from_numpy(inp["q_pos"]).cuda()
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws_t = torch.empty(cskv.index_topk_workspace_size(B, N, k), dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(max(1, cskv.attend_workspace_size(B, H, k + W)), dtype=torch.uint8, device="cuda")

    def run(ev):
        ev[0].record()
        cskv.index_topk(qI, kI, k, q_pos=qp, m=4, idx_scale=scale, idx_out=idx, workspace=ws_t)
        ev[1].record()
        cskv.sparse_attend(q, ent, win, idx, q_pos=qp, win_pos0=inp["win_pos0"], W=W, out=out,
                           lse=lse, workspace=ws_a)
        ev[2].record()

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for _ in range(2):
        run(mk())
    steps = max(3, args.steps // 4)
    evs = [mk() for _ in range(steps)]
    torch.cuda.synchronize()
    for e in evs:
        run(e)
    torch.cuda.synchronize()
    t_sel = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    t_att = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    n_vis = np.minimum((inp["q_pos"] + 1) // 4, N)
    pairs = int(n_vis.sum())                                   # visible (query, entry) scores
    idx_flops = 2 * pairs * I
    att_flops = 2 * B * H * (k + W) * (E + D)
    return {
        "workload": "csa_prefill", "queries": B, "entries": N, "top_k": k, "window": W,
        "ms": round(t_sel + t_att, 4),
        "entries_attended_per_s": round(B * k / ((t_sel + t_att) * 1e-3), 1),
        "indexer_topk_ms": round(t_sel, 4),
        "indexer_TFLOPs": round(idx_flops / (t_sel * 1e-3) / 1e12, 2),
        "indexer_frac_bf16_peak": round(idx_flops / (t_sel * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "indexer_frac_fp8_peak": round(idx_flops / (t_sel * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
        "attention_ms": round(t_att, 4),
        "attention_roofline": {"bound": "mfma", "achieved": round(att_flops / (t_att * 1e-3) / 1e12, 1),
                               "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(att_flops / (t_att * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
    }


def bench_hca_prefill(args, cskv, wl, dev, torch, np):
    """HCA at the same prefill chunk: 4,096 causal queries at positions
    1,044,480..1,048,575 attend densely over the 8,192 m'=128 entries they
    see ((i+1)*128 <= pos+1: 8,160..8,192 of them)."""
    cfg = wl.CONFIGS["hca_prefill"]
    inp = wl.make_inputs(cfg, seed=args.seed)
    B, H, N, m = cfg.B, cfg.H, cfg.N_hca, cfg.m_hca
    q, ent = dev(inp["q_hca"]), dev(inp["entries_hca"])
    qp = torch.from_numpy(inp["q_pos"]).cuda()
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, cskv.hca_workspace_size(B, H, N)), dtype=torch.uint8, device="cuda")
    run = lambda: cskv.hca_attend(q, ent, q_pos=qp, m=m, out=out, lse=lse, workspace=ws)
    for _ in range(2):
        run()
    steps = max(3, args.steps // 4)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / steps
    n_vis = np.minimum((inp["q_pos"] + 1) // m, N)
    flops = 2 * H * int(n_vis.sum()) * (E + D)
    return {
        "workload": "hca_prefill", "queries": B, "entries": N, "ms": round(t, 4),
        "entries_attended_per_s": round(int(n_vis.sum()) / (t * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(flops / (t * 1e-3) / 1e12, 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / (t * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
    }


def bench_mxfp4_topk(args, cskv, wl, inp, cfg, torch, np, bf16_ms):
    """The decode step's indexer selection with MXFP4 queries and keys: the
    same draws as the bf16 indexer inputs, quantised per 32-element block
    (34 bytes per key instead of 128)."""
    B, N, k = cfg.B, cfg.N_csa, cfg.k
    qc, qs = wl.mxfp4_encode(wl.bf16_bits_to_f32(inp["qI"].raw))
    kc, ks = wl.mxfp4_encode(wl.bf16_bits_to_f32(inp["kI"].raw))
    qc, qs, kc, ks = (torch.from_numpy(a).cuda() for a in (qc, qs, kc, ks))
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    ws = torch.empty(cskv.index_topk_workspace_size(B, N, k), dtype=torch.uint8, device="cuda")
    run = lambda: cskv.index_topk_mxfp4(qc, qs, kc, ks, k, idx_out=idx, workspace=ws)
    for _ in range(3):
        run()
    steps = max(20, args.steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / steps
    nbytes = N * 34 + B * 34 + B * k * 4
    return {
        "workload": "layer_1m decode indexer, MXFP4", "queries": B, "entries": N, "k": k,
        "ms": round(t, 4), "bf16_ms": bf16_ms,
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (t * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }


def bench_mxfp4_attend(args, cskv, inp, cfg, dev, torch, np, part_ms):
    """The decode step's two attentions over MXFP4 entries (306 bytes a row
    instead of 1,152): CSA over 1,024 selected of 262,144 entries plus the
    128 window rows, and HCA over 8,192 entries, 32 queries x 128 heads.
    Each call includes the decode of the rows it reads to bf16.
    The codes are uniform random bytes and the scales 2^-2..2^0 (the
    kernels' time does not depend on the values); the selection is a random
    sorted one per query."""
    B, H, k, W = cfg.B, cfg.H, cfg.k, cfg.W
    rng = np.random.default_rng(5)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    c4 = up(rng.integers(0, 256, (cfg.N_csa, E // 2), dtype=np.uint8))
    s4 = up(rng.integers(125, 128, (cfg.N_csa, E // 32), dtype=np.uint8))
    c128 = up(rng.integers(0, 256, (cfg.N_hca, E // 2), dtype=np.uint8))
    s128 = up(rng.integers(125, 128, (cfg.N_hca, E // 32), dtype=np.uint8))
    idx = up(np.sort(np.stack([rng.choice(cfg.N_csa, k, replace=False) for _ in range(B)]),
                     axis=1).astype(np.int32))
    q, qh, win = dev(inp["q"]), dev(inp["q_hca"]), dev(inp["window"])
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    lib = cskv.binding.library()
    ws = torch.empty(max(lib.cskv_sparse_attend_mxfp4_workspace_size(B, H, W, k),
                         lib.cskv_hca_attend_mxfp4_workspace_size(B, H, cfg.N_hca, 0)),
                     dtype=torch.uint8, device="cuda")
    runs = {
        "csa_attend": lambda: cskv.sparse_attend_mxfp4(q, c4, s4, win, idx, out=out, lse=lse,
                                                       workspace=ws),
        "hca_attend": lambda: cskv.hca_attend_mxfp4(qh, c128, s128, out=out, lse=lse, workspace=ws),
    }
    res = {"workload": "layer_1m decode attention, MXFP4 entries", "queries": B, "heads": H}
    for name, run in runs.items():
        for _ in range(3):
            run()
        steps = max(20, args.steps)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / steps
        rows = k + W if name == "csa_attend" else cfg.N_hca
        flops = 2 * B * H * rows * (E + D)
        res[name] = {"ms": round(t, 4), "bf16_entries_ms": round(part_ms[name], 4),
                     "roofline": {"bound": "mfma", "achieved": round(flops / (t * 1e-3) / 1e12, 1),
                                  "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(flops / (t * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}}
    return res


def cpu_baseline(args, inp, cfg, gpu_ms, np):
    """The oracle (plain fp64 C, OpenMP over independent outputs) on the same
    step: a small calibration sample predicts the whole step's time, then the
    largest fraction of the step that fits --cpu-seconds (the whole step when
    it fits) is run and timed, and scaled to a whole step.  Attention runs
    over the oracle's own compressed entries."""
    import oracle
    import workloads as wl
    threads = oracle.max_threads()
    T, B, H, k = cfg.T, cfg.B, cfg.H, cfg.k
    N4, N128 = T // 4, T // 128
    rng = np.random.default_rng(0)

    def ids(n, total):
        return np.arange(total) if n >= total else np.sort(rng.choice(total, n, replace=False))

    def entries(ids_, m, bias):
        return oracle.compress(inp["x"].raw, inp["z"].raw, wl.DT_BF16, bias, m, entry_ids=ids_)

    def run(f):
        """Times of each part on fraction f of the step, scaled to the step."""
        n4, n128 = max(64, int(N4 * f)), max(4, int(N128 * f))
        nq, nh = max(1, int(round(B * f))), max(8, int(H * f)) if f < 1 else H
        i4, i128 = ids(n4, N4), ids(n128, N128)
        t = time.perf_counter()
        c4 = entries(i4, 4, inp["b4"].raw)
        t_c4 = (time.perf_counter() - t) * N4 / len(i4)
        t = time.perf_counter()
        c128 = entries(i128, 128, inp["b128"].raw)
        t_c128 = (time.perf_counter() - t) * N128 / len(i128)
        # entries for attention: the computed ones where sampled, the rest a
        # constant (the oracle's attention cost does not depend on values)
        ent = np.full((N4, E), 0x3f80, np.uint16)
        ent[i4, :D] = wl.bf16_bits(c4.astype(np.float32))
        ent[:, D:] = inp["rope4"].raw
        ent128 = np.full((N128, E), 0x3f80, np.uint16)
        ent128[i128, :D] = wl.bf16_bits(c128.astype(np.float32))
        ent128[:, D:] = inp["rope128"].raw
        t = time.perf_counter()
        sc, vis = oracle.index_scores(inp["qI"].raw[:nq], inp["kI"].raw, wl.DT_BF16)
        sel = oracle.topk(sc, vis, k)
        t_sel = (time.perf_counter() - t) * B / nq
        t = time.perf_counter()
        oracle.csa_attend(inp["q"].raw[:nq], ent, inp["window"].raw, wl.DT_BF16, sel)
        t_csa = (time.perf_counter() - t) * B / nq
        t = time.perf_counter()
        oracle.hca_attend(inp["q_hca"].raw[:nq, :nh], ent128, wl.DT_BF16)
        t_hca = (time.perf_counter() - t) * B * H / (nq * nh)
        return (t_c4, t_c128, t_sel, t_csa, t_hca), (n4, n128, nq, nh)

    est, _ = run(1.0 / 64)
    frac = min(1.0, args.cpu_seconds / max(sum(est), 1e-9))
    # the whole step when it fits, repeated while the budget allows (at most 3 runs)
    t0 = time.perf_counter()
    runs = [run(frac)]
    while (frac >= 1.0 and len(runs) < 3 and
           (time.perf_counter() - t0) * (len(runs) + 1) / len(runs) <= args.cpu_seconds):
        runs.append(run(frac))
    reps = len(runs)
    sample_s = time.perf_counter() - t0
    # one core: a sample sized for about half the budget (the all-core
    # calibration times the thread count), the same parts scaled to the step
    oracle.set_threads(1)
    try:
        f1 = min(1.0, 0.5 * args.cpu_seconds / max(sum(est) * threads, 1e-9))
        f1 = max(f1, 1.0 / 4096)
        t1 = time.perf_counter()
        r1 = run(f1)
        s1 = time.perf_counter() - t1
    finally:
        oracle.set_threads(threads)
    step1 = float(sum(r1[0]))
    n4s, n128s, nqs, nhs = r1[1]
    (n4, n128, nq, nh) = runs[0][1]
    parts = tuple(float(np.mean([r[0][i] for r in runs])) for i in range(5))
    t_c4, t_c128, t_sel, t_csa, t_hca = parts
    step_s = sum(parts)
    pairs = B * k + B * N128
    whole = n4 >= N4 and n128 >= N128 and nq >= B and nh >= H
    return {
        "value": round(pairs / step_s, 2), "unit": "entries/s", "cores": threads, "kind": "oracle",
        "sample": (f"the whole step, {reps} time(s)" if whole else
                   f"compress {n4} of {N4} m=4 entries and {n128} of {N128} m'=128 entries; "
                   f"indexer+top-k and CSA attention for {nq} of {B} queries (all {H} heads); "
                   f"HCA for {nq} queries x {nh} of {H} heads; each part scaled to the full step")
                  + f" ({sample_s:.1f} s of oracle time, after a 1/64 calibration sample)",
        "step_s_extrapolated": round(step_s, 2),
        "parts_s": {"compress_m4": round(t_c4, 2), "compress_m128": round(t_c128, 2),
                    "csa_topk": round(t_sel, 2), "csa_attend": round(t_csa, 2),
                    "hca_attend": round(t_hca, 2)},
        "gpu_speedup": round(step_s / (gpu_ms * 1e-3), 1),
        "single_core": {
            "value": round(pairs / step1, 2), "unit": "entries/s", "cores": 1, "kind": "oracle",
            "sample": (f"compress {n4s} of {N4} m=4 entries and {n128s} of {N128} m'=128 entries; "
                       f"indexer+top-k and CSA attention for {nqs} of {B} queries; HCA for {nqs} "
                       f"queries x {nhs} of {H} heads; each part scaled to the full step "
                       f"({s1:.1f} s of oracle time on one thread)"),
            "step_s_extrapolated": round(step1, 2),
            "parts_s": dict(zip(("compress_m4", "compress_m128", "csa_topk", "csa_attend",
                                 "hca_attend"), (round(float(v), 2) for v in r1[0]))),
        },
    }

if __name__ == "__main__":
    main()
