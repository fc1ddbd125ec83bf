#!/usr/bin/env python3
"""Benchmark of the absorbed-MLA hot path on one MI355X.

One step = the whole path over one batch: mla_absorb_q -> mla_latent_attn_up_v (split kernel,
then the log-sum-exp merge of the splits fused into the value up-projection), on the
single-token decode workload with batch 32, cache length 8192, 64 heads, 256-dim heads, latent
512 (bf16 inputs, fp32 outputs).  Inputs are resident in HBM before the timed region; three
input sets rotate so the 256 MB Infinity Cache cannot hold the 256 MiB latent cache between
steps.

Prints ONE JSON line: value = latent-cache GB/s over whole steps (bytes of latent rows the
path reads per step / step time).  `roofline` is the dominant call, the latent attention
(mla_latent_attn: split kernel + log-sum-exp merge), timed with HIP events on the stream it is
launched on; the projections are not counted in it.  `fused_attn_up_v` gives the call the step
actually runs, attention with the merge fused into the up-projection, against the bytes it must
move.  `secondary` is the 6-position verification pass (batch 16, cache 32768) in TFLOP/s
against the bf16 matrix-core peak.
`cpu_baseline` is the fp64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix-core peak
WEIGHT_ROTATION_BYTES = 384 << 20   # weight copies a step rotates over: more than the Infinity Cache
NSETS = 3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_text(src: str) -> str:
    """C++ source with comments removed and whitespace collapsed: what the compiler sees.  (The
    sources hold no comment markers inside string literals.)"""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_digest() -> str:
    """Digest of the attention kernels' code (comments and layout excluded), recorded beside the
    counter measurements so that they are used only while the code they measured is unchanged."""
    h = hashlib.sha256()
    for f in ("latent_attn.hip", "up_v.hip", "mla_device.h", "mla_internal.h", "mla_api.hip"):
        h.update(code_text(open(os.path.join(ROOT, "mla_latent_cache_absorb_amd", "csrc", f)).read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, if recorded for this exact kernel
    source (profiles/traffic_<workload>.md holds 'key: value' lines)."""
    path = os.path.join(ROOT, "profiles", f"traffic_latent_attn_{workload}.md")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_digest") != kernel_source_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def warm_up(call, min_calls: int, min_ms: float = 20.0) -> int:
    """Untimed calls of call(k), in batches of at least `min_calls`, until about `min_ms` of wall
    time has passed with the device busy: an idle device drops its clock, and work issued right
    after an idle spell runs below the steady clock for a few milliseconds (a 4 x 131,072 decode
    call measured 124-136 us after 20 warm-up calls against 112-117 us after 100).  The collector
    runs first, before the device is busy.  Returns the number of calls made."""
    import torch
    gc.collect()
    t0 = time.perf_counter()
    k = 0
    while True:
        for _ in range(max(1, min_calls)):
            call(k)
            k += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms:
            return k


def chunked_ms(call, steps: int, stream=None, nchunk: int = 5):
    """`steps` calls of call(k) launched back to back in `nchunk` chunks, an event between chunks
    (an event does not stop the stream).  Returns (average over every call, per-call average of the
    median chunk).  The first is the figure reported; the second, beside it, shows whether one
    stall of the host or the device set it.  The collector is off meanwhile; it is not run here:
    the device would idle meanwhile and the timed calls would start below the steady clock (the
    callers run it before their warm-up calls)."""
    import torch
    nchunk = nchunk if steps >= 2 * nchunk else 1
    sizes = [steps // nchunk + (1 if c < steps % nchunk else 0) for c in range(nchunk)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nchunk + 1)]
    was_enabled = gc.isenabled()
    gc.disable()
    try:
        if stream is None:
            ev[0].record()
        else:
            ev[0].record(stream)
        done = 0
        for c in range(nchunk):
            for k in range(sizes[c]):
                call(done + k)
            done += sizes[c]
            if stream is None:
                ev[c + 1].record()
            else:
                ev[c + 1].record(stream)
        torch.cuda.synchronize()
    finally:
        if was_enabled:
            gc.enable()
    chunk = sorted(ev[c].elapsed_time(ev[c + 1]) / sizes[c] for c in range(nchunk))
    return ev[0].elapsed_time(ev[nchunk]) / steps, chunk[nchunk // 2]


def visible_rows(w) -> int:
    """Latent rows the attention reads: every visible position of every query (dense), or every
    listed position (indexed).  Queries of one sequence share rows in the dense case."""
    import numpy as np
    if w.idx is not None:
        return int(w.idx_len.sum())
    B, Q = w.q.shape[:2]
    return int(np.sum(w.cache_len.astype(np.int64)))  # the longest query's prefix covers the others


def attended_positions(w) -> int:
    """Sum over queries of the positions each attends to (for FLOP counts)."""
    import numpy as np
    if w.idx is not None:
        return int(w.idx_len.astype(np.int64).sum())
    B, Q = w.q.shape[:2]
    return int(sum(int(w.cache_len[b]) - Q + i + 1 for b in range(B) for i in range(Q)))


def attn_up_v_bytes(w) -> int:
    """Bytes mla_latent_attn_up_v must move: the latent rows, U^V once, the absorbed queries in,
    the outputs and log-sum-exps out."""
    B, Q, H, D = w.q.shape
    R = w.cache.shape[2]
    return visible_rows(w) * R * 2 + H * D * R * 2 + B * Q * H * (R * 2 + D * 4 + 4)


def attn_up_v_flops(w) -> int:
    """FLOPs of mla_latent_attn_up_v: 4 H R per (query, attended position) for the scores and the
    value sum, and 2 H D R per query for the up-projection."""
    B, Q, H, D = w.q.shape
    R = w.cache.shape[2]
    return 4 * H * R * attended_positions(w) + 2 * H * D * R * B * Q


def to_device(w, dev):
    import numpy as np
    import torch
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    d = dict(q=bf(w.q), cache=bf(w.cache), w_k=bf(w.w_k), w_v=bf(w.w_v),
             cache_len=torch.from_numpy(w.cache_len).to(dev))
    if w.idx is not None:
        d["idx"] = torch.from_numpy(w.idx).to(dev)
        d["idx_len"] = torch.from_numpy(w.idx_len).to(dev)
    return d


def time_path(name: str, steps: int, warmup: int, nsets: int):
    """Run the path; returns per-step and per-stage times (ms) and the workload."""
    import torch
    from mla_latent_cache_absorb_amd import binding, workloads as wl

    dev = torch.device("cuda:0")
    log(f"[bench] generating {nsets} input set(s) for {name}")
    ws = [wl.make_workload(name, set_index=s) for s in range(nsets)]
    sets = [to_device(w, dev) for w in ws]
    w0 = ws[0]
    B, Q, H, D = w0.q.shape
    R = w0.cache.shape[2]
    Lmax = int(w0.cache.shape[1])
    indexed = w0.idx is not None
    K_max = w0.idx.shape[2] if indexed else Lmax
    splits = binding.mla_latent_attn_num_splits(B, Q, H, K_max, 0, indexed=indexed)
    q_abs = torch.empty((B, Q, H, R), dtype=torch.bfloat16, device=dev)
    o_lat = torch.empty((B, Q, H, R), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=dev)
    out = torch.empty((B, Q, H, D), dtype=torch.float32, device=dev)
    ws_bytes = max(binding.mla_latent_attn_workspace_size(B, Q, H, R, K_max, 0, indexed=indexed),
                   binding.mla_latent_attn_up_v_workspace_size(B, Q, H, R, K_max, 0, indexed=indexed))
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    # Weights rotate over copies holding WEIGHT_ROTATION_BYTES or more, so that a step never finds
    # its layer's W^UK / W^UV in the 256 MB Infinity Cache from an earlier step: in a model a
    # layer's weights come back only after every other layer's weights and caches have streamed.
    # (The caches' non-temporal stream leaves the cache to data that is reused, and three weight
    # sets of 32 MiB would otherwise stay resident.)
    wts = [(d["w_k"], d["w_v"]) for d in sets]
    pair_bytes = wts[0][0].numel() * 2 + wts[0][1].numel() * 2
    while len(wts) * pair_bytes < WEIGHT_ROTATION_BYTES:
        wk, wv = wts[len(wts) % nsets]
        wts.append((wk.clone(), wv.clone()))
    nw = len(wts)

    def attn_up_v(d, s):
        binding.mla_latent_attn_up_v(q_abs, d["cache"], d["cache_len"], Lmax, w0.scale, wts[s % nw][1], d.get("idx"),
                                     d.get("idx_len"), 0, out=out, lse=lse, workspace=workspace)

    def step(s):
        d = sets[s % nsets]
        binding.mla_absorb_q(d["q"], wts[s % nw][0], q_abs=q_abs)
        attn_up_v(d, s)

    # no collector pauses inside the timed regions: it runs now, before the warm-up (run between the
    # warm-up and the timing, it would leave the device idle and the first timed steps below the
    # steady clock), and again after them
    gc.collect()
    gc.disable()
    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    # whole steps, back to back
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(steps):
        step(warmup + s)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / steps
    # per-stage durations, each stage's `steps` calls (input sets rotating as in the steps) between
    # two events.  The attention calls take longer on the GPU than the Python call that launches
    # them, so their calls are launched back to back; the short projections would measure the
    # launch rate that way, so theirs are captured in a HIP graph and replayed.  The separate
    # attention call (merge kernel writing o_lat) and up-projection are timed for comparison.
    def one_stage(k, s):
        d = sets[s % nsets]
        if k == "absorb_q":
            binding.mla_absorb_q(d["q"], wts[s % nw][0], q_abs=q_abs)
        elif k == "latent_attn_up_v":
            attn_up_v(d, s)
        elif k == "latent_attn" and indexed:
            binding.mla_latent_attn_indexed(q_abs, d["cache"], d["cache_len"], d["idx"], d["idx_len"], Lmax,
                                            w0.scale, 0, o_lat=o_lat, lse=lse, workspace=workspace)
        elif k == "latent_attn":
            binding.mla_latent_attn(q_abs, d["cache"], d["cache_len"], Lmax, w0.scale, 0, o_lat=o_lat, lse=lse,
                                    workspace=workspace)
        else:
            binding.mla_up_v(o_lat, wts[s % nw][1], out=out)

    stage, pct, stage_med = {}, {}, {}
    for k in ("absorb_q", "latent_attn_up_v", "latent_attn", "up_v"):
        if k.startswith("latent_attn"):
            warm_up(lambda s: one_stage(k, s), 3)
            # back to back: the average over every call, and beside it the median chunk's (chunked_ms)
            stage[k], stage_med[k] = chunked_ms(lambda s: one_stage(k, s), steps, stream)
            # the spread: each call between its own pair of events
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
            ev[0].record(stream)
            for s in range(steps):
                one_stage(k, s)
                ev[s + 1].record(stream)
            torch.cuda.synchronize()
            per = sorted(ev[s].elapsed_time(ev[s + 1]) for s in range(steps))
            pct[k] = [per[int(f * (steps - 1) + 0.5)] for f in (0.1, 0.5, 0.9)]
            continue
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for s in range(steps):
                one_stage(k, s)
        warm_up(lambda s: graph.replay(), 1)  # untimed replays (the capture left the device idle)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        stage[k] = e0.elapsed_time(e1) / steps
        del graph
    gc.enable()
    del sets, wts
    torch.cuda.empty_cache()
    return dict(weight_sets_rotated=nw, ms_step=ms_step, wall_s=wall, stage_ms=stage, stage_median_chunk_ms=stage_med, stage_pct_ms=pct,
                splits=splits, workload=w0)


def time_latency(name: str = "decode_b1_l256", samples: int = 200):
    """Per-call latency of the path at batch 1 (Module 05 section 5's decode-shaped workload,
    one sequence whose cache grows by one position per call): absorb_q, the fused attention with
    up-projection, and the two together.  Each is captured in a HIP graph of one call; every
    sample is one replay between its own pair of HIP events, started behind a short GPU spin so
    that the events bracket the kernels rather than the host's launch.  Reports p10 / p50 / p90
    and the mean of back-to-back replays of a graph of `samples` calls (launch gaps hidden)."""
    import torch
    from mla_latent_cache_absorb_amd import binding

    dev = torch.device("cuda:0")
    from mla_latent_cache_absorb_amd import workloads as wl
    w = wl.make_workload(name)
    d = to_device(w, dev)
    B, Q, H, D = w.q.shape
    R = w.cache.shape[2]
    Lmax = int(w.cache.shape[1])
    q_abs = torch.empty((B, Q, H, R), dtype=torch.bfloat16, device=dev)
    out = torch.empty((B, Q, H, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(binding.mla_latent_attn_up_v_workspace_size(B, Q, H, R, Lmax, 0), 1), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()
    calls = {
        "absorb_q": lambda: binding.mla_absorb_q(d["q"], d["w_k"], q_abs=q_abs),
        "latent_attn_up_v": lambda: binding.mla_latent_attn_up_v(q_abs, d["cache"], d["cache_len"], Lmax, w.scale,
                                                                 d["w_v"], out=out, lse=lse, workspace=ws),
    }
    calls["path"] = lambda: (calls["absorb_q"](), calls["latent_attn_up_v"]())
    spin = getattr(torch.cuda, "_sleep", None)
    res = {"workload": name, "batch": B, "q_len": Q, "cache_len": Lmax,
           "splits": binding.mla_latent_attn_num_splits(B, Q, H, Lmax, 0)}
    for k, fn in calls.items():
        fn()
        torch.cuda.synchronize()
        g1 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g1):
            fn()
        gn = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gn):
            for _ in range(samples):
                fn()
        for _ in range(10):
            g1.replay()
        gn.replay()
        torch.cuda.synchronize()
        per = []
        for _ in range(samples):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if spin is not None:
                spin(20000)
            e0.record(stream)
            g1.replay()
            e1.record(stream)
            e1.synchronize()
            per.append(e0.elapsed_time(e1))
        per.sort()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        gn.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        res[k] = {"p10_p50_p90_ms": [round(per[int(f * (samples - 1) + 0.5)], 6) for f in (0.1, 0.5, 0.9)],
                  "mean_back_to_back_ms": round(e0.elapsed_time(e1) / samples, 6)}
        del g1, gn
    res["sample_note"] = ("each sample one graph replay between its own events, behind a GPU spin"
                          if spin is not None else "each sample one graph replay between its own events")
    return res


def time_read_ceiling(mib: int = 256, nsets: int = 3, calls: int = 30):
    """The device's plain streaming-read rate (mla_stream_read): `calls` reads of `mib` MiB, the
    `nsets` buffers rotating so that the 256 MB Infinity Cache cannot serve them, launched back to
    back between two HIP events on the launch stream (as the attention calls are timed), and the
    spread of single calls, each between its own events behind a short GPU spin so that the events
    bracket the kernel rather than the host's launch.  The ceiling beside the published 8 TB/s
    against which the cache streams of the attention kernels are read."""
    import torch
    from mla_latent_cache_absorb_amd import binding

    dev = torch.device("cuda:0")
    bufs = [torch.full((mib << 20,), s + 1, dtype=torch.uint8, device=dev) for s in range(nsets)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    warm_up(lambda k: binding.mla_stream_read(bufs[k % nsets], sink), 4 * nsets)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(calls):
        binding.mla_stream_read(bufs[k % nsets], sink)
    e1.record(stream)
    torch.cuda.synchronize()
    avg = e0.elapsed_time(e1) / calls
    spin = getattr(torch.cuda, "_sleep", None)
    per = []
    for k in range(calls):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if spin is not None:
            spin(20000)
        a.record(stream)
        binding.mla_stream_read(bufs[k % nsets], sink)
        b.record(stream)
        b.synchronize()
        per.append(a.elapsed_time(b))
    per.sort()
    nbytes = mib << 20
    gbs = lambda ms: round(nbytes / (ms * 1e-3) / 1e9, 1)
    del bufs
    torch.cuda.empty_cache()
    return {"kernel": "stream_read_kernel", "bytes_per_call": nbytes, "buffers_rotated": nsets,
            "avg_launch_ms": round(avg, 6), "GB/s": gbs(avg), "frac_of_peak": round(gbs(avg) / HBM_PEAK_GBS, 4),
            "single_call_ms_p10_p50_p90": [round(per[int(f * (calls - 1) + 0.5)], 6) for f in (0.1, 0.5, 0.9)],
            "small_reads": time_small_reads()}


def time_small_reads(sizes_mib=(16, 32), rotate_mib: int = 384):
    """The floor for a kernel that pulls one weight matrix from HBM: plain streaming reads
    (mla_stream_read) of 16 and 32 MiB, captured back to back in one graph and replayed, over
    enough buffers (`rotate_mib` in all) that none is still in the 256 MB Infinity Cache when it
    is read again ("cold"), and of one buffer read again and again ("warm": served by the caches).
    16 MiB is the size of W_k or W_v at 64 heads; the absorption reads W_k, the fused merge and
    up-projection W_v and as much again of split partials at decode."""
    import torch
    from mla_latent_cache_absorb_amd import binding

    dev = torch.device("cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    out = []
    for mib in sizes_mib:
        nsets = max(2, -(-rotate_mib // mib))
        bufs = [torch.full((mib << 20,), s + 1, dtype=torch.uint8, device=dev) for s in range(nsets)]
        res = {"MiB": mib}
        for kind, n, pick in (("cold", nsets, lambda k: bufs[k % nsets]), ("warm", 40, lambda k: bufs[0])):
            g = torch.cuda.CUDAGraph()
            binding.mla_stream_read(pick(0), sink)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                for k in range(n):
                    binding.mla_stream_read(pick(k), sink)
            warm_up(lambda k: g.replay(), 2)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 5
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / (reps * n) * 1e3
            res[f"{kind}_us"] = round(us, 3)
            res[f"{kind}_GB/s"] = round((mib << 20) / (us * 1e-6) / 1e9, 1)
            del g
        out.append(res)
        del bufs
        torch.cuda.empty_cache()
    return out


def time_indexer(name: str, steps: int, warmup: int):
    """The k-pooled indexer on the sequences of `name`: pooled keys (a full build, and a decode
    step's build of each sequence's newest pool), pool scores for all queries, top-k selection
    into position lists; per-kernel times from HIP events on the launch stream."""
    import numpy as np
    import torch
    from mla_latent_cache_absorb_amd import binding, workloads as wl

    dev = torch.device("cuda:0")
    spec = wl.WORKLOADS[name]
    lens = wl.cache_lengths(spec)
    ix = wl.make_indexer_inputs(spec, lens)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, g = bf(ix.q), bf(ix.k), bf(ix.g)
    cl = torch.from_numpy(lens).to(dev)
    Lmax = int(spec.cache_len)
    B, Q, d = ix.q.shape
    max_pools = Lmax // ix.pool
    pooled = torch.empty((B, max_pools, d), dtype=torch.float32, device=dev)
    scores = torch.empty((B, Q, max_pools), dtype=torch.float32, device=dev)
    idx = torch.empty((B, Q, ix.topk + ix.pool - 1), dtype=torch.int32, device=dev)
    idx_len = torch.empty((B, Q), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    # a decode step only pools what its new positions complete: the last pool of each sequence
    last_pool = torch.from_numpy(np.maximum(lens // ix.pool - 1, 0).astype(np.int32)).to(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        binding.mla_kpool_keys(k, g, cl, Lmax, ix.pool, pooled=pooled)
        if ev is not None:
            ev[1].record(stream)
        binding.mla_kpool_keys(k, g, cl, Lmax, ix.pool, pooled=pooled, pool_begin=last_pool)
        if ev is not None:
            ev[2].record(stream)
        binding.mla_indexer_scores(q, pooled, cl, Lmax, ix.pool, scores=scores)
        if ev is not None:
            ev[3].record(stream)
        binding.mla_indexer_select(scores, cl, Lmax, ix.pool, ix.topk, True, idx=idx, idx_len=idx_len)
        if ev is not None:
            ev[4].record(stream)

    warm_up(lambda k: step(), warmup)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for s in range(steps):
        step(evs[s])
    torch.cuda.synchronize()
    stage = {kname: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps
             for j, kname in enumerate(("kpool_keys_full", "kpool_keys_step", "scores", "select"))}
    npools = (lens // ix.pool).astype(np.int64)
    # algorithmic bytes of the score kernel: every pooled key read once per sequence, one score
    # written per (query, pool)
    score_bytes = int(npools.sum()) * d * 4 + int(npools.sum()) * Q * 4
    # the full pooled-key build: keys and gate logits of every complete pool read, keys written
    kpool_bytes = int(npools.sum()) * (2 * ix.pool * d * 2 + d * 4)
    achieved = score_bytes / (stage["scores"] * 1e-3) / 1e9
    return {
        "workload": name, "pool": ix.pool, "topk": ix.topk, "dim": d, "queries": B * Q,
        "stages_ms": {kname: round(v, 6) for kname, v in stage.items()},
        # one decode step: pool the newly completed pools, score, select (the full build is a
        # prefill-time cost, reported on its own)
        "ms_per_step": round(stage["kpool_keys_step"] + stage["scores"] + stage["select"], 6),
        "kpool_full_roofline": {"kernel": "kpool_kernel", "bound": "hbm",
                                "achieved": round(kpool_bytes / (stage["kpool_keys_full"] * 1e-3) / 1e9, 2),
                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(kpool_bytes / (stage["kpool_keys_full"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                "algorithmic_bytes_per_launch": kpool_bytes},
        "roofline": {"kernel": "score_kernel", "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_launch": score_bytes, "avg_launch_ms": round(stage["scores"], 6)},
    }


def time_append(steps: int, warmup: int):
    """The latent down-projection with cache append at three pass shapes: the decode batch
    (32 sequences x 1 token), the verification batch (16 x 6) and a 4096-token prefill chunk of
    one sequence.  Per-call time from HIP events around a graph replay of `steps` calls.  The two small passes are
    bound by reading the projection (4 MiB) and the hidden states; the chunk by the matrix cores
    (2 * 4096 * 512 flops per token)."""
    import numpy as np
    import torch
    from mla_latent_cache_absorb_amd import binding, workloads as wl

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    out = {}
    for label, wname, rows in (("decode_b32_q1", "decode_b32_l8192", None),
                               ("verify_b16_q6", "verify_b16_q6_l32768", None),
                               ("prefill_chunk_4096", "decode_b32_l8192", 4096)):
        spec = wl.WORKLOADS[wname]
        inp = wl.make_append_inputs(spec, rows=rows)
        B, Q, hidden = inp.h.shape if rows is None else (1, rows, wl.HIDDEN)
        h = bf(inp.h.reshape(B, Q, hidden))
        w = bf(inp.w_dkv)
        L = 8192 if rows is None else rows
        cache = torch.zeros((B, L, wl.LATENT), dtype=torch.bfloat16, device=dev)
        cl = torch.full((B,), L, dtype=torch.int32, device=dev)
        warm_up(lambda k: binding.mla_latent_append(h, w, cache, cl, L), warmup)
        # a call takes a few microseconds on the GPU, less than the Python call that launches it:
        # the timed calls are captured in a HIP graph and replayed, so the events see GPU time
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(steps):
                binding.mla_latent_append(h, w, cache, cl, L)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        del graph
        n = B * Q
        nbytes = wl.LATENT * hidden * 2 + n * hidden * 2 + n * wl.LATENT * 2
        flops = 2 * n * hidden * wl.LATENT
        entry = {"tokens": n, "ms": round(ms, 6)}
        if rows is None:
            ach = nbytes / (ms * 1e-3) / 1e9
            entry["roofline"] = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(ach / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": nbytes}
        else:
            ach = flops / (ms * 1e-3) / 1e12
            entry["roofline"] = {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4), "flops_per_launch": flops}
        out[label] = entry
        del cache
    return out


CROSSOVER_SHAPES = (("decode", 1, 4096), ("decode", 1, 32768), ("prefill", 1024, 1024), ("prefill", 4096, 4096),
                    ("prefill", 8192, 8192))


def time_crossover(reps: int = 3):
    """Module 05 section 5's comparison: the absorbed path (absorb_q, latent attention, up_v) and
    the naive path (expand every cached key and value, then multi-head attention) on one sequence,
    decode-shaped (one query against a cache of L) and prefill-shaped (L queries, each over its
    own prefix).  Each form is captured in a HIP graph of `reps` calls and replayed; per-call time
    from HIP events.  Inputs: torch.randn on the GPU with the workloads' distributions (timing
    only)."""
    import torch
    from mla_latent_cache_absorb_amd import binding, workloads as wl

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0x5C)
    H, D, R = wl.HEADS, wl.HEAD_DIM, wl.LATENT
    bf = lambda *shape, std=1.0: (torch.randn(*shape, generator=gen, device=dev) * std).to(torch.bfloat16)
    w_k, w_v = bf(H, D, R, std=wl.W_STD), bf(H, D, R, std=wl.W_STD)
    rows = []
    for kind, Q, L in CROSSOVER_SHAPES:
        q, cache = bf(1, Q, H, D), bf(1, L, R)
        cl = torch.full((1,), L, dtype=torch.int32, device=dev)
        visible = Q * (L - Q) + Q * (Q + 1) // 2        # sum over queries of the positions each sees
        forms = {
            "absorbed": lambda: binding.mla_forward(q, w_k, w_v, cache, cl, L, wl.SCALE),
            "naive": lambda: binding.mla_naive_forward(q, w_k, w_v, cache, cl, L, wl.SCALE),
        }
        entry = {"shape": kind, "queries": Q, "cache_len": L}
        for name, fn in forms.items():
            fn()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(reps):
                    fn()
            graph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            entry[name + "_ms"] = round(e0.elapsed_time(e1) / reps, 4)
            del graph
            torch.cuda.empty_cache()
        wbytes = 2 * H * D * R * 2                        # U^K and U^V, read once
        io = Q * H * D * 2 + Q * H * D * 4                # queries in, outputs out
        entry["absorbed_flops"] = 2 * 2 * Q * H * D * R + 4 * H * R * visible
        entry["naive_flops"] = 2 * 2 * L * H * D * R + 4 * H * D * visible
        entry["absorbed_bytes"] = L * R * 2 + wbytes + io
        # the expanded keys and values are written once and read back once
        entry["naive_bytes"] = L * R * 2 + wbytes + io + 2 * L * H * D * 2 * 2
        entry["winner"] = "absorbed" if entry["absorbed_ms"] <= entry["naive_ms"] else "naive"
        rows.append(entry)
        del q, cache
        torch.cuda.empty_cache()
    return rows


QLEN_SWEEP = (16, 32768, (1, 2, 3, 4, 5, 6, 7, 8))   # batch, cache length, query counts


def time_qlen_sweep(steps: int = 20, warmup: int = 20):
    """The latent attention (mla_latent_attn, split kernel + merge) at one to eight query
    positions per pass (draft depths 0..7) on 16 sequences of 32,768 positions.  Intensity is
    128 Q FLOP/B: HBM-bound at Q = 1 and 2, matrix-core-bound from Q = 3 on (the ridge is
    2.5e15 / 8e12 = 312 FLOP/B).  Each depth is timed over `steps` back-to-back calls (the
    median of five chunks, chunked_ms), two caches alternating.  Inputs: torch.randn on the GPU with the workloads'
    distributions (timing only)."""
    import torch
    from mla_latent_cache_absorb_amd import binding, workloads as wl

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0x51)
    B, L, qs = QLEN_SWEEP
    H, R = wl.HEADS, wl.LATENT
    caches = [(torch.randn(B, L, R, generator=gen, device=dev)).to(torch.bfloat16) for _ in range(2)]
    cl = torch.full((B,), L, dtype=torch.int32, device=dev)
    rows = []
    for Q in qs:
        # absorbed queries: q ~ N(0, 1) through U^K ~ N(0, 1/512) over 256 dims gives N(0, 1/2)
        q_abs = (torch.randn(B, Q, H, R, generator=gen, device=dev) * 0.5 ** 0.5).to(torch.bfloat16)
        o = torch.empty((B, Q, H, R), dtype=torch.float32, device=dev)
        lse = torch.empty((B, Q, H), dtype=torch.float32, device=dev)
        ws = torch.empty(max(binding.mla_latent_attn_workspace_size(B, Q, H, R, L, 0), 1), dtype=torch.uint8,
                         device=dev)
        call = lambda k: binding.mla_latent_attn(q_abs, caches[k & 1], cl, L, wl.SCALE, 0, o_lat=o, lse=lse,
                                                 workspace=ws)
        warm_up(call, warmup)
        ms, _ = chunked_ms(call, steps)
        visible = B * (Q * (L - Q) + Q * (Q + 1) // 2)
        flops = 4 * H * R * visible
        lat_bytes = B * L * R * 2
        tf = flops / (ms * 1e-3) / 1e12
        gbs = lat_bytes / (ms * 1e-3) / 1e9
        bound = "hbm" if 128 * Q < BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1000 else "mfma"
        rows.append({"q_len": Q, "ms": round(ms, 5), "splits": binding.mla_latent_attn_num_splits(B, Q, H, L, 0),
                     "TFLOP/s": round(tf, 2), "latent_GB/s": round(gbs, 2), "bound": bound,
                     "frac": round(gbs / HBM_PEAK_GBS if bound == "hbm" else tf / BF16_PEAK_TFLOPS, 4)})
        del q_abs, o, lse, ws
    del caches
    torch.cuda.empty_cache()
    return {"batch": B, "cache_len": L, "rows": rows}


def time_query_terms(name: str, terms=(1, 2), steps: int = 20, warmup: int = 20, gen=None):
    """The dense attention call (mla_latent_attn) at a full-size decode workload, with the absorbed
    query in one and/or two bf16 terms.  decode_b4_l131072_spiked: 4 sequences of 131,072
    positions with 1% of each sequence's latents scaled by 8 (the workload that needs the second
    term to meet the parity bar); decode_b32_l8192: the headline decode shape.  Inputs are drawn on
    the GPU with those shapes and structures (timing only; the parity tests use the seeded CPU
    workloads); the second term is a remainder below half a bf16 step of the first.  Two input
    sets alternate; each call is timed over `steps` back-to-back calls (the median of five chunks,
    chunked_ms)."""
    import torch
    from mla_latent_cache_absorb_amd import binding, workloads as wl

    dev = torch.device("cuda:0")
    if gen is None:
        gen = torch.Generator(device=dev)
        gen.manual_seed(0xC3)
    H, R = wl.HEADS, wl.LATENT
    B, Q, L, spiked = {"decode_b4_l131072_spiked": (4, 1, 131072, True),
                       "decode_b32_l8192": (32, 1, 8192, False)}[name]
    sets = []
    for _ in range(2):
        c = torch.randn(B, L, R, generator=gen, device=dev)
        if spiked:
            for b in range(B):
                pos = torch.randperm(L, generator=gen, device=dev)[: round(0.01 * L)]
                c[b, pos] *= 8.0
        qa = (torch.randn(B, Q, H, R, generator=gen, device=dev) * 0.5 ** 0.5).to(torch.bfloat16)
        q_lo = (qa.float() * torch.randn(qa.shape, generator=gen, device=dev) * 2.0 ** -10).to(torch.bfloat16)
        sets.append((c.to(torch.bfloat16), qa, q_lo))
        del c
    cl = torch.full((B,), L, dtype=torch.int32, device=dev)
    o = torch.empty((B, Q, H, R), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(binding.mla_latent_attn_workspace_size(B, Q, H, R, L, 0), 1), dtype=torch.uint8, device=dev)
    lat = B * L * R * 2
    out = []
    for nt in terms:
        def call(k):
            c, qa, q_lo = sets[k % 2]
            binding.mla_latent_attn(qa, c, cl, L, wl.SCALE, 0, o_lat=o, lse=lse, workspace=ws,
                                    q_abs_lo=q_lo if nt == 2 else None)
        warm_up(call, warmup)
        ms, ms_med = chunked_ms(call, steps)
        gbs = lat / (ms * 1e-3) / 1e9
        out.append({"workload": name, "call": "mla_latent_attn", "query_terms": nt, "ms": round(ms, 5),
                    "median_chunk_ms": round(ms_med, 5), "splits": binding.mla_latent_attn_num_splits(B, Q, H, L, 0),
                    "latent_bytes": lat, "GB/s": round(gbs, 2), "bound": "hbm", "frac": round(gbs / HBM_PEAK_GBS, 4)})
    del sets, o, lse, ws
    torch.cuda.empty_cache()
    return out


def time_other_configs(steps: int = 20, warmup: int = 20, two_term: bool = True):
    """The headline attention call on the two other full-size workloads: the spiked decode of 4
    sequences of 131,072 positions (time_query_terms: with one query term, and with two unless
    two_term is False), and mla_latent_attn_indexed on the indexed verification of 32 sequences
    (4 queries, lengths uniform in [4096, 65536]) over 2,048 positions drawn per query from the
    committed prefix plus the causal tail; then, with two_term, the headline decode shape with one
    and two query terms.  Inputs are drawn on the GPU with those shapes and structures (timing
    only; the parity tests use the seeded CPU workloads).  Two input sets alternate; each call is
    timed over `steps` back-to-back calls (the median of five chunks, chunked_ms)."""
    import torch
    from mla_latent_cache_absorb_amd import binding, workloads as wl

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0xC3)
    H, R = wl.HEADS, wl.LATENT

    def run(call, nsets):
        warm_up(lambda k: call(k % nsets), warmup)
        return chunked_ms(lambda k: call(k % nsets), steps)

    out = time_query_terms("decode_b4_l131072_spiked", (1, 2) if two_term else (1,), steps, warmup, gen)

    # indexed verification, 32 x 4, ragged
    B, Q, Lmax, n_index = 32, 4, 65536, 2048
    K = n_index + Q
    g_cpu = torch.Generator()
    g_cpu.manual_seed(0xC4)
    lens = torch.randint(4096, Lmax + 1, (B,), generator=g_cpu, dtype=torch.int32)
    idx = torch.full((B, Q, K), -1, dtype=torch.int32)
    idx_len = torch.empty((B, Q), dtype=torch.int32)
    for b in range(B):
        first_new = int(lens[b]) - Q
        for i in range(Q):
            drawn = torch.sort(torch.randperm(first_new, generator=g_cpu)[:n_index]).values
            row = torch.cat([drawn, torch.arange(first_new, first_new + i + 1)])
            idx[b, i, : row.numel()] = row.to(torch.int32)
            idx_len[b, i] = row.numel()
    idx, idx_len, cl = idx.to(dev), idx_len.to(dev), lens.to(dev)
    sets = [((torch.randn(B, Lmax, R, generator=gen, device=dev)).to(torch.bfloat16),
             (torch.randn(B, Q, H, R, generator=gen, device=dev) * 0.5 ** 0.5).to(torch.bfloat16)) for _ in range(2)]
    o = torch.empty((B, Q, H, R), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(binding.mla_latent_attn_workspace_size(B, Q, H, R, K, 0, indexed=True), 1),
                     dtype=torch.uint8, device=dev)
    ms, ms_med = run(lambda k: binding.mla_latent_attn_indexed(sets[k][1], sets[k][0], cl, idx, idx_len, Lmax,
                                                               wl.SCALE, 0, o_lat=o, lse=lse, workspace=ws), 2)
    rows = int(idx_len.sum())
    lat = rows * R * 2
    flops = 4 * H * R * rows
    gbs = lat / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    out.append({"workload": "indexed_verify_b32_q4_ragged", "call": "mla_latent_attn_indexed", "ms": round(ms, 5),
                "median_chunk_ms": round(ms_med, 5),
                "splits": binding.mla_latent_attn_num_splits(B, Q, H, K, 0, indexed=True), "latent_bytes": lat,
                "index_bytes": B * Q * K * 4, "GB/s": round(gbs, 2), "bound": "hbm",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "TFLOP/s": round(tf, 2),
                "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)})
    del sets, o, lse, ws, idx, idx_len
    torch.cuda.empty_cache()
    if two_term:
        out += time_query_terms("decode_b32_l8192", (1, 2), steps, warmup, gen)
    return out


def cpu_baseline(name: str, budget_s: float = 12.0):
    """The fp64 oracle (expanded form) on whole sequences of the same workload, until about
    budget_s of CPU time has been spent."""
    import numpy as np
    import oracle
    from mla_latent_cache_absorb_amd import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    w = wl.make_workload(name)
    B = w.q.shape[0]
    done, rows, t0 = 0, 0, time.perf_counter()
    while done < B and time.perf_counter() - t0 < budget_s:
        oracle.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, w.scale, idx=w.idx, idx_len=w.idx_len,
                             batches=[done])
        rows += int(w.cache_len[done]) if w.idx is None else int(w.idx_len[done].sum())
        done += 1
    dt = time.perf_counter() - t0
    gbs = rows * w.cache.shape[2] * 2 / dt / 1e9
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count()
    # cores = the BLAS threads the oracle ran on; the host's own core counts are stated beside it
    return {"value": round(gbs, 6), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "host_cpus": os.cpu_count(), "host_cpus_usable": affinity,
            "sample": f"{done} of {B} sequences of {name} (all {w.q.shape[2]} heads, expanded fp64), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the GPU reaches its steady clock only after some tens of milliseconds of work: 200 decode
    # steps (about 18 ms) come before the timed ones
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="decode_b32_l8192")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-indexer", action="store_true")
    ap.add_argument("--no-append", action="store_true")
    ap.add_argument("--no-crossover", action="store_true")
    ap.add_argument("--no-qlen-sweep", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true")
    ap.add_argument("--no-two-term", action="store_true",
                    help="other configs: leave out the two-term query timings (one kernel per workload per run)")
    ap.add_argument("--query-terms-only", metavar="WORKLOAD", default=None,
                    help="only the attention call at this decode workload with one and two query terms")
    ap.add_argument("--no-latency", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true")
    ap.add_argument("--read-ceiling-only", action="store_true",
                    help="time only the plain streaming read of 256 MiB (the device's read ceiling)")
    ap.add_argument("--latency-only", action="store_true",
                    help="time only the batch-1 decode latency (256 positions), for profiling it on its own")
    ap.add_argument("--other-configs-only", action="store_true",
                    help="time only the attention on the 131,072-position decode and the indexed verification")
    ap.add_argument("--qlen-sweep-only", action="store_true",
                    help="time only the latent attention at 1..8 query positions (for profiling it on its own)")
    ap.add_argument("--crossover-only", action="store_true",
                    help="time only the absorbed / naive comparison (for profiling it on its own)")
    ap.add_argument("--append-only", action="store_true",
                    help="time only the down-projection with cache append (for profiling it on its own)")
    ap.add_argument("--indexer-only", action="store_true",
                    help="time only the k-pooled indexer (for profiling it on its own)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device-to-device three times (a plain copy of known size, "
                         "so that hardware byte counters can be scaled)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from mla_latent_cache_absorb_amd import binding, build as libbuild
    if not os.path.exists(binding.LIB_PATH):
        libbuild.build()
    binding.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 18  # int32 elements
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.calibrate_copy} MiB three times")
        del src, dst
        torch.cuda.empty_cache()
    if args.read_ceiling_only:
        print(json.dumps({"read_ceiling": time_read_ceiling()}), flush=True)
        return
    if args.latency_only:
        print(json.dumps({"latency_b1": time_latency()}), flush=True)
        return
    if args.other_configs_only:
        print(json.dumps({"other_configs": time_other_configs(two_term=not args.no_two_term)}), flush=True)
        return
    if args.query_terms_only:
        print(json.dumps({"query_terms": time_query_terms(args.query_terms_only)}), flush=True)
        return
    if args.qlen_sweep_only:
        print(json.dumps({"qlen_sweep": time_qlen_sweep()}), flush=True)
        return
    if args.crossover_only:
        print(json.dumps({"crossover": time_crossover()}), flush=True)
        return
    if args.append_only:
        print(json.dumps({"append": time_append(args.steps, args.warmup)}), flush=True)
        return
    if args.indexer_only:
        print(json.dumps({"indexer": time_indexer("indexed_verify_b32_q4_ragged", args.steps, args.warmup)}),
              flush=True)
        return
    r = time_path(args.workload, args.steps, args.warmup, NSETS)
    w = r["workload"]
    B, Q, H, D = w.q.shape
    R = w.cache.shape[2]
    latent_bytes = visible_rows(w) * R * 2
    gbs = latent_bytes / (r["ms_step"] * 1e-3) / 1e9
    attn_ms = r["stage_ms"]["latent_attn"]
    achieved = latent_bytes / (attn_ms * 1e-3) / 1e9
    fused_ms = r["stage_ms"]["latent_attn_up_v"]
    fused_bytes = attn_up_v_bytes(w)
    fused_gbs = fused_bytes / (fused_ms * 1e-3) / 1e9
    traffic = read_traffic(args.workload)
    result = {
        "metric": "absorbed-MLA attn: latent-cache GB/s (q_len=1) + TFLOP/s (q_len=6) vs roofline",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "q_len": Q, "cache_len": int(w.cache.shape[1]),
                   "heads": H, "head_dim": D, "latent": R, "softmax_scale": w.scale, "splits": r["splits"],
                   "input_sets_rotated": NSETS, "weight_sets_rotated": r["weight_sets_rotated"],
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "mla_latent_attn (split kernel + merge)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic / (attn_ms * 1e-3) / 1e9, 2),
                     "algorithmic_bytes_per_launch": latent_bytes, "avg_launch_ms": round(attn_ms, 6),
                     "median_chunk_ms": round(r["stage_median_chunk_ms"]["latent_attn"], 6),
                     "launch_ms_p10_p50_p90": [round(x, 6) for x in r["stage_pct_ms"]["latent_attn"]]},
        "fused_attn_up_v": {"call": "mla_latent_attn_up_v (split kernel + merge fused into the up-projection)",
                            "avg_launch_ms": round(fused_ms, 6),
                            "median_chunk_ms": round(r["stage_median_chunk_ms"]["latent_attn_up_v"], 6),
                            "launch_ms_p10_p50_p90": [round(x, 6) for x in r["stage_pct_ms"]["latent_attn_up_v"]],
                            "algorithmic_bytes_per_launch": fused_bytes,
                            "achieved": round(fused_gbs, 2), "unit": "GB/s",
                            "frac": round(fused_gbs / HBM_PEAK_GBS, 4)},
        "stages_ms": {k: round(v, 6) for k, v in r["stage_ms"].items()},
        "tokens_per_s": round(B * Q / (r["ms_step"] * 1e-3), 1),
    }
    if not args.no_secondary:
        torch.cuda.empty_cache()
        # at least 100 untimed passes first (about 60 ms of verification work): the first calls of a
        # process run below the steady clock
        s = time_path("verify_b16_q6_l32768", max(10, args.steps // 5), max(100, args.warmup), 1)
        ws2 = s["workload"]
        flops = 4 * ws2.q.shape[2] * ws2.cache.shape[2] * attended_positions(ws2)
        t_attn = s["stage_ms"]["latent_attn"] * 1e-3
        tf = flops / t_attn / 1e12
        # the call the path runs: attention with the merge fused into the up-projection
        fused_flops = attn_up_v_flops(ws2)
        tf_fused = fused_flops / (s["stage_ms"]["latent_attn_up_v"] * 1e-3) / 1e12
        result["secondary"] = {
            "workload": "verify_b16_q6_l32768", "metric": "latent attention TFLOP/s (q_len=6)",
            "value": round(tf, 2), "unit": "TFLOP/s", "peak": BF16_PEAK_TFLOPS, "bound": "mfma",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4), "attn_flops": flops,
            "ms_per_step": round(s["ms_step"], 6), "stages_ms": {k: round(v, 6) for k, v in s["stage_ms"].items()},
            "splits": s["splits"],
            "launch_ms_p10_p50_p90": [round(x, 6) for x in s["stage_pct_ms"]["latent_attn"]],
            "fused_attn_up_v": {"value": round(tf_fused, 2), "unit": "TFLOP/s",
                                "frac": round(tf_fused / BF16_PEAK_TFLOPS, 4), "flops": fused_flops}}
    if not args.no_read_ceiling:
        log("[bench] timing the plain streaming read (read ceiling)")
        result["read_ceiling"] = time_read_ceiling()
        result["roofline"]["frac_of_read_ceiling"] = round(achieved / result["read_ceiling"]["GB/s"], 4)
    if not args.no_latency:
        log("[bench] timing the batch-1 decode latency")
        result["latency_b1"] = time_latency()
    if not args.no_indexer:
        torch.cuda.empty_cache()
        log("[bench] timing the k-pooled indexer")
        result["indexer"] = time_indexer("indexed_verify_b32_q4_ragged", max(5, args.steps // 5), 3)
    if not args.no_append:
        log("[bench] timing the down-projection with cache append")
        result["append"] = time_append(max(10, args.steps // 2), 3)
    if not args.no_crossover:
        log("[bench] timing the absorbed and naive forms at decode and prefill shapes")
        result["crossover"] = time_crossover()
    if not args.no_qlen_sweep:
        log("[bench] timing the latent attention at 1..8 query positions")
        result["qlen_sweep"] = time_qlen_sweep()
    if not args.no_other_configs:
        log("[bench] timing the attention on the long-context decode and the indexed verification")
        result["other_configs"] = time_other_configs()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
