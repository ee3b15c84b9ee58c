#!/usr/bin/env python3
"""Benchmark of the routed top-k sparse-attention hot path on one MI355X.

Default workload: sparse decode at 128K context, batch 8, 28 layers (32 query
heads, 4 KV heads, head dim 128, bf16 KV cache = 56 GiB resident in HBM),
int8 indexer (4 heads x 64) with top-2048 and one index per group of 4
layers (7 indexer calls per step).  One step = the whole hot path for one
new token per sequence: 7 x (indexer scores + top-k select) + 28 x sparse
attention, captured in a HIP graph and replayed.  value = tokens/s = B /
step time (median over the timed replays).  Inputs are seeded synthetic
tensors generated directly in HBM.  The same line carries the metric's second
half, ``prefill_indexer``: the causal index of one 64K-token group (int8 TOP/s
against the int8 MFMA peak).

Prints one JSON line.  Other workloads (``--config``) are for exploration:
``decode_32k``, ``decode_1m``, ``gsa_128k`` and ``prefill_64k`` (indexer int8
TOPS of the causal scorer).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, vendor figure
INT8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, vendor figure
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, vendor figure
ADDR_PEAK_GBS = 256 * 64 * 2.4  # vector-memory address rate: 256 CUs x 64 B/clk x 2.4 GHz (GB/s)
MIB = 1 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------ byte model ----

def decode_step_bytes(cfg) -> dict:
    """Algorithmic bytes of one decode step.

    Indexer keys are read once per group (B x L x HD bytes); each layer reads
    the selected K and V rows (B x Lq x k x Hkv x D x 2 bytes x 2).  With one
    KV cache for all layers the layers of a group gather the very same rows
    (one index, one cache), so those bytes count once per group.  Queries,
    index sets, outputs and scratch are not counted.
    """
    idx_per_call = cfg.B * cfg.L * cfg.HD
    kv_per_layer = cfg.B * cfg.Lq * min(cfg.topk, cfg.L) * cfg.Hkv * cfg.D * 2 * 2
    kv_reads = cfg.n_groups if getattr(cfg, "shared_kv", False) else cfg.n_layers
    total = cfg.n_groups * idx_per_call + kv_reads * kv_per_layer
    return {"indexer_per_call": idx_per_call, "kv_per_layer": kv_per_layer, "total": total}


def gsa_step_bytes(cfg) -> dict:
    """Routing keys (every gist key; with coarse-to-fine routing the meta-gist
    keys and the chosen groups' gist keys), then per (b, h): chosen chunks'
    raw K and V, gist V, tail K and V."""
    BH = cfg.B * cfg.H
    rows = (cfg.Nm + cfg.km * cfg.group) if cfg.group else cfg.Nc
    gk = BH * rows * cfg.D * 2
    sel = BH * cfg.kc * (cfg.chunk * 2 + 1) * cfg.D * 2 + BH * cfg.tail_len * 2 * cfg.D * 2
    return {"gist_keys": gk, "selected": sel, "total": gk + sel}


def causal_pairs(L: int) -> int:
    return L * (L + 1) // 2


# --------------------------------------------------------------- helpers ----

def _timed_loop(fn, iters, stream):
    """Average ms per call of ``fn``: events around back-to-back calls on ``stream``."""
    import torch
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(iters):
        fn()
    e.record(stream)
    e.synchronize()
    return s.elapsed_time(e) / iters  # ms


def _timed_each(fn, iters, stream):
    """Per-call ms of ``iters`` back-to-back calls of ``fn``: an event on
    ``stream`` between consecutive calls (no host wait in between), so each
    interval is one call as the stream runs it.  Returns (median, mean)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    ev[0].record(stream)
    for i in range(iters):
        fn()
        ev[i + 1].record(stream)
    ev[-1].synchronize()
    t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(iters))
    return t[len(t) // 2], ev[0].elapsed_time(ev[-1]) / iters


def _graph_of(fns, stream):
    """One HIP graph holding the calls ``fns`` in order (each already run once)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    g.replay()
    torch.cuda.synchronize()
    return g


def _timed_graph(fn, iters, stream):
    """Average ms per call of ``fn`` with ``iters`` calls captured in one HIP
    graph (no host launch overhead); events on the capturing stream."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = _graph_of([fn] * iters, stream)
    return _timed_loop(g.replay, 1, stream) / iters


def _rotating_ms(fns, reps, stream):
    """ms per call when ``fns`` (calls on different data, e.g. the 7 groups'
    indexer keys) run back to back in one graph, so that each call finds its
    data cold in the 256 MiB Infinity Cache, as inside a step.  Median over
    ``reps`` replays of the whole rotation."""
    import torch
    for f in fns:
        f()
    torch.cuda.synchronize()
    g = _graph_of(fns, stream)
    med, _ = _timed_each(g.replay, reps, stream)
    return med / len(fns)


def host_info():
    """CPU model and the number of threads this process may run on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return model, n


def _flush(buf):
    """Evict the 256 MiB Infinity Cache between small timed launches."""
    buf.add_(1)


def _timed_flushed(fn, iters, stream, flush_buf):
    """Median ms of ``iters`` calls of ``fn``, each timed alone with events on
    ``stream`` after a 1 GiB write has evicted the Infinity Cache (the flush
    is outside the timed interval)."""
    import torch
    t = []
    for _ in range(iters):
        _flush(flush_buf)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        t.append(e0.elapsed_time(e1))
    t.sort()
    return t[len(t) // 2]


SCORER_SOURCES = ["long_context_top_amd/csrc/idx_score.hip", "long_context_top_amd/csrc/common.h",
                  "long_context_top_amd/csrc/kernels.h"]
PROFILE_128K = os.path.join(ROOT, "profiles", "decode_128k_b8_kernels.txt")


def scorer_traffic():
    """HBM bytes per launch of the indexer scorer from the committed counter
    profile (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when the
    scorer's sources changed since the counters were taken."""
    import hashlib
    if not os.path.exists(PROFILE_128K):
        return None
    h = hashlib.sha256()
    for f in SCORER_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    vals, sha = {}, None
    for line in open(PROFILE_128K):
        parts = line.split()
        if len(parts) == 4 and parts[0] == "traffic" and parts[1] == "k_idx_score_stream":
            vals[parts[2]] = parts[3]
        if len(parts) == 3 and parts[0] == "source_sha256" and parts[1] == "k_idx_score_stream":
            sha = parts[2]
    if sha != h.hexdigest():
        return None
    try:
        return int(vals["fetch_bytes_per_launch"]) + int(vals["write_bytes_per_launch"])
    except KeyError:
        return None


def _decode_oracle_inputs(cfg, b=0):
    """Host copies of one sequence's inputs (generated once, outside any timing)."""
    import concurrent.futures as cf

    import numpy as np

    import synth
    from synth import configs as C

    with cf.ThreadPoolExecutor(8) as ex:
        qi = list(ex.map(lambda g: C.rows(cfg, cfg.qi_spec(g), (np.array([b]),)), range(cfg.n_groups)))
        ki = list(ex.map(lambda g: C.rows(cfg, cfg.ki_spec(g), (np.array([b]),)), range(cfg.n_groups)))
    q = [synth.as_float(synth.BF16N, C.rows(cfg, cfg.q_spec(l), (np.array(b), np.array(0))))
         for l in range(cfg.n_layers)]
    return qi, ki, q


def _decode_oracle_step(cfg, qi, ki, q, kv_cache, b=0):
    """One whole decode step of the oracle for one sequence: every group's
    indexer scores and top-k select, every layer's sparse attention.  The
    gathered K/V rows are generated on first use and kept (kv_cache)."""
    import numpy as np

    import oracle
    import synth
    from synth import configs as C

    idx_all = []
    for g in range(cfg.n_groups):
        s = oracle.index_scores(qi[g], ki[g], cfg.H_idx)
        idx_all.append(oracle.select_topk(s[0], cfg.topk, cfg.L))
    if not kv_cache:
        for l in range(cfg.n_layers):
            idx = idx_all[l // cfg.group]
            sel = idx[0][idx[0] >= 0].astype(np.int64)
            lead = (np.full_like(sel, b), sel)
            kv_cache.append((synth.as_float(synth.BF16N, C.rows(cfg, cfg.k_spec(l), lead)),
                             synth.as_float(synth.BF16N, C.rows(cfg, cfg.v_spec(l), lead))))
    for l in range(cfg.n_layers):
        oracle.sparse_attention_gqa(q[l], kv_cache[l][0], kv_cache[l][1], cfg.scale)


def cpu_baseline_decode(cfg, budget_s=6.0):
    """The oracle, as it stands (int64 scores, stable-sort top-k, float64
    attention), on whole decode steps of one sequence, timed on this host:
    once on one thread (steps in a row until budget_s), once on every
    thread this process may use (that many steps at a time in a thread pool,
    numpy releasing the interpreter lock inside its loops, until budget_s).
    tokens/s = steps / wall time.  Inputs are generated once, outside the
    timing (regenerating a sequence's 32 MiB of indexer keys per group costs
    the host more than the oracle itself)."""
    import concurrent.futures as cf

    from threadpoolctl import threadpool_limits

    model, nthreads = host_info()
    qi, ki, q = _decode_oracle_inputs(cfg)
    kv = []
    with threadpool_limits(limits=1):
        _decode_oracle_step(cfg, qi, ki, q, kv)        # gathers the K/V rows once (untimed)
        steps1, t0 = 0, time.perf_counter()
        while steps1 == 0 or time.perf_counter() - t0 < budget_s:
            _decode_oracle_step(cfg, qi, ki, q, kv)
            steps1 += 1
        t1 = time.perf_counter() - t0
        stepsn, t0 = 0, time.perf_counter()
        with cf.ThreadPoolExecutor(nthreads) as ex:
            while stepsn == 0 or time.perf_counter() - t0 < budget_s:
                list(ex.map(lambda _: _decode_oracle_step(cfg, qi, ki, q, kv), range(nthreads)))
                stepsn += nthreads
        tn = time.perf_counter() - t0
    return {"value": stepsn / tn, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "cpu_model": model, "one_thread": {"value": steps1 / t1, "unit": "tokens/s", "cores": 1},
            "sample": (f"sequence b=0, whole decode steps ({cfg.n_groups} groups: int64 indexer scores over "
                       f"{cfg.L} positions + stable-sort top-{cfg.topk}; {cfg.n_layers} layers of float64 sparse "
                       f"attention), one token each: {steps1} steps in {t1:.1f} s on 1 thread, {stepsn} steps "
                       f"in {tn:.1f} s on {nthreads} threads ({nthreads} steps at a time)")}


def cpu_baseline_prefill(cfg, n_rows=16, budget_rows=None):
    """The oracle (int64 scores of a query row against every key, stable-sort
    top-k with the causal valid length) on a sample of the 64K group's rows,
    spread over the sequence, on one thread and on every thread; its cost per
    row does not depend on the row (it scores all L keys), so the group's
    time is the sample's time x L / n_rows, and the figure is the group's
    int8 ops (the causal pairs') over that extrapolated time."""
    import concurrent.futures as cf

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from synth import configs as C

    model, nthreads = host_info()
    qi = C.rows(cfg, cfg.qi_spec(0), (np.array([0]),))          # [1, L, HD]
    ki = C.rows(cfg, cfg.ki_spec(0), (np.array([0]),))
    rows = (np.arange(n_rows) * (cfg.L // n_rows) + cfg.L // (2 * n_rows)).astype(np.int64)
    ops = 2 * cfg.HD * causal_pairs(cfg.L)

    def block(rs):
        s = oracle.index_scores(qi[:, rs], ki, cfg.H_idx)[0]
        return oracle.select_topk(s, cfg.topk, rs + 1)

    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for r in rows:
            block(np.array([r]))
        t1 = time.perf_counter() - t0
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(lambda r: block(np.array([r])), list(rows) * nthreads))
        tn = (time.perf_counter() - t0) / nthreads
    g1, gn = t1 * cfg.L / n_rows, tn * cfg.L / n_rows
    return {"value": ops / gn / 1e12, "unit": "int8 TOP/s (causal-pair ops of the group / extrapolated time)",
            "cores": nthreads, "kind": "oracle", "cpu_model": model,
            "one_thread": {"value": ops / g1 / 1e12, "cores": 1, "s_per_group_extrapolated": g1},
            "s_per_group_extrapolated": gn,
            "sample": (f"{n_rows} query rows spread over the {cfg.L} (one every {cfg.L // n_rows}), each scored "
                       f"against all {cfg.L} keys and selected: {t1:.1f} s on 1 thread, {tn * nthreads:.1f} s for "
                       f"{nthreads} x the sample on {nthreads} threads; extrapolated x{cfg.L // n_rows} to the group")}


# ---------------------------------------------------------------- decode ----

def bench_decode(cfg, steps, warmup, want_cpu):
    import torch

    import long_context_top_amd as lct
    import synth.device as sd

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t0 = time.time()
    ng = cfg.n_groups
    qi = [sd.make(cfg, cfg.qi_spec(g), dev) for g in range(ng)]
    ki = [sd.make(cfg, cfg.ki_spec(g), dev) for g in range(ng)]
    q = [sd.make(cfg, cfg.q_spec(l), dev) for l in range(cfg.n_layers)]
    # one cache tensor per distinct KV layer (all layers share layer 0's with shared_kv)
    kv = {}
    for l in range(cfg.n_layers):
        j = cfg.kv_layer(l)
        if j not in kv:
            kv[j] = (sd.make(cfg, cfg.k_spec(l), dev), sd.make(cfg, cfg.v_spec(l), dev))
    k = [kv[cfg.kv_layer(l)][0] for l in range(cfg.n_layers)]
    v = [kv[cfg.kv_layer(l)][1] for l in range(cfg.n_layers)]
    out = [torch.empty((cfg.B, cfg.Lq, cfg.Hq, cfg.D), dtype=torch.float32, device=dev)
           for _ in range(cfg.n_layers)]
    idx_out = [torch.empty((cfg.B, cfg.Lq, cfg.topk), dtype=torch.int32, device=dev) for _ in range(ng)]
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated)")
    run = lct.GroupRun(qi, ki, q, k, v, out, cfg.topk, cfg.group, cfg.scale, idx_out=idx_out)
    stream = torch.cuda.current_stream()
    run()
    torch.cuda.synchronize()

    # one step as a HIP graph (84 kernels for 28 layers / 7 groups)
    g = _graph_of([run], stream)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    log(f"warmup done ({warmup} steps)")
    ms, ms_mean = _timed_each(g.replay, steps, stream)
    torch.cuda.synchronize()

    # the dominant kernels as they run inside a step: rotations over the 7
    # groups' indexer keys (1.75 GiB) and the 28 layers' KV caches, so that every
    # launch reads cold data as in the step (not the warm 256 MiB Infinity Cache)
    bytes_ = decode_step_bytes(cfg)
    scores = torch.empty((cfg.B, cfg.Lq, cfg.L), dtype=torch.int32, device=dev)
    rot = 7
    ms_score = _rotating_ms([lambda g=g_: lct.idx_score(qi[g % ng], ki[g % ng], out=scores)
                             for g_ in range(3 * rot)], max(5, steps // 10), stream)
    ws = lct.Workspace(dev)
    ms_attn = _rotating_ms([lambda l=l_: lct.sparse_attn_gather(q[l], k[l], v[l], idx_out[l // cfg.group],
                                                                cfg.scale, out=out[l], ws=ws)
                            for l_ in range(cfg.n_layers)], max(5, steps // 10), stream)
    torch.cuda.synchronize()
    score_gbs = bytes_["indexer_per_call"] / (ms_score * 1e-3) / 1e9
    attn_gbs = bytes_["kv_per_layer"] / (ms_attn * 1e-3) / 1e9
    step_gbs = bytes_["total"] / (ms * 1e-3) / 1e9
    res = {
        "metric": "sparse-decode tokens/s + HBM GB/s at 128K ctx; prefill indexer int8 TOPS",
        "value": cfg.B * cfg.Lq / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": ms, "ms_per_step_mean": ms_mean,
        "timing": f"median of {steps} graph replays of one step, an event between consecutive replays",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64 inputs generated in HBM; random-init, no trained weights)",
        "config": {"workload": cfg.name, "global_batch": cfg.B, "seq_len": cfg.L,
                   "layers": cfg.n_layers, "layers_per_index": cfg.group, "q_heads": cfg.Hq,
                   "kv_heads": cfg.Hkv, "head_dim": cfg.D, "indexer": f"int8 {cfg.H_idx}x{cfg.d_idx}",
                   "topk": cfg.topk, "kv_cache": "one shared by all layers" if cfg.shared_kv else "per layer",
                   "parallelism": "single GPU"},
        "hbm_gbs_step": step_gbs, "hbm_frac_step": step_gbs / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": bytes_["total"],
        "roofline": {"bound": "hbm", "kernel": "k_idx_score_stream (indexer scores, one group)",
                     "achieved": score_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": score_gbs / HBM_PEAK_GBS, "traffic": scorer_traffic(),
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "us_per_launch": ms_score * 1e3, "bytes_per_launch": bytes_["indexer_per_call"],
                     "timing": "launches rotating over the 7 groups' keys (cold Infinity Cache), graph-replayed"},
        "attention_kernel": {"kernel": "k_sparse_attn + k_split_merge (one layer)", "achieved": attn_gbs,
                             "unit": "GB/s", "frac": attn_gbs / HBM_PEAK_GBS,
                             "us_per_launch": ms_attn * 1e3, "bytes_per_launch": bytes_["kv_per_layer"],
                             "timing": "launches rotating over the 28 layers' KV caches, graph-replayed"},
    }
    del g, scores, ws
    if want_cpu:
        log("timing the CPU oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline_decode(cfg)
    return res


# ------------------------------------------------------------------- GSA ----

def bench_gsa(cfg, steps, warmup, want_cpu=False):
    """One GSA decode step (gist scores, chunk select, unfold attention), or
    the coarse-to-fine H-GSA step, captured in a HIP graph; each replay timed
    alone after the Infinity Cache has been evicted (the step's gist keys are
    512 MiB, the selected rows 132 MiB: a warm cache would serve part of them)."""
    import torch

    import long_context_top_amd as lct
    import synth.device as sd

    dev = torch.device("cuda", 0)
    BH = cfg.B * cfg.H

    def mk(spec):
        t = sd.make(cfg, spec, dev)
        return t.view((BH,) + tuple(t.shape[2:]))

    qv, gk, gv, rk, rv = mk(cfg.q_spec()), mk(cfg.gk_spec()), mk(cfg.gv_spec()), mk(cfg.rk_spec()), mk(cfg.rv_spec())
    out = torch.empty((BH, cfg.D), dtype=torch.float32, device=dev)
    cidx = torch.empty((BH, cfg.kc), dtype=torch.int32, device=dev)
    ws = lct.Workspace(dev)
    if cfg.group:  # coarse-to-fine routing through the meta-gists
        mkeys = mk(cfg.mk_spec())
        step = lambda: lct.hgsa_decode(qv, mkeys, gk, gv, rk, rv, cfg.group, cfg.km, cfg.kc, cfg.tail_len,
                                       cfg.scale, idx_out=cidx, out=out, ws=ws)
    else:
        step = lambda: lct.gsa_decode(qv, gk, gv, rk, rv, cfg.kc, cfg.tail_len, cfg.scale, idx_out=cidx,
                                      out=out, ws=ws)
    step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    g = _graph_of([step], stream)
    for _ in range(warmup):
        g.replay()
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    ms = _timed_flushed(g.replay, steps, stream, flush)
    b = gsa_step_bytes(cfg)
    gbs = b["total"] / (ms * 1e-3) / 1e9
    res = {"workload": cfg.name, "ms_per_step": ms, "tokens_per_s": BH // cfg.H * 1.0 / (ms * 1e-3),
           "hbm_gbs_step": gbs, "hbm_frac_step": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_step": b["total"],
           "routing_key_bytes": b["gist_keys"],
           "timing": f"median of {steps} graph replays, each alone after a 1 GiB write evicted the Infinity Cache"}
    if not cfg.group:
        gs = torch.empty((BH, cfg.Nc), dtype=torch.float32, device=dev)
        lct.gist_score(qv, gk, out=gs)
        ms_gs = _timed_flushed(lambda: lct.gist_score(qv, gk, out=gs), max(5, steps // 2), stream, flush)
        res["roofline"] = {"bound": "hbm", "kernel": "k_gist_score (every gist key once)",
                           "achieved": b["gist_keys"] / (ms_gs * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": b["gist_keys"] / (ms_gs * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "us_per_launch": ms_gs * 1e3, "bytes_per_launch": b["gist_keys"]}
    del g, flush, qv, gk, gv, rk, rv, out, cidx, ws
    torch.cuda.empty_cache()
    if want_cpu:
        res["cpu_baseline"] = cpu_baseline_gsa(cfg)
    return res


def cpu_baseline_gsa(cfg, n_pairs=16):
    """The oracle's GSA (or H-GSA) decode on a sample of (batch, head) pairs,
    on one thread and on every thread; every pair costs the oracle the same
    (it regenerates and scores the pair's gist keys, then unfolds its chunks),
    so the step's time is the sample's x (B x H) / n_pairs."""
    import concurrent.futures as cf

    from threadpoolctl import threadpool_limits

    import oracle

    model, nthreads = host_info()
    step = oracle.driver.hgsa_step if cfg.group else oracle.driver.gsa_step
    pairs = [(b, h) for b in range(cfg.B) for h in range(cfg.H)][:: (cfg.B * cfg.H) // n_pairs][:n_pairs]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        step(cfg, pairs)
        t1 = time.perf_counter() - t0
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(lambda p: step(cfg, [p]), pairs * max(1, nthreads // 4)))
        tn = (time.perf_counter() - t0) / max(1, nthreads // 4)
    scale = cfg.B * cfg.H / len(pairs)
    return {"value": cfg.B / (tn * scale), "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "cpu_model": model, "one_thread": {"value": cfg.B / (t1 * scale), "unit": "tokens/s", "cores": 1},
            "sample": (f"{len(pairs)} (batch, head) pairs of the {cfg.B * cfg.H}: {t1:.1f} s on 1 thread; "
                       f"{max(1, nthreads // 4)} x the sample on {nthreads} threads in {tn * max(1, nthreads // 4):.1f} s; "
                       f"a step is {cfg.B * cfg.H} pairs (extrapolated x{scale:.0f})")}


# ----------------------------------------------------------- GSA prefill ----

def gsa_prefill_pairs(cfg) -> int:
    """Visible (query, key) pairs under the gist mask for one (batch, head):
    raw token i of chunk c sees c gists and i + 1 raw tokens, gist c sees
    c + 1 gists and the chunk's raw tokens."""
    nc, ch = cfg.Nc, cfg.chunk
    raw = ch * nc * (nc - 1) // 2 + nc * ch * (ch + 1) // 2
    gist = nc * (nc + 1) // 2 + nc * ch
    return raw + gist


def cpu_baseline_gsa_prefill(cfg, n_raw=512, n_gist=128):
    """The oracle's GSA prefill on sampled rows of one (batch, head): raw and
    gist queries spread over the sequence, each attending over its visible
    keys (oracle.gsa_prefill_rows).  The oracle's cost per query grows with
    its visible keys, so the whole prefill's time is the sample's scaled by
    (visible pairs of all rows and heads) / (visible pairs of the sample)."""
    import concurrent.futures as cf

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import synth
    from synth import configs as C

    model, nthreads = host_info()
    n_rows = cfg.Nc * cfg.chunk
    raw_rows = [int(x) for x in np.linspace(0, n_rows - 1, n_raw)]
    gist_rows = [int(x) for x in np.linspace(0, cfg.Nc - 1, n_gist)]
    idx = (np.array(0), np.array(0))
    args = [synth.as_float(spec[0], C.rows(cfg, spec, idx)) for spec in
            (cfg.qr_spec(), cfg.qg_spec(), cfg.rk_spec(), cfg.rv_spec(), cfg.gk_spec(), cfg.gv_spec())]
    args[2], args[3] = args[2][:n_rows], args[3][:n_rows]
    ch = cfg.chunk
    pairs = sum((t // ch) + (t % ch) + 1 for t in raw_rows) + sum(c + 1 + ch for c in gist_rows)
    run = lambda rr, gr: oracle.gsa_prefill_rows(*args, ch, cfg.scale, raw_rows=rr, gist_rows=gr)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        run(raw_rows, gist_rows)
        t1 = time.perf_counter() - t0
        reps = max(1, nthreads // 4)
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(lambda i: run(raw_rows[i::nthreads], gist_rows[i::nthreads]), list(range(nthreads)) * reps))
        tn = (time.perf_counter() - t0) / reps
    scale = gsa_prefill_pairs(cfg) * cfg.B * cfg.H / pairs
    tokens = cfg.B * cfg.Nc * (cfg.chunk + 1)
    return {"value": tokens / (tn * scale), "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "cpu_model": model, "one_thread": {"value": tokens / (t1 * scale), "unit": "tokens/s", "cores": 1},
            "sample": (f"{n_raw} raw and {n_gist} gist queries of one (batch, head) spread over the sequence, "
                       f"each over its visible keys: {t1:.1f} s on 1 thread; {reps} x the sample on {nthreads} "
                       f"threads in {tn * reps:.1f} s; extrapolated by visible pairs (x{scale:.0f})")}


def bench_gsa_prefill(cfg, steps, warmup, want_cpu=False):
    """Every raw and gist token of the sequence attends under the gist mask
    (lct_gsa_prefill).  Throughput: bf16 flops of the visible pairs (QK and
    PV: 4 per pair and feature) against the dense bf16 MFMA peak."""
    import torch

    import long_context_top_amd as lct
    import synth.device as sd

    dev = torch.device("cuda", 0)
    BH = cfg.B * cfg.H

    def mk(spec):
        t = sd.make(cfg, spec, dev)
        return t.view((BH,) + tuple(t.shape[2:]))

    qr, qg, rk, rv, gk, gv = (mk(cfg.qr_spec()), mk(cfg.qg_spec()), mk(cfg.rk_spec()), mk(cfg.rv_spec()),
                              mk(cfg.gk_spec()), mk(cfg.gv_spec()))
    out_r = torch.empty((BH, cfg.Nc * cfg.chunk, cfg.D), dtype=torch.float32, device=dev)
    out_g = torch.empty((BH, cfg.Nc, cfg.D), dtype=torch.float32, device=dev)
    f = lambda: lct.gsa_prefill(qr, qg, rk, rv, gk, gv, cfg.scale, out_raw=out_r, out_gist=out_g)
    for _ in range(max(warmup, 1)):
        f()
    torch.cuda.synchronize()
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    ms = _timed_flushed(f, steps, torch.cuda.current_stream(), flush)
    del flush
    flops = 4.0 * cfg.D * gsa_prefill_pairs(cfg) * BH
    tf = flops / (ms * 1e-3) / 1e12
    tokens = cfg.B * cfg.Nc * (cfg.chunk + 1)
    res = {"workload": cfg.name, "ms_per_prefill": ms, "tokens_per_s": tokens / (ms * 1e-3),
           "roofline": {"bound": "mfma", "kernel": "k_gsa_prefill (raw and gist queries)", "achieved": tf,
                        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tf / BF16_PEAK_TFLOPS,
                        "flops_per_launch": flops, "us_per_launch": ms * 1e3}}
    if want_cpu:
        del qr, qg, rk, rv, gk, gv, out_r, out_g
        torch.cuda.empty_cache()
        log("timing the CPU oracle on sampled GSA prefill rows ...")
        res["cpu_baseline"] = cpu_baseline_gsa_prefill(cfg)
    return res


# --------------------------------------------------------------- prefill ----

def bench_prefill_indexer(cfg, steps, warmup, want_cpu=False, attention=True):
    """Causal index of one group at full length: int8 MFMA scores of every
    earlier position, filtered on the fly, exact top-k per row
    (lct_prefill_index_i8).  Throughput over the causal pairs' int8 ops."""
    import torch

    import long_context_top_amd as lct
    import synth.device as sd

    dev = torch.device("cuda", 0)
    qi = sd.make(cfg, cfg.qi_spec(0), dev)[0]
    ki = sd.make(cfg, cfg.ki_spec(0), dev)[0]
    out = torch.empty((cfg.L, cfg.topk), dtype=torch.int32, device=dev)
    ws = lct.Workspace(dev)
    stats = {}
    lct.prefill_index(qi, ki, cfg.topk, out=out, ws=ws, stats=stats)      # rows on the whole-row path
    torch.cuda.synchronize()
    f = lambda: lct.prefill_index(qi, ki, cfg.topk, out=out, ws=ws)
    stream = torch.cuda.current_stream()
    g = _graph_of([f], stream)
    for _ in range(max(warmup, 1)):
        g.replay()
    torch.cuda.synchronize()
    ms, ms_mean = _timed_each(g.replay, steps, stream)
    pairs = causal_pairs(cfg.L)
    ops = 2 * cfg.HD * pairs
    tops = ops / (ms * 1e-3) / 1e12
    res = {"workload": cfg.name + " indexer (one group, fused score filter + exact top-k)",
           "ms_per_group": ms, "ms_per_group_mean": ms_mean, "int8_tops": tops,
           "rows_on_plain_path": stats.get("n_fallback"),
           "timing": f"median of {steps} graph replays of one call, an event between consecutive replays",
           "roofline": {"bound": "mfma", "kernel": "k_pf_filter + k_pf_select (+ short-row block)",
                        "achieved": tops, "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                        "frac": tops / INT8_PEAK_TOPS, "ops_per_launch": ops,
                        "us_per_launch": ms * 1e3}}
    del g
    if attention:
        attn = bench_prefill_attention(cfg, out, max(5, steps), warmup)
        res["attention"] = attn
    del qi, ki, out, ws
    torch.cuda.empty_cache()
    if attention:
        # the whole prefill of the 28-layer stack: one layer group through the
        # driver (its index, then its layers' attention), times the groups
        grp = bench_prefill_group(cfg, max(3, steps // 5), 1)
        step_ms = cfg.n_groups * grp["ms_per_group"]
        res.update({"group_run": grp, "prefill_ms_all_layers": step_ms,
                    "prefill_tokens_per_s": cfg.L / (step_ms * 1e-3)})
    if want_cpu:
        log("timing the CPU oracle on sampled prefill rows ...")
        res["cpu_baseline"] = cpu_baseline_prefill(cfg)
    return res


def bench_prefill_group(cfg, steps, warmup):
    """One layer group of the causal prefill through the layer-group driver
    (lct_group_run, causal): the group's index, then each of its layers'
    sparse attention over that index (the Shared layers reuse the segment
    bounds and block-union lists the first layer derived from it)."""
    import torch

    import long_context_top_amd as lct
    import synth.device as sd

    dev = torch.device("cuda", 0)
    n = cfg.group
    qi = [sd.make(cfg, cfg.qi_spec(0), dev)]
    ki = [sd.make(cfg, cfg.ki_spec(0), dev)]
    q = [sd.make(cfg, cfg.q_spec(l), dev) for l in range(n)]
    k = [sd.make(cfg, cfg.k_spec(l), dev) for l in range(n)]
    v = [sd.make(cfg, cfg.v_spec(l), dev) for l in range(n)]
    out = [torch.empty((1, cfg.L, cfg.Hq, cfg.D), dtype=torch.float32, device=dev) for _ in range(n)]
    run = lct.GroupRun(qi, ki, q, k, v, out, cfg.topk, cfg.group, cfg.scale, causal=True)
    for _ in range(max(warmup, 1)):
        run()
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sorted(times)[len(times) // 2]
    del run, qi, ki, q, k, v, out
    torch.cuda.empty_cache()
    return {"ms_per_group": ms, "layers": n,
            "timing": f"median of {steps} lct_group_run calls (causal: the index, then {n} layers)"}


def bench_prefill_attention(cfg, idx, steps, warmup):
    """Sparse attention of one layer over the causal index sets (every row
    its own top-k positions): the position-segment path of
    lct_sparse_attn_gather.  Throughput over the selected pairs' bf16 flops
    (QK and PV, 4 flops per pair, query head and feature)."""
    import torch

    import long_context_top_amd as lct
    import synth.device as sd

    dev = idx.device
    q = sd.make(cfg, cfg.q_spec(0), dev)
    k = sd.make(cfg, cfg.k_spec(0), dev)
    v = sd.make(cfg, cfg.v_spec(0), dev)
    out = torch.empty((1, cfg.L, cfg.Hq, cfg.D), dtype=torch.float32, device=dev)
    ws = lct.Workspace(dev)
    ix = idx.view(1, cfg.L, cfg.topk)
    f = lambda: lct.sparse_attn_gather(q, k, v, ix, cfg.scale, out=out, ws=ws)
    for _ in range(max(warmup, 1)):
        f()
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        f()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sorted(times)[len(times) // 2]
    sel = sum(min(cfg.topk, r + 1) for r in range(cfg.L))
    flops = 4.0 * cfg.Hq * cfg.D * sel
    gathered = sel * cfg.Hkv * cfg.D * 2 * 2
    # the same layer when neighbouring queries share their sets: every row of
    # a 16-row block reuses the set its first row selected (valid for every
    # row of the block: those positions precede the block)
    ix_sh = ix[:, ::16].repeat_interleave(16, dim=1)[:, : cfg.L].contiguous()
    f2 = lambda: lct.sparse_attn_gather(q, k, v, ix_sh, cfg.scale, out=out, ws=ws)
    f2()
    torch.cuda.synchronize()
    t2 = []
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        f2()
        e1.record()
        torch.cuda.synchronize()
        t2.append(e0.elapsed_time(e1))
    ms2 = sorted(t2)[len(t2) // 2]
    sel2 = int((ix_sh >= 0).sum().item())
    del q, k, v, out, ws, ix_sh
    return {"kernel": "k_seg_bounds + k_union_plan + k_union_attn + k_sparse_attn_seg + k_seg_merge",
            "ms_per_layer": ms,
            "shared_sets_ms_per_layer": ms2,
            "shared_sets_bf16_tflops": 4.0 * cfg.Hq * cfg.D * sel2 / (ms2 * 1e-3) / 1e12,
            "shared_sets_note": "every row of a 16-row block attends over its first row's set: the block-union path",
            "bf16_tflops": flops / (ms * 1e-3) / 1e12, "frac_of_bf16_peak": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "gathered_gb_per_s": gathered / (ms * 1e-3) / 1e9,
            # the vector address unit takes 64 bytes (a quad of 16-byte lanes) per
            # cycle per CU: 256 CUs x 64 B x 2.4 GHz
            "address_rate_peak_gb_per_s": ADDR_PEAK_GBS,
            "frac_of_address_rate": gathered / (ms * 1e-3) / 1e9 / ADDR_PEAK_GBS,
            "note": "selected K/V rows are re-read by many rows: the gathers run from L2/MALL, "
                    "bounded by the per-CU address rate (64 B/clk), not HBM"}


def copy_calibration(steps):
    """A plain device copy of known size (1 GiB read + 1 GiB written per launch),
    used to scale the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"mode": "copy_calibration", "bytes_read_per_launch": src.numel() * 4,
            "bytes_written_per_launch": dst.numel() * 4, "launches": steps}


def summarize_profile(stats_csv, pmc_csvs, calib_csvs, trace_csv=None):
    """Text summary of rocprofv3 output: per-kernel average duration, and the
    average counter value per dispatch for each kernel, scaled by the copy
    calibration (counter units per byte of a known plain copy)."""
    import csv
    lines = []
    rows = list(csv.DictReader(open(stats_csv)))
    lines.append(f"{'kernel':30s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'share':>7s}")
    for r in rows:
        lines.append(f"{r['Name'][:30]:30s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:9.2f} "
                     f"{float(r['MinNs'])/1e3:9.2f} {float(r['MaxNs'])/1e3:9.2f} {float(r['Percentage']):6.2f}%")

    def per_kernel(path):
        acc = {}
        for r in csv.DictReader(open(path)):
            key = (r["Kernel_Name"], r["Counter_Name"])
            acc.setdefault(key, {})
            d = r.get("Dispatch_Id") or r.get("Correlation_Id")
            acc[key][d] = acc[key].get(d, 0.0) + float(r["Counter_Value"])
        return {k: sum(v.values()) / len(v) for k, v in acc.items()}

    scale = {}
    for c in calib_csvs:
        for (kname, cname), val in per_kernel(c).items():
            if "elementwise" in kname or "copy" in kname.lower():
                want = 1 << 30  # bytes read (FETCH) or written (WRITE) per copy launch
                scale[cname] = want / (val * 1024.0)
    traffic = {}
    if pmc_csvs:
        lines.append("")
        lines.append("counters per dispatch (KiB as read) -> bytes after copy calibration")
        for c in pmc_csvs:
            for (kname, cname), val in sorted(per_kernel(c).items()):
                if kname.startswith("k_fill") or "elementwise" in kname:
                    continue
                sc = scale.get(cname, 1.0)
                lines.append(f"{kname[:30]:30s} {cname:12s} {val:14.1f} KiB  x{sc:.4f} = {val*1024*sc/2**20:10.2f} MiB")
                short = kname.split("(")[0].split("<")[0].replace("void ", "").replace("lct::", "")
                traffic[(short, cname)] = val * 1024 * sc
    if trace_csv:
        lines.append("")
        lines.extend(step_breakdown(trace_csv))
    if ("k_idx_score_stream", "FETCH_SIZE") in traffic and ("k_idx_score_stream", "WRITE_SIZE") in traffic:
        import hashlib
        h = hashlib.sha256()
        for f in SCORER_SOURCES:
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
        lines.append("")
        lines.append(f"traffic k_idx_score_stream fetch_bytes_per_launch {int(traffic[('k_idx_score_stream', 'FETCH_SIZE')])}")
        lines.append(f"traffic k_idx_score_stream write_bytes_per_launch {int(traffic[('k_idx_score_stream', 'WRITE_SIZE')])}")
        lines.append(f"source_sha256 k_idx_score_stream {h.hexdigest()}")
    return "\n".join(lines)


def step_breakdown(trace_csv, n_steps=5):
    """Per-kernel durations inside graph-replayed decode steps (the last
    n_steps complete steps of the trace): a step starts at a scorer launch
    that is followed by the select's first kernel."""
    import csv
    rows = list(csv.DictReader(open(trace_csv)))
    seq = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                  r["Kernel_Name"].split("(")[0].replace("void ", "").replace("lct::", "").split("<")[0])
                 for r in rows)
    names = [x[2] for x in seq]
    starts = [i for i in range(len(seq) - 1)
              if names[i] == "k_idx_score_stream" and names[i + 1] == "k_topk_hist"]
    if len(starts) < 2:
        return ["(no graph-replayed steps found in the trace)"]
    groups = 7
    per_step = groups
    sel = starts[-per_step * n_steps:]
    first, last = sel[0], sel[-1]
    end = last + 1
    while end < len(seq) and names[end] != "k_idx_score_stream":
        end += 1
    agg = {}
    for i in range(first, end):
        s0, e0, n = seq[i]
        agg.setdefault(n, []).append((e0 - s0) / 1e3)
    span = (seq[end - 1][1] - seq[first][0]) / 1e3
    out = [f"steady-state decode steps (last {n_steps} graph-replayed steps of the trace)",
           f"{'kernel':24s} {'launches/step':>13s} {'mean_us':>9s} {'us/step':>9s}"]
    total = 0.0
    for n, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        ps = sum(v) / n_steps
        total += ps
        out.append(f"{n:24s} {len(v) / n_steps:13.1f} {sum(v) / len(v):9.2f} {ps:9.1f}")
    out.append(f"{'sum of kernel time':24s} {'':13s} {'':9s} {total:9.1f}")
    out.append(f"{'step span (first start to last end)':38s} {span / n_steps:9.1f} us/step")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="decode_128k",
                    choices=["decode_128k", "decode_32k", "decode_1m", "gsa_128k", "prefill_64k", "tiny",
                             "decode_128k_shared_kv", "hgsa_128k", "gsa_prefill_128k"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="decode_128k: leave out the prefill indexer object of the default line")
    ap.add_argument("--no-gsa", action="store_true",
                    help="decode_128k: leave out the GSA / H-GSA / GSA-prefill objects of the default line")
    ap.add_argument("--mode", default="bench", choices=["bench", "copy"],
                    help="copy: a plain 1 GiB device copy used to calibrate HBM byte counters")
    ap.add_argument("--summarize", nargs="+", metavar="CSV",
                    help="print a summary of rocprofv3 CSVs: STATS [TRACE] [PMC ...] [--calib CSV ...]")
    args, rest = ap.parse_known_args()
    if args.summarize:
        files = args.summarize + rest
        calib = files[files.index("--calib") + 1:] if "--calib" in files else []
        main_files = files[:files.index("--calib")] if "--calib" in files else files
        trace = [f for f in main_files[1:] if f.endswith("kernel_trace.csv")]
        pmc = [f for f in main_files[1:] if not f.endswith("kernel_trace.csv")]
        print(summarize_profile(main_files[0], pmc, calib, trace[0] if trace else None))
        return
    if rest:
        ap.error(f"unknown arguments {rest}")
    if args.mode == "copy":
        print(json.dumps(copy_calibration(args.steps)))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(every workload runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    from synth import configs as C
    cfgs = {"decode_128k": C.DECODE_128K, "decode_32k": C.DECODE_32K, "decode_1m": C.DECODE_1M,
            "gsa_128k": C.GSA_128K, "prefill_64k": C.PREFILL_64K, "tiny": C.TINY,
            "decode_128k_shared_kv": C.DECODE_128K_SHARED_KV, "hgsa_128k": C.HGSA_128K,
            "gsa_prefill_128k": C.GSA_PREFILL_128K}
    cfg = cfgs[args.config]
    if args.config in ("gsa_128k", "hgsa_128k"):
        res = bench_gsa(cfg, args.steps, args.warmup, want_cpu=not args.no_cpu_baseline)
    elif args.config == "gsa_prefill_128k":
        res = bench_gsa_prefill(cfg, args.steps, args.warmup, want_cpu=not args.no_cpu_baseline)
    elif args.config == "prefill_64k":
        res = bench_prefill_indexer(cfg, args.steps, args.warmup, want_cpu=not args.no_cpu_baseline)
    else:
        headline = args.config == "decode_128k"
        res = bench_decode(cfg, args.steps, args.warmup, want_cpu=not args.no_cpu_baseline and headline)
        if headline and not args.no_prefill:
            # the metric's second half: the causal prefill indexer at 64K
            import gc

            import torch
            gc.collect()
            torch.cuda.empty_cache()
            log("prefill indexer, one 64K group ...")
            res["prefill_indexer"] = bench_prefill_indexer(C.PREFILL_64K, args.steps, args.warmup,
                                                           want_cpu=not args.no_cpu_baseline)
        if headline and not args.no_gsa:
            # the gist-chunk workloads beside it (the select-and-unfold decode, its
            # coarse-to-fine variant, the prefill under the gist mask)
            import gc

            import torch
            gc.collect()
            torch.cuda.empty_cache()
            log("GSA workloads ...")
            gsteps = max(10, args.steps)
            res["gsa_decode"] = bench_gsa(C.GSA_128K, gsteps, 2, want_cpu=not args.no_cpu_baseline)
            res["hgsa_decode"] = bench_gsa(C.HGSA_128K, gsteps, 2, want_cpu=not args.no_cpu_baseline)
            res["gsa_prefill"] = bench_gsa_prefill(C.GSA_PREFILL_128K, max(5, args.steps), 1,
                                                   want_cpu=not args.no_cpu_baseline)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
