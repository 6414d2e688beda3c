"""Decode-step throughput of the two-level sparse attention operator on one
MI355X, with the HBM roofline of its dominant kernel and the CPU oracle
timed beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gqa48k]

A step is one decode step of one attention layer over the whole batch:
append the new token, block scores over the full context, top-K_b, label
scores over the kept blocks, top-K_t, exact attention and the split merge.
Inputs are resident in HBM before timing starts. Steps rotate over several
copies of the cache (distinct addresses, as consecutive layers would be) so
the 256 MB Infinity Cache cannot serve a step from the previous one. Steps
are captured as HIP graphs of several consecutive steps each (as a model's
decode graph holds all its layers) and replayed; the rate with one graph
launch per step is reported beside it.

Prints one JSON line.
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

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from hierarchical_sparse_attention_block_amd import hsab as H  # noqa: E402
from hierarchical_sparse_attention_block_amd import workloads as W  # noqa: E402

METRIC = "sparse-attn decode queries/s (batch×heads) at 48k/96k ctx; % HBM roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
COUNTERS = os.path.join(ROOT, "profiles", "block_score_{wl}_counters.json")
# what the block-score kernel is built from: its sources and the build
# options (per-source compiler flags), so counters taken on another build
# are not reported
SCORE_SOURCES = ["hierarchical_sparse_attention_block_amd/csrc/score.hip",
                 "hierarchical_sparse_attention_block_amd/csrc/common.h",
                 "hierarchical_sparse_attention_block_amd/build.py"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dims_of(w):
    agg = H.AGG_HEAD if w.per_head else (H.AGG_SUM if w.agg_sum else H.AGG_MAX)
    return H.dims(w.batch, w.n_q_heads, w.n_kv_heads, w.d_k, w.d_v, w.v_alias_k, w.block, w.r,
                  w.k_blocks, w.k_tokens, w.max_ctx, w.sm_scale, H.META_FP8 if w.meta_fp8 else H.META_BF16,
                  agg, w.sink_blocks, w.local_blocks, H.LABEL_FP8 if w.label_fp8 else H.LABEL_BF16)


def meta_value_bytes(w):
    return 1 if w.meta_fp8 else 2


def step_bytes(w):
    """Algorithmic HBM bytes of one decode step (every unit at full context):
    block metadata, label rows of the kept blocks, gathered K/V rows of the
    kept tokens, queries and outputs."""
    U, nb = w.units, -(-w.ctx // w.block)
    meta = U * nb * 2 * w.d_k * meta_value_bytes(w)
    labels = U * min(w.k_blocks, nb) * w.block * w.r * 2
    kv_row = (w.d_k if w.v_alias_k else w.d_k + w.d_v) * 2
    gather = U * min(w.k_tokens, min(w.k_blocks, nb) * w.block) * kv_row
    qo = w.batch * w.n_q_heads * (w.d_k * 2 + w.d_v * 4)
    return {"meta": meta, "labels": labels, "gather": gather, "q_out": qo,
            "total": meta + labels + gather + qo}


def score_kernel_bytes(w):
    """Algorithmic bytes of one block-score launch: every metadata row read
    once, the queries read once, one fp32 score written per block."""
    U, nb = w.units, -(-w.ctx // w.block)
    return U * nb * (2 * w.d_k * meta_value_bytes(w) + 4) + w.batch * w.n_q_heads * w.d_k * 2


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Replica:
    def __init__(self, d, base, clone_from=None):
        src = clone_from or base
        self.K = src["K"].clone()
        self.V = None if src["V"] is None else src["V"].clone()
        self.meta = src["meta"].clone()
        self.klabel = src["klabel"].clone()
        self.blk = torch.empty(d.batch * d.n_kv_heads * d.k_blocks, dtype=torch.int32, device="cuda")
        self.tok = torch.empty(d.batch * d.n_kv_heads * d.k_tokens, dtype=torch.int32, device="cuda")
        self.out = torch.empty(d.batch * d.n_q_heads * d.d_v, device="cuda")
        self.lse = torch.empty(d.batch * d.n_q_heads, device="cuda")
        self.ws = H.alloc_workspace(d)
        self.score = torch.empty(d.batch * d.n_kv_heads * d.nb_cap, device="cuda")


def stage(w, threads):
    """Host generation of the seeded inputs, upload, and prefill metadata."""
    t0 = time.time()
    q = W.queries(w)
    K, V = W.full_cache(w, q, threads=threads)
    k_new, v_new = W.new_token(w)
    lab = W.label_channels(w)
    log(f"[bench] generated {w.name} inputs in {time.time() - t0:.1f}s")
    dev16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    d = dims_of(w)
    U = w.units
    base = {
        "q": dev16(q), "K": dev16(K), "V": None if V is None else dev16(V),
        "k_new": dev16(k_new), "v_new": dev16(v_new),
        "label": torch.from_numpy(lab).cuda(),
        "ctx": torch.full((w.batch,), w.ctx, dtype=torch.int32, device="cuda"),
        "ctx_prefill": torch.full((w.batch,), w.ctx - 1, dtype=torch.int32, device="cuda"),
        "meta": H.alloc_meta(d),
        "klabel": H.alloc_klabel(d),
    }
    H.build_meta(d, base["K"], base["ctx_prefill"], base["label"], base["meta"], base["klabel"])
    torch.cuda.synchronize()
    host = {"q": q, "K": K, "V": V, "k_new": k_new, "v_new": v_new, "label": lab}
    return d, base, host


def graph_group(steps, cap=16):
    """Steps per captured graph: the largest divisor of `steps` up to cap,
    so that exactly `steps` steps are timed."""
    return max(g for g in range(1, min(cap, steps) + 1) if steps % g == 0)


def time_replays(fns, stream, warmup, steps, graphs=True, group=1, spread=False):
    """Average ms per call of fns[i % len(fns)] over `steps` calls (after an
    eager warmup call of every fn and about `warmup` untimed calls). With
    graphs, calls are captured as HIP graphs of `group` consecutive calls
    each (len(fns) graphs, graph k holding calls k*group .. k*group+group-1,
    so replaying them in turn continues the rotation over fns) and
    steps / group graphs are replayed; group must divide steps. spread
    (graphs only): also return the median, p10 and p90 of ms per call from
    a second pass that brackets every replay with its own events (after the
    timed region, which holds no events between its replays)."""
    assert steps % group == 0
    with torch.cuda.stream(stream):
        for f in fns:
            f()
    torch.cuda.synchronize()
    n = len(fns)
    gr = []
    if graphs:
        for k in range(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for j in range(group):
                    fns[(k * group + j) % n]()
            gr.append(g)
        torch.cuda.synchronize()
        calls, call = steps // group, (lambda i: gr[i % n].replay())
        wcalls = max(1, -(-warmup // group))
    else:
        calls, call, wcalls = steps, (lambda i: fns[i % n]()), warmup
    with torch.cuda.stream(stream):
        for i in range(wcalls):
            call(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for i in range(calls):
            call(i)
        ev1.record(stream)
    torch.cuda.synchronize()
    avg = ev0.elapsed_time(ev1) / steps
    if not (spread and graphs):
        return avg
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    with torch.cuda.stream(stream):
        for i in range(calls):
            evs[i][0].record(stream)
            call(i)
            evs[i][1].record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) / group for a, b in evs])
    return avg, {"median_ms": round(float(np.median(per)), 6), "p10_ms": round(float(np.percentile(per, 10)), 6),
                 "p90_ms": round(float(np.percentile(per, 90)), 6), "samples": int(calls), "steps_per_sample": group}


_COPY_GBS = []


def copy_reference():
    """measured_copy_gbs(), measured once per process."""
    if not _COPY_GBS:
        _COPY_GBS.append(measured_copy_gbs())
        log(f"[bench] device copy: {_COPY_GBS[0]:.0f} GB/s (read + write)")
    return _COPY_GBS[0]


def measured_h2d_gbs(pinned, n_bytes=256 << 20, reps=4):
    """Rate of one large host-to-device copy from pinned host memory (best
    of reps after one untimed copy): the measured link reference beside the
    PCIe peak."""
    src = pinned.view(torch.uint8)[:n_bytes]
    dst = torch.empty(n_bytes, dtype=torch.uint8, device="cuda")
    best = float("inf")
    for i in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src, non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
        if i:
            best = min(best, e0.elapsed_time(e1))
    del dst
    return n_bytes / (best * 1e-3) / 1e9


def measured_copy_gbs(n_bytes=1 << 30, reps=5):
    """Device-to-device copy rate of this GPU (bytes read plus bytes
    written per second, best of reps after one untimed copy): the measured
    stream-copy reference beside the published HBM peak."""
    a = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    best = float("inf")
    for i in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        if i:
            best = min(best, e0.elapsed_time(e1))
    del a, b
    torch.cuda.empty_cache()
    return 2 * n_bytes / (best * 1e-3) / 1e9


def time_score_launches(d, base, metas, reps, stream, steps):
    """us per block-score launch: a graph of 8 launches per cache copy,
    back to back, replayed; HIP events on the launching stream."""
    R = len(reps)
    n_score = 8 * R
    with torch.cuda.stream(stream):
        for m, r in zip(metas, reps):
            H.score_blocks(d, base["q"], m, base["ctx"], r.score, stream=stream)
    torch.cuda.synchronize()
    gs = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gs, stream=stream):
        for i in range(n_score):
            H.score_blocks(d, base["q"], metas[i % R], base["ctx"], reps[i % R].score, stream=stream)
    with torch.cuda.stream(stream):
        gs.replay()
    torch.cuda.synchronize()
    n_rep = max(1, steps // n_score)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(n_rep):
            gs.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) * 1e3 / (n_rep * n_score)


def fp8_meta_leg(w, base, reps, stream, args, ms_step_bf16):
    """The same decode step with block metadata in outward-rounded fp8 e4m3
    (half the bytes of the block-score stream): own metadata per cache copy,
    built from the same keys; the rest of the step is unchanged."""
    w8 = dataclasses.replace(w, meta_fp8=True)
    d8 = dims_of(w8)
    metas = []
    for r in reps:
        m = H.alloc_meta(d8)
        H.build_meta(d8, r.K, base["ctx_prefill"], base["label"], m, r.klabel)
        metas.append(m)
    torch.cuda.synchronize()

    def dec(i):
        r = reps[i]
        return lambda: H.decode_step(d8, base["q"], base["k_new"], base["v_new"], r.K, r.V, metas[i], r.klabel,
                                     base["label"], base["ctx"], r.blk, r.tok, r.out, r.lse, r.ws, stream=stream)
    ms = time_replays([dec(i) for i in range(len(reps))], stream, args.warmup, args.steps, not args.no_graph,
                      graph_group(args.steps))
    us_score = time_score_launches(d8, base, metas, reps, stream, args.steps)
    kb = score_kernel_bytes(w8)
    ach = kb / (us_score * 1e-6) / 1e9
    log(f"[bench] fp8 metadata: {ms * 1e3:.1f} us/step, block score {us_score:.2f} us/launch ({ach:.0f} GB/s)")
    # the same step with the label rows in nearest-rounded e4m3 as well
    w88 = dataclasses.replace(w8, label_fp8=True)
    d88 = dims_of(w88)
    lab8 = []
    for r, m in zip(reps, metas):
        kl = H.alloc_klabel(d88)
        H.build_meta(d88, r.K, base["ctx_prefill"], base["label"], H.alloc_meta(d88), kl)
        lab8.append(kl)
    torch.cuda.synchronize()

    def dec8(i):
        r = reps[i]
        return lambda: H.decode_step(d88, base["q"], base["k_new"], base["v_new"], r.K, r.V, metas[i], lab8[i],
                                     base["label"], base["ctx"], r.blk, r.tok, r.out, r.lse, r.ws, stream=stream)
    ms88 = time_replays([dec8(i) for i in range(len(reps))], stream, args.warmup, args.steps, not args.no_graph,
                        graph_group(args.steps))
    log(f"[bench] fp8 metadata and label rows: {ms88 * 1e3:.1f} us/step")
    return {"format": "e4m3, max rounded up, min rounded down", "ms_per_step": round(ms, 6),
            "queries_per_s": round(w.batch * w.n_q_heads / (ms * 1e-3), 1),
            "step_speedup_vs_bf16_meta": round(ms_step_bf16 / ms, 3),
            "block_score": {"us_per_launch": round(us_score, 3), "algorithmic_bytes": kb,
                            "achieved": round(ach, 1), "frac": round(ach / HBM_PEAK_GBS, 4)},
            "with_fp8_labels": {"label_format": "e4m3, nearest", "ms_per_step": round(ms88, 6),
                                "queries_per_s": round(w.batch * w.n_q_heads / (ms88 * 1e-3), 1),
                                "step_speedup_vs_bf16": round(ms_step_bf16 / ms88, 3)}}


def variants_leg(w, base, reps, stream, args, ms_step):
    """Cost of the opt-in selection variants (group sum, one sink block and
    two local blocks) on the same step, and of one label-channel
    calibration over 1024 sampled (query, key) rows of every KV head."""
    wv = dataclasses.replace(w, agg_sum=True, sink_blocks=1, local_blocks=2)
    dv = dims_of(wv)

    def dec(r):
        return lambda: H.decode_step(dv, base["q"], base["k_new"], base["v_new"], r.K, r.V, r.meta, r.klabel,
                                     base["label"], base["ctx"], r.blk, r.tok, r.out, r.lse, r.ws, stream=stream)
    ms = time_replays([dec(r) for r in reps], stream, args.warmup, args.steps, not args.no_graph,
                      graph_group(args.steps))
    S = 1024
    gen = torch.Generator(device="cuda").manual_seed(5)
    qs = torch.randn(S * w.n_q_heads * w.d_k, generator=gen, device="cuda").to(torch.bfloat16)
    ks = torch.randn(S * w.n_kv_heads * w.d_k, generator=gen, device="cuda").to(torch.bfloat16)
    imp = torch.empty(w.n_kv_heads * w.d_k, device="cuda")
    lab = torch.empty(w.n_kv_heads * w.r, dtype=torch.int32, device="cuda")
    d = dims_of(w)
    ms_cal = time_replays([lambda: H.calibrate_labels(d, qs, ks, S, imp, lab, stream=stream)], stream, 3, 20,
                          not args.no_graph, graph_group(20))
    cal_bytes = S * (w.n_q_heads + w.n_kv_heads) * w.d_k * 2
    log(f"[bench] variants step {ms * 1e3:.1f} us; calibration {ms_cal * 1e3:.1f} us")
    res = {"agg_sum_sink1_local2": {"ms_per_step": round(ms, 6), "vs_default_step": round(ms / ms_step, 3)},
           "calibration": {"samples": S, "us_per_call": round(ms_cal * 1e3, 2), "bytes_read": cal_bytes,
                           "achieved_gbs": round(cal_bytes / (ms_cal * 1e-3) / 1e9, 1)}}
    if not w.v_alias_k:
        res["per_head"] = per_head_leg(w, base, reps, stream, args, ms_step)
    return res


def per_head_leg(w, base, reps, stream, args, ms_step):
    """The same step with per-query-head selection (every head selects its
    own blocks and tokens; the attention gathers the union of a KV head's
    token sets once): step time, and how many rows the union holds per KV
    head against K_t (one shared set) and G*K_t (every head gathering its
    own rows)."""
    wh = dataclasses.replace(w, per_head=True)
    dh = dims_of(wh)
    S = w.batch * w.n_q_heads
    bufs = [{"blk": torch.empty(S * w.k_blocks, dtype=torch.int32, device="cuda"),
             "tok": torch.empty(S * w.k_tokens, dtype=torch.int32, device="cuda"),
             "ws": H.alloc_workspace(dh)} for _ in reps]

    def dec(r, x):
        return lambda: H.decode_step(dh, base["q"], base["k_new"], base["v_new"], r.K, r.V, r.meta, r.klabel,
                                     base["label"], base["ctx"], x["blk"], x["tok"], r.out, r.lse, x["ws"],
                                     stream=stream)
    ms = time_replays([dec(r, x) for r, x in zip(reps, bufs)], stream, args.warmup, args.steps, not args.no_graph,
                      graph_group(args.steps))
    tok = bufs[0]["tok"].cpu().numpy().reshape(w.units, w.group, w.k_tokens)
    union = [len(np.unique(u[u >= 0])) for u in tok]
    log(f"[bench] per-head selection step {ms * 1e3:.1f} us, union {np.mean(union):.0f} rows per KV head")
    return {"ms_per_step": round(ms, 6), "vs_default_step": round(ms / ms_step, 3),
            "union_rows_per_kv_head": round(float(np.mean(union)), 1),
            "union_vs_k_tokens": round(float(np.mean(union)) / w.k_tokens, 3),
            "union_vs_heads_times_k_tokens": round(float(np.mean(union)) / (w.group * w.k_tokens), 3)}


def decode(d, base, rep, stream):
    H.decode_step(d, base["q"], base["k_new"], base["v_new"], rep.K, rep.V, rep.meta, rep.klabel,
                  base["label"], base["ctx"], rep.blk, rep.tok, rep.out, rep.lse, rep.ws, stream=stream)


_CPU_JOB = None   # (workload, prepared units) shared with forked workers


def _cpu_decode_loop(k, n_workers, budget_s):
    """Oracle decodes of units k, k + n_workers, ... of the prepared sample,
    one BLAS thread, for about budget_s seconds. Returns (units, seconds)."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    w, units = _CPU_JOB
    done, spent, i = 0, 0.0, k
    with threadpool_limits(limits=1):
        while spent < budget_s:
            q, K, V, meta, lab = units[i % len(units)]
            t0 = time.perf_counter()
            O.decode_unit(q, K, V, w.ctx, w.block, w.k_blocks, lab, w.k_tokens, w.sm_scale, meta=meta)
            spent += time.perf_counter() - t0
            done += 1
            i += n_workers
    return done, spent


def _cpu_worker(a):
    return _cpu_decode_loop(*a)


def cpu_baseline(w, host, budget_s=10.0, max_workers=16):
    """The CPU oracle on a bounded sample of the same step: the first units
    of the batch, converted to fp64 with metadata prebuilt outside the
    timed region, decoded repeatedly for about budget_s seconds, once on one
    core and once on every core this process may use (at most max_workers
    worker processes, one BLAS thread each, each cycling over its own units;
    rate = all queries decoded / wall time)."""
    import multiprocessing as mp
    import oracle as O
    global _CPU_JOB
    cpus = os.cpu_count()
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else cpus
    n_workers = max(1, min(avail, max_workers))
    G, n = w.group, w.ctx
    units = []
    for u in range(min(max(4, n_workers), w.units)):
        b, g = divmod(u, w.n_kv_heads)
        Kb = host["K"][b, g, :n].copy()
        Kb[n - 1] = host["k_new"][b, g]
        K = O.bf16_to_f64(Kb)
        if w.v_alias_k:
            V = K[:, : w.d_v]
        else:
            Vb = host["V"][b, g, :n].copy()
            Vb[n - 1] = host["v_new"][b, g]
            V = O.bf16_to_f64(Vb)
        q = O.bf16_to_f64(host["q"][b, g * G:(g + 1) * G])
        meta_fn = O.block_meta_e4m3 if w.meta_fp8 else O.block_meta
        units.append((q, K, V, meta_fn(K, n, w.block), host["label"][g]))
    _CPU_JOB = (w, units)
    done1, spent1 = _cpu_decode_loop(0, 1, budget_s)
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(n_workers) as pool:
        parts = pool.map(_cpu_worker, [(k, n_workers, budget_s) for k in range(n_workers)])
    wall = time.perf_counter() - t0
    done_all = sum(p[0] for p in parts)
    _CPU_JOB = None
    return {"value": round(done_all * G / wall, 2), "unit": "queries/s", "cores": n_workers, "kind": "oracle",
            "os_cpu_count": cpus, "cores_available": avail,
            "single_core": {"value": round(done1 * G / spent1, 2), "cores": 1,
                            "sample": f"{done1} unit decodes cycling over the first {len(units)} units, {spent1:.1f}s"},
            "sample": f"{done_all} unit decodes by {n_workers} worker processes (one BLAS thread each) over the first "
                      f"{len(units)} (batch, KV head) units of the {w.name} step ({done_all * G} queries), fp64 "
                      f"NumPy, metadata prebuilt, {wall:.1f}s wall"}


PCIE_PEAK_GBS = 64.0   # PCIe 5.0 x16, one direction


def offload_bench(args, lite=False):
    """The multi-step offload run: 16 decode steps with drifting queries;
    the full cache sits in a pinned host pool, the GPU holds metadata,
    label rows and a block cache. One JSON line with the step rate over
    the steady steps (1..15), the delta bytes per step, the copy time and
    how much of it the compute stream did not wait for (overlap), next to
    the same 16 steps on an HBM-resident cache. lite: host and GPU
    planning only (no runtime-copy mode, no multi-layer loop, no CPU
    baseline), returned instead of printed."""
    w = W.WORKLOADS["offload96k"]
    if args.meta == "fp8":
        w = dataclasses.replace(w, meta_fp8=True)
    steps = W.OFFLOAD_STEPS
    d = dims_of(w)
    U, B, Hkv, bs = w.units, w.batch, w.n_kv_heads, w.block
    nb_cap, be = d.nb_cap, H.block_elems(d)
    n_slots = 2 * w.k_blocks + 2
    prefill = W.offload_prefill(w, steps)
    t0 = time.time()
    q0 = W.queries(w)
    pool = torch.zeros(U * nb_cap * be, dtype=torch.int16, pin_memory=True)
    pv = pool.numpy().view(np.uint16).reshape(U, nb_cap, be)
    Kd = torch.zeros(U * w.max_ctx * w.d_k, dtype=torch.int16, device="cuda")
    Vd = torch.zeros(U * w.max_ctx * w.d_v, dtype=torch.int16, device="cuda")
    Kv, Vv = Kd.view(U, w.max_ctx, w.d_k), Vd.view(U, w.max_ctx, w.d_v)

    def fill(u):
        b, g = divmod(u, Hkv)
        n = int(prefill[b])
        kb, vb = W.unit_kv(w, b, g, q0, n)
        nbk = -(-n // bs)
        for src, lo, width in ((kb, 0, w.d_k), (vb, bs * w.d_k, w.d_v)):
            pad = np.zeros((nbk * bs, width), np.uint16)
            pad[:n] = src
            pv[u, :nbk, lo:lo + bs * width] = pad.reshape(nbk, bs * width)
        return u, kb, vb

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=args.threads) as ex:
        for u, kb, vb in ex.map(fill, range(U)):
            n = kb.shape[0]
            Kv[u, :n] = torch.from_numpy(kb.view(np.int16))
            Vv[u, :n] = torch.from_numpy(vb.view(np.int16))
    label = torch.from_numpy(W.label_channels(w)).cuda()
    meta0 = H.alloc_meta(d)
    klabel0 = torch.zeros(U * w.max_ctx * w.r, dtype=torch.int16, device="cuda")
    H.build_meta(d, Kd, torch.from_numpy(prefill).cuda(), label, meta0, klabel0)
    qs = [q0]
    for t in range(1, steps):
        qs.append(W.f32_to_bf16_bits(W.drift_queries(W.bf16_bits_to_f32(qs[-1]), w, t)))
    dev16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    q_d = [dev16(q) for q in qs]
    news = [W.new_token(w, t) for t in range(steps)]
    kn_d = [dev16(k) for k, _ in news]
    vn_d = [dev16(v) for _, v in news]
    ctx_h = [torch.from_numpy(prefill + t + 1) for t in range(steps)]
    ctx_d = [c.cuda() for c in ctx_h]
    torch.cuda.synchronize()
    log(f"[bench] offload run: prefill {prefill.tolist()}, pool {pool.numel() * 2 / 1e9:.2f} GB pinned, "
        f"staged in {time.time() - t0:.1f}s")
    h2d_gbs = measured_h2d_gbs(pool)
    log(f"[bench] pinned host-to-device copy of 256 MiB: {h2d_gbs:.1f} GB/s")

    meta, klabel = meta0.clone(), klabel0.clone()
    cache = torch.zeros(U * n_slots * be, dtype=torch.int16, device="cuda")
    slot_of = torch.full((U * nb_cap,), -1, dtype=torch.int32, device="cuda")
    tok = torch.empty(U * w.k_tokens, dtype=torch.int32, device="cuda")
    out = torch.empty(B * w.n_q_heads * w.d_v, device="cuda")
    lse = torch.empty(B * w.n_q_heads, device="cuda")
    ws = H.alloc_workspace(d)
    cs, xs = torch.cuda.Stream(), torch.cuda.Stream()
    full_bytes = U * w.k_blocks * be * 2

    def timed_runs(copy_mode):
        eng = H.OffloadEngine(d, n_slots, copy_mode)
        runs = []
        # run 0 warms up; the timed runs record no GPU timestamps (each
        # timed event is a marker the GPU processes, several us per step);
        # one more run with timestamps gives the copy / wait breakdown
        for run in range(args.offload_runs + 2):
            instrumented = run == args.offload_runs + 1
            eng.set_timing(instrumented)
            meta.copy_(meta0)
            klabel.copy_(klabel0)
            torch.cuda.synchronize()
            eng.begin(torch.from_numpy(prefill.copy()), pool, cache, slot_of, stream=cs)
            stats = []
            t_start = time.perf_counter()
            for t in range(steps):
                if t == 1:
                    torch.cuda.synchronize()
                    t_steady = time.perf_counter()
                h0 = time.perf_counter()
                stats.append(eng.step(q_d[t], kn_d[t], vn_d[t], pool, cache, meta, klabel, label, ctx_d[t],
                                      ctx_h[t], slot_of, tok, out, lse, ws, compute_stream=cs,
                                      copy_stream=xs).as_dict())
                stats[-1]["host_call_ms"] = (time.perf_counter() - h0) * 1e3
            torch.cuda.synchronize()
            t_end = time.perf_counter()
            for t, x in enumerate(stats):   # planned on the GPU (kernel copies): read back now
                x["delta_bytes"], x["cold_bytes"] = eng.delta(t)
                if x["n_copies"] < 0:
                    x["n_copies"] = x["delta_bytes"] // (H.block_elems(d) * 2)
            if instrumented:
                tim = [eng.timing(t) for t in range(steps)]
                timed_ms = (t_end - t_steady) * 1e3 / (steps - 1)
            else:
                runs.append({"cold_s": t_steady - t_start, "steady_s": t_end - t_steady, "stats": stats})
        eng.close()
        runs = runs[1:]
        best = min(runs, key=lambda r: r["steady_s"])
        ms_step = best["steady_s"] * 1e3 / (steps - 1)
        st = best["stats"]
        delta = np.array([x["delta_bytes"] for x in st[1:]], np.float64)
        copy_ms = np.array([x["copy_ms"] for x in tim[1:]], np.float64)
        # the compute stream of step t+1 waits for step t's copies; what it
        # did not wait is hidden behind compute
        waits = np.array([x["copy_wait_ms"] for x in tim[2:]], np.float64)
        hidden = 1.0 - waits.sum() / max(copy_ms[:-1].sum(), 1e-9)
        link_gbs = delta.sum() / max(copy_ms.sum() * 1e-3, 1e-12) / 1e9
        return ms_step, {
            "copy_mode": {H.COPY_KERNEL: "gather_kernel", H.COPY_DMA: "dma_memcpy",
                          H.COPY_KERNEL_GPU_PLAN: "gather_kernel_gpu_plan"}[copy_mode],
            "ms_per_step": round(ms_step, 6), "runs": len(runs),
            "ms_per_step_with_timestamps": round(timed_ms, 6),
            "cold_ms": round(best["cold_s"] * 1e3, 3), "cold_bytes": st[0]["cold_bytes"],
            "delta_bytes_per_step": delta.tolist(), "delta_bytes_mean": float(delta.mean()),
            "full_set_bytes_per_step": full_bytes,
            "delta_frac_of_full": round(float(delta.mean()) / full_bytes, 4),
            "copies_mean": float(np.mean([x["n_copies"] for x in st[1:]])),
            "copy_ms_mean": round(float(copy_ms.mean()), 4), "copy_wait_ms_mean": round(float(waits.mean()), 4),
            "overlap_hidden_frac": round(float(hidden), 4),
            "link": {"achieved": round(link_gbs, 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                     "frac": round(link_gbs / PCIE_PEAK_GBS, 4), "measured_h2d_gbs": round(h2d_gbs, 2),
                     "frac_of_measured_h2d": round(link_gbs / h2d_gbs, 4)},
            "compute_ms_mean": round(float(np.mean([x["compute_ms"] for x in tim[1:]])), 4),
            "breakdown_from": "one extra run with per-step GPU timestamps (copy, wait, compute, link)",
            "host_wait_ms_mean": round(float(np.mean([x["host_wait_ms"] for x in st[1:]])), 4),
            "host_plan_ms_mean": round(float(np.mean([x["host_plan_ms"] for x in st[1:]])), 4),
            "host_call_ms_mean": round(float(np.mean([x["host_call_ms"] for x in st[1:]])), 4),
        }

    ms_step, off_k = timed_runs(H.COPY_KERNEL)
    off_d = None if lite else timed_runs(H.COPY_DMA)[1]
    _, off_g = timed_runs(H.COPY_KERNEL_GPU_PLAN)

    def multilayer(n_layers):
        """n_layers layers stepped in turn each decode step on one compute
        and one copy stream (gather copies): each has its own queries,
        metadata, label rows, block cache and engine and reads the shared
        pool (the appended rows are the same for every layer), so one
        layer's block delta is copied while the next layers compute."""
        L = []
        for l in range(n_layers):
            wl = dataclasses.replace(w, seed=w.seed + 1000 * (l + 1))
            ql = [W.queries(wl)]
            for t in range(1, steps):
                ql.append(W.f32_to_bf16_bits(W.drift_queries(W.bf16_bits_to_f32(ql[-1]), wl, t)))
            L.append({"q": [dev16(q) for q in ql], "meta": meta0.clone(), "klabel": klabel0.clone(),
                      "cache": torch.zeros_like(cache), "slot_of": torch.full_like(slot_of, -1),
                      "tok": torch.empty_like(tok), "out": torch.empty_like(out), "lse": torch.empty_like(lse),
                      "ws": H.alloc_workspace(d), "eng": H.OffloadEngine(d, n_slots, H.COPY_KERNEL)})
        best, tim = None, None
        for run in range(args.offload_runs + 2):   # as timed_runs: the last run records timestamps
            instrumented = run == args.offload_runs + 1
            for x in L:
                x["eng"].set_timing(instrumented)
                x["meta"].copy_(meta0)
                x["klabel"].copy_(klabel0)
            torch.cuda.synchronize()
            for x in L:
                x["eng"].begin(torch.from_numpy(prefill.copy()), pool, x["cache"], x["slot_of"], stream=cs)
            torch.cuda.synchronize()
            for t in range(steps):
                if t == 1:
                    torch.cuda.synchronize()
                    t_steady = time.perf_counter()
                for x in L:
                    x["eng"].step(x["q"][t], kn_d[t], vn_d[t], pool, x["cache"], x["meta"], x["klabel"], label,
                                  ctx_d[t], ctx_h[t], x["slot_of"], x["tok"], x["out"], x["lse"], x["ws"],
                                  compute_stream=cs, copy_stream=xs)
            torch.cuda.synchronize()
            steady = time.perf_counter() - t_steady
            if instrumented:
                tim = [[x["eng"].timing(t) for t in range(steps)] for x in L]
            elif run > 0 and (best is None or steady < best):
                best = steady
        for x in L:
            x["eng"].close()
        steady = best
        ms = steady * 1e3 / (steps - 1)
        copy_ms = sum(float(np.sum([x["copy_ms"] for x in tl[1:-1]])) for tl in tim)
        waits = sum(float(np.sum([x["copy_wait_ms"] for x in tl[2:]])) for tl in tim)
        return {"layers": n_layers, "ms_per_step": round(ms, 6), "ms_per_layer": round(ms / n_layers, 6),
                "per_layer_vs_single_layer_step": round(ms / n_layers / ms_step, 3),
                "copy_ms_per_layer_step": round(copy_ms / (n_layers * (steps - 2)), 4),
                "overlap_hidden_frac": round(1.0 - waits / max(copy_ms, 1e-9), 4)}

    multi = None if lite else multilayer(4)
    if multi:
        log(f"[bench] 4 layers: {multi['ms_per_step'] * 1e3:.1f} us/step, {multi['ms_per_layer'] * 1e3:.1f} "
            f"us/layer, {100 * multi['overlap_hidden_frac']:.0f}% of copies hidden")

    # the same 16 steps on an HBM-resident cache (no offload), for reference
    meta.copy_(meta0)
    klabel.copy_(klabel0)
    blk = torch.empty(U * w.k_blocks, dtype=torch.int32, device="cuda")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    with torch.cuda.stream(cs):
        for t in range(steps):
            if t == 1:
                evs[0].record(cs)
            H.decode_step(d, q_d[t], kn_d[t], vn_d[t], Kd, Vd, meta, klabel, label, ctx_d[t], blk, tok, out,
                          lse, ws, stream=cs)
        evs[1].record(cs)
    torch.cuda.synchronize()
    resident_ms = evs[0].elapsed_time(evs[1]) / (steps - 1)
    # overlap of the copies with compute: (t_compute + t_copy - t_step) /
    # min(t_compute, t_copy), with the resident step as t_compute (1: fully
    # overlapped, 0: in series)
    for o in (off_k, off_d, off_g):
        if o:
            tc, tx = resident_ms, o["copy_ms_mean"]
            o["overlap_ratio"] = round((tc + tx - o["ms_per_step"]) / max(min(tc, tx), 1e-9), 4)

    queries = B * w.n_q_heads
    res = {
        "metric": "offload decode queries/s (batch×heads), 16-step drifting run, 8k-96k ctx",
        "value": round(queries / (ms_step * 1e-3), 1), "unit": "queries/s", "n_gpus": 1,
        "steps": steps - 1, "warmup": 1, "ms_per_step": round(ms_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": w.n_q_heads, "kv_heads": Hkv, "d_k": w.d_k,
                   "prefill": prefill.tolist(), "block": bs, "k_blocks": w.k_blocks, "r": w.r,
                   "k_tokens": w.k_tokens, "n_slots": n_slots, "parallelism": "none (1 GPU)"},
        "resident_ms_per_step": round(resident_ms, 6),
        "offload": off_k,
        "offload_dma": off_d,
        "offload_gpu_plan": off_g,
        "multilayer": multi,
    }
    if lite:
        return res
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = offload_cpu_baseline(w, prefill, qs, news, Kv, Vv)
    print(json.dumps(res), flush=True)


def offload_summary(args):
    """The offload run's figures for the default bench line: step time and
    rate with host and with GPU planning, delta bytes per step, link rate
    and the share of the copy time hidden behind compute."""
    r = offload_bench(args, lite=True)
    out = {"workload": "offload96k", "prefill": r["config"]["prefill"], "steps": W.OFFLOAD_STEPS,
           "resident_ms_per_step": r["resident_ms_per_step"]}
    for key, src in (("host_plan", r["offload"]), ("gpu_plan", r["offload_gpu_plan"])):
        out[key] = {"ms_per_step": src["ms_per_step"],
                    "queries_per_s": round(r["config"]["batch"] * r["config"]["q_heads"]
                                           / (src["ms_per_step"] * 1e-3), 1),
                    "delta_bytes_mean": src["delta_bytes_mean"], "delta_frac_of_full": src["delta_frac_of_full"],
                    "link_gbs": src["link"]["achieved"], "link_frac": src["link"]["frac"],
                    "measured_h2d_gbs": src["link"]["measured_h2d_gbs"],
                    "overlap_hidden_frac": src["overlap_hidden_frac"], "overlap_ratio": src["overlap_ratio"],
                    "copy_ms_mean": src["copy_ms_mean"],
                    "host_call_ms_mean": src["host_call_ms_mean"]}
    log(f"[bench] offload: host plan {out['host_plan']['ms_per_step'] * 1e3:.1f} us/step, GPU plan "
        f"{out['gpu_plan']['ms_per_step'] * 1e3:.1f} us/step, resident {out['resident_ms_per_step'] * 1e3:.1f}")
    return out


def offload_cpu_baseline(w, prefill, qs, news, Kv, Vv, budget_s=10.0):
    """The oracle's offload_run on unit (0, 0) over the 16 steps, repeated
    for about budget_s seconds (one thread)."""
    import oracle as O
    from threadpoolctl import threadpool_limits

    G, n0, steps = w.group, int(prefill[0]), len(qs)
    K = Kv[0, : n0 + steps].cpu().numpy().view(np.uint16).copy()
    V = Vv[0, : n0 + steps].cpu().numpy().view(np.uint16).copy()
    for t, (kn, vn) in enumerate(news):
        K[n0 + t], V[n0 + t] = kn[0, 0], vn[0, 0]
    Kf, Vf = O.bf16_to_f64(K), O.bf16_to_f64(V)
    lab = W.label_channels(w)[0]
    seq = [(O.bf16_to_f64(qs[t][0, :G]), Kf, Vf, n0 + t + 1, w.k_blocks, lab, w.k_tokens, w.sm_scale)
           for t in range(steps)]
    with threadpool_limits(limits=1):
        done, spent = 0, 0.0
        while spent < budget_s:
            t0 = time.perf_counter()
            O.offload_run(seq, w.block, w.d_k, w.d_v)
            spent += time.perf_counter() - t0
            done += 1
    return {"value": done * steps * G / spent, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} x offload_run of unit (0,0) (prefill {n0}) over {steps} steps "
                      f"({done * steps * G} queries), fp64 NumPy, {spent:.1f}s"}


def layer_leg(w, args, full):
    """Stage workload w, time its decode step (grouped graph replay and one
    graph launch per step) and its block-score launches; full: also the
    dense reference, the fp8 and the selection-variant legs. Returns the
    result dict and the host arrays (for the CPU baseline)."""
    d, base, host = stage(w, args.threads)
    sb = step_bytes(w)
    R = args.replicas or max(4, math.ceil(768e6 / sb["total"]))
    reps = [Replica(d, base)]
    for _ in range(R - 1):
        reps.append(Replica(d, base, clone_from={"K": reps[0].K, "V": reps[0].V, "meta": reps[0].meta,
                                                 "klabel": reps[0].klabel}))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()

    # the timed loop replays graphs of `group` consecutive steps (the way a
    # model captures the layers of one token step in one graph); one graph
    # launch per step is timed too and reported beside it
    group = graph_group(args.steps) if not args.no_graph else 1
    step_fns = [(lambda r=r: decode(d, base, r, stream)) for r in reps]
    ms_step = time_replays(step_fns, stream, args.warmup, args.steps, not args.no_graph, group,
                           spread=not args.no_graph)
    ms_step, spread = ms_step if isinstance(ms_step, tuple) else (ms_step, None)
    ms_step_single = time_replays(step_fns, stream, args.warmup, args.steps, True, 1) if not args.no_graph else None
    log(f"[bench] {w.name}: {args.steps} steps: {ms_step * 1e3:.1f} us/step (events)")

    # dominant kernel alone: a graph of back-to-back block-score launches
    us_score = time_score_launches(d, base, [r.meta for r in reps], reps, stream, args.steps)
    copy_gbs = copy_reference()
    kb = score_kernel_bytes(w)
    achieved = kb / (us_score * 1e-6) / 1e9

    traffic = None
    cpath = COUNTERS.format(wl=w.name + ("_fp8" if w.meta_fp8 else ""))
    if os.path.exists(cpath):
        c = json.load(open(cpath))
        if c.get("source_hash") == source_hash(SCORE_SOURCES):
            traffic = c.get("bytes_per_launch")

    queries = w.batch * w.n_q_heads
    res = {
        "value": round(queries / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 6),
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads,
                   "d_k": w.d_k, "d_v": w.d_v, "ctx": w.ctx, "block": w.block, "k_blocks": w.k_blocks,
                   "r": w.r, "k_tokens": w.k_tokens, "meta": "fp8_e4m3_outward" if w.meta_fp8 else "bf16",
                   "cache_replicas": R, "hip_graph": not args.no_graph, "steps_per_graph": group,
                   "parallelism": "none (1 GPU)"},
        "ms_per_step_one_graph_per_step": None if ms_step_single is None else round(ms_step_single, 6),
        "hbm_frac_step": round(sb["total"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_bytes": sb["total"],
        "step_ms_spread": spread,
        "roofline": {"kernel": "block_score", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": kb, "us_per_launch": round(us_score, 3),
                     "measured_copy_gbs": round(copy_gbs, 1), "frac_of_measured_copy": round(achieved / copy_gbs, 4)},
    }
    if w.group > 1:
        # the block score as a matrix product on the matrix cores: G heads x
        # 2 d_k stacked channels per block, 2 flops per multiply-add
        flops = 2 * w.group * 2 * w.d_k * w.units * (-(-w.ctx // w.block))
        tf = flops / (us_score * 1e-6) / 1e12
        res["score_gemm"] = {"flops_per_launch": flops, "achieved_tflops": round(tf, 2),
                             "peak_tflops_bf16_dense": MFMA_PEAK_TFLOPS,
                             "frac_of_mfma_peak": round(tf / MFMA_PEAK_TFLOPS, 4),
                             "flop_per_byte": round(flops / kb, 2)}
        # matrix-core busy share from the committed rocprofv3 counters of this
        # kernel (reported while the hash of its sources matches)
        mpath = os.path.join(ROOT, "profiles", f"block_score_{w.name}_mfma_counters.json")
        if not w.meta_fp8 and os.path.exists(mpath):
            c = json.load(open(mpath))
            if c.get("source_hash") == source_hash(SCORE_SOURCES):
                res["score_gemm"]["mfma_busy_frac_counters"] = round(c["mfma_busy_frac"], 4)
                res["score_gemm"]["mfma_flops_executed_per_launch"] = int(c["mfma_flops_executed"])
    if full:
        # full attention over every token on the same caches: the operator the
        # sparse step replaces (the pages report the sparse speedup over it)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dws = H.dense_workspace_bytes(d)
        if dws:
            dout = torch.empty(w.batch * w.n_q_heads * w.d_v, device="cuda")
            dlse = torch.empty(w.batch * w.n_q_heads, device="cuda")
            dwsb = torch.empty(dws, dtype=torch.uint8, device="cuda")
            gd = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                H.dense_attend(d, base["q"], reps[0].K, reps[0].V, base["ctx"], dout, dlse, dwsb, stream=stream)
            torch.cuda.synchronize()
            with torch.cuda.graph(gd, stream=stream):
                for r in reps:
                    H.dense_attend(d, base["q"], r.K, r.V, base["ctx"], dout, dlse, dwsb, stream=stream)
            with torch.cuda.stream(stream):
                gd.replay()
            torch.cuda.synchronize()
            n_rep = max(1, args.steps // (4 * R))
            with torch.cuda.stream(stream):
                ev0.record(stream)
                for _ in range(n_rep):
                    gd.replay()
                ev1.record(stream)
            torch.cuda.synchronize()
            ms_dense = ev0.elapsed_time(ev1) / (n_rep * R)
            dbytes = w.units * w.ctx * (w.d_k + (0 if w.v_alias_k else w.d_v)) * 2
            res["dense_reference"] = {"ms_per_call": round(ms_dense, 6), "kv_bytes": dbytes,
                                      "achieved_gbs": round(dbytes / (ms_dense * 1e-3) / 1e9, 1),
                                      "speedup_sparse_step_vs_dense": round(ms_dense / ms_step, 3)}
            log(f"[bench] dense attention {ms_dense * 1e3:.1f} us/call, sparse step {ms_step * 1e3:.1f} us "
                f"({ms_dense / ms_step:.2f}x)")
        if not w.meta_fp8 and not args.no_fp8_leg and w.d_k % 32 == 0:
            res["meta_fp8"] = fp8_meta_leg(w, base, reps, stream, args, ms_step)
        if not args.no_fp8_leg:
            res["variants"] = variants_leg(w, base, reps, stream, args, ms_step)
    del reps, base
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, host


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gqa48k", choices=sorted(W.WORKLOADS))
    ap.add_argument("--replicas", type=int, default=0, help="cache copies to rotate (0: auto)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of graph replay")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--threads", type=int, default=16)
    ap.add_argument("--meta", default="bf16", choices=["bf16", "fp8"],
                    help="block metadata format of the timed step (fp8: e4m3, rounded outward)")
    ap.add_argument("--no-fp8-leg", action="store_true",
                    help="skip the extra timings (fp8 metadata, selection variants, calibration)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the 96k, latent and offload legs of the default run")
    ap.add_argument("--offload-runs", type=int, default=3, help="timed 16-step runs of the offload workload")
    ap.add_argument("--score-only", type=int, default=0,
                    help="only launch the block-score kernel this many times (for counter runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the operator is measured on a "
              f"single MI355X and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    w = W.WORKLOADS[args.workload]
    if args.meta == "fp8":
        w = dataclasses.replace(w, meta_fp8=True)
    torch.cuda.set_device(0)
    if w.name == "offload96k":
        offload_bench(args)
        return
    if args.score_only:
        score_only(w, args)
        return

    leg, host = layer_leg(w, args, full=True)
    res = {"metric": METRIC, "value": leg.pop("value"), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": leg.pop("ms_per_step"), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    res.update(leg)
    if args.workload == "gqa48k" and args.meta == "bf16" and not args.no_extra:
        # the other layers the metric is quoted on, measured in the same run
        for key, name in (("ctx96k", "gqa96k"), ("mla64k", "mla64k")):
            sub, _ = layer_leg(W.WORKLOADS[name], args, full=False)
            sub["queries_per_s"] = sub.pop("value")
            res[key] = sub
        res["offload"] = offload_summary(args)
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(w, host)
    print(json.dumps(res), flush=True)


def score_only(w, args):
    """Block-score launches alone (for counter runs), then a plain copy of
    known size as the last kernel, for calibrating the counters."""
    d, base, host = stage(w, args.threads)
    sb = step_bytes(w)
    R = args.replicas or max(4, math.ceil(768e6 / sb["total"]))
    reps = [Replica(d, base)]
    for _ in range(R - 1):
        reps.append(Replica(d, base, clone_from={"K": reps[0].K, "V": reps[0].V, "meta": reps[0].meta,
                                                 "klabel": reps[0].klabel}))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(args.score_only):
            r = reps[i % R]
            H.score_blocks(d, base["q"], r.meta, base["ctx_prefill"], r.score, stream=stream)
        # plain copy of known size for counter calibration: 1 GiB of
        # initialized data, the last kernel this mode launches
        a = torch.ones(256 << 20, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] score-only: {args.score_only} launches, then a copy of {a.numel() * 4} bytes")


if __name__ == "__main__":
    main()
