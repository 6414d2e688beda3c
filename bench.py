"""Decode-step throughput of the two-level sparse attention operator on one
MI355X, with the HBM roofline of its dominant kernel and the CPU oracle
timed beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gqa48k]

A step is one decode step of one attention layer over the whole batch:
append the new token, block scores over the full context, top-K_b, label
scores over the kept blocks, top-K_t, exact attention and the split merge.
Inputs are resident in HBM before timing starts. Steps rotate over several
copies of the cache (distinct addresses, as consecutive layers would be) so
the 256 MB Infinity Cache cannot serve a step from the previous one; each
copy's step is captured once as a HIP graph and replayed.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
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
COUNTERS = os.path.join(ROOT, "profiles", "block_score_{wl}_counters.json")
SCORE_SOURCES = ["hierarchical_sparse_attention_block_amd/csrc/score.hip",
                 "hierarchical_sparse_attention_block_amd/csrc/common.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dims_of(w):
    return H.dims(w.batch, w.n_q_heads, w.n_kv_heads, w.d_k, w.d_v, w.v_alias_k, w.block, w.r,
                  w.k_blocks, w.k_tokens, w.max_ctx, w.sm_scale)


def step_bytes(w):
    """Algorithmic HBM bytes of one decode step (every unit at full context):
    block metadata, label rows of the kept blocks, gathered K/V rows of the
    kept tokens, queries and outputs."""
    U, nb = w.units, -(-w.ctx // w.block)
    meta = U * nb * 2 * w.d_k * 2
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
    return U * nb * (2 * w.d_k * 2 + 4) + w.batch * w.n_q_heads * w.d_k * 2


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
        "meta": torch.zeros(U * d.nb_cap * 2 * w.d_k, dtype=torch.int16, device="cuda"),
        "klabel": torch.zeros(U * w.max_ctx * w.r, dtype=torch.int16, device="cuda"),
    }
    H.build_meta(d, base["K"], base["ctx_prefill"], base["label"], base["meta"], base["klabel"])
    torch.cuda.synchronize()
    host = {"q": q, "K": K, "V": V, "k_new": k_new, "v_new": v_new, "label": lab}
    return d, base, host


def decode(d, base, rep, stream):
    H.decode_step(d, base["q"], base["k_new"], base["v_new"], rep.K, rep.V, rep.meta, rep.klabel,
                  base["label"], base["ctx"], rep.blk, rep.tok, rep.out, rep.lse, rep.ws, stream=stream)


def cpu_baseline(w, host, budget_s=10.0, n_units=4):
    """The CPU oracle on a bounded sample of the same step: the first
    n_units (batch, KV head) units, converted to fp64 and with metadata
    prebuilt outside the timed region, decoded repeatedly until about
    budget_s seconds of oracle work. One thread (BLAS pinned to 1)."""
    import oracle as O
    from threadpoolctl import threadpool_limits

    G, n = w.group, w.ctx
    units = []
    for u in range(min(n_units, w.units)):
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
        units.append((q, K, V, O.block_meta(K, n, w.block), host["label"][g]))
    done, spent = 0, 0.0
    with threadpool_limits(limits=1):
        while spent < budget_s:
            q, K, V, meta, lab = units[done % len(units)]
            t0 = time.perf_counter()
            O.decode_unit(q, K, V, n, w.block, w.k_blocks, lab, w.k_tokens, w.sm_scale, meta=meta)
            spent += time.perf_counter() - t0
            done += 1
    return {"value": done * G / spent, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} unit decodes cycling over the first {len(units)} (batch, KV head) units of "
                      f"the {w.name} step ({done * G} queries), fp64 NumPy, metadata prebuilt, {spent:.1f}s"}


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
    ap.add_argument("--score-only", type=int, default=0,
                    help="only launch the block-score kernel this many times (for counter runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the operator is measured on a "
              f"single MI355X and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    w = W.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    d, base, host = stage(w, args.threads)
    sb = step_bytes(w)
    R = args.replicas or max(4, math.ceil(768e6 / sb["total"]))
    reps = [Replica(d, base)]
    for _ in range(R - 1):
        reps.append(Replica(d, base, clone_from={"K": reps[0].K, "V": reps[0].V, "meta": reps[0].meta,
                                                 "klabel": reps[0].klabel}))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()

    if args.score_only:
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
        return

    # eager warmup (loads code objects before any capture)
    with torch.cuda.stream(stream):
        for r in reps:
            decode(d, base, r, stream)
    torch.cuda.synchronize()

    graphs = []
    if not args.no_graph:
        for r in reps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                decode(d, base, r, stream)
            graphs.append(g)
        torch.cuda.synchronize()

    def run(i):
        if graphs:
            graphs[i % R].replay()
        else:
            decode(d, base, reps[i % R], stream)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            run(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(args.steps):
            run(i)
        ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log(f"[bench] {args.steps} steps: {ms_step * 1e3:.1f} us/step (events), wall {wall / args.steps * 1e6:.1f} us/step")

    # dominant kernel alone: a graph of back-to-back block-score launches
    n_score = 8 * R
    gs = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        for r in reps:
            H.score_blocks(d, base["q"], r.meta, base["ctx"], r.score, stream=stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(gs, stream=stream):
        for i in range(n_score):
            r = reps[i % R]
            H.score_blocks(d, base["q"], r.meta, base["ctx"], r.score, stream=stream)
    with torch.cuda.stream(stream):
        gs.replay()
    torch.cuda.synchronize()
    reps_score = max(1, args.steps // n_score)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(reps_score):
            gs.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    us_score = ev0.elapsed_time(ev1) * 1e3 / (reps_score * n_score)
    kb = score_kernel_bytes(w)
    achieved = kb / (us_score * 1e-6) / 1e9

    traffic = None
    cpath = COUNTERS.format(wl=w.name)
    if os.path.exists(cpath):
        c = json.load(open(cpath))
        if c.get("source_hash") == source_hash(SCORE_SOURCES):
            traffic = c.get("bytes_per_launch")

    queries = w.batch * w.n_q_heads
    value = queries / (ms_step * 1e-3)
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads,
                   "d_k": w.d_k, "d_v": w.d_v, "ctx": w.ctx, "block": w.block, "k_blocks": w.k_blocks,
                   "r": w.r, "k_tokens": w.k_tokens, "cache_replicas": R, "hip_graph": bool(graphs),
                   "parallelism": "none (1 GPU)"},
        "hbm_frac_step": round(sb["total"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_bytes": sb["total"],
        "roofline": {"kernel": "block_score", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": kb, "us_per_launch": round(us_score, 3)},
    }
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(w, host)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
