"""Selection variants on the GPU against the oracle: group scores summed
over the query heads (HSAB_AGG_SUM) and always-kept sink / local blocks,
alone and together, also with fp8 metadata."""
import numpy as np
import pytest
import torch

import oracle as O
from hierarchical_sparse_attention_block_amd import workloads as W
from tests import hsab_testlib as T

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _wl(**kw):
    base = dict(name="var", batch=2, n_q_heads=8, n_kv_heads=2, d_k=128, d_v=128, v_alias_k=False,
                block=16, r=16, k_blocks=16, k_tokens=64, ctx=1000, max_ctx=1024, scaled_keys=True,
                label_mode="top_scale", n_planted=4, seed=29)
    base.update(kw)
    return W.Workload(**base)


def _decode(w):
    ctx = np.array([w.ctx, max(2, (w.ctx * 5) // 7)], np.int32)
    say(f"[variant decode_step] {w}")
    h = T.host_inputs(w, ctx_len=ctx)
    dev = T.Device(w, h)
    dev.prefill_meta()
    dev.decode_step()
    r = dev.results()
    K, V = T.appended_cache(w, h)
    G = w.group
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            T.oracle_unit_vs_gpu(w, h["q"], K, V, h["ctx"], h["label"], b, g, r["blk"][b, g], r["tok"][b, g],
                                 r["out"][b, g * G:(g + 1) * G], r["lse"][b, g * G:(g + 1) * G])
    return r


@pytest.mark.parametrize("kw", [dict(), dict(n_q_heads=16, n_kv_heads=2, d_k=64, d_v=64),
                                dict(n_q_heads=32, n_kv_heads=1, d_k=576, d_v=512, v_alias_k=True, block=32,
                                     r=32, k_blocks=8, k_tokens=100, n_planted=0)])
def test_sum_aggregation_decode(kw):
    _decode(_wl(agg_sum=True, **kw))


@pytest.mark.parametrize("sink,local,kb", [(1, 2, 16), (4, 0, 8), (0, 3, 3), (2, 2, 4), (1, 1, 64)])
def test_forced_blocks_decode(sink, local, kb):
    r = _decode(_wl(sink_blocks=sink, local_blocks=local, k_blocks=kb))
    for b, n in enumerate([1000, (1000 * 5) // 7]):
        nb = -(-n // 16)
        for g in range(2):
            blk = r["blk"][b, g]
            assert set(range(min(sink, nb))) <= set(blk.tolist())
            assert set(range(max(0, nb - local), nb)) <= set(blk.tolist())


def test_all_variants_with_fp8_metadata_latent():
    _decode(_wl(n_q_heads=32, n_kv_heads=1, d_k=576, d_v=512, v_alias_k=True, block=32, r=32, k_blocks=8,
                k_tokens=100, n_planted=0, agg_sum=True, sink_blocks=1, local_blocks=2, meta_fp8=True))


@pytest.mark.parametrize("G,dk", [(4, 128), (8, 256), (32, 576), (3, 128)])
def test_summed_block_scores_within_fp32_bound(G, dk):
    w = _wl(n_q_heads=2 * G, n_kv_heads=2, d_k=dk, d_v=dk if dk != 576 else 512, v_alias_k=dk == 576,
            max_ctx=1500, ctx=1500, n_planted=0, agg_sum=True)
    ctx = np.array([1500, 1093], np.int32)
    h = T.host_inputs(w, ctx_len=ctx)
    dev = T.Device(w, h)
    dev.prefill_meta()
    d = dev.d
    sc = torch.full((w.units * d.nb_cap,), float("nan"), device="cuda")
    dev.H.score_blocks(d, dev.q, dev.meta, dev.ctx_prefill, sc)
    sc = sc.cpu().numpy().reshape(w.batch, w.n_kv_heads, d.nb_cap)
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            n = int(ctx[b]) - 1
            q = O.bf16_to_f64(h["q"][b, g * G:(g + 1) * G])
            kmax, kmin = O.block_meta(O.bf16_to_f64(h["K"][b, g, :n]), n, w.block)
            want = O.block_scores(q, kmax, kmin, "sum")
            # each head's fp32 bound error, summed, plus the G-term sum itself
            tol = sum(T.score_tolerance(q[i:i + 1], kmax, kmin) for i in range(G)) \
                + G * 2.0 ** -24 * np.abs(O.quest_bound(q, kmax, kmin)).sum(axis=0)
            err = np.abs(sc[b, g, :len(want)] - want)
            assert np.all(err <= tol), f"unit ({b},{g}) worst {np.max(err / tol):.3g}x the bound"


def test_select_blocks_entry_point_with_forced_blocks():
    """hsab_select_blocks alone (score + block stage) keeps the forced blocks."""
    w = _wl(sink_blocks=2, local_blocks=1, k_blocks=6, n_planted=0)
    ctx = np.array([1000, 700], np.int32)
    h = T.host_inputs(w, ctx_len=ctx)
    dev = T.Device(w, h)
    dev.prefill_meta()
    dev.H.select_blocks(dev.d, dev.q, dev.meta, dev.ctx_prefill, dev.blk, ws=dev.ws)
    torch.cuda.synchronize()
    blk = dev.blk.cpu().numpy().reshape(w.batch, w.n_kv_heads, w.k_blocks)
    for b in range(w.batch):
        n = int(ctx[b]) - 1
        for g in range(w.n_kv_heads):
            q = O.bf16_to_f64(h["q"][b, g * 4:(g + 1) * 4])
            kmax, kmin = O.block_meta(O.bf16_to_f64(h["K"][b, g, :n]), n, w.block)
            T.check_block_set(O.block_scores(q, kmax, kmin), blk[b, g], w.k_blocks, 2, 1, f"unit ({b},{g})")
