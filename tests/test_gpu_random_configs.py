"""Seeded sweep of small decode configurations over every option at once:
group size, head dims, block size, label width, budgets (including ones
beyond the context), ragged context lengths, bf16 / fp8 metadata and
label rows, group max / sum / per-head selection, forced blocks and the
absorbed latent layout. Each draw runs one decode step and is checked unit
by unit (head by head for per-head selection) against the oracle under
the parity rules. A second, smaller set of draws uses capacities of 2k-32k
tokens with budgets up to 2048 blocks and tokens, which reach the paths
small contexts never take (the token stage split over several workgroups
per unit, the wider selector instances, several tiles per score wave)."""
import numpy as np
import pytest

from hierarchical_sparse_attention_block_amd import workloads as W
from tests import hsab_testlib as T

pytestmark = pytest.mark.gpu

N_DRAWS = 48


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    latent = rng.random() < 0.2
    if latent:
        G, Hkv, dk, dv, r = 32, 1, 576, 512, 32
    else:
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.integers(1, 4))
        dk = int(rng.choice([64, 128, 256]))
        dv = dk
        r = int(rng.choice([16, 32, 64] if dk >= 64 else [16, 32]))
    block = int(rng.choice([1, 4, 8, 16, 32]))
    max_ctx = int(rng.integers(64, 1500))
    nb_cap = -(-max_ctx // block)
    kb = int(rng.integers(1, min(nb_cap + 4, 8192 // block) + 1))
    kt = int(rng.integers(1, 400))
    agg = rng.choice(["max", "sum", "head"] if not latent else ["max", "sum"])
    forced = int(rng.integers(0, 3)) if kb >= 3 else 0
    sink = int(rng.integers(0, forced + 1))
    w = W.Workload(name=f"draw{i}", batch=int(rng.integers(1, 4)), n_q_heads=G * Hkv, n_kv_heads=Hkv, d_k=dk,
                   d_v=dv, v_alias_k=latent, block=block, r=r, k_blocks=kb, k_tokens=kt, ctx=max_ctx,
                   max_ctx=max_ctx, scaled_keys=bool(rng.random() < 0.5), label_mode="random",
                   n_planted=int(rng.integers(0, 3)), seed=int(rng.integers(1 << 30)),
                   meta_fp8=bool(rng.random() < 0.4 and dk % 32 == 0), agg_sum=agg == "sum",
                   sink_blocks=sink, local_blocks=forced - sink, per_head=agg == "head",
                   label_fp8=bool(rng.random() < 0.4))
    ctx = rng.integers(1, max_ctx + 1, size=w.batch).astype(np.int32)
    ctx[0] = max_ctx
    return w, ctx


def _draw_large(i):
    rng = np.random.default_rng(90000 + i)
    latent = rng.random() < 0.2
    if latent:
        G, Hkv, dk, dv, r = 32, 1, 576, 512, 32
    else:
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.integers(1, 3))
        dk = int(rng.choice([64, 128, 256]))
        dv = dk
        r = int(rng.choice([16, 32, 64]))
    block = int(rng.choice([8, 16, 32]))
    max_ctx = int(rng.integers(2000, 32768))
    nb_cap = -(-max_ctx // block)
    kb = int(rng.integers(1, min(nb_cap, 8192 // block, 2048) + 1))
    kt = int(rng.integers(1, 2048))
    agg = rng.choice(["max", "sum", "head"] if not latent else ["max", "sum"])
    forced = int(rng.integers(0, 3)) if kb >= 3 else 0
    sink = int(rng.integers(0, forced + 1))
    w = W.Workload(name=f"large{i}", batch=int(rng.integers(1, 3)), n_q_heads=G * Hkv, n_kv_heads=Hkv, d_k=dk,
                   d_v=dv, v_alias_k=latent, block=block, r=r, k_blocks=kb, k_tokens=kt, ctx=max_ctx,
                   max_ctx=max_ctx, scaled_keys=bool(rng.random() < 0.5), label_mode="random",
                   n_planted=int(rng.integers(0, 3)), seed=int(rng.integers(1 << 30)),
                   meta_fp8=bool(rng.random() < 0.4 and dk % 32 == 0), agg_sum=agg == "sum",
                   sink_blocks=sink, local_blocks=forced - sink, per_head=agg == "head",
                   label_fp8=bool(rng.random() < 0.4))
    ctx = rng.integers(1, max_ctx + 1, size=w.batch).astype(np.int32)
    ctx[0] = max_ctx
    return w, ctx


@pytest.mark.parametrize("i", range(N_DRAWS))
def test_random_config(i):
    _check_draw(*_draw(i), f"random config {i}")


@pytest.mark.parametrize("i", range(8))
def test_random_larger_config(i):
    _check_draw(*_draw_large(i), f"larger random config {i}")


def _check_draw(w, ctx, label):
    print(f"[{label}] {w} ctx={ctx.tolist()}", flush=True)
    h = T.host_inputs(w, ctx_len=ctx)
    dev = T.Device(w, h)
    dev.prefill_meta()
    dev.decode_step()
    r = dev.results()
    K, V = T.appended_cache(w, h)
    G = w.group
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            if w.per_head:
                for hh in range(G):
                    a = g * G + hh
                    T.oracle_unit_vs_gpu(w, h["q"], K, V, h["ctx"], h["label"], b, g, r["blk"][b, a],
                                         r["tok"][b, a], r["out"][b, a:a + 1], r["lse"][b, a:a + 1], head=hh)
            else:
                T.oracle_unit_vs_gpu(w, h["q"], K, V, h["ctx"], h["label"], b, g, r["blk"][b, g], r["tok"][b, g],
                                     r["out"][b, g * G:(g + 1) * G], r["lse"][b, g * G:(g + 1) * G])
