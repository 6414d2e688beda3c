"""Seeded sweep of small offload runs (AsyncTLS, gist.science/de explainer
section 2.B; gist.science/es explainer section 2.B: only the block delta
crosses the host link, copied beside the compute): group size, head dims
or the absorbed latent layout, block size, budgets, ragged prefill lengths
(some inside a first block, some on a block edge), the number of steps,
bf16 / fp8 metadata and label rows, all three copy modes, and steps either
synchronised one by one or enqueued back to back. Every unit at every step
is checked against the oracle's lagged schedule under the parity rules,
and the per-step delta bytes exactly."""
import numpy as np
import pytest

from hierarchical_sparse_attention_block_amd import workloads as W
from test_gpu_offload import _check_against_oracle, _run_offload

pytestmark = pytest.mark.gpu

N_DRAWS = 24


def _draw(i):
    rng = np.random.default_rng(7000 + i)
    latent = rng.random() < 0.2
    if latent:
        G, Hkv, dk, dv, r = 32, 1, 576, 512, 32
        block = int(rng.choice([16, 32]))
    else:
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.integers(1, 4))
        dk = int(rng.choice([64, 128, 256]))
        dv = dk
        r = int(rng.choice([16, 32]))
        block = int(rng.choice([4, 8, 16, 32]))
    steps = int(rng.integers(2, 11))
    max_ctx = int(rng.integers(max(4 * block, 64), 1500))
    nb_cap = -(-max_ctx // block)
    kb = int(rng.integers(1, min(16, nb_cap) + 1))
    w = W.Workload(name=f"offdraw{i}", batch=int(rng.integers(1, 4)), n_q_heads=G * Hkv, n_kv_heads=Hkv, d_k=dk,
                   d_v=dv, v_alias_k=latent, block=block, r=r, k_blocks=kb, k_tokens=int(rng.integers(1, 200)),
                   ctx=max_ctx, max_ctx=max_ctx, scaled_keys=bool(rng.random() < 0.5), label_mode="random",
                   n_planted=0, seed=int(rng.integers(1 << 30)),
                   meta_fp8=bool(rng.random() < 0.3 and dk % 32 == 0), label_fp8=bool(rng.random() < 0.3))
    prefill = rng.integers(1, max_ctx - steps + 1, size=w.batch)
    if w.batch > 1:
        prefill[1] = max(block, (prefill[1] // block) * block)   # a row whose prefill ends on a block edge
    copy_mode = int(rng.integers(0, 3))
    pipelined = bool(rng.random() < 0.5)
    return w, prefill.astype(np.int32), steps, copy_mode, pipelined


@pytest.mark.parametrize("i", range(N_DRAWS))
def test_offload_random_config(i):
    w, prefill, steps, copy_mode, pipelined = _draw(i)
    print(f"[offload draw {i}] {w} prefill={prefill.tolist()} steps={steps} copy_mode={copy_mode} "
          f"pipelined={pipelined}", flush=True)
    K, V, qs, res = _run_offload(w, prefill.tolist(), steps, copy_mode=copy_mode, pipelined=pipelined)
    _check_against_oracle(w, prefill, K, V, qs, res)
