"""Attention with 128-token splits: where 64-token splits would need more
than 1,024 workgroups (one resident round), the GQA attention of heads up
to 128 wide takes 128 list entries per workgroup (gist.science/es
explainer section 2.A item 2: the final attention over the kept tokens).
Shapes on both sides of that rule, with ragged contexts (some shorter than
K_t, so lists end in -1 padding), a K_t that leaves the last split
partial, every group size, both head widths, per-head selection (masked
union lists), and a wider head that keeps 64-token splits; every unit
against the oracle under the parity rules."""
import numpy as np
import pytest

from hierarchical_sparse_attention_block_amd import workloads as W
from tests import hsab_testlib as T
from test_gpu_random_configs import _check_draw

pytestmark = pytest.mark.gpu


def _wl(**kw):
    base = dict(name="long", batch=32, n_q_heads=16, n_kv_heads=4, d_k=128, d_v=128, v_alias_k=False,
                block=16, r=16, k_blocks=128, k_tokens=1000, ctx=3000, max_ctx=3000, scaled_keys=True,
                label_mode="random", n_planted=2, seed=77)
    base.update(kw)
    return W.Workload(**base)


def _ctx(w, seed):
    rng = np.random.default_rng(seed)
    ctx = rng.integers(200, w.max_ctx + 1, size=w.batch).astype(np.int32)
    ctx[0] = w.max_ctx
    ctx[1] = 300   # fewer candidates than K_t: the list ends in padding
    return ctx


@pytest.mark.parametrize("kw", [
    dict(),                                                                  # G = 4, d = 128, partial last split
    dict(n_q_heads=64, n_kv_heads=8, d_k=64, d_v=64, batch=16, k_blocks=64, k_tokens=1024, seed=78),  # G = 8, d = 64
    dict(n_q_heads=4, n_kv_heads=4, k_tokens=1024, seed=79),                # G = 1
    dict(n_q_heads=8, n_kv_heads=4, k_tokens=777, seed=80, meta_fp8=True),  # G = 2, fp8 metadata
    dict(batch=8, n_q_heads=32, n_kv_heads=8, k_tokens=512, per_head=True, seed=81),   # masked union lists
    dict(d_k=256, d_v=256, r=32, seed=82),                                  # wide heads: 64-token splits
])
def test_long_splits(kw):
    w = _wl(**kw)
    _check_draw(w, _ctx(w, w.seed), "long splits")
