"""The allocation-free decode step (hsab_decode_step_noalloc, for callers
that cannot allocate device memory) against hsab_decode_step on the same
inputs: two calls in a row on the library's static scratch, the second on
a smaller layer, each bit-identical to the step with a caller workspace
(the same kernels run on the same inputs); and a shape whose workspace
exceeds the scratch refused before any launch."""
import numpy as np
import pytest
import torch

from hierarchical_sparse_attention_block_amd import workloads as W
from tests import hsab_testlib as T

pytestmark = pytest.mark.gpu


def _wl(**kw):
    base = dict(name="noalloc", batch=4, n_q_heads=16, n_kv_heads=4, d_k=128, d_v=128, v_alias_k=False,
                block=16, r=16, k_blocks=32, k_tokens=256, ctx=6000, max_ctx=6144, scaled_keys=True,
                label_mode="top_scale", n_planted=4, seed=31)
    base.update(kw)
    return W.Workload(**base)


def _both(w, ctx):
    from hierarchical_sparse_attention_block_amd import hsab as H
    print(f"[noalloc] {w.name} B={w.batch} heads={w.n_q_heads}/{w.n_kv_heads} d_k={w.d_k} ctx={ctx.tolist()} "
          f"workspace {H.workspace_bytes(T.dims_of(w))} B of {H.SCRATCH_BYTES}", flush=True)
    h = T.host_inputs(w, ctx_len=ctx)
    ref, got = T.Device(w, h), T.Device(w, h)
    ref.prefill_meta()
    got.prefill_meta()
    ref.decode_step()
    H.decode_step_noalloc(got.d, got.q, got.k_new, got.v_new, got.K, got.V, got.meta, got.klabel, got.label,
                          got.ctx, got.blk, got.tok, got.out, got.lse)
    a, b = ref.results(), got.results()
    for k in ("blk", "tok", "out", "lse"):
        assert np.array_equal(a[k], b[k]), f"{w.name}: {k} differs from hsab_decode_step"
    assert torch.equal(ref.meta, got.meta) and torch.equal(ref.K, got.K), "appended cache differs"
    return a


def test_noalloc_matches_decode_step_twice_then_refuses_oversize():
    from hierarchical_sparse_attention_block_amd import hsab as H
    a = _both(_wl(), np.array([6000, 4099, 5000, 17], np.int32))
    assert np.all(np.isfinite(a["out"]))
    # a smaller layer on the same scratch right after (its counters and
    # partials must not carry over from the first call)
    _both(_wl(name="noalloc_small", batch=2, n_q_heads=8, n_kv_heads=2, ctx=1500, max_ctx=1536, k_blocks=12,
              k_tokens=100, seed=32), np.array([1500, 333], np.int32))
    # the absorbed latent layout on the same scratch
    _both(_wl(name="noalloc_latent", batch=2, n_q_heads=32, n_kv_heads=1, d_k=576, d_v=512, v_alias_k=True,
              block=32, r=32, k_blocks=16, k_tokens=128, ctx=2048, max_ctx=2048, n_planted=0, seed=33),
          np.array([2048, 1111], np.int32))
    # per-head selection at 96k needs ~40 MiB of workspace: refused up front
    big = W.WORKLOADS["gqa96k"].replace(per_head=True)
    d = T.dims_of(big)
    assert H.workspace_bytes(d) > H.SCRATCH_BYTES
    z16 = torch.zeros(1, dtype=torch.int16, device="cuda")
    z32 = torch.zeros(1, dtype=torch.int32, device="cuda")
    zf = torch.zeros(1, device="cuda")
    p = lambda t: H.ctypes.c_void_p(t.data_ptr())
    rc = H.raw_call("hsab_decode_step_noalloc", H.ctypes.byref(d), p(z16), p(z16), p(z16), p(z16), p(z16), p(z16),
                    p(z16), p(z32), p(z32), p(z32), p(z32), p(zf), p(zf), None)
    assert rc == H.HSAB_ESCRATCH
    torch.cuda.synchronize()
