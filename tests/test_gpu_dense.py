"""Dense decode attention (full attention over every token, the reference
the sparse operator is measured against) on the GPU against the oracle's
attention over all tokens."""
import numpy as np
import pytest
import torch

import oracle as O
from hierarchical_sparse_attention_block_amd import workloads as W
from tests import hsab_testlib as T

pytestmark = pytest.mark.gpu


def _wl(**kw):
    base = dict(name="dense", batch=3, n_q_heads=8, n_kv_heads=2, d_k=128, d_v=128, v_alias_k=False,
                block=16, r=16, k_blocks=8, k_tokens=64, ctx=3072, max_ctx=3072, scaled_keys=True,
                label_mode="top_scale", n_planted=0, seed=31)
    base.update(kw)
    return W.Workload(**base)


def _run(w, ctx):
    from hierarchical_sparse_attention_block_amd import hsab as H
    print(f"[dense] {w} ctx={list(ctx)}", flush=True)
    h = T.host_inputs(w, ctx_len=np.asarray(ctx, np.int32) + 1)   # prefill holds ctx tokens
    d = T.dims_of(w)
    q, K = T.dev16(h["q"]), T.dev16(h["K"])
    V = None if w.v_alias_k else T.dev16(h["V"])
    ctx_d = torch.from_numpy(np.asarray(ctx, np.int32)).cuda()
    out = torch.full((w.batch * w.n_q_heads * w.d_v,), float("nan"), device="cuda")
    lse = torch.full((w.batch * w.n_q_heads,), float("nan"), device="cuda")
    ws = H.alloc_dense_workspace(d)
    H.dense_attend(d, q, K, V, ctx_d, out, lse, ws)
    torch.cuda.synchronize()
    out = out.cpu().numpy().reshape(w.batch, w.n_q_heads, w.d_v)
    lse = lse.cpu().numpy().reshape(w.batch, w.n_q_heads)
    G = w.group
    for b in range(w.batch):
        n = int(ctx[b])
        for g in range(w.n_kv_heads):
            qq = O.bf16_to_f64(h["q"][b, g * G:(g + 1) * G])
            Kf = O.bf16_to_f64(h["K"][b, g, :n])
            Vf = Kf[:, :w.d_v] if w.v_alias_k else O.bf16_to_f64(h["V"][b, g, :n])
            o, l = O.attend(qq, Kf, Vf, w.sm_scale)
            err = np.max(np.abs(o - out[b, g * G:(g + 1) * G]))
            assert err <= T.OUT_ATOL, f"unit ({b},{g}) n={n}: max-abs {err:.3g}"
            np.testing.assert_allclose(lse[b, g * G:(g + 1) * G], l, rtol=T.LSE_RTOL, atol=T.LSE_ATOL)
    return out, lse


def test_dense_ragged_chunks():
    """Contexts across the 1024-token chunk boundary, a single token, and
    a full-capacity row."""
    _run(_wl(), [3072, 1025, 1])


@pytest.mark.parametrize("G,d", [(8, 64), (1, 256), (2, 128)])
def test_dense_shapes(G, d):
    w = _wl(n_q_heads=2 * G, d_k=d, d_v=d, batch=2, ctx=2100, max_ctx=2100)
    _run(w, [2100, 1024])


def test_dense_equals_sparse_dense_limit():
    """With K_b covering every block and K_t every token, the sparse step's
    output is the dense attention over the same (appended) cache."""
    from hierarchical_sparse_attention_block_amd import hsab as H
    w = _wl(batch=2, ctx=640, max_ctx=640, k_blocks=40, k_tokens=640)
    ctx = np.array([640, 333], np.int32)
    h = T.host_inputs(w, ctx_len=ctx)
    dev = T.Device(w, h)
    dev.prefill_meta()
    dev.decode_step()
    r = dev.results()
    out = torch.empty(w.batch * w.n_q_heads * w.d_v, device="cuda")
    lse = torch.empty(w.batch * w.n_q_heads, device="cuda")
    H.dense_attend(dev.d, dev.q, dev.K, dev.V, dev.ctx, out, lse, H.alloc_dense_workspace(dev.d))
    torch.cuda.synchronize()
    out = out.cpu().numpy().reshape(r["out"].shape)
    lse = lse.cpu().numpy().reshape(r["lse"].shape)
    assert np.max(np.abs(out - r["out"])) <= 1e-5
    np.testing.assert_allclose(lse, r["lse"], rtol=1e-5)


@pytest.mark.parametrize("B,dk,dv,ctx", [(2, 576, 512, [2100, 33]), (1, 1024, 512, [1031]),
                                         (3, 128, 64, [1, 1056, 32])])
def test_dense_latent(B, dk, dv, ctx):
    """Absorbed latent layout (32 query heads on one latent key, values its
    first d_v dims): ragged rounds of 32 tokens and 1024-token chunks."""
    w = _wl(batch=B, n_q_heads=32, n_kv_heads=1, d_k=dk, d_v=dv, v_alias_k=True, block=32, r=32,
            k_blocks=4, k_tokens=64, ctx=max(ctx), max_ctx=max(ctx))
    _run(w, ctx)


def test_dense_rejects_unsupported():
    from hierarchical_sparse_attention_block_amd import hsab as H
    w = _wl(n_q_heads=12, n_kv_heads=4, d_k=96, d_v=96)
    assert H.dense_workspace_bytes(T.dims_of(w)) == 0
