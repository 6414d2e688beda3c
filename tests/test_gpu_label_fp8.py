"""Label rows in fp8 e4m3 (HSAB_LABEL_FP8) on the GPU against the oracle:
the rounding of every finite bf16 value, the rows the prefill build and the
step's append write, decode steps (16- and 32-channel label steps, GQA and
latent layouts, with fp8 metadata and per-head selection) and an offload
run, all under the parity rules with the oracle's label scores computed on
the rounded rows."""
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
    base = dict(name="lab8", batch=2, n_q_heads=8, n_kv_heads=2, d_k=128, d_v=128, v_alias_k=False,
                block=16, r=16, k_blocks=16, k_tokens=64, ctx=1000, max_ctx=1024, scaled_keys=True,
                label_mode="top_scale", n_planted=4, seed=53, label_fp8=True)
    base.update(kw)
    return W.Workload(**base)


def _label_values(dev):
    w = dev.w
    v = dev.klabel.cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return v.reshape(w.batch, w.n_kv_heads, w.max_ctx, w.r)


def test_label_rounding_of_every_bf16_value():
    """The label channels of 8192 one-token rows hold every finite bf16
    pattern (saturation past 448, subnormals, zeros of both signs)."""
    w = _wl(batch=1, n_q_heads=1, n_kv_heads=1, d_k=32, d_v=32, block=16, r=16, k_blocks=8, k_tokens=8,
            ctx=8192, max_ctx=8192, n_planted=0, label_mode="random")
    bits = np.arange(65536, dtype=np.uint32)
    pat = bits[np.isfinite(O.bf16_to_f64(bits.astype(np.uint16)))].astype(np.uint16)
    h = T.host_inputs(w)
    lab = h["label"][0]
    K = np.zeros((1, 1, 8192, 32), np.uint16)
    flat = np.zeros(8192 * 16, np.uint16)
    flat[: pat.size] = pat
    K[0, 0][:, lab] = flat.reshape(8192, 16)
    h["K"] = K
    dev = T.Device(w, h)
    dev.ctx_prefill = torch.full((1,), 8192, dtype=torch.int32, device="cuda")
    say(f"[fp8 labels] {pat.size} bf16 values")
    dev.prefill_meta()
    torch.cuda.synchronize()
    got = _label_values(dev)[0, 0]
    np.testing.assert_array_equal(got, O.e4m3_round_nearest(O.bf16_to_f64(K[0, 0][:, lab])))


@pytest.mark.parametrize("kw", [dict(), dict(d_k=64, d_v=64, block=8, r=32),
                                dict(n_q_heads=32, n_kv_heads=1, d_k=576, d_v=512, v_alias_k=True, block=32,
                                     r=32, k_blocks=8, k_tokens=64, n_planted=0)])
def test_label_rows_of_build_and_append(kw):
    w = _wl(**kw)
    ctx = np.array([1000, 333], np.int32)
    h = T.host_inputs(w, ctx_len=ctx)
    dev = T.Device(w, h)
    dev.prefill_meta()
    dev.decode_step()
    torch.cuda.synchronize()
    got = _label_values(dev)
    K, _ = T.appended_cache(w, h)
    for b in range(w.batch):
        n = int(ctx[b])
        for g in range(w.n_kv_heads):
            want = O.e4m3_round_nearest(O.bf16_to_f64(K[b, g, :n][:, h["label"][g]]))
            np.testing.assert_array_equal(got[b, g, :n], want, err_msg=f"unit ({b},{g})")


def _decode(w):
    ctx = np.array([w.ctx, max(2, (w.ctx * 5) // 7)], np.int32)[: w.batch]
    say(f"[fp8 labels decode_step] {w}")
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


@pytest.mark.parametrize("kw", [dict(), dict(r=32), dict(r=64, d_k=256, d_v=256, block=8, k_blocks=40),
                                dict(n_q_heads=32, n_kv_heads=1, d_k=576, d_v=512, v_alias_k=True, block=32,
                                     r=32, k_blocks=8, k_tokens=100, n_planted=0),
                                dict(meta_fp8=True, agg_sum=True, sink_blocks=1, local_blocks=1),
                                dict(per_head=True)])
def test_decode_with_fp8_labels(kw):
    _decode(_wl(**kw))


def test_offload_with_fp8_labels():
    from tests.test_gpu_offload import _run_offload, _check_against_oracle
    w = W.WORKLOADS["tiny4k"].replace(name="offload_lab8", batch=2, n_q_heads=8, n_kv_heads=2, k_blocks=8,
                                      k_tokens=64, ctx=1024, max_ctx=1024, scaled_keys=True, n_planted=0,
                                      seed=26, label_fp8=True)
    prefill = [300, 511]
    K, V, qs, res = _run_offload(w, prefill, steps=8, copy_mode=0)
    _check_against_oracle(w, np.array(prefill), K, V, qs, res)
