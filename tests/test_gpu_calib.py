"""Label-channel calibration on the GPU against the oracle's
``calibrate_labels``: channel weights within their fp32 summation bound,
the label set under the near-tie rule, and a bit-identical rerun."""
import numpy as np
import pytest
import torch

import oracle as O
from hierarchical_sparse_attention_block_amd import workloads as W
from tests import hsab_testlib as T

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("Hq,Hkv,dk,r,S", [(32, 8, 128, 16, 300), (32, 1, 576, 32, 97), (4, 2, 1024, 128, 40),
                                          (2, 2, 64, 64, 5)])
def test_calibration_matches_oracle(Hq, Hkv, dk, r, S):
    from hierarchical_sparse_attention_block_amd import hsab as H
    w = W.Workload("cal", 1, Hq, Hkv, dk, dk, False, 16, r, 4, 16, 64, 64, True, "top_scale", 0, 41)
    d = T.dims_of(w)
    print(f"[calibrate] Hq={Hq} Hkv={Hkv} d_k={dk} r={r} samples={S}", flush=True)
    rng = np.random.default_rng(41 + dk)
    scales = np.stack([W.key_scales(w, g) for g in range(Hkv)])                  # [Hkv, dk]
    q = W.f32_to_bf16_bits(rng.standard_normal((S, Hq, dk)).astype(np.float32))
    k = W.f32_to_bf16_bits((rng.standard_normal((S, Hkv, dk)) * scales).astype(np.float32))
    imp = torch.full((Hkv * dk,), float("nan"), device="cuda")
    lab = torch.full((Hkv * r,), -7, dtype=torch.int32, device="cuda")
    H.calibrate_labels(d, T.dev16(q), T.dev16(k), S, imp, lab)
    torch.cuda.synchronize()
    imp1, lab1 = imp.cpu().numpy().reshape(Hkv, dk), lab.cpu().numpy().reshape(Hkv, r)
    G = Hq // Hkv
    for g in range(Hkv):
        qf = O.bf16_to_f64(q[:, g * G:(g + 1) * G])
        kf = O.bf16_to_f64(k[:, g])
        want = O.label_importance(qf, kf)
        # fp32 sum of S*G non-negative exact products: relative error <= n 2^-24
        np.testing.assert_allclose(imp1[g], want, rtol=S * G * 2.0 ** -24 + 1e-7, atol=1e-30)
        ref = O.calibrate_labels(qf, kf, r)
        got, tie = T.check_index_set(want, lab1[g], r, f"label set of KV head {g}")
        assert len(got) == len(ref) == min(r, dk)
        if not tie:   # a clear cut: the GPU's set is the oracle's, entry by entry
            np.testing.assert_array_equal(lab1[g], ref)
    # fixed summation order: a rerun is bit-identical
    H.calibrate_labels(d, T.dev16(q), T.dev16(k), S, imp, lab)
    torch.cuda.synchronize()
    assert np.array_equal(imp.cpu().numpy().reshape(Hkv, dk), imp1)
    assert np.array_equal(lab.cpu().numpy().reshape(Hkv, r), lab1)
