"""Pins of the CPU oracle against facts fixed outside the oracle itself:
hand-worked examples, algebraic identities, the Quest bound property,
special cases that reduce to exact top-k or dense attention (checked against
torch's scaled_dot_product_attention), brute-force selection, and the
offload delta count. CPU only."""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from hierarchical_sparse_attention_block_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    vals = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        k, v = [x.strip() for x in line.split("=", 1)]
        rows = []
        for part in v.split(";"):
            rows.append([eval(t, {"exp": math.exp, "log": math.log}) for t in part.split()])
        vals[k] = rows if len(rows) > 1 else rows[0]
    return vals


def _bf16(x, rng_=None):
    """float64 values that are exactly representable in bf16."""
    return O.bf16_to_f64(W.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def _rand_unit(seed, G, d, n, dv=None, scale=1.0):
    r = np.random.default_rng(seed)
    q = _bf16(r.standard_normal((G, d)))
    K = _bf16(scale * r.standard_normal((n, d)))
    V = _bf16(r.standard_normal((n, dv or d)))
    return q, K, V


# ------------------------------------------------------------------ bf16 input
def test_bf16_to_f64_matches_torch_on_every_pattern():
    """The oracle's bf16 decoder against torch's own bfloat16 type on all
    65,536 bit patterns: every finite value, both zeros (with their signs)
    and both infinities equal torch's widening; NaN patterns decode to NaN."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):        # NaN patterns pass through the fp32 widening
        got = O.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127                      # exponent all ones, mantissa nonzero
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # landmarks of the format: 1.0, -2.0, the largest finite value, the
    # smallest normal and subnormal numbers
    for b, v in [(0x3F80, 1.0), (0xC000, -2.0), (0x7F7F, (2 - 2 ** -7) * 2.0 ** 127),
                 (0x0080, 2.0 ** -126), (0x0001, 2.0 ** -133), (0x7F80, np.inf)]:
        assert O.bf16_to_f64(np.array([b], np.uint16))[0] == v


# ------------------------------------------------------------ golden examples
def test_worked_example_every_stage():
    g = _read_golden("worked_example.txt")
    q = np.array([g["q0"], g["q1"]], dtype=np.float64)
    K = np.array([g[f"k{i}"] for i in range(5)], dtype=np.float64)
    V = np.array([g[f"v{i}"] for i in range(5)], dtype=np.float64)
    kmax, kmin = O.block_meta(K, 5, 2)
    np.testing.assert_array_equal(kmax, np.array(g["kmax"]))
    np.testing.assert_array_equal(kmin, np.array(g["kmin"]))
    ub = O.quest_bound(q, kmax, kmin)
    np.testing.assert_array_equal(ub, np.array([g["ub0"], g["ub1"]]))
    r = O.decode_unit(q, K, V, 5, 2, 2, np.array([0]), 2, 1.0)
    np.testing.assert_array_equal(r["blk_score"], g["blk_score"])
    np.testing.assert_array_equal(r["blk_idx"], g["blk_idx"])
    np.testing.assert_array_equal(r["cand"], g["cand"])
    np.testing.assert_array_equal(r["tok_score"], g["tok_score"])
    np.testing.assert_array_equal(r["tok_idx"], g["tok_idx"])
    np.testing.assert_allclose(r["out"], np.array([g["out0"], g["out1"]]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(r["lse"], [g["lse0"][0], g["lse1"][0]], rtol=1e-15)


def test_tie_example_lower_index_wins():
    g = _read_golden("tie_example.txt")
    q = np.array([[g["q0"]]], dtype=np.float64)
    K = np.array(g["k"], dtype=np.float64)[:, None]
    kmax, kmin = O.block_meta(K, 6, 1)
    s = O.block_scores(q, kmax, kmin)
    np.testing.assert_array_equal(O.topk_stable(s, 3), g["blk_idx"])
    np.testing.assert_array_equal(O.topk_stable(s, 4), g["blk_idx_k4"])
    np.testing.assert_array_equal(O.topk_stable(s, 5), g["blk_idx_k5"])


# ---------------------------------------------------------- metadata (step 2)
@pytest.mark.parametrize("n,bs", [(1, 16), (15, 16), (16, 16), (17, 16), (100, 16), (65, 32), (7, 1)])
def test_block_meta_brackets_every_key(n, bs):
    """Every valid key lies inside its block's [kmin, kmax], and both bounds
    are attained by some key of the block (closed form of channelwise max/min)."""
    _, K, _ = _rand_unit(n * 7 + bs, 1, 8, n)
    kmax, kmin = O.block_meta(K, n, bs)
    assert kmax.shape[0] == -(-n // bs)
    for t in range(n):
        j = t // bs
        assert np.all(kmin[j] <= K[t]) and np.all(K[t] <= kmax[j])
    for j in range(kmax.shape[0]):
        rows = K[j * bs: min(n, (j + 1) * bs)]
        assert np.all((rows == kmax[j]).any(axis=0)) and np.all((rows == kmin[j]).any(axis=0))


@pytest.mark.parametrize("bs", [1, 4, 16])
def test_incremental_meta_equals_bulk(bs):
    _, K, _ = _rand_unit(bs, 1, 16, 70)
    kmax, kmin = O.block_meta(K, 1, bs)
    for pos in range(1, 70):
        kmax, kmin = O.append_meta(kmax, kmin, K[pos], pos, bs)
        bmax, bmin = O.block_meta(K, pos + 1, bs)
        np.testing.assert_array_equal(kmax, bmax)
        np.testing.assert_array_equal(kmin, bmin)


# ------------------------------------------------------- block bound (step 3)
@pytest.mark.parametrize("seed", range(4))
def test_gemm_form_equals_elementwise_quest_bound(seed):
    q, K, _ = _rand_unit(seed, 5, 24, 203)
    kmax, kmin = O.block_meta(K, 203, 16)
    a = O.quest_bound(q, kmax, kmin)
    b = O.quest_bound_gemm(q, kmax, kmin)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n,bs,scale", [(200, 16, 1.0), (97, 8, 3.0), (33, 32, 1.0)])
def test_bound_dominates_true_block_max(n, bs, scale):
    """Quest property: every head's bound is >= the largest q.k in the block,
    so the group score is >= every head's true block maximum."""
    q, K, _ = _rand_unit(n + bs, 4, 32, n, scale=scale)
    kmax, kmin = O.block_meta(K, n, bs)
    ub = O.quest_bound(q, kmax, kmin)
    s = O.block_scores(q, kmax, kmin)
    for j in range(kmax.shape[0]):
        true = q @ K[j * bs: min(n, (j + 1) * bs)].T     # [G, tokens]
        assert np.all(ub[:, j] >= true.max(axis=1) - 1e-12)
        assert s[j] >= true.max() - 1e-12


def test_bound_is_tight_for_a_single_token_block():
    """With one token per block, kmax = kmin = k and the bound is exactly q.k."""
    q, K, _ = _rand_unit(9, 3, 16, 40)
    kmax, kmin = O.block_meta(K, 40, 1)
    np.testing.assert_allclose(O.quest_bound(q, kmax, kmin), q @ K.T, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("G", [1, 4])
def test_block1_reduces_to_exact_token_topk(G):
    """Block size 1: the block stage is an exact top-K over tokens of
    max_h q_h.k, which we rank with an independent full sort."""
    q, K, V = _rand_unit(G, G, 16, 300)
    r = O.decode_unit(q, K, V, 300, 1, 37, np.arange(4), 10, 0.25)
    true = (q @ K.T).max(axis=0)
    want = np.sort(np.lexsort((np.arange(300), -true))[:37])
    np.testing.assert_array_equal(r["blk_idx"], want)


# ------------------------------------------------------------- top-k (4, 5)
def test_topk_stable_brute_force_with_ties():
    """Exhaustive check on small integer scores with many ties: index i is
    kept iff fewer than k indices beat it, where j beats i when s_j > s_i or
    (s_j == s_i and j < i)."""
    rng = np.random.default_rng(0)
    for n in range(1, 9):
        for trial in range(30):
            s = rng.integers(-2, 3, size=n).astype(np.float64)
            for k in range(0, n + 3):
                got = O.topk_stable(s, k)
                want = [i for i in range(n)
                        if sum((s[j] > s[i]) or (s[j] == s[i] and j < i) for j in range(n)) < k]
                assert list(got) == want


def test_topk_matches_enumeration_of_subsets():
    """The kept set maximises the score sum over all subsets of size k and,
    among maximisers, is the lexicographically smallest index set."""
    s = np.array([3., 1., 3., 2., 2., 0., 3.])
    for k in range(len(s) + 1):
        best = max(itertools.combinations(range(len(s)), k),
                   key=lambda c: (sum(s[list(c)]), [-i for i in c]))
        assert tuple(O.topk_stable(s, k)) == best


# --------------------------------------------------------- token stage (5)
def test_label_score_is_exact_dot_when_keys_live_on_label_channels():
    """If keys are zero outside the label channels, the label score equals
    the exact max_h q_h.k (full-vector dot), whatever the channel order."""
    rng = np.random.default_rng(3)
    q, K, _ = _rand_unit(3, 4, 32, 50)
    ch = np.sort(rng.choice(32, size=6, replace=False))
    Km = np.zeros_like(K)
    Km[:, ch] = K[:, ch]
    np.testing.assert_allclose(O.label_scores(q, Km, ch), (q @ Km.T).max(axis=0), rtol=1e-13, atol=1e-13)


def test_full_label_set_equals_exact_scores():
    q, K, _ = _rand_unit(4, 4, 16, 64)
    np.testing.assert_allclose(O.label_scores(q, K, np.arange(16)), (q @ K.T).max(axis=0),
                               rtol=1e-13, atol=1e-13)


def test_candidates_cover_valid_tokens_of_kept_blocks():
    c = O.candidate_tokens(np.array([4, 0, 2]), 37, 8)
    np.testing.assert_array_equal(c, list(range(0, 8)) + list(range(16, 24)) + list(range(32, 37)))


# ------------------------------------------------------------ attention (6)
def _sdpa(q, K, V, scale):
    qt = torch.tensor(q)[None, :, None, :]                     # [1, G, 1, d]
    kt = torch.tensor(K)[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.tensor(V)[None, None].expand(1, q.shape[0], -1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    lse = torch.logsumexp(scale * (torch.tensor(q) @ torch.tensor(K).T), dim=1)
    return out[0, :, 0].numpy(), lse.numpy()


@pytest.mark.parametrize("n,bs,G,dk,dv", [(1, 16, 4, 16, 16), (37, 16, 4, 32, 32), (64, 8, 2, 24, 16), (70, 32, 8, 40, 32)])
def test_dense_limit_equals_sdpa(n, bs, G, dk, dv):
    """K_b >= number of blocks and K_t >= n keep every token: the operator is
    then dense attention, checked against torch's SDPA in fp64."""
    q, K, V = _rand_unit(n + G, G, dk, n, dv=dv)
    r = O.decode_unit(q, K, V, n, bs, 10 ** 6, np.arange(min(4, dk)), 10 ** 6, 1 / math.sqrt(dk))
    np.testing.assert_array_equal(r["tok_idx"], np.arange(n))
    out, lse = _sdpa(q, K, V, 1 / math.sqrt(dk))
    np.testing.assert_allclose(r["out"], out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse, rtol=1e-13)


def test_decode_all_maps_query_heads_to_kv_heads():
    """GQA grouping: query head h attends KV head h // G. With every token
    kept, decode_all equals SDPA with K/V repeated per group (an independent
    formulation of the same mapping)."""
    B, Hq, Hkv, d, n = 2, 6, 3, 16, 21
    rng = np.random.default_rng(11)
    qb = W.f32_to_bf16_bits(rng.standard_normal((B, Hq, d)).astype(np.float32))
    Kb = W.f32_to_bf16_bits(rng.standard_normal((B, Hkv, 32, d)).astype(np.float32))
    Vb = W.f32_to_bf16_bits(rng.standard_normal((B, Hkv, 32, d)).astype(np.float32))
    ctx = np.array([n, n - 5])
    res = O.decode_all(qb, Kb, Vb, ctx, Hkv, 4, 100, np.tile(np.arange(4), (Hkv, 1)), 100, 0.3)
    q = torch.tensor(O.bf16_to_f64(qb))
    K = torch.tensor(O.bf16_to_f64(Kb)).repeat_interleave(Hq // Hkv, dim=1)
    V = torch.tensor(O.bf16_to_f64(Vb)).repeat_interleave(Hq // Hkv, dim=1)
    for b in range(B):
        nb_ = int(ctx[b])
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[b][:, None], K[b, :, :nb_], V[b, :, :nb_], scale=0.3)[:, 0]
        got = np.concatenate([res[(b, g)]["out"] for g in range(Hkv)])
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)


def test_decode_all_aliased_values_equal_sdpa():
    """Absorbed latent layout: values are the first d_v dims of each key row
    (decode_all given the int d_v instead of a V array). With every token
    kept the result is SDPA with V = K[:, :d_v], per batch row, for every
    query head of the one latent KV head."""
    B, Hq, d, dv, n = 2, 4, 24, 16, 19
    rng = np.random.default_rng(12)
    qb = W.f32_to_bf16_bits(rng.standard_normal((B, Hq, d)).astype(np.float32))
    Kb = W.f32_to_bf16_bits(rng.standard_normal((B, 1, 32, d)).astype(np.float32))
    ctx = np.array([n, 7])
    res = O.decode_all(qb, Kb, dv, ctx, 1, 4, 100, np.arange(4)[None, :], 100, 0.2)
    q = torch.tensor(O.bf16_to_f64(qb))
    K = torch.tensor(O.bf16_to_f64(Kb))
    for b in range(B):
        m = int(ctx[b])
        k = K[b, 0, :m]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[b][:, None], k[None].expand(Hq, -1, -1), k[None, :, :dv].expand(Hq, -1, -1), scale=0.2)[:, 0]
        assert res[(b, 0)]["out"].shape == (Hq, dv)
        np.testing.assert_allclose(res[(b, 0)]["out"], ref.numpy(), rtol=0, atol=1e-12)


def test_lse_merges_disjoint_token_sets():
    """lse is the true log-partition: attention over A u B equals the
    lse-weighted merge of attention over A and over B."""
    q, K, V = _rand_unit(5, 3, 16, 40)
    oa, la = O.attend(q, K[:17], V[:17], 0.7)
    ob, lb = O.attend(q, K[17:], V[17:], 0.7)
    o, l = O.attend(q, K, V, 0.7)
    M = np.logaddexp(la, lb)
    np.testing.assert_allclose(M, l, rtol=1e-14)
    np.testing.assert_allclose(oa * np.exp(la - M)[:, None] + ob * np.exp(lb - M)[:, None], o, atol=1e-14)


def test_single_selected_token_returns_its_value():
    q, K, V = _rand_unit(6, 2, 8, 10)
    o, l = O.attend(q, K[3:4], V[3:4], 0.5)
    np.testing.assert_array_equal(o, np.repeat(V[3:4], 2, axis=0))
    np.testing.assert_allclose(l, 0.5 * (q @ K[3]), rtol=1e-15)


# ------------------------------------------------------------ clamps, edges
def test_budgets_clamp_to_what_exists():
    q, K, V = _rand_unit(8, 2, 16, 20)
    r = O.decode_unit(q, K, V, 20, 16, 5, np.arange(4), 999, 0.25)
    np.testing.assert_array_equal(r["blk_idx"], [0, 1])
    np.testing.assert_array_equal(r["tok_idx"], np.arange(20))


# -------------------------------------------------------------- planted keys
def test_planted_keys_survive_both_stages_tiny4k():
    w = W.WORKLOADS["tiny4k"]
    qb = W.queries(w)
    kb, vb = W.unit_kv(w, 0, 0, qb)
    knew, vnew = W.new_token(w)
    K = O.bf16_to_f64(np.concatenate([kb, knew[0, :, :]]))
    V = O.bf16_to_f64(np.concatenate([vb, vnew[0, :, :]]))
    q = O.bf16_to_f64(qb[0])
    lab = W.label_channels(w)[0]
    r = O.decode_unit(q, K, V, w.ctx, w.block, w.k_blocks, lab, w.k_tokens, w.sm_scale)
    pos, _ = W.planted_positions(w, 0, 0)
    assert set(pos // w.block) <= set(r["blk_idx"])
    assert set(pos) <= set(r["tok_idx"])
    # margin: every planted block bound exceeds every unplanted block score
    planted_blk = set(pos // w.block)
    others = [s for j, s in enumerate(r["blk_score"]) if j not in planted_blk]
    assert min(r["blk_score"][list(planted_blk)]) > 1.5 * max(others)


# ------------------------------------------------------------------ offload
def test_offload_delta_bytes_hand_sequence():
    """Selections {1,2,3} -> {2,3,4} -> {2,3,4} -> {0,4,5}: the transfers are
    1, 0 and 2 blocks (set differences). Bytes per block at block=16,
    d_k=d_v=128 in bf16: 16*256*2 = 8192."""
    assert list(O.offload_delta([1, 2, 3], [2, 3, 4])) == [4]
    assert list(O.offload_delta([2, 3, 4], [2, 3, 4])) == []
    assert list(O.offload_delta([2, 3, 4], [0, 4, 5])) == [0, 5]


def test_offload_schedule_hand_sequence_with_tail_rollover():
    """Hand-worked lagged schedule, block 4, prefill of 9 tokens (blocks
    0,1 full, block 2 holds token 8). Steps append tokens 9..12, so the
    contexts are 10, 11, 12, 13 tokens; block 3 opens at step 3.
      held(n): n=10..12 -> {2} (block 1 was never appended to); n=13 -> {3, 2}
      sel:  t0 {0,1,2}  t1 {1,2}  t2 {0,2}  t3 {1,3}
      cold = {0,1,2} - held(10) = {0,1}
      t0: R_slot = {0,1}; held(11) = {2}; delta = {0,1,2} - {0,1,2} = {}
      t1: R_slot = {0,1,2} - held(11) = {0,1}; held(12) = {2}; delta = {1,2} - {0,1,2} = {}
      t2: R_slot = {1,2} - {2} = {1}; held(13) = {2,3}; delta = {0,2} - {1,2,3} = {0}
      t3: R_slot = {0,2} - held(13) = {0}; held(14) = {2,3}; delta = {1,3} - {0,2,3} = {1}"""
    sels = [[0, 1, 2], [1, 2], [0, 2], [1, 3]]
    cold, deltas = O.offload_schedule(sels, [10, 11, 12, 13], 9, 4)
    assert list(cold) == [0, 1]
    assert [list(d) for d in deltas] == [[], [], [0], [1]]
    assert O.offload_held(13, 9, 4) == {2, 3}
    assert O.offload_held(10, 9, 4) == {2}


def test_offload_run_attends_over_previous_selection():
    rng = np.random.default_rng(1)
    G, d, bs, n0 = 2, 8, 4, 31
    K = _bf16(rng.standard_normal((n0 + 4, d)))
    V = _bf16(rng.standard_normal((n0 + 4, d)))
    qs = [_bf16(rng.standard_normal((G, d))) for _ in range(4)]
    steps = [(qs[t], K, V, n0 + 1 + t, 3, np.arange(2), 6, 0.3) for t in range(4)]
    res = O.offload_run(steps, bs, d, d)
    for t, r in enumerate(res):
        if t == 0:
            np.testing.assert_array_equal(r["resident"], r["sel"])
        else:
            np.testing.assert_array_equal(r["resident"], res[t - 1]["sel"])
        # the token stage ran on the resident set only
        assert set(np.asarray(r["tok_idx"]) // bs) <= set(r["resident"])
        assert r["delta_bytes"] == len(r["delta"]) * bs * 2 * d * 2
        # every transferred block was selected at this step
        assert set(r["delta"]) <= set(r["sel"])


def test_offload_run_bytes_on_forced_selections():
    """offload_run end to end on a unit whose block selections are forced:
    block j (block 4) holds keys A*e_j, so the bound of block j for a 0/1
    query is A where the query has a one at channel j and 0 elsewhere, and
    top-K_b with K_b = the query's weight keeps exactly those blocks. The
    selections are the hand-worked schedule above ({0,1,2}, {1,2}, {0,2},
    {1,3}; prefill 9, contexts 10..13), so the transfers are counted by
    hand: cold fill blocks {0,1}, then 0, 0, 1 and 1 blocks. A block is
    4 tokens of d_k + d_v = 8 + 8 bf16 values: 4 * 16 * 2 = 128 bytes
    (64 with values aliased to the keys)."""
    d, bs, A = 8, 4, 5.0
    K = np.zeros((16, d))
    for j in range(4):
        K[4 * j:4 * j + 4, j] = A
    V = _bf16(np.random.default_rng(3).standard_normal((16, d)))
    want = [[0, 1, 2], [1, 2], [0, 2], [1, 3]]
    steps = []
    for t, sel in enumerate(want):
        q = np.zeros((2, d))
        q[0, sel] = 1.0
        steps.append((q, K, V, 10 + t, len(sel), np.arange(4), 8, 0.5))
    for alias, per_block in [(False, 128), (True, 64)]:
        res = O.offload_run(steps, bs, d, d, v_alias=alias)
        assert [list(r["sel"]) for r in res] == want
        assert res[0]["cold_bytes"] == 2 * per_block
        assert [r["delta_bytes"] for r in res] == [0, 0, per_block, per_block]
        assert [r["cold_bytes"] for r in res[1:]] == [0, 0, 0]


# ------------------------------------------- quantised metadata (fp8 e4m3)
def test_e4m3_grid_matches_an_independent_decoder():
    """The grid built from the bit-field definition equals torch's
    float8_e4m3fn decode of the same 256 codes (NaN codes excluded)."""
    codes, vals = O.e4m3_grid()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().double().numpy()
    assert len(codes) == 254 and 0x7F not in codes and 0xFF not in codes
    assert np.all(np.isnan(ref[[0x7F, 0xFF]]))
    np.testing.assert_array_equal(vals, ref[codes])


def test_e4m3_landmarks_of_the_format():
    """Largest finite 448 (0x7e), smallest normal 2^-6 (0x08), smallest
    subnormal 2^-9 (0x01), one at 0x38 with a step of 1/8 above it."""
    codes, vals = O.e4m3_grid()
    v = dict(zip(codes.tolist(), vals.tolist()))
    assert v[0x7E] == 448.0 and vals.max() == 448.0 and vals.min() == -448.0
    assert v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9 and v[0x38] == 1.0 and v[0x39] == 1.125
    assert v[0x80 | 0x38] == -1.0


def test_e4m3_outward_rounding_brute_force():
    """round_up(x) is the smallest grid value >= x and round_down(x) the
    largest <= x (by a scan of the grid), saturating at +-448; grid values
    map to themselves; torch's round-to-nearest result lies between them."""
    _, vals = O.e4m3_grid()
    r = np.random.default_rng(3)
    x = np.concatenate([r.uniform(-500, 500, 3000), r.uniform(-0.05, 0.05, 2000),
                        r.standard_normal(2000) * 2.0 ** r.integers(-12, 9, 2000), vals])
    x = O.bf16_to_f64(W.f32_to_bf16_bits(x.astype(np.float32)))
    up, dn = O.e4m3_round(x, True), O.e4m3_round(x, False)
    for xi, u, d in zip(x, up, dn):
        above, below = vals[vals >= xi], vals[vals <= xi]
        assert u == (above.min() if above.size else 448.0)
        assert d == (below.max() if below.size else -448.0)
    on = np.isin(x, vals)
    np.testing.assert_array_equal(up[on], x[on])
    np.testing.assert_array_equal(dn[on], x[on])
    inr = np.abs(x) <= 448
    rne = torch.from_numpy(x[inr]).float().to(torch.float8_e4m3fn).double().numpy()
    assert np.all((dn[inr] <= rne) & (rne <= up[inr]))
    assert np.all((rne == dn[inr]) | (rne == up[inr]))


@pytest.mark.parametrize("n,bs,scale", [(200, 16, 1.0), (97, 8, 30.0), (64, 32, 0.01)])
def test_quantised_bound_dominates_exact_bound_and_true_max(n, bs, scale):
    """Outward-rounded metadata keeps the Quest property: its bound is >= the
    exact-metadata bound, which is >= the true block maximum of q.k."""
    q, K, _ = _rand_unit(n + 7 * bs, 4, 32, n, scale=scale)
    kmax, kmin = O.block_meta(K, n, bs)
    qmax, qmin = O.block_meta_e4m3(K, n, bs)
    assert np.all(qmax >= kmax) and np.all(qmin <= kmin)
    ub, ubq = O.quest_bound(q, kmax, kmin), O.quest_bound(q, qmax, qmin)
    assert np.all(ubq >= ub - 1e-12)
    for j in range(kmax.shape[0]):
        true = q @ K[j * bs: min(n, (j + 1) * bs)].T
        assert np.all(ubq[:, j] >= true.max(axis=1) - 1e-12)


def test_quantised_meta_is_exact_for_keys_on_the_grid():
    """Keys that are e4m3 values give the same metadata either way."""
    _, vals = O.e4m3_grid()
    r = np.random.default_rng(8)
    K = r.choice(vals[np.abs(vals) <= 64], size=(50, 16))
    for a, b in zip(O.block_meta(K, 50, 8), O.block_meta_e4m3(K, 50, 8)):
        np.testing.assert_array_equal(a, b)


# ------------------------------------ selection variants: forced blocks, sum
@pytest.mark.parametrize("scores,k,sink,local,want", [
    # worked by hand: block 0 and block 5 are forced, one slot left -> the best other (9 at block 2)
    ([5, 1, 9, 3, 7, 2], 3, 1, 1, [0, 2, 5]),
    ([5, 1, 9, 3, 7, 2], 2, 1, 1, [0, 5]),                 # no slot left beyond the forced ones
    ([5, 1, 9, 3, 7, 2], 6, 1, 1, [0, 1, 2, 3, 4, 5]),     # budget covers everything
    ([5, 1, 9, 3, 7, 2], 3, 2, 0, [0, 1, 2]),              # two sink blocks, then 9
    ([5, 1, 9, 3, 7, 2], 4, 0, 2, [0, 2, 4, 5]),           # blocks 4, 5 forced, then 9 (2) and 5 (0)
    ([3, 8], 2, 1, 1, [0, 1]),                             # the forced sets overlap the whole range
    ([1, 2, 3], 3, 2, 2, [0, 1, 2]),                       # sink and local windows overlap
    ([4, 4, 4, 4], 2, 0, 1, [0, 3]),                       # tie among the others: the lower index
])
def test_forced_blocks_hand_examples(scores, k, sink, local, want):
    np.testing.assert_array_equal(O.select_blocks(np.array(scores, float), k, sink, local), want)


def test_forced_blocks_brute_force():
    """The kept set holds every forced block, has min(K_b, nb) entries, and
    no dropped block beats a kept non-forced one (ties: lower index kept)."""
    r = np.random.default_rng(4)
    for _ in range(400):
        nb = int(r.integers(1, 12))
        s = r.integers(0, 5, nb).astype(float)      # many ties
        sink, local = int(r.integers(0, 4)), int(r.integers(0, 4))
        forced = set(range(min(sink, nb))) | set(range(max(0, nb - local), nb))
        k = int(r.integers(len(forced), nb + 3)) if len(forced) <= nb + 2 else len(forced)
        got = O.select_blocks(s, k, sink, local)
        assert forced <= set(got.tolist()) and len(got) == min(k, nb) and np.all(np.diff(got) > 0)
        kept = [j for j in got if j not in forced]
        dropped = [j for j in range(nb) if j not in set(got.tolist())]
        for a in kept:
            for b in dropped:
                assert s[a] > s[b] or (s[a] == s[b] and a < b)
    with pytest.raises(ValueError):
        O.select_blocks(np.zeros(8), 2, 2, 1)


def test_sum_aggregation_closed_forms():
    """One token per block: every head's bound is exact, so the summed group
    bound is (sum_h q_h).k; the summed label score over all channels is the
    same number; with one head, sum and max agree."""
    q, K, _ = _rand_unit(12, 4, 16, 30)
    kmax, kmin = O.block_meta(K, 30, 1)
    np.testing.assert_allclose(O.block_scores(q, kmax, kmin, "sum"), K @ q.sum(axis=0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.label_scores(q, K, np.arange(16), "sum"), K @ q.sum(axis=0), rtol=1e-12,
                               atol=1e-12)
    np.testing.assert_array_equal(O.block_scores(q[:1], kmax, kmin, "sum"), O.block_scores(q[:1], kmax, kmin))


def test_sum_aggregated_bound_dominates_summed_block_maxima():
    q, K, _ = _rand_unit(13, 4, 32, 120, scale=2.0)
    kmax, kmin = O.block_meta(K, 120, 16)
    s = O.block_scores(q, kmax, kmin, "sum")
    for j in range(kmax.shape[0]):
        true = (q @ K[j * 16: (j + 1) * 16].T).max(axis=1).sum()
        assert s[j] >= true - 1e-12


# ------------------------------------------------- label-channel calibration
def test_calibration_hand_example():
    """Two samples, one head, four channels: |q*k| per channel sums to
    [0.5+0, 4+1, 0+3, 1+1] = [0.5, 5, 3, 2] -> the two heaviest are 1 and 2."""
    q = np.array([[[1.0, -2.0, 0.0, 1.0]], [[0.0, 1.0, 3.0, -1.0]]])
    k = np.array([[0.5, 2.0, 7.0, 1.0], [4.0, -1.0, 1.0, 1.0]])
    np.testing.assert_array_equal(O.calibrate_labels(q, k, 2), [1, 2])
    np.testing.assert_array_equal(O.calibrate_labels(q, k, 3), [1, 2, 3])


def test_calibration_brute_force_and_symmetries():
    """The chosen set has the largest total importance among all r-subsets
    (enumerated); it is unchanged by scaling the samples and follows a
    permutation of the channels; r = d keeps every channel."""
    r_ = np.random.default_rng(6)
    for _ in range(30):
        d, G, S, r = 8, int(r_.integers(1, 4)), int(r_.integers(1, 6)), int(r_.integers(1, 8))
        q = r_.standard_normal((S, G, d)) * r_.uniform(0.1, 3, d)
        k = r_.standard_normal((S, d)) * r_.uniform(0.1, 3, d)
        imp = np.abs(q * k[:, None, :]).sum(axis=(0, 1))
        got = O.calibrate_labels(q, k, r)
        best = max(itertools.combinations(range(d), r), key=lambda c: imp[list(c)].sum())
        assert math.isclose(imp[got].sum(), imp[list(best)].sum(), rel_tol=1e-12)
        np.testing.assert_array_equal(O.calibrate_labels(3.5 * q, 0.25 * k, r), got)
        perm = r_.permutation(d)
        np.testing.assert_array_equal(np.sort(perm[O.calibrate_labels(q[:, :, perm], k[:, perm], r)]), got)
    q = r_.standard_normal((3, 2, 6))
    np.testing.assert_array_equal(O.calibrate_labels(q, r_.standard_normal((3, 6)), 6), np.arange(6))


def test_calibration_recovers_outlier_channels():
    """Keys with a few large-scale channels (the workloads' scaled keys):
    those channels dominate |q*k| and are the label set."""
    r_ = np.random.default_rng(7)
    d, r = 64, 8
    scale = np.full(d, 0.2)
    hot = r_.choice(d, r, replace=False)
    scale[hot] = 10.0
    q = r_.standard_normal((256, 4, d))
    k = r_.standard_normal((256, d)) * scale
    np.testing.assert_array_equal(O.calibrate_labels(q, k, r), np.sort(hot))


# ------------------------------------------------ per-query-head selection
def test_per_head_selection_hand_example():
    """Two heads that prefer different one-token blocks: with one block and
    one token per head, each head keeps and attends its own token, while the
    group maximum gives both heads the first one (hand-worked values)."""
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    K = np.array([[3.0, 0.0], [0.0, 3.0], [1.0, 1.0], [2.0, 2.0]])
    V = np.array([[1.0, 0.0], [0.0, 1.0], [5.0, 5.0], [7.0, 7.0]])
    r = O.decode_unit_heads(q, K, V, 4, 1, 1, np.array([0, 1]), 1, 0.5)
    np.testing.assert_array_equal(r["heads"][0]["blk_score"], [3, 0, 1, 2])
    np.testing.assert_array_equal(r["heads"][1]["blk_score"], [0, 3, 1, 2])
    assert [list(h["tok_idx"]) for h in r["heads"]] == [[0], [1]]
    np.testing.assert_array_equal(r["out"], [[1.0, 0.0], [0.0, 1.0]])
    np.testing.assert_array_equal(r["lse"], [1.5, 1.5])
    np.testing.assert_array_equal(r["union"], [0, 1])
    np.testing.assert_array_equal(r["mask"], [1, 2])
    g = O.decode_unit(q, K, V, 4, 1, 1, np.array([0, 1]), 1, 0.5)
    np.testing.assert_array_equal(g["tok_idx"], [0])
    np.testing.assert_array_equal(g["out"], [[1.0, 0.0], [1.0, 0.0]])


def test_per_head_single_head_equals_group_mode():
    q, K, V = _rand_unit(31, 1, 32, 90)
    a = O.decode_unit_heads(q, K, V, 90, 8, 4, np.arange(0, 32, 4), 12, 0.2)
    b = O.decode_unit(q, K, V, 90, 8, 4, np.arange(0, 32, 4), 12, 0.2)
    np.testing.assert_array_equal(a["heads"][0]["blk_idx"], b["blk_idx"])
    np.testing.assert_array_equal(a["union"], b["tok_idx"])
    np.testing.assert_array_equal(a["out"], b["out"])
    np.testing.assert_array_equal(a["mask"], np.ones(len(b["tok_idx"])))


@pytest.mark.parametrize("G,n,kt", [(2, 40, 5), (4, 64, 9), (8, 33, 33)])
def test_per_head_exact_limit_is_topk_of_each_heads_logits(G, n, kt):
    """One-token blocks make the block bound the exact q_h.k, and a label set
    of every channel makes the label score exact too: each head then keeps
    the K_t keys of largest q_h.k (torch.topk on the logits, no ties in
    continuous data) and attends over them (torch SDPA)."""
    d = 16
    q, K, V = _rand_unit(100 + G, G, d, n)
    r = O.decode_unit_heads(q, K, V, n, 1, n, np.arange(d), kt, 0.3)
    for h in range(G):
        want = np.sort(torch.topk(torch.tensor(q[h] @ K.T), min(kt, n)).indices.numpy())
        np.testing.assert_array_equal(r["heads"][h]["tok_idx"], want)
        out, lse = _sdpa(q[h:h + 1], K[want], V[want], 0.3)
        np.testing.assert_allclose(r["out"][h], out[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["lse"][h], lse[0], rtol=1e-13)


def test_token_union_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(50):
        G = int(rng.integers(1, 9))
        sets = [np.sort(rng.choice(60, size=int(rng.integers(0, 20)), replace=False)) for _ in range(G)]
        u, m = O.token_union(sets)
        assert list(u) == sorted(set().union(*[set(s.tolist()) for s in sets]))
        for x, bits in zip(u, m):
            assert all(((int(bits) >> h) & 1) == (int(x) in set(s.tolist())) for h, s in enumerate(sets))


def test_per_head_forced_blocks_apply_to_every_head():
    q, K, V = _rand_unit(77, 3, 16, 100)
    r = O.decode_unit_heads(q, K, V, 100, 10, 4, np.arange(4), 20, 0.25, sink=1, local=1)
    for h in r["heads"]:
        assert 0 in h["blk_idx"] and 9 in h["blk_idx"] and len(h["blk_idx"]) == 4


# ------------------------------------------------------ fp8 label rows
def test_e4m3_nearest_matches_torch_on_every_bf16_value():
    """Round-to-nearest-even onto e4m3 equals torch's float8_e4m3fn
    conversion for every finite bf16 value up to 464 in magnitude (the
    halfway point above 448, where torch stops rounding to the grid)."""
    bits = np.arange(65536, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= 464)]
    ours = O.e4m3_round_nearest(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_nearest_landmarks_and_saturation():
    got = O.e4m3_round_nearest(np.array([0.0, 448.0, 450.0, 464.0, 465.0, 1e6, -1e6, 2.0 ** -9, 2.0 ** -10,
                                         3 * 2.0 ** -10, 0.0625 + 0.00390625]))
    # 2^-9 is the smallest subnormal; 2^-10 is halfway to 0 (tie to even: 0);
    # 3*2^-10 is halfway between 2^-9 and 2^-8 (even mantissa: 2^-8);
    # 0.0625 + 2^-8 is halfway between 0.0625 (m=0) and 0.0703125 (m=1): 0.0625
    np.testing.assert_array_equal(got, [0.0, 448.0, 448.0, 448.0, 448.0, 448.0, -448.0, 2.0 ** -9, 0.0,
                                        2.0 ** -8, 0.0625])


def test_e4m3_nearest_error_within_half_spacing():
    _, vals = O.e4m3_grid()
    grid = np.unique(vals)
    x = np.random.default_rng(0).uniform(-448, 448, 20000)
    r = O.e4m3_round_nearest(x)
    assert np.all(np.isin(r, grid))
    i = np.searchsorted(grid, x)
    gap = grid[np.minimum(i, grid.size - 1)] - grid[np.maximum(i - 1, 0)]
    assert np.all(np.abs(r - x) <= gap / 2 + 1e-12)
    np.testing.assert_array_equal(O.e4m3_round_nearest(grid), grid)


def test_fp8_labels_change_only_the_token_stage():
    """Quantised label rows leave the block stage and the attention rows
    alone: the blocks equal the bf16 run's, and the tokens are the top-K_t
    of the label scores recomputed on rounded rows."""
    q, K, V = _rand_unit(55, 4, 32, 300)
    a = O.decode_unit(q, K, V, 300, 16, 6, np.arange(0, 32, 2), 20, 0.2)
    b = O.decode_unit(q, K, V, 300, 16, 6, np.arange(0, 32, 2), 20, 0.2, label_fp8=True)
    np.testing.assert_array_equal(a["blk_idx"], b["blk_idx"])
    want = O.label_scores(q, O.e4m3_round_nearest(K[b["cand"]]), np.arange(0, 32, 2))
    np.testing.assert_array_equal(b["tok_score"], want)
    np.testing.assert_array_equal(b["tok_idx"], b["cand"][O.topk_stable(want, 20)])
