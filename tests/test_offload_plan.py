"""Host planner of the offload engine (hsab_offload_plan) against the
oracle's lagged schedule (AsyncTLS, gist.science/de explainer section 2.B;
gist.science/es explainer section 2.B).

The planner runs on the host only, so these tests need no GPU. A simulated
block cache follows every copy and every append and checks that each block
the attention reads at step t sits in the slot the slot table names, and
that no copy of step t lands in a slot step t reads.
"""
import numpy as np
import pytest
import torch

from oracle import hsab_oracle as O

H = pytest.importorskip("hierarchical_sparse_attention_block_amd.hsab")


def _dims(B, Hkv, kb, bs, max_ctx, d=64):
    return H.dims(B, Hkv * 4, Hkv, d, d, False, bs, 16, kb, 8 * bs, max_ctx, 0.125)


def _drift_sels(rng, ns, bs, kb, p_keep=0.8):
    """S_b sequence with temporal locality: most blocks survive a step."""
    sels, prev = [], None
    for n in ns:
        nb = -(-n // bs)
        k = min(kb, nb)
        if prev is None:
            cur = set(rng.choice(nb, size=k, replace=False).tolist())
        else:
            cur = {b for b in prev if rng.random() < p_keep and b < nb}
            if rng.random() < 0.5:
                cur.add(nb - 1)   # the tail block is often selected
            cur = set(sorted(cur)[-k:]) if len(cur) > k else cur
            pool = [b for b in range(nb) if b not in cur]
            rng.shuffle(pool)
            cur |= set(pool[: max(0, k - len(cur))])
        sels.append(np.array(sorted(cur), dtype=np.int64))
        prev = cur
    return sels


def _held(n, jp, bs):
    j = (n - 1) // bs
    t = [-1, -1]
    t[j & 1] = j
    if j - 1 >= jp:
        t[(j - 1) & 1] = j - 1
    return t


def _pad(rows, kb):
    out = np.full((len(rows), kb), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        out[i, : len(r)] = r
    return out


def _run(seed, B=2, Hkv=2, kb=6, bs=4, steps=24, n_slots=None):
    rng = np.random.default_rng(seed)
    max_ctx = 512
    d = _dims(B, Hkv, kb, bs, max_ctx)
    U, nb_cap = B * Hkv, d.nb_cap
    n_slots = n_slots or 2 * kb + 2
    n_norm = n_slots - 2
    n_pre = rng.integers(bs, 200, size=B)
    n_pre[0] = 4 * bs          # prefill ends on a block boundary
    unit_sels, unit_ns = [], []
    for u in range(U):
        ns = [int(n_pre[u // Hkv]) + 1 + t for t in range(steps)]
        unit_ns.append(ns)
        unit_sels.append(_drift_sels(rng, ns, bs, kb))
    expect = [O.offload_schedule(unit_sels[u], unit_ns[u], int(n_pre[u // Hkv]), bs) for u in range(U)]

    slot_map = torch.full((U * nb_cap,), -1, dtype=torch.int32)
    plan = torch.empty(U * kb * 3, dtype=torch.int32)
    content = [dict() for _ in range(U)]          # slot -> block it holds
    jp = [(int(n) - 1) // bs for n in n_pre]
    for u in range(U):                            # engine begin: last prefill block in its tail slot
        j = jp[u // Hkv]
        content[u][n_norm + (j & 1)] = j
        slot_map[u * nb_cap + j] = n_norm + (j & 1)
    blk_bytes = bs * (d.d_k + d.d_v) * 2

    def do_plan(resident, selected, tails):
        nbytes = H.offload_plan(d, n_slots, torch.from_numpy(resident.ravel().copy()),
                                torch.from_numpy(selected.ravel().copy()),
                                torch.tensor(np.array(tails, dtype=np.int32).ravel()), slot_map, plan)
        P = plan.view(U, kb, 3).numpy().copy()
        return nbytes, P

    def apply(P, reads):
        """Apply a plan's copies to the simulated cache; `reads` holds the
        slots the concurrent attention reads per unit."""
        copied = [[] for _ in range(U)]
        for u in range(U):
            used = []
            for blk, slot, cp in P[u]:
                if blk < 0:
                    continue
                used.append(slot)
                if cp:
                    assert 0 <= slot < n_norm, "copies go to block slots"
                    assert slot not in reads[u], "a copy overwrites a slot the step reads"
                    content[u][slot] = blk
                    copied[u].append(int(blk))
            assert len(set(used)) == len(used), "two selected blocks share a slot"
        return copied

    prev_sel = None
    for t in range(steps):
        n = [unit_ns[u][t] for u in range(U)]
        # append: the new token's block takes its tail slot
        for u in range(U):
            j = (n[u] - 1) // bs
            content[u][n_norm + (j & 1)] = j
        sel = _pad([unit_sels[u][t] for u in range(U)], kb)
        if t == 0:
            tails = [_held(n[u], jp[u // Hkv], bs) for u in range(U)]
            nbytes, P = do_plan(np.full((U, kb), -1, np.int32), sel, tails)
            cold = apply(P, [set() for _ in range(U)])
            for u in range(U):
                assert cold[u] == expect[u][0].tolist()
            assert nbytes == sum(len(c) for c in cold) * blk_bytes
            resident = sel
        else:
            resident = prev_sel
        # the attention of step t reads R(t) through the current slot table
        reads = []
        for u in range(U):
            rs = set()
            for blk in resident[u]:
                if blk < 0:
                    continue
                slot = int(slot_map[u * nb_cap + blk])
                assert content[u].get(slot) == blk, f"step {t} unit {u}: block {blk} not in slot {slot}"
                rs.add(slot)
            reads.append(rs)
        old_map = slot_map.clone()
        tails = [_held(n[u] + 1, jp[u // Hkv], bs) for u in range(U)]
        nbytes, P = do_plan(resident, sel, tails)
        delta = apply(P, reads)
        for u in range(U):
            assert delta[u] == expect[u][1][t].tolist(), f"step {t} unit {u}"
            for blk, slot, cp in P[u]:   # held-next blocks sit in their tail slot
                if blk >= 0 and blk in tails[u]:
                    assert slot == n_norm + (blk & 1) and cp == 0
            # a block whose slot the patch changes while step t reads it
            # must be whole in both slots
            for blk in resident[u]:
                if blk >= 0 and int(old_map[u * nb_cap + blk]) != int(slot_map[u * nb_cap + blk]):
                    assert content[u][int(slot_map[u * nb_cap + blk])] == blk
        assert nbytes == sum(len(x) for x in delta) * blk_bytes
        prev_sel = sel


@pytest.mark.parametrize("seed", range(6))
def test_plan_matches_schedule(seed):
    _run(seed)


def test_plan_block_size_one_and_wide_kb():
    _run(11, kb=12, bs=1, steps=30)


def test_plan_extra_slots():
    _run(12, n_slots=40)


def test_plan_rejects_too_few_slots():
    d = _dims(1, 1, 4, 4, 64)
    z = torch.full((4,), -1, dtype=torch.int32)
    st = H.raw_call("hsab_offload_plan", __import__("ctypes").byref(d), 9, None, None, None, None, None, None)
    assert st == H.HSAB_EINVAL
    with pytest.raises(H.HsabError):
        H.offload_plan(d, 9, z, z, torch.full((2,), -1, dtype=torch.int32),
                       torch.full((d.nb_cap,), -1, dtype=torch.int32), torch.empty(12, dtype=torch.int32))
