"""The opt-in variants at the full 48k GQA size, in the launch configuration
the benchmark times for each: e4m3 block metadata and label rows
(quantised index data, gist.science/de explainer section 2.A "Stufe 2"),
the group score summed over the query heads with one sink and two local
blocks always kept, and per-query-head selection. Every unit is checked
for structure; sampled units of every batch row and KV head are checked
against the oracle under the parity rules."""
import dataclasses
import sys

import numpy as np
import pytest

from hierarchical_sparse_attention_block_amd import workloads as W
from tests import hsab_testlib as T

pytestmark = pytest.mark.gpu

# one unit of every batch row and of every KV head, plus one more
SAMPLED = [(b, b) for b in range(8)] + [(3, 5)]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _decode(w):
    say(f"[full-size variant] {w}")
    h = T.host_inputs(w)
    dev = T.Device(w, h)
    dev.prefill_meta()
    dev.decode_step()
    return h, dev.results()


def _structure(w, lists_blk, lists_tok):
    """Ascending, in range, tokens inside their kept blocks, -1 padding only
    at the end."""
    nb = -(-w.ctx // w.block)
    for blk, tok in zip(lists_blk, lists_tok):
        kb = blk[blk >= 0]
        kt = tok[tok >= 0]
        assert np.all(blk[len(kb):] == -1) and np.all(tok[len(kt):] == -1)
        assert np.all(np.diff(kb) > 0) and np.all(np.diff(kt) > 0)
        assert kb.size and kb[-1] < nb and kt.size and kt[-1] < w.ctx
        assert set((kt // w.block).tolist()) <= set(kb.tolist())


def _oracle_units(w, h, r, units, head=None):
    K, V = T.appended_cache(w, h)
    G = w.group
    stats = []
    for b, g in units:
        say(f"  oracle check of unit ({b},{g})" + ("" if head is None else f" head {head}"))
        if head is None:
            a, rows = g, slice(g * G, (g + 1) * G)
        else:
            a, rows = g * G + head, slice(g * G + head, g * G + head + 1)
        stats.append(T.oracle_unit_vs_gpu(w, h["q"], K, V, h["ctx"], h["label"], b, g, r["blk"][b, a],
                                          r["tok"][b, a], r["out"][b, rows], r["lse"][b, rows], head=head))
    return stats


def test_gqa48k_fp8_metadata_and_labels_full_size():
    w = dataclasses.replace(W.WORKLOADS["gqa48k"], meta_fp8=True, label_fp8=True)
    h, r = _decode(w)
    _structure(w, r["blk"].reshape(-1, w.k_blocks), r["tok"].reshape(-1, w.k_tokens))
    assert np.all(np.isfinite(r["out"])) and np.all(np.isfinite(r["lse"]))
    say("gqa48k fp8 sampled", _oracle_units(w, h, r, SAMPLED))


def test_gqa48k_summed_group_scores_with_forced_blocks_full_size():
    w = dataclasses.replace(W.WORKLOADS["gqa48k"], agg_sum=True, sink_blocks=1, local_blocks=2)
    h, r = _decode(w)
    _structure(w, r["blk"].reshape(-1, w.k_blocks), r["tok"].reshape(-1, w.k_tokens))
    nb = -(-w.ctx // w.block)
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            assert {0, nb - 2, nb - 1} <= set(r["blk"][b, g].tolist()), f"forced blocks missing in ({b},{g})"
    assert np.all(np.isfinite(r["out"])) and np.all(np.isfinite(r["lse"]))
    say("gqa48k sum+forced sampled", _oracle_units(w, h, r, SAMPLED))


def test_gqa48k_per_head_selection_full_size():
    w = dataclasses.replace(W.WORKLOADS["gqa48k"], per_head=True)
    h, r = _decode(w)
    G = w.group
    _structure(w, r["blk"].reshape(-1, w.k_blocks), r["tok"].reshape(-1, w.k_tokens))
    assert np.all(np.isfinite(r["out"])) and np.all(np.isfinite(r["lse"]))
    # the heads of a group select different token sets somewhere
    differ = sum(len({tuple(r["tok"][b, g * G + hh]) for hh in range(G)}) > 1
                 for b in range(w.batch) for g in range(w.n_kv_heads))
    assert differ > 0
    st = []
    for i, (b, g) in enumerate(SAMPLED[:4]):
        st += _oracle_units(w, h, r, [(b, g)], head=i % G)
    say("gqa48k per-head sampled", st)


def test_gqa96k_fp8_metadata_full_size():
    """The 96k layer with e4m3 metadata (the benchmark's fp8 leg at 96k):
    6,144 blocks and 4,096 candidates per unit; one unit of every batch row
    and every KV head against the oracle."""
    w = dataclasses.replace(W.WORKLOADS["gqa96k"], meta_fp8=True)
    h, r = _decode(w)
    _structure(w, r["blk"].reshape(-1, w.k_blocks), r["tok"].reshape(-1, w.k_tokens))
    assert np.all(np.isfinite(r["out"])) and np.all(np.isfinite(r["lse"]))
    say("gqa96k fp8 sampled", _oracle_units(w, h, r, [(b, b % 8) for b in range(16)]))


def test_mla64k_fp8_metadata_full_size():
    """The latent layer with e4m3 metadata (split-row block score widening
    e4m3 rows), all eight units against the oracle."""
    w = dataclasses.replace(W.WORKLOADS["mla64k"], meta_fp8=True)
    h, r = _decode(w)
    _structure(w, r["blk"].reshape(-1, w.k_blocks), r["tok"].reshape(-1, w.k_tokens))
    assert np.all(np.isfinite(r["out"])) and np.all(np.isfinite(r["lse"]))
    say("mla64k fp8 all units", _oracle_units(w, h, r, [(b, 0) for b in range(w.batch)]))
