"""CPU oracle for the AsyncTLS two-level sparse-attention decode operator.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this module. The product path
(the HIP library and its Python binding) never imports or calls it.

Plain, slow, fp64 NumPy. Every function works on one unit u = (batch b,
KV head g) and follows the method's steps in the order the pages give:

1. The KV cache of a unit is cut into fixed-size token blocks
   [AsyncTLS, gist.science/de explainer, section 2.A "Stufe 1";
   gist.science/es explainer, section 2.A item 1].
2. Each block is summarised by its channelwise key maximum and minimum
   [gist.science/de, section 2.A "Stufe 1": Max/Min der Keys].
3. Block importance is the Quest upper bound of q.k over the block,
   sum_c max(q_c*Kmax_c, q_c*Kmin_c) [gist.science/es, section 2.A item 1,
   "based on Quest"; Quest is in the "Builds on" list of the mlsanity index
   page]. The same bound written as the dense product q+ . Kmax + q- . Kmin
   (the GEMM form the pages introduce for shared-KV heads; gist.science/de
   section 2.A "Optimierung", gist.science/es section 2.A "Innovacion") is
   given by ``quest_bound_gemm``; the two are the same number up to rounding.
4. The top K_b blocks are kept [gist.science/es, section 2.A item 1].
5. Inside the kept blocks, tokens are scored on a few label channels of q
   and k (Double Sparsity) and the top K_t tokens are kept
   [gist.science/de, section 2.A "Stufe 2"; gist.science/es section 2.A
   item 2].
6. Exact softmax attention runs over the kept tokens [gist.science/es,
   section 2.A item 2, "final attention"].

Readings where the pages are silent (all fixed here, none printed there):
* query heads that share one KV head are combined by the MAX over the group,
  for both block and token scores; one selection per (batch, KV head);
* top-k ties go to the lower index, and results are returned ascending;
* the last, partial block is summarised over its valid tokens only; K_b and
  K_t clamp to what exists, unused output slots hold -1;
* label scores are the plain bf16-valued dot product on the label channels
  (no quantisation);
* attention logits are sm_scale * q.k; out is fp64 here (fp32 on the GPU);
  lse is the natural-log logsumexp of those logits.

Selection variants (``agg="sum"``, ``select_blocks`` with sink and local
blocks): the pages combine no query-head scores and force no tokens; their
related-work list names StreamingLLM (attention sinks) [mlsanity index
page, "Builds on"]. Readings taken here, both opt-in: a group score may be
the SUM of the heads' scores instead of the max (a query group's total
attention mass rather than its most demanding head), and the first
`sink` blocks and the last `local` blocks (the newest, holding the
appended token) may be kept unconditionally, the remaining K_b - forced
slots going to the best of the other blocks.

Per-query-head selection (``decode_unit_heads``): the pages score blocks
for the heads that share a KV head in one product and say nothing of
combining them; Quest, which the pages build on, selects per query head.
Reading taken here (opt-in): every query head of the group runs both
selection stages on its own scores, exactly as a group of one head, and
attends over its own tokens; the rows a KV head needs are then the union
of its heads' token sets.

Label-channel calibration (``calibrate_labels``): the fine stage scores
tokens on a few important channels chosen offline (Double Sparsity)
[gist.science/de, section 2.A "Stufe 2"; gist.science/es, section 2.A item
2]; the pages do not define "important". Reading taken here: channel c of
a KV head weighs sum |q_c * k_c| over sampled (query, key) pairs of that
head's group, and the r heaviest channels form the label set.

Quantised block metadata (``e4m3_*``, ``block_meta_e4m3``): the pages name
quantisation of the index data as a way to cut the indexing cost
[gist.science/de, section 2.A "Stufe 2"] and give no scheme. Reading taken
here: the block max row rounded up and the min row rounded down to the fp8
e4m3 grid (OCP "fn" variant: bias 7, 3 mantissa bits, subnormals, no
infinities, largest finite 448, saturating), so every block bound stays an
upper bound of the true block maximum. These functions are pinned to the
format's bit-field definition, to an independent fp8 decoder and to that
bound invariant; against the pages themselves the scheme is a reading
(parity unpinned: the pages print no quantised value).

Quantised label rows (``e4m3_round_nearest``, ``label_fp8``): Double
Sparsity keeps its label cache in a few bits, and the pages count
quantisation among the ways to cut the indexing cost [gist.science/de,
section 2.A "Stufe 2"]. Reading taken here (opt-in): label rows rounded to
the nearest e4m3 value (ties to the even mantissa, saturating at +-448);
the label score is an estimate, so no direction of rounding is needed.
Pinned to an independent fp8 converter on every bf16 value up to the
format's rounding limit; against the pages, parity unpinned.

Offload (``offload_*``): the fine stage of step t runs over the blocks
selected at step t-1 while step t's new blocks are fetched; only the set
difference of consecutive block selections is transferred
[gist.science/de, section 2.B; gist.science/es, section 2.B]. Reading: the
block being appended to (and the one completed just before it) stays on the
GPU in a tail slot and never crosses the host link.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f64", "n_blocks", "block_meta", "append_meta", "quest_bound",
    "quest_bound_gemm", "block_scores", "topk_stable", "candidate_tokens",
    "label_scores", "attend", "select_tokens_unit", "decode_unit", "select_blocks",
    "e4m3_grid", "e4m3_round", "e4m3_round_nearest", "block_meta_e4m3", "label_importance", "calibrate_labels",
    "decode_unit_heads", "token_union", "decode_all", "offload_delta", "offload_held", "offload_schedule", "offload_run",
]


# ---------------------------------------------------------------- bf16 input
def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ------------------------------------------------------------ step 1: blocks
def n_blocks(n: int, bs: int) -> int:
    """Number of blocks covering n tokens: block j holds [j*bs, min((j+1)*bs, n))."""
    return -(-n // bs)


# ---------------------------------------------------------- step 2: metadata
def block_meta(K: np.ndarray, n: int, bs: int):
    """Channelwise max and min of the keys of every block, over valid tokens.

    K: [>=n, d] float64 keys of one unit. Returns (kmax, kmin), each [nb, d]."""
    nb = n_blocks(n, bs)
    d = K.shape[1]
    kmax = np.empty((nb, d))
    kmin = np.empty((nb, d))
    for j in range(nb):
        rows = K[j * bs: min((j + 1) * bs, n)]
        kmax[j] = rows.max(axis=0)
        kmin[j] = rows.min(axis=0)
    return kmax, kmin


def append_meta(kmax: np.ndarray, kmin: np.ndarray, k: np.ndarray, pos: int, bs: int):
    """Metadata after appending key k at position pos (incremental update):
    a new block starts with k as both bounds, otherwise the tail block's
    bounds widen to include k. Returns new (kmax, kmin) arrays."""
    j = pos // bs
    kmax = kmax.copy()
    kmin = kmin.copy()
    if pos % bs == 0:
        if j != kmax.shape[0]:
            raise ValueError("a new block must be appended right after the last one")
        kmax = np.vstack([kmax, k[None, :]])
        kmin = np.vstack([kmin, k[None, :]])
    else:
        kmax[j] = np.maximum(kmax[j], k)
        kmin[j] = np.minimum(kmin[j], k)
    return kmax, kmin


# ------------------------------------------- quantised metadata (fp8 e4m3)
def e4m3_grid():
    """Every finite fp8 e4m3 ("fn") value by code: sign bit, exponent field
    e (4 bits, bias 7), mantissa m (3 bits); e = 0 is subnormal, m/8 * 2^-6;
    otherwise (1 + m/8) * 2^(e-7); codes 0x7f and 0xff are NaN.

    Returns (codes uint8 [254], values float64 [254])."""
    codes, vals = [], []
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        sgn, e, m = c >> 7, (c >> 3) & 0xF, c & 0x7
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        codes.append(c)
        vals.append(-v if sgn else v)
    return np.array(codes, np.uint8), np.array(vals, np.float64)


def e4m3_round(x, up: bool) -> np.ndarray:
    """Outward rounding to the e4m3 grid: up = the smallest grid value >= x,
    down = the largest grid value <= x; beyond the largest magnitude (448)
    the result saturates at +-448."""
    _, vals = e4m3_grid()
    grid = np.unique(vals)                          # sorted, +0 and -0 merged
    x = np.asarray(x, np.float64)
    if up:
        i = np.searchsorted(grid, x, side="left")   # first grid value >= x
        return grid[np.minimum(i, grid.size - 1)]
    i = np.searchsorted(grid, x, side="right") - 1  # last grid value <= x
    return grid[np.maximum(i, 0)]


def e4m3_round_nearest(x) -> np.ndarray:
    """Rounding to the nearest e4m3 value; a value halfway between two grid
    values goes to the one whose mantissa field is even; beyond the largest
    magnitude the nearest finite value is +-448 (saturation)."""
    codes, vals = e4m3_grid()
    even = {}
    for c, v in zip(codes, vals):
        even[float(v)] = even.get(float(v), False) or (int(c) & 1) == 0
    grid = np.unique(vals)
    ev = np.array([even[float(v)] for v in grid])
    x = np.asarray(x, np.float64)
    hi = np.minimum(np.searchsorted(grid, x, side="left"), grid.size - 1)   # first grid value >= x (or the top)
    lo = np.maximum(hi - 1, 0)
    gl, gh = grid[lo], grid[hi]
    dl, dh = np.abs(x - gl), np.abs(gh - x)
    pick_hi = (dh < dl) | ((dh == dl) & ev[hi] & ~ev[lo])
    out = np.where(pick_hi, gh, gl)
    return np.where(x >= gh, gh, np.where(x <= grid[0], grid[0], out))


def block_meta_e4m3(K: np.ndarray, n: int, bs: int):
    """Block metadata quantised outward to e4m3: (round_up(kmax),
    round_down(kmin)) of ``block_meta``."""
    kmax, kmin = block_meta(K, n, bs)
    return e4m3_round(kmax, True), e4m3_round(kmin, False)


# ----------------------------------------------------- step 3: block scoring
def quest_bound(q: np.ndarray, kmax: np.ndarray, kmin: np.ndarray) -> np.ndarray:
    """Quest upper bound, elementwise definition.

    q: [G, d], kmax/kmin: [nb, d]. UB[h, j] = sum_c max(q[h,c]*kmax[j,c], q[h,c]*kmin[j,c])."""
    G, nb = q.shape[0], kmax.shape[0]
    ub = np.empty((G, nb))
    for h in range(G):
        ub[h] = np.maximum(q[h] * kmax, q[h] * kmin).sum(axis=1)
    return ub


def quest_bound_gemm(q: np.ndarray, kmax: np.ndarray, kmin: np.ndarray) -> np.ndarray:
    """The same bound as one dense product: [q+, q-] @ [kmax; kmin]^T with
    q+ = max(q, 0) and q- = min(q, 0)."""
    qq = np.concatenate([np.maximum(q, 0.0), np.minimum(q, 0.0)], axis=1)   # [G, 2d]
    kk = np.concatenate([kmax, kmin], axis=1)                               # [nb, 2d]
    return qq @ kk.T


def block_scores(q: np.ndarray, kmax: np.ndarray, kmin: np.ndarray, agg: str = "max") -> np.ndarray:
    """Block score of a KV head shared by the query heads q [G, d]: the
    largest Quest bound over the group (agg="max"), or their sum
    (agg="sum", a selection variant)."""
    ub = quest_bound(q, kmax, kmin)
    return ub.sum(axis=0) if agg == "sum" else ub.max(axis=0)


# --------------------------------------------------------- steps 4, 5: top-k
def topk_stable(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the min(k, len) largest scores; on equal scores the lower
    index wins. Returned in ascending index order (int64)."""
    s = np.asarray(scores, dtype=np.float64)
    k = min(int(k), s.shape[0])
    order = np.argsort(-s, kind="stable")      # stable: equal keys keep index order
    return np.sort(order[:k])


def select_blocks(s_blk: np.ndarray, k_blocks: int, sink: int = 0, local: int = 0) -> np.ndarray:
    """Block stage with forced blocks: the first `sink` and the last `local`
    blocks are kept whatever their scores; the other K_b - (forced count)
    slots take the best remaining blocks (ties to the lower index).
    Ascending. Without forced blocks this is ``topk_stable``."""
    nb = len(s_blk)
    forced = sorted(set(range(min(sink, nb))) | set(range(max(0, nb - local), nb)))
    if len(forced) > k_blocks:
        raise ValueError("more forced blocks than the block budget")
    others = np.array([j for j in range(nb) if j not in set(forced)], np.int64)
    pick = others[topk_stable(np.asarray(s_blk)[others], k_blocks - len(forced))] if others.size else others
    return np.sort(np.concatenate([np.array(forced, np.int64), pick]))


def candidate_tokens(blk_idx: np.ndarray, n: int, bs: int) -> np.ndarray:
    """Valid token positions of the kept blocks, ascending."""
    toks = [np.arange(j * bs, min((j + 1) * bs, n)) for j in np.sort(np.asarray(blk_idx))]
    return np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)


def label_scores(q: np.ndarray, K_rows: np.ndarray, label_ch: np.ndarray, agg: str = "max") -> np.ndarray:
    """Approximate token scores on the label channels: for each key row,
    the largest over the group of sum_{c in label_ch} q[h,c]*k[c] (or the
    sum over the group with agg="sum")."""
    qc = q[:, label_ch]                  # [G, r]
    kc = K_rows[:, label_ch]             # [T, r]
    s = qc @ kc.T
    return s.sum(axis=0) if agg == "sum" else s.max(axis=0)


def label_importance(q_samples: np.ndarray, k_samples: np.ndarray) -> np.ndarray:
    """Channel importance of one KV head from sampled activations: for each
    channel c the sum over samples s and the group's query heads h of
    |q[s,h,c] * k[s,c]|. q_samples [S, G, d], k_samples [S, d] float64;
    returns [d]."""
    return np.abs(q_samples * k_samples[:, None, :]).sum(axis=(0, 1))


def calibrate_labels(q_samples: np.ndarray, k_samples: np.ndarray, r: int) -> np.ndarray:
    """Label channels of one KV head: the r channels of largest
    ``label_importance``, ties to the lower channel, ascending."""
    return topk_stable(label_importance(q_samples, k_samples), r)


# ------------------------------------------------------ step 6: attention
def attend(q: np.ndarray, K_sel: np.ndarray, V_sel: np.ndarray, sm_scale: float):
    """Exact softmax attention of each query head over the selected rows.

    q [G, d_k], K_sel [T, d_k], V_sel [T, d_v]. Returns (out [G, d_v], lse [G])
    with logits z = sm_scale * q.k and lse = log(sum exp z)."""
    G = q.shape[0]
    if K_sel.shape[0] == 0:
        return np.zeros((G, V_sel.shape[1])), np.full(G, -np.inf)
    z = sm_scale * (q @ K_sel.T)                         # [G, T]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ V_sel) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


# -------------------------------------------------------- whole-unit pipeline
def select_tokens_unit(q, K, n, bs, blk_idx, label_ch, k_tokens, agg="max"):
    """Token stage given a block set: candidates, label scores, top-K_t.
    Returns (tok_idx ascending positions, cand positions, label scores of cand)."""
    cand = candidate_tokens(blk_idx, n, bs)
    s_tok = label_scores(q, K[cand], label_ch, agg)
    keep = topk_stable(s_tok, k_tokens)
    return cand[keep], cand, s_tok


def decode_unit(q, K, V, n, bs, k_blocks, label_ch, k_tokens, sm_scale, meta=None, meta_fp8=False,
                agg="max", sink=0, local=0, label_fp8=False):
    """One decode step of one unit over its first n tokens (the appended
    token included). q [G, d_k] float64; K [>=n, d_k], V [>=n, d_v] float64.
    meta_fp8: block metadata quantised outward to e4m3 (``block_meta_e4m3``);
    label_fp8: label rows rounded to the nearest e4m3 value
    (``e4m3_round_nearest``) before the label scores;
    agg, sink, local: the selection variants (group sum, forced blocks).

    Returns a dict with the intermediate results of every stage."""
    if meta is None:
        meta = block_meta_e4m3(K, n, bs) if meta_fp8 else block_meta(K, n, bs)
    kmax, kmin = meta
    s_blk = block_scores(q, kmax, kmin, agg)
    blk = select_blocks(s_blk, k_blocks, sink, local)
    Klab = e4m3_round_nearest(K) if label_fp8 else K
    tok, cand, s_tok = select_tokens_unit(q, Klab, n, bs, blk, label_ch, k_tokens, agg)
    out, lse = attend(q, K[tok], V[tok], sm_scale)
    return {"blk_score": s_blk, "blk_idx": blk, "cand": cand, "tok_score": s_tok,
            "tok_idx": tok, "out": out, "lse": lse, "kmax": kmax, "kmin": kmin}


def decode_unit_heads(q, K, V, n, bs, k_blocks, label_ch, k_tokens, sm_scale, meta=None, meta_fp8=False,
                      sink=0, local=0, label_fp8=False):
    """Per-query-head selection (a selection variant): query head h of the
    group runs ``decode_unit`` on its own query as a group of one, so its
    block and token scores are its own bounds and label scores. Returns
    {"heads": [decode_unit result per head], "out" [G, d_v], "lse" [G],
    "union": the ascending union of the heads' token sets, "mask": for each
    union entry the bit set of the heads that selected it}."""
    if meta is None:
        meta = block_meta_e4m3(K, n, bs) if meta_fp8 else block_meta(K, n, bs)
    heads = [decode_unit(q[h:h + 1], K, V, n, bs, k_blocks, label_ch, k_tokens, sm_scale, meta=meta,
                         agg="max", sink=sink, local=local, label_fp8=label_fp8) for h in range(q.shape[0])]
    union, mask = token_union([r["tok_idx"] for r in heads])
    return {"heads": heads, "out": np.concatenate([r["out"] for r in heads]),
            "lse": np.concatenate([r["lse"] for r in heads]), "union": union, "mask": mask}


def token_union(token_sets):
    """Ascending union of the heads' token sets and, per union entry, the
    bit mask of the heads (bit h for set h) that hold it."""
    union = np.unique(np.concatenate([np.asarray(s, np.int64) for s in token_sets])) if token_sets else \
        np.zeros(0, np.int64)
    mask = np.zeros(union.shape[0], np.int64)
    for h, s in enumerate(token_sets):
        mask |= np.isin(union, np.asarray(s)).astype(np.int64) << h
    return union, mask


def decode_all(q_bits, K_bits, V_bits, ctx_len, n_kv_heads, bs, k_blocks, label_ch,
               k_tokens, sm_scale, units=None, meta_fp8=False):
    """Decode step over all (or the listed) units of a batch.

    q_bits [B, Hq, d_k]; K_bits [B, Hkv, cap, d_k]; V_bits [B, Hkv, cap, d_v],
    or the int d_v when values are the first d_v key dims (absorbed MLA);
    ctx_len [B]; label_ch [Hkv, r]. Query head h reads KV head h // G.
    Returns {(b, g): decode_unit result}."""
    B, Hq, _ = q_bits.shape
    G = Hq // n_kv_heads
    res = {}
    todo = units if units is not None else [(b, g) for b in range(B) for g in range(n_kv_heads)]
    for b, g in todo:
        n = int(ctx_len[b])
        q = bf16_to_f64(q_bits[b, g * G:(g + 1) * G])
        K = bf16_to_f64(K_bits[b, g, :n])
        if isinstance(V_bits, (int, np.integer)):
            V = K[:, : int(V_bits)]
        else:
            V = bf16_to_f64(V_bits[b, g, :n])
        res[(b, g)] = decode_unit(q, K, V, n, bs, k_blocks, np.asarray(label_ch[g]),
                                  k_tokens, sm_scale, meta_fp8=meta_fp8)
    return res


# ------------------------------------------------------------------ offload
def offload_delta(prev_blocks, cur_blocks) -> np.ndarray:
    """Blocks that must cross the host link at a step: selected now, not
    resident from the previous step (set difference, ascending)."""
    return np.setdiff1d(np.asarray(cur_blocks), np.asarray(prev_blocks))


def offload_held(n: int, n_prefill: int, bs: int) -> set:
    """Blocks kept on the GPU outside the selection when the context holds n
    tokens: the block being appended to, and the block before it if that
    one was itself appended to during the run (two tail slots). The first
    such block is the one holding the last prefill token."""
    jp = (n_prefill - 1) // bs if n_prefill > 0 else 0
    j = (n - 1) // bs
    return {j} | ({j - 1} if j - 1 >= jp else set())


def offload_schedule(sels, ns, n_prefill, bs):
    """Transfer schedule of the lagged offload engine from the block
    selections alone. sels[t] = S_b(t) (selected at step t from the context
    of ns[t] tokens); step t attends over R(t) = S_b(t-1) (R(0) = S_b(0),
    filled synchronously before step 0). After the step-t selection the
    blocks of S_b(t) that are neither resident in a block slot nor held in
    a tail slot at step t+1 are copied:
        delta(t) = S_b(t) - (R_slot(t) | held(t+1)),
        R_slot(t) = R(t) - held(t)   (t >= 1),  R_slot(0) = S_b(0) - held(0).
    Returns (cold blocks, [delta(t)] per step)."""
    cold = set(sels[0]) - offload_held(ns[0], n_prefill, bs)
    out = []
    for t, sel in enumerate(sels):
        if t == 0:
            r_slot = cold
        else:
            r_slot = set(sels[t - 1]) - offload_held(ns[t], n_prefill, bs)
        held_next = offload_held(ns[t] + 1, n_prefill, bs)
        out.append(np.array(sorted(set(sel) - (r_slot | held_next)), dtype=np.int64))
    return np.array(sorted(cold), dtype=np.int64), out


def offload_run(steps, bs, d_k, d_v, v_alias=False):
    """Lagged offload schedule over a sequence of decode steps of one unit.

    ``steps`` is a list of (q [G,d_k], K [>=n,d_k], V [>=n,d_v], n, k_blocks,
    label_ch, k_tokens, sm_scale), with n growing by one per step. Step t
    selects S_b(t) from its own query, but its token stage and attention run
    over the resident set R(t) = S_b(t-1) (R(0) = S_b(0): the cold start is
    a synchronous fill). Transfers follow offload_schedule. Bytes per block
    = bs * (d_k + d_v) * 2 (bf16; d_k only when values alias keys).
    Returns a list of per-step dicts."""
    row_bytes = (d_k if v_alias else d_k + d_v) * 2
    sels, ns, res = [], [], []
    prev = None
    for t, (q, K, V, n, k_blocks, label_ch, k_tokens, sm_scale) in enumerate(steps):
        kmax, kmin = block_meta(K, n, bs)
        cur = topk_stable(block_scores(q, kmax, kmin), k_blocks)
        resident = cur if prev is None else prev
        tok, _, _ = select_tokens_unit(q, K, n, bs, resident, label_ch, k_tokens)
        o, lse = attend(q, K[tok], V[tok], sm_scale)
        res.append({"sel": cur, "resident": resident, "tok_idx": tok, "out": o, "lse": lse, "n": n})
        sels.append(cur)
        ns.append(n)
        prev = cur
    cold, deltas = offload_schedule(sels, ns, steps[0][3] - 1, bs)
    for t, r in enumerate(res):
        r["delta"] = deltas[t]
        r["delta_bytes"] = int(len(deltas[t])) * bs * row_bytes
        r["cold"] = cold if t == 0 else None
        r["cold_bytes"] = int(len(cold)) * bs * row_bytes if t == 0 else 0
    return res
