"""Seeded synthetic inputs for the two-level sparse decode operator.

This module is shared by the HIP path (tests, bench, smoke) and by the CPU
oracle's tests. It holds none of the operator's arithmetic: it only draws
random numbers, rounds them to bf16 bit patterns and places them in the
layouts the library documents.

Workloads (sizes follow the decode configurations the operator is measured
on; the pages evaluate Qwen3-8B (GQA) and GLM-4.7-Flash (MLA) at 48k-96k
context, see the AsyncTLS abstract and the German explainer, section 4):

* ``tiny4k``  - B=1, 4 query heads on 1 KV head, d=128, n=4096, block 16,
  K_b=16, r=16 (seeded random channel set), K_t=128; q, k, v ~ N(0,1) and
  8 planted keys.
* ``gqa48k``  - B=8, 32/8 heads, d=128, n=49152, block 16, K_b=128, r=16,
  K_t=512; keys carry per-(KV head, channel) log-uniform scales in [0.1, 10]
  (outlier channels), label set = the r largest scales, 64 planted keys per
  (batch, KV head).
* ``gqa96k``  - as gqa48k with B=16, n=98304, K_b=256, K_t=1024.
* ``mha48k``  - as gqa48k with one query head per KV head: B=2, 32/32
  heads (64 units and the same metadata bytes as gqa48k).
* ``mla64k``  - B=8, 32 query heads sharing one 576-dim latent key
  (512 latent + 64 rope), values = first 512 key dims, n=65536, block 32,
  K_b=128, r=32, K_t=1024, scaled keys as above, no planted keys.
* ``offload96k`` - the offload run: B=4, 32/8 heads, d=128, per-row prefill
  lengths uniform in 8k-96k, 16 decode steps whose queries drift as
  q_t = sqrt(d) * normalize(q_{t-1} + 0.1 N(0,1)); layer settings as gqa48k
  (block 16, K_b=128, r=16, K_t=512, scaled keys), no planted keys.

Random streams are keyed by ``SeedSequence([seed, stream, ...])`` so each
(batch, KV head) unit can be regenerated on its own; this lets a test
rebuild one unit of a large workload on the CPU without the rest.

Planted keys (reading of "keys set to 3*q/|q| so they must be selected"):
a planted key is ``3 * knorm * q_h / |q_h|`` with ``knorm = sqrt(sum_c s_c^2)``
the typical key norm (sqrt(d) when all scales are 1). The literal unit-norm
reading gives a q.k of only ~3 sigma of the random q.k spread, which cannot
guarantee selection; the scaled reading keeps the planted tokens far above
every random block bound.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# stream ids for SeedSequence keys; fixed order, never reused
_S_Q, _S_K, _S_V, _S_SCALE, _S_LABEL, _S_PLANT, _S_NEW, _S_DRIFT, _S_CTX = range(9)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    d_k: int
    d_v: int
    v_alias_k: bool      # values are the first d_v dims of the key row (absorbed MLA)
    block: int
    r: int
    k_blocks: int
    k_tokens: int
    ctx: int             # tokens after this step's append (the new token sits at ctx-1)
    max_ctx: int         # cache capacity per (batch, KV head)
    scaled_keys: bool    # per-(KV head, channel) log-uniform key scales
    label_mode: str      # "random" (seeded channel set) or "top_scale"
    n_planted: int       # planted keys per (batch, KV head)
    seed: int
    meta_fp8: bool = False   # block metadata as outward-rounded fp8 e4m3 instead of bf16
    agg_sum: bool = False    # group scores summed over the query heads (selection variant)
    sink_blocks: int = 0     # always-kept first blocks (selection variant)
    local_blocks: int = 0    # always-kept last blocks (selection variant)
    per_head: bool = False   # every query head selects its own blocks and tokens (selection variant)
    label_fp8: bool = False  # label rows rounded to the nearest fp8 e4m3 value instead of bf16

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_k)

    @property
    def units(self) -> int:
        return self.batch * self.n_kv_heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny4k": Workload("tiny4k", 1, 4, 1, 128, 128, False, 16, 16, 16, 128,
                       4096, 4096, False, "random", 8, 1),
    "gqa48k": Workload("gqa48k", 8, 32, 8, 128, 128, False, 16, 16, 128, 512,
                       49152, 49152, True, "top_scale", 64, 2),
    "gqa96k": Workload("gqa96k", 16, 32, 8, 128, 128, False, 16, 16, 256, 1024,
                       98304, 98304, True, "top_scale", 64, 3),
    "mha48k": Workload("mha48k", 2, 32, 32, 128, 128, False, 16, 16, 128, 512,
                       49152, 49152, True, "top_scale", 64, 6),
    "mla64k": Workload("mla64k", 8, 32, 1, 576, 512, True, 32, 32, 128, 1024,
                       65536, 65536, True, "top_scale", 0, 4),
    # multi-step offload run; ctx is the capacity, per-row prefill lengths
    # come from offload_prefill
    "offload96k": Workload("offload96k", 4, 32, 8, 128, 128, False, 16, 16, 128, 512,
                           98304, 98304, True, "top_scale", 0, 5),
}

OFFLOAD_STEPS = 16
OFFLOAD_CTX_RANGE = (8192, 98304)


def offload_prefill(w: Workload, steps: int = OFFLOAD_STEPS) -> np.ndarray:
    """Prefill length of each batch row of a multi-step offload run, drawn
    uniformly from [8192, 98304 - steps] so every row has room for the run."""
    lo, hi = OFFLOAD_CTX_RANGE
    hi = min(hi, w.max_ctx) - steps
    return rng(w.seed, _S_CTX).integers(lo, hi + 1, size=w.batch).astype(np.int32)


def rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16. Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def key_scales(w: Workload, g: int) -> np.ndarray:
    """Per-channel key scale of KV head g: 1 everywhere, or log-uniform in [0.1, 10]."""
    if not w.scaled_keys:
        return np.ones(w.d_k, dtype=np.float32)
    u = rng(w.seed, _S_SCALE, g).uniform(math.log(0.1), math.log(10.0), w.d_k)
    return np.exp(u).astype(np.float32)


def label_channels(w: Workload) -> np.ndarray:
    """[Hkv, r] int32, ascending: the label channel set of each KV head.

    ``random``: r distinct channels drawn from the seed (shared by all KV heads).
    ``top_scale``: the r channels with the largest key scale of that head.
    """
    out = np.empty((w.n_kv_heads, w.r), dtype=np.int32)
    for g in range(w.n_kv_heads):
        if w.label_mode == "random":
            ch = rng(w.seed, _S_LABEL).choice(w.d_k, size=w.r, replace=False)
        else:
            s = key_scales(w, g)
            ch = np.argsort(-s, kind="stable")[: w.r]
        out[g] = np.sort(ch)
    return out


def queries(w: Workload) -> np.ndarray:
    """[B, Hq, d_k] bf16 bits, N(0,1)."""
    z = rng(w.seed, _S_Q).standard_normal((w.batch, w.n_q_heads, w.d_k), dtype=np.float32)
    return f32_to_bf16_bits(z)


def planted_positions(w: Workload, b: int, g: int) -> tuple[np.ndarray, np.ndarray]:
    """Positions of the planted keys of unit (b, g) and the query head (within
    the group) each one targets. Each planted key sits in its own full block of
    the prefill region [0, ctx-1), at a uniform offset inside that block."""
    if w.n_planted == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    n_full = (w.ctx - 1) // w.block
    if w.n_planted > n_full:
        raise ValueError("more planted keys than full blocks")
    r_ = rng(w.seed, _S_PLANT, b, g)
    blocks = np.sort(r_.choice(n_full, size=w.n_planted, replace=False))
    offs = r_.integers(0, w.block, size=w.n_planted)
    heads = np.arange(w.n_planted) % w.group
    return blocks * w.block + offs, heads


def _unit_keys_f32(w: Workload, b: int, g: int, n: int, q_bits: np.ndarray) -> np.ndarray:
    z = rng(w.seed, _S_K, b, g).standard_normal((n, w.d_k), dtype=np.float32)
    z *= key_scales(w, g)[None, :]
    pos, heads = planted_positions(w, b, g)
    if len(pos):
        s = key_scales(w, g).astype(np.float64)
        knorm = math.sqrt(float(np.sum(s * s)))
        qg = bf16_bits_to_f32(q_bits[b, g * w.group:(g + 1) * w.group]).astype(np.float64)
        for p, h in zip(pos, heads):
            if p < n:
                qh = qg[h]
                z[p] = (3.0 * knorm * qh / np.linalg.norm(qh)).astype(np.float32)
    return z


def unit_kv(w: Workload, b: int, g: int, q_bits: np.ndarray, n: int | None = None):
    """Prefill K (and V unless aliased) of unit (b, g): the first ``n`` rows
    (default ctx-1, i.e. everything before this step's appended token).
    Returns (K [n, d_k] bf16 bits, V [n, d_v] bf16 bits or None)."""
    n = w.ctx - 1 if n is None else n
    kb = f32_to_bf16_bits(_unit_keys_f32(w, b, g, n, q_bits))
    if w.v_alias_k:
        return kb, None
    v = rng(w.seed, _S_V, b, g).standard_normal((n, w.d_v), dtype=np.float32)
    return kb, f32_to_bf16_bits(v)


def new_token(w: Workload, step: int = 0):
    """The appended (k_new [B, Hkv, d_k], v_new [B, Hkv, d_v]) of decode step
    ``step``: scaled N(0,1) keys and N(0,1) values, bf16 bits."""
    r_ = rng(w.seed, _S_NEW, step)
    k = r_.standard_normal((w.batch, w.n_kv_heads, w.d_k), dtype=np.float32)
    for g in range(w.n_kv_heads):
        k[:, g, :] *= key_scales(w, g)[None, :]
    v = r_.standard_normal((w.batch, w.n_kv_heads, w.d_v), dtype=np.float32)
    return f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def full_cache(w: Workload, q_bits: np.ndarray, threads: int = 8, max_ctx: int | None = None):
    """Dense cache arrays for all units, prefilled with ctx-1 tokens:
    K [B, Hkv, max_ctx, d_k] and V [B, Hkv, max_ctx, d_v] (V is None when
    aliased), bf16 bits, rows >= ctx-1 zero."""
    cap = w.max_ctx if max_ctx is None else max_ctx
    K = np.zeros((w.batch, w.n_kv_heads, cap, w.d_k), dtype=np.uint16)
    V = None if w.v_alias_k else np.zeros((w.batch, w.n_kv_heads, cap, w.d_v), dtype=np.uint16)

    def fill(u):
        b, g = divmod(u, w.n_kv_heads)
        kb, vb = unit_kv(w, b, g, q_bits)
        K[b, g, : w.ctx - 1] = kb
        if V is not None:
            V[b, g, : w.ctx - 1] = vb

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(fill, range(w.units)))
    return K, V


def drift_queries(q_prev_f32: np.ndarray, w: Workload, step: int, noise: float = 0.1) -> np.ndarray:
    """Query drift for multi-step runs: q_t = sqrt(d) * normalize(q_{t-1} + noise*N(0,1)),
    per head; returns float32 (caller rounds to bf16)."""
    e = rng(w.seed, _S_DRIFT, step).standard_normal(q_prev_f32.shape, dtype=np.float32)
    x = q_prev_f32.astype(np.float64) + noise * e
    x *= math.sqrt(w.d_k) / np.linalg.norm(x, axis=-1, keepdims=True)
    return x.astype(np.float32)
