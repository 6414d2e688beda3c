"""Python binding of libhsab.so: argument marshalling only.

Each function takes torch tensors that live on the GPU, checks that every
buffer has the dtype, contiguity and size the C ABI documents (the library
itself only sees raw pointers), and forwards the pointers. All computation
happens in the HIP kernels. There is no fallback: if the shared library is
missing or cannot be loaded, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhsab.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m hierarchical_sparse_attention_block_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

HSAB_OK, HSAB_EINVAL, HSAB_EHIP, HSAB_EUNSUPPORTED, HSAB_ESCRATCH = 0, -1, -2, -3, -4
SCRATCH_BYTES = 16 << 20   # HSAB_SCRATCH_BYTES: the static workspace of decode_step_noalloc
COPY_KERNEL, COPY_DMA, COPY_KERNEL_GPU_PLAN = 0, 1, 2   # HSAB_OFFLOAD_COPY_*
EXPORTS = ("hsab_workspace_bytes", "hsab_status_string", "hsab_last_hip_error", "hsab_build_meta",
           "hsab_score_blocks", "hsab_select_blocks", "hsab_select_tokens", "hsab_sparse_attend",
           "hsab_decode_step", "hsab_decode_step_noalloc", "hsab_offload_append", "hsab_offload_plan", "hsab_offload_copy", "hsab_offload_create",
           "hsab_offload_destroy", "hsab_offload_begin", "hsab_offload_step", "hsab_offload_timing",
           "hsab_offload_set_timing", "hsab_offload_selection", "hsab_offload_step_selection", "hsab_offload_step_delta",
           "hsab_dense_workspace_bytes", "hsab_dense_attend",
           "hsab_calibrate_labels")


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("v_alias_k", ctypes.c_int32),
                ("block", ctypes.c_int32), ("r", ctypes.c_int32), ("k_blocks", ctypes.c_int32),
                ("k_tokens", ctypes.c_int32), ("max_ctx", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("meta_format", ctypes.c_int32), ("group_agg", ctypes.c_int32), ("sink_blocks", ctypes.c_int32),
                ("local_blocks", ctypes.c_int32), ("label_format", ctypes.c_int32)]

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def nb_cap(self):
        return -(-self.max_ctx // self.block)

    def __repr__(self):
        return "Dims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


META_BF16, META_FP8 = 0, 1   # block metadata formats (HSAB_META_BF16 / HSAB_META_FP8)
AGG_MAX, AGG_SUM = 0, 1      # group score combination (HSAB_AGG_MAX / HSAB_AGG_SUM)
AGG_HEAD = 2                 # per-query-head selection (HSAB_AGG_HEAD)
LABEL_BF16, LABEL_FP8 = 0, 1  # label row formats (HSAB_LABEL_BF16 / HSAB_LABEL_FP8)


def dims(batch, n_q_heads, n_kv_heads, d_k, d_v, v_alias_k, block, r, k_blocks, k_tokens, max_ctx,
         sm_scale, meta_format=META_BF16, group_agg=AGG_MAX, sink_blocks=0, local_blocks=0,
         label_format=LABEL_BF16) -> Dims:
    return Dims(batch, n_q_heads, n_kv_heads, d_k, d_v, int(bool(v_alias_k)), block, r, k_blocks,
                k_tokens, max_ctx, float(sm_scale), int(meta_format), int(group_agg), int(sink_blocks),
                int(local_blocks), int(label_format))


_vp, _sz, _i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
_D = ctypes.POINTER(Dims)
_lib.hsab_workspace_bytes.argtypes = [_D]
_lib.hsab_workspace_bytes.restype = _sz
_lib.hsab_status_string.argtypes = [ctypes.c_int]
_lib.hsab_status_string.restype = ctypes.c_char_p
_lib.hsab_last_hip_error.argtypes = []
_lib.hsab_last_hip_error.restype = ctypes.c_int
_lib.hsab_build_meta.argtypes = [_D, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.hsab_score_blocks.argtypes = [_D, _vp, _vp, _vp, _vp, _vp]
_lib.hsab_select_blocks.argtypes = [_D, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.hsab_select_tokens.argtypes = [_D, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.hsab_sparse_attend.argtypes = [_D, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp]
_lib.hsab_decode_step.argtypes = [_D, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _sz, _vp]
_lib.hsab_decode_step_noalloc.argtypes = [_D, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                          _vp, _vp]
_lib.hsab_offload_append.argtypes = [_D, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.hsab_offload_plan.argtypes = [_D, _i32, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.hsab_offload_copy.argtypes = [_D, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp]


class OffloadStats(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int64), ("delta_bytes", ctypes.c_int64), ("cold_bytes", ctypes.c_int64),
                ("delta_blocks", ctypes.c_int32), ("n_copies", ctypes.c_int32),
                ("host_wait_ms", ctypes.c_float), ("host_plan_ms", ctypes.c_float)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib.hsab_offload_create.argtypes = [_D, _i32, _i32, ctypes.POINTER(_vp)]
_lib.hsab_calibrate_labels.argtypes = [_D, _vp, _vp, _i32, _vp, _vp, _vp]
_lib.hsab_dense_workspace_bytes.argtypes = [_D]
_lib.hsab_dense_attend.argtypes = [_D, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.hsab_offload_destroy.argtypes = [_vp]
_lib.hsab_offload_begin.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp]
_lib.hsab_offload_step.argtypes = [_vp] * 16 + [_sz, _vp, _vp, ctypes.POINTER(OffloadStats)]
_lib.hsab_offload_timing.argtypes = [_vp, ctypes.c_int64, _vp]
_lib.hsab_offload_set_timing.argtypes = [_vp, ctypes.c_int32]
_lib.hsab_offload_selection.argtypes = [_vp, _vp]
_lib.hsab_offload_step_selection.argtypes = [_vp, ctypes.c_int64, _vp]
_lib.hsab_offload_step_delta.argtypes = [_vp, ctypes.c_int64, _vp, _vp]
for _f in EXPORTS[3:]:
    getattr(_lib, _f).restype = ctypes.c_int
_lib.hsab_offload_destroy.restype = None
_lib.hsab_dense_workspace_bytes.restype = _sz


class HsabError(RuntimeError):
    def __init__(self, fn, status):
        msg = _lib.hsab_status_string(status).decode()
        if status == HSAB_EHIP:
            msg += f" (hipError {_lib.hsab_last_hip_error()})"
        super().__init__(f"{fn}: {msg}")
        self.status = status


def _check(fn, status):
    if status != HSAB_OK:
        raise HsabError(fn, status)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


_u16, _i, _f = torch.uint16, torch.int32, torch.float32
# bf16 buffers may be passed as bfloat16 tensors or as raw 16-bit patterns
_BF16_BITS = (torch.bfloat16, torch.int16, torch.uint16)


def _buf(name, t, dtype, numel, allow_none=False):
    """Pointer of a device buffer after checking dtype, layout and size."""
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    ok = t.dtype in _BF16_BITS if dtype is _u16 else t.dtype == dtype
    if not ok:
        raise ValueError(f"{name} must be {'bf16 bits' if dtype is _u16 else dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _hbuf(name, t, dtype, numel, pinned=False, allow_none=False):
    """Pointer of a host buffer after checking dtype, layout and size."""
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.is_cuda:
        raise ValueError(f"{name} must be a host tensor")
    ok = t.dtype in _BF16_BITS if dtype is _u16 else t.dtype == dtype
    if not ok:
        raise ValueError(f"{name} must be {'bf16 bits' if dtype is _u16 else dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if pinned and not t.is_pinned():
        raise ValueError(f"{name} must be pinned host memory")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def workspace_bytes(d: Dims) -> int:
    return int(_lib.hsab_workspace_bytes(ctypes.byref(d)))


def status_string(status: int) -> str:
    return _lib.hsab_status_string(status).decode()


def alloc_workspace(d: Dims, device="cuda") -> torch.Tensor:
    n = workspace_bytes(d)
    if n == 0:
        raise ValueError(f"invalid dims {d}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def selections(d: Dims) -> int:
    """Selections per step: one per (batch, KV head), or one per (batch,
    query head) with per-head selection (AGG_HEAD)."""
    return d.batch * (d.n_q_heads if d.group_agg == AGG_HEAD else d.n_kv_heads)


def _sizes(d: Dims):
    U = d.batch * d.n_kv_heads
    S = selections(d)
    return {
        "q": d.batch * d.n_q_heads * d.d_k, "K": U * d.max_ctx * d.d_k, "V": U * d.max_ctx * d.d_v,
        "meta": U * d.nb_cap * 2 * d.d_k, "klabel": U * d.max_ctx * d.r, "label": d.n_kv_heads * d.r,
        "ctx": d.batch, "blk": S * d.k_blocks, "tok": S * d.k_tokens, "score": S * d.nb_cap,
        "tscore": S * d.k_blocks * d.block, "out": d.batch * d.n_q_heads * d.d_v,
        "lse": d.batch * d.n_q_heads, "knew": U * d.d_k, "vnew": U * d.d_v,
    }


def _meta(d: Dims, meta):
    """Metadata buffer: bf16 bits, or uint8 e4m3 bytes with fp8 metadata;
    B*Hkv*nb_cap*2*d_k values either way."""
    n = d.batch * d.n_kv_heads * d.nb_cap * 2 * d.d_k
    return _buf("meta", meta, torch.uint8 if d.meta_format == META_FP8 else _u16, n)


def _klabel(d: Dims, klabel):
    """Label rows: bf16 bits, or uint8 e4m3 bytes with fp8 label rows;
    B*Hkv*max_ctx*r values either way."""
    n = d.batch * d.n_kv_heads * d.max_ctx * d.r
    return _buf("klabel", klabel, torch.uint8 if d.label_format == LABEL_FP8 else _u16, n)


def alloc_klabel(d: Dims, device="cuda") -> torch.Tensor:
    n = d.batch * d.n_kv_heads * d.max_ctx * d.r
    return torch.zeros(n, dtype=torch.uint8 if d.label_format == LABEL_FP8 else torch.int16, device=device)


def alloc_meta(d: Dims, device="cuda") -> torch.Tensor:
    n = d.batch * d.n_kv_heads * d.nb_cap * 2 * d.d_k
    return torch.zeros(n, dtype=torch.uint8 if d.meta_format == META_FP8 else torch.int16, device=device)


def _ws(d, ws):
    if ws is None:
        raise ValueError("workspace is required (alloc_workspace)")
    return _buf("ws", ws, torch.uint8, workspace_bytes(d)), ctypes.c_size_t(ws.numel())


def build_meta(d: Dims, K, ctx_len, label_ch, meta, klabel, stream=None):
    s = _sizes(d)
    _check("hsab_build_meta", _lib.hsab_build_meta(
        ctypes.byref(d), _buf("K", K, _u16, s["K"]), _buf("ctx_len", ctx_len, _i, s["ctx"]),
        _buf("label_ch", label_ch, _i, s["label"]), _meta(d, meta),
        _klabel(d, klabel), _stream(stream)))


def score_blocks(d: Dims, q, meta, ctx_len, blk_score, stream=None):
    s = _sizes(d)
    _check("hsab_score_blocks", _lib.hsab_score_blocks(
        ctypes.byref(d), _buf("q", q, _u16, s["q"]), _meta(d, meta),
        _buf("ctx_len", ctx_len, _i, s["ctx"]), _buf("blk_score", blk_score, _f, s["score"]),
        _stream(stream)))


def select_blocks(d: Dims, q, meta, ctx_len, blk_idx, blk_score=None, ws=None, stream=None):
    s = _sizes(d)
    if blk_score is None:
        wp, wn = _ws(d, ws)
    else:
        wp, wn = (None, 0) if ws is None else _ws(d, ws)
    _check("hsab_select_blocks", _lib.hsab_select_blocks(
        ctypes.byref(d), _buf("q", q, _u16, s["q"]), _meta(d, meta),
        _buf("ctx_len", ctx_len, _i, s["ctx"]), _buf("blk_idx", blk_idx, _i, s["blk"]),
        _buf("blk_score", blk_score, _f, s["score"], allow_none=True), wp, wn, _stream(stream)))


def select_tokens(d: Dims, q, klabel, label_ch, blk_idx, ctx_len, tok_idx, tok_score=None, ws=None,
                  stream=None):
    s = _sizes(d)
    wp, wn = (None, 0) if ws is None else _ws(d, ws)
    _check("hsab_select_tokens", _lib.hsab_select_tokens(
        ctypes.byref(d), _buf("q", q, _u16, s["q"]), _klabel(d, klabel),
        _buf("label_ch", label_ch, _i, s["label"]), _buf("blk_idx", blk_idx, _i, s["blk"]),
        _buf("ctx_len", ctx_len, _i, s["ctx"]), _buf("tok_idx", tok_idx, _i, s["tok"]),
        _buf("tok_score", tok_score, _f, s["tscore"], allow_none=True), wp, wn, _stream(stream)))


def sparse_attend(d: Dims, q, K, V, tok_idx, ctx_len, out, lse, ws, slot_of=None, n_slots=0,
                  stream=None):
    s = _sizes(d)
    U = d.batch * d.n_kv_heads
    if slot_of is None:
        kn, vn = s["K"], s["V"]
    else:   # block cache: key rows then value rows per slot, V unused
        kn, vn, V = U * n_slots * block_elems(d), 0, None
    wp, wn = _ws(d, ws)
    _check("hsab_sparse_attend", _lib.hsab_sparse_attend(
        ctypes.byref(d), _buf("q", q, _u16, s["q"]), _buf("K", K, _u16, kn),
        _buf("V", V, _u16, vn, allow_none=bool(d.v_alias_k) or slot_of is not None),
        _buf("tok_idx", tok_idx, _i, s["tok"]),
        _buf("ctx_len", ctx_len, _i, s["ctx"]),
        _buf("slot_of", slot_of, _i, U * d.nb_cap, allow_none=True), ctypes.c_int32(n_slots),
        _buf("out", out, _f, s["out"]), _buf("lse", lse, _f, s["lse"]), wp, wn, _stream(stream)))


def decode_step(d: Dims, q, k_new, v_new, K, V, meta, klabel, label_ch, ctx_len, blk_idx, tok_idx,
                out, lse, ws, stream=None):
    s = _sizes(d)
    alias = bool(d.v_alias_k)
    wp, wn = _ws(d, ws)
    _check("hsab_decode_step", _lib.hsab_decode_step(
        ctypes.byref(d), _buf("q", q, _u16, s["q"]), _buf("k_new", k_new, _u16, s["knew"]),
        _buf("v_new", v_new, _u16, s["vnew"], allow_none=alias), _buf("K", K, _u16, s["K"]),
        _buf("V", V, _u16, s["V"], allow_none=alias), _meta(d, meta),
        _klabel(d, klabel), _buf("label_ch", label_ch, _i, s["label"]),
        _buf("ctx_len", ctx_len, _i, s["ctx"]), _buf("blk_idx", blk_idx, _i, s["blk"]),
        _buf("tok_idx", tok_idx, _i, s["tok"]), _buf("out", out, _f, s["out"]),
        _buf("lse", lse, _f, s["lse"]), wp, wn, _stream(stream)))


def decode_step_noalloc(d: Dims, q, k_new, v_new, K, V, meta, klabel, label_ch, ctx_len, blk_idx, tok_idx,
                        out, lse, stream=None):
    """decode_step on the library's static per-GPU workspace (no workspace
    argument; raises with HSAB_ESCRATCH when the shape needs more than
    SCRATCH_BYTES)."""
    s = _sizes(d)
    alias = bool(d.v_alias_k)
    _check("hsab_decode_step_noalloc", _lib.hsab_decode_step_noalloc(
        ctypes.byref(d), _buf("q", q, _u16, s["q"]), _buf("k_new", k_new, _u16, s["knew"]),
        _buf("v_new", v_new, _u16, s["vnew"], allow_none=alias), _buf("K", K, _u16, s["K"]),
        _buf("V", V, _u16, s["V"], allow_none=alias), _meta(d, meta),
        _klabel(d, klabel), _buf("label_ch", label_ch, _i, s["label"]),
        _buf("ctx_len", ctx_len, _i, s["ctx"]), _buf("blk_idx", blk_idx, _i, s["blk"]),
        _buf("tok_idx", tok_idx, _i, s["tok"]), _buf("out", out, _f, s["out"]),
        _buf("lse", lse, _f, s["lse"]), _stream(stream)))


def block_elems(d: Dims) -> int:
    """bf16 elements of one block in the host pool and the block cache."""
    return d.block * (d.d_k if d.v_alias_k else d.d_k + d.d_v)


def offload_append(d: Dims, n_slots, k_new, v_new, cache, meta, klabel, label_ch, ctx_len, stream=None):
    s = _sizes(d)
    U = d.batch * d.n_kv_heads
    alias = bool(d.v_alias_k)
    _check("hsab_offload_append", _lib.hsab_offload_append(
        ctypes.byref(d), ctypes.c_int32(n_slots), _buf("k_new", k_new, _u16, s["knew"]),
        _buf("v_new", v_new, _u16, s["vnew"], allow_none=alias),
        _buf("cache", cache, _u16, U * n_slots * block_elems(d)), _meta(d, meta),
        _klabel(d, klabel), _buf("label_ch", label_ch, _i, s["label"]),
        _buf("ctx_len", ctx_len, _i, s["ctx"]), _stream(stream)))


def offload_plan(d: Dims, n_slots, resident, selected, tail, slot_map, plan) -> int:
    """Host planner; every argument is a host int32 tensor. Returns the
    bytes the plan copies."""
    U = d.batch * d.n_kv_heads
    nb = ctypes.c_int64(0)
    _check("hsab_offload_plan", _lib.hsab_offload_plan(
        ctypes.byref(d), ctypes.c_int32(n_slots), _hbuf("resident", resident, _i, U * d.k_blocks),
        _hbuf("selected", selected, _i, U * d.k_blocks), _hbuf("tail", tail, _i, U * 2),
        _hbuf("slot_map", slot_map, _i, U * d.nb_cap), _hbuf("plan", plan, _i, U * d.k_blocks * 3),
        ctypes.byref(nb)))
    return int(nb.value)


def offload_copy(d: Dims, n_slots, host_pool, cache, plan, plan_dev, slot_of, copy_stream, done=None,
                 copy_mode=COPY_KERNEL) -> int:
    """Enqueue a plan's copies on copy_stream; returns the blocks gathered
    (kernel mode) or copies issued (DMA mode). host_pool and plan are
    pinned host tensors; done is a torch.cuda.Event (recorded on
    copy_stream) or None."""
    U = d.batch * d.n_kv_heads
    nc = ctypes.c_int32(0)
    ev = None
    if done is not None:
        ev = ctypes.c_void_p(done.cuda_event)
    _check("hsab_offload_copy", _lib.hsab_offload_copy(
        ctypes.byref(d), ctypes.c_int32(n_slots),
        _hbuf("host_pool", host_pool, _u16, U * d.nb_cap * block_elems(d), pinned=True),
        _buf("cache", cache, _u16, U * n_slots * block_elems(d)),
        _hbuf("plan", plan, _i, U * d.k_blocks * 3, pinned=True),
        _buf("plan_dev", plan_dev, _i, U * d.k_blocks * 3), _buf("slot_of", slot_of, _i, U * d.nb_cap),
        ctypes.c_int32(copy_mode), _stream(copy_stream), ev, ctypes.byref(nc)))
    return int(nc.value)


class OffloadEngine:
    """Handle of a native offload engine (hsab_offload_create). The caller
    owns the pool (pinned host), the block cache, metadata and outputs."""

    def __init__(self, d: Dims, n_slots: int, copy_mode: int = COPY_KERNEL):
        self.d, self.n_slots, self.copy_mode = d, int(n_slots), int(copy_mode)
        h = ctypes.c_void_p()
        _check("hsab_offload_create", _lib.hsab_offload_create(ctypes.byref(d), ctypes.c_int32(n_slots),
                                                               ctypes.c_int32(copy_mode), ctypes.byref(h)))
        self._h = h

    def close(self):
        if self._h:
            _lib.hsab_offload_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def begin(self, n_prefill, host_pool, cache, slot_of, stream=None):
        d = self.d
        U = d.batch * d.n_kv_heads
        _check("hsab_offload_begin", _lib.hsab_offload_begin(
            self._h, _hbuf("n_prefill", n_prefill, _i, d.batch),
            _hbuf("host_pool", host_pool, _u16, U * d.nb_cap * block_elems(d), pinned=True),
            _buf("cache", cache, _u16, U * self.n_slots * block_elems(d)),
            _buf("slot_of", slot_of, _i, U * d.nb_cap), _stream(stream)))

    def step(self, q, k_new, v_new, host_pool, cache, meta, klabel, label_ch, ctx_len, ctx_len_host, slot_of,
             tok_idx, out, lse, ws, compute_stream=None, copy_stream=None) -> OffloadStats:
        d = self.d
        s = _sizes(d)
        U = d.batch * d.n_kv_heads
        wp, wn = _ws(d, ws)
        st = OffloadStats()
        if copy_stream is None:
            raise ValueError("copy_stream is required")
        _check("hsab_offload_step", _lib.hsab_offload_step(
            self._h, _buf("q", q, _u16, s["q"]), _buf("k_new", k_new, _u16, s["knew"]),
            _buf("v_new", v_new, _u16, s["vnew"], allow_none=bool(d.v_alias_k)),
            self._pool(host_pool, U * d.nb_cap * block_elems(d)),
            _buf("cache", cache, _u16, U * self.n_slots * block_elems(d)), _meta(d, meta),
            _klabel(d, klabel), _buf("label_ch", label_ch, _i, s["label"]),
            _buf("ctx_len", ctx_len, _i, s["ctx"]), _hbuf("ctx_len_host", ctx_len_host, _i, d.batch),
            _buf("slot_of", slot_of, _i, U * d.nb_cap), _buf("tok_idx", tok_idx, _i, s["tok"]),
            _buf("out", out, _f, s["out"]), _buf("lse", lse, _f, s["lse"]), wp, wn, _stream(compute_stream),
            _stream(copy_stream), ctypes.byref(st)))
        return st

    def _pool(self, host_pool, numel):
        """The pool's pointer; whether it is pinned is checked once per
        tensor (the query goes to the HIP runtime), the rest every call."""
        key = (host_pool.data_ptr(), host_pool.numel()) if isinstance(host_pool, torch.Tensor) else None
        if key is not None and key == getattr(self, "_pool_ok", None):
            return _hbuf("host_pool", host_pool, _u16, numel)
        p = _hbuf("host_pool", host_pool, _u16, numel, pinned=True)
        self._pool_ok = key
        return p

    def set_timing(self, enable: bool):
        """Record per-step GPU timestamps (for timing()) from the next step on."""
        _check("hsab_offload_set_timing", _lib.hsab_offload_set_timing(self._h, int(bool(enable))))

    def timing(self, step):
        ms = (ctypes.c_float * 5)()
        _check("hsab_offload_timing", _lib.hsab_offload_timing(self._h, ctypes.c_int64(step), ms))
        return {"compute_ms": ms[0], "copy_ms": ms[1], "copy_start_ms": ms[2], "copy_end_ms": ms[3],
                "copy_wait_ms": ms[4]}

    def selection(self) -> torch.Tensor:
        d = self.d
        outb = torch.empty(d.batch * d.n_kv_heads * d.k_blocks, dtype=torch.int32)
        _check("hsab_offload_selection", _lib.hsab_offload_selection(self._h, ctypes.c_void_p(outb.data_ptr())))
        return outb.view(d.batch, d.n_kv_heads, d.k_blocks)

    def step_selection(self, step) -> torch.Tensor:
        """S_b [B][Hkv][K_b] of a step among the last 32 (waits for it)."""
        d = self.d
        outb = torch.empty(d.batch * d.n_kv_heads * d.k_blocks, dtype=torch.int32)
        _check("hsab_offload_step_selection", _lib.hsab_offload_step_selection(
            self._h, ctypes.c_int64(step), ctypes.c_void_p(outb.data_ptr())))
        return outb.view(d.batch, d.n_kv_heads, d.k_blocks)

    def delta(self, step) -> tuple:
        """(delta_bytes, cold_bytes) of a step among the last 32 (waits for
        that step's copies when the GPU planned them)."""
        db, cb = ctypes.c_int64(0), ctypes.c_int64(0)
        _check("hsab_offload_step_delta", _lib.hsab_offload_step_delta(self._h, ctypes.c_int64(step),
                                                                       ctypes.byref(db), ctypes.byref(cb)))
        return int(db.value), int(cb.value)


def dense_workspace_bytes(d: Dims) -> int:
    return int(_lib.hsab_dense_workspace_bytes(ctypes.byref(d)))


def alloc_dense_workspace(d: Dims, device="cuda") -> torch.Tensor:
    n = dense_workspace_bytes(d)
    if n == 0:
        raise ValueError(f"dense attention unsupported or invalid dims {d}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def dense_attend(d: Dims, q, K, V, ctx_len, out, lse, ws, stream=None):
    """Full attention over every token (the reference the sparse operator
    is measured against)."""
    s = _sizes(d)
    _check("hsab_dense_attend", _lib.hsab_dense_attend(
        ctypes.byref(d), _buf("q", q, _u16, s["q"]), _buf("K", K, _u16, s["K"]),
        _buf("V", V, _u16, s["V"], allow_none=bool(d.v_alias_k)),
        _buf("ctx_len", ctx_len, _i, s["ctx"]), _buf("out", out, _f, s["out"]), _buf("lse", lse, _f, s["lse"]),
        _buf("ws", ws, torch.uint8, dense_workspace_bytes(d)), ctypes.c_size_t(ws.numel()), _stream(stream)))


def raw_call(name, *args):
    """Call an exported entry point with raw ctypes arguments and return its
    status (used by the host-side error-path tests)."""
    return getattr(_lib, name)(*args)


def calibrate_labels(d: Dims, q_samples, k_samples, n_samples, importance, label_ch, stream=None):
    """Label channels per KV head from n_samples sampled query rows
    [n][Hq][d_k] and key rows [n][Hkv][d_k] (bf16 bits); writes importance
    [Hkv][d_k] fp32 and label_ch [Hkv][r] int32."""
    n = int(n_samples)
    _check("hsab_calibrate_labels", _lib.hsab_calibrate_labels(
        ctypes.byref(d), _buf("q_samples", q_samples, _u16, n * d.n_q_heads * d.d_k),
        _buf("k_samples", k_samples, _u16, n * d.n_kv_heads * d.d_k), ctypes.c_int32(n),
        _buf("importance", importance, _f, d.n_kv_heads * d.d_k), _buf("label_ch", label_ch, _i, d.n_kv_heads * d.r),
        _stream(stream)))
