"""C ABI of libhsab on the host: the library loads, exports every function
include/hsab.h declares, sizes its workspace, and rejects bad arguments
before it touches a GPU. No kernel runs here."""
import ctypes
import os
import re

import pytest

H = pytest.importorskip("hierarchical_sparse_attention_block_amd.hsab")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hsab.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(hsab_\w+)\s*\(", text, flags=re.M)))


def _dims(**kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, d_k=128, d_v=128, v_alias_k=False, block=16, r=16,
                k_blocks=8, k_tokens=64, max_ctx=1024, sm_scale=0.125)
    base.update(kw)
    return H.dims(**base)


def test_every_declared_function_is_exported():
    names = _declared()
    assert len(names) >= 18, names
    lib = ctypes.CDLL(H.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in hsab.h but not exported"
    assert sorted(H.EXPORTS) == names, "binding EXPORTS out of step with the header"


def test_workspace_layout():
    d = _dims()
    U, Hq = 4, 16
    splits = -(-64 // 64)
    al = lambda x: (x + 255) // 256 * 256
    # block scores, split (max, sum), split accumulators, selection keys
    # (K_b * block candidates per unit), selection arrival counters
    want = (al(U * d.nb_cap * 4) + al(Hq * splits * 2 * 4) + al(Hq * splits * 128 * 4)
            + al(U * d.k_blocks * d.block * 4) + al(U * 4))
    assert H.workspace_bytes(d) == want
    assert H.workspace_bytes(_dims(n_q_heads=7)) == 0          # Hq % Hkv != 0
    # per-head selection: one selection per query head, splits over the
    # union of the heads' lists (G * K_t entries), the union and its masks
    dh = _dims(group_agg=H.AGG_HEAD)
    S, G = U * 4, 4
    sh = -(-(G * 64) // 64)
    want_h = (al(S * d.nb_cap * 4) + al(Hq * sh * 2 * 4) + al(Hq * sh * 128 * 4)
              + al(S * d.k_blocks * d.block * 4) + al(S * 4) + 2 * al(U * G * 64 * 4))
    assert H.workspace_bytes(dh) == want_h
    # one head per group: per-head selection is the group mode, no union
    assert H.workspace_bytes(_dims(n_q_heads=2, group_agg=H.AGG_HEAD)) == \
        H.workspace_bytes(_dims(n_q_heads=2))


def test_workspace_splits_follow_the_resident_round():
    """64-token attention splits while units x splits fit one round of 1,024
    resident workgroups; 128-token splits beyond it for d <= 128; 64 for
    wider heads. The split count sizes the two partial arrays."""
    al = lambda x: (x + 255) // 256 * 256

    def partials(d, splits):
        Hq = d.batch * d.n_q_heads
        return al(Hq * splits * 2 * 4) + al(Hq * splits * d.d_v * 4)

    def ws_without_partials(d):
        U = d.batch * d.n_kv_heads
        return al(U * d.nb_cap * 4) + al(U * d.k_blocks * d.block * 4) + al(U * 4)

    # 128 units x 16 splits of 64 = 2,048 workgroups: 8 splits of 128
    d = _dims(batch=16, n_q_heads=32, n_kv_heads=8, k_blocks=256, k_tokens=1024, max_ctx=98304)
    assert H.workspace_bytes(d) == ws_without_partials(d) + partials(d, 8)
    # 64 units x 8 splits = 512 workgroups: 64-token splits
    d = _dims(batch=8, n_q_heads=32, n_kv_heads=8, k_blocks=128, k_tokens=512, max_ctx=49152)
    assert H.workspace_bytes(d) == ws_without_partials(d) + partials(d, 8)
    # exactly 1,024 workgroups still fit the round
    d = _dims(batch=16, n_q_heads=32, n_kv_heads=8, k_blocks=128, k_tokens=512, max_ctx=49152)
    assert H.workspace_bytes(d) == ws_without_partials(d) + partials(d, 8)
    # d = 256 keeps 64-token splits
    d = _dims(batch=16, n_q_heads=32, n_kv_heads=8, d_k=256, d_v=256, k_blocks=256, k_tokens=1024,
              max_ctx=98304)
    assert H.workspace_bytes(d) == ws_without_partials(d) + partials(d, 16)


@pytest.mark.parametrize("bad", [
    dict(batch=0), dict(n_q_heads=7), dict(n_q_heads=128, n_kv_heads=2), dict(d_k=100), dict(d_k=2048),
    dict(d_v=12), dict(r=24), dict(r=256), dict(k_blocks=0), dict(k_blocks=4096), dict(k_blocks=1024, block=16),
    dict(k_tokens=0), dict(max_ctx=0), dict(max_ctx=16 * 8193), dict(v_alias_k=True, d_v=256, d_k=128),
    dict(sm_scale=float("inf")), dict(meta_format=2), dict(meta_format=1, d_k=48), dict(group_agg=3), dict(label_format=2),
    dict(sink_blocks=-1), dict(local_blocks=-1), dict(sink_blocks=5, local_blocks=4),
])
def test_bad_dims_rejected(bad):
    d = _dims(**bad)
    p = ctypes.c_void_p(16)   # never dereferenced: the shape check comes first
    assert H.raw_call("hsab_workspace_bytes", ctypes.byref(d)) == 0
    assert H.raw_call("hsab_score_blocks", ctypes.byref(d), p, p, p, p, None) == H.HSAB_EINVAL
    assert H.raw_call("hsab_build_meta", ctypes.byref(d), p, p, p, p, p, None) == H.HSAB_EINVAL
    h = ctypes.c_void_p()
    assert H.raw_call("hsab_offload_create", ctypes.byref(d), 64, 0, ctypes.byref(h)) == H.HSAB_EINVAL
    assert not h.value


def test_null_pointers_rejected():
    d = _dims()
    p = ctypes.c_void_p(16)
    n = None
    assert H.raw_call("hsab_build_meta", ctypes.byref(d), n, p, p, p, p, None) == H.HSAB_EINVAL
    assert H.raw_call("hsab_score_blocks", ctypes.byref(d), p, n, p, p, None) == H.HSAB_EINVAL
    assert H.raw_call("hsab_select_blocks", ctypes.byref(d), p, p, p, n, p, p, 1 << 20, None) == H.HSAB_EINVAL
    assert H.raw_call("hsab_decode_step", ctypes.byref(d), n, p, p, p, p, p, p, p, p, p, p, p, p, p,
                      1 << 20, None) == H.HSAB_EINVAL
    assert H.raw_call("hsab_offload_step", n, *([p] * 15), 1 << 20, None, None, None) == H.HSAB_EINVAL
    assert H.raw_call("hsab_offload_begin", n, p, p, p, p, None) == H.HSAB_EINVAL
    assert H.raw_call("hsab_offload_timing", n, 0, p) == H.HSAB_EINVAL
    assert H.raw_call("hsab_offload_set_timing", n, 1) == H.HSAB_EINVAL
    assert H.raw_call("hsab_offload_selection", n, p) == H.HSAB_EINVAL
    # unknown copy mode, misaligned pool
    assert H.raw_call("hsab_offload_copy", ctypes.byref(d), 18, p, p, p, p, p, 7, None, None, None) == H.HSAB_EINVAL
    q = ctypes.c_void_p(18)
    assert H.raw_call("hsab_offload_copy", ctypes.byref(d), 18, q, p, p, p, p, 0, None, None, None) == H.HSAB_EINVAL
    h = ctypes.c_void_p()
    assert H.raw_call("hsab_offload_create", ctypes.byref(d), 18, 3, ctypes.byref(h)) == H.HSAB_EINVAL


def test_small_workspace_and_unsupported_shape():
    d = _dims()
    p = ctypes.c_void_p(16)
    ws = H.workspace_bytes(d)
    # sparse_attend: workspace one byte short, then an attention shape with no kernel
    assert H.raw_call("hsab_sparse_attend", ctypes.byref(d), p, p, p, p, p, None, 0, p, p, p, ws - 1,
                      None) == H.HSAB_EINVAL
    d96 = _dims(d_k=96, d_v=96)
    ws96 = H.workspace_bytes(d96)
    assert H.raw_call("hsab_sparse_attend", ctypes.byref(d96), p, p, p, p, p, None, 0, p, p, p, ws96,
                      None) == H.HSAB_EUNSUPPORTED
    h = ctypes.c_void_p()
    assert H.raw_call("hsab_offload_create", ctypes.byref(d96), 64, 0, ctypes.byref(h)) == H.HSAB_EUNSUPPORTED
    # the offload engine needs 2 K_b + 2 slots
    assert H.raw_call("hsab_offload_create", ctypes.byref(d), 17, 0, ctypes.byref(h)) == H.HSAB_EINVAL


def test_status_strings():
    assert H.status_string(H.HSAB_OK) == "ok"
    for s in (H.HSAB_EINVAL, H.HSAB_EHIP, H.HSAB_EUNSUPPORTED):
        assert H.status_string(s) not in ("ok", "unknown status")
    assert H.status_string(12345) == "unknown status"
    assert H.raw_call("hsab_last_hip_error") == 0


def test_noalloc_refuses_oversize_before_any_gpu_call():
    """hsab_decode_step_noalloc checks the workspace a shape needs against
    its static scratch before touching a GPU: per-head selection at 96k
    needs more and is refused with HSAB_ESCRATCH."""
    from hierarchical_sparse_attention_block_amd import workloads as W
    from tests.hsab_testlib import dims_of
    d = dims_of(W.WORKLOADS["gqa96k"].replace(per_head=True))
    assert H.workspace_bytes(d) > H.SCRATCH_BYTES
    p = ctypes.c_void_p(16)
    assert H.raw_call("hsab_decode_step_noalloc", ctypes.byref(d), p, p, p, p, p, p, p, p, p, p, p, p, p,
                      None) == H.HSAB_ESCRATCH
    assert b"static scratch" in H._lib.hsab_status_string(H.HSAB_ESCRATCH)
