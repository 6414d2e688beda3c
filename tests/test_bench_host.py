"""Host-side logic of bench.py (no GPU): the one-GPU guard, how steps are
grouped into captured graphs, and the algorithmic byte counts that the
roofline and the step's HBM fraction divide by, against figures worked out
by hand from the layouts (48k GQA layer: 64 units of 3072 blocks, 2 x 128
bf16 metadata values per block, one fp32 score per block)."""
import dataclasses
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from hierarchical_sparse_attention_block_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("steps,group", [(200, 10), (7, 7), (17, 1), (32, 16), (1, 1), (48, 16), (90, 15)])
def test_graph_group_divides_steps(steps, group):
    g = bench.graph_group(steps)
    assert g == group
    assert steps % g == 0 and g <= 16


def test_block_score_bytes_48k():
    w = W.WORKLOADS["gqa48k"]
    # 64 units x 3072 blocks x (256 bf16 values + one fp32 score) + 8 x 32 query rows of 128 bf16
    assert bench.score_kernel_bytes(w) == 64 * 3072 * (256 * 2 + 4) + 8 * 32 * 128 * 2 == 101_515_264
    w8 = dataclasses.replace(w, meta_fp8=True)
    assert bench.score_kernel_bytes(w8) == 64 * 3072 * (256 + 4) + 8 * 32 * 128 * 2 == 51_183_616


def test_step_bytes_48k():
    w = W.WORKLOADS["gqa48k"]
    b = bench.step_bytes(w)
    assert b["meta"] == 64 * 3072 * 256 * 2
    assert b["labels"] == 64 * 128 * 16 * 16 * 2            # K_b blocks of 16 rows of r = 16 label values
    assert b["gather"] == 64 * 512 * (128 + 128) * 2        # K_t key and value rows
    assert b["q_out"] == 8 * 32 * (128 * 2 + 128 * 4)       # bf16 queries in, fp32 outputs out
    assert b["total"] == 121_831_424


def test_step_bytes_latent_values_alias_keys():
    w = W.WORKLOADS["mla64k"]
    b = bench.step_bytes(w)
    # 8 units, 2048 blocks of 32 tokens; one 576-dim row per kept token (values are its first 512 dims)
    assert b["meta"] == 8 * 2048 * 2 * 576 * 2
    assert b["gather"] == 8 * 1024 * 576 * 2
