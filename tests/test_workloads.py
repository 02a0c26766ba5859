"""The seeded input generator: recipes, determinism, layouts and poisoning."""

import math

import numpy as np
import pytest
import torch

from paged_mla_decode_04_amd import workloads as wl
from paged_mla_decode_04_amd.workloads import D_QK, WORKLOADS, draw


def _seqlens(name, seed=0):
    g = torch.Generator().manual_seed(seed)
    return wl._draw_seqlens(WORKLOADS[name], g)


def test_tiny_workload_shapes():
    inp = draw("tiny")
    assert inp.cache_seqlens.tolist() == [37, 130]
    assert inp.meta["max_seqlen_pad"] == 256
    assert tuple(inp.block_table.shape) == (2, 4)
    assert sorted(inp.block_table.flatten().tolist()) == list(range(8))
    assert tuple(inp.q.shape) == (2, 1, 16, 576) and inp.q.dtype == torch.bfloat16
    assert tuple(inp.blocked_k.shape) == (8, 64, 1, 576)


def test_draws_are_deterministic():
    a, b = draw("tiny"), draw("tiny")
    assert torch.equal(a.q, b.q) and torch.equal(a.k_storage, b.k_storage)
    assert torch.equal(a.block_table, b.block_table)
    c = draw("tiny", seed=1)
    assert not torch.equal(a.q, c.q)


def test_length_recipes():
    s = _seqlens("v2lite")
    assert s.numel() == 32 and int(s.min()) >= 1024 and int(s.max()) <= 4096
    s = _seqlens("wide")
    assert s.numel() == 128 and int(s.min()) >= 1 and int(s.max()) <= 8192
    assert abs(float(s.float().mean()) - 4096) < 3 * 1024 / math.sqrt(128)
    s = _seqlens("mtp")
    assert s.numel() == 64 and int(s.min()) >= 4096 and int(s.max()) <= 12288
    s = _seqlens("skewed")
    assert s.numel() == 16 and int(s.max()) == 32768 and int(s.min()) >= 1


def test_wide_workload_uses_identity_table():
    w = WORKLOADS["wide"]
    small = wl.Workload(**{**w.__dict__, "batch": 3, "seqlens": "fixed",
                           "fixed_seqlens": (10, 300, 5)})
    inp = draw(small)
    assert torch.equal(inp.block_table.flatten(), torch.arange(inp.block_table.numel(),
                                                                dtype=torch.int32))


def test_640_pitch_is_a_strided_view():
    w = WORKLOADS["mtp"]
    small = wl.Workload(**{**w.__dict__, "batch": 2, "seqlens": "fixed",
                           "fixed_seqlens": (100, 200)})
    inp = draw(small)
    assert inp.k_storage.shape[-1] == 640
    assert inp.blocked_k.shape[-1] == D_QK
    assert inp.blocked_k.stride() == (64 * 640, 640, 640, 1)
    assert inp.blocked_k.data_ptr() == inp.k_storage.data_ptr()


def test_poison_marks_exactly_the_unused_bytes():
    w = wl.Workload("p", batch=3, s_q=1, h_q=2, causal=False, seqlens="fixed",
                    fixed_seqlens=(1, 64, 130), pitch=640)
    inp = draw(w, poison=True)
    k = inp.k_storage.float()
    assert torch.isnan(k[..., D_QK:]).all()
    used_rows = 0
    for b, n in enumerate([1, 64, 130]):
        pages = (n + 63) // 64
        assert (inp.block_table[b, pages:] == -1).all()
        for t in range(n):
            row = k[int(inp.block_table[b, t // 64]), t % 64, :, :D_QK]
            assert torch.isfinite(row).all()
            used_rows += 1
    assert int(torch.isfinite(k[..., 0]).sum()) == used_rows


def test_bench_overrides_rename_the_workload():
    """bench.py's layout/shape overrides change only what they name, and rename the
    workload so that no counter summary of the plain workload is attached to it."""
    import sys

    import bench
    argv = sys.argv
    try:
        sys.argv = ["bench.py", "--workload", "wide"]
        plain = bench.chosen_workload(bench.parse())
        sys.argv = ["bench.py", "--workload", "wide", "--pitch", "640", "--table", "randperm",
                    "--seqlen-mean", "2048", "--s-q", "2", "--causal", "yes"]
        w = bench.chosen_workload(bench.parse())
    finally:
        sys.argv = argv
    assert plain == WORKLOADS["wide"]
    assert w.name != "wide" and w.name.startswith("wide+")
    assert (w.pitch, w.table, w.seqlens, w.s_q, w.causal) == (640, "randperm", "normal_2048_512", 2, True)
    assert (w.batch, w.h_q, w.h_kv) == (plain.batch, plain.h_q, plain.h_kv)
    s = draw(w).cache_seqlens
    assert int(s.min()) >= 1 and int(s.max()) <= 4096
