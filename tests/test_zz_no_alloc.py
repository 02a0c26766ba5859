"""The no-allocation decode entry point against the workspace one.

mla_decode_with_kvcache_noalloc runs the same kernels as
mla_decode_with_kvcache with the plan and the split partials in the
library's static scratch, so on the same inputs (and the same default part
count) its results are bit-identical.  Two calls in a row, the second on a
smaller input, show that nothing a call reads from the scratch is left over
from the one before; both kernel families (more and fewer than 64 query rows
per kv head) are covered, with the plan made inside the call and passed in.
"""

import ctypes
import sys

import pytest
import torch

from paged_mla_decode_04_amd import _lib, get_mla_metadata, mla_decode_with_kvcache
from paged_mla_decode_04_amd.workloads import D_V, Workload, draw

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def decode(g, no_alloc, with_plan):
    w = g.workload
    meta = get_mla_metadata(g.cache_seqlens, w.s_q * w.h_q, w.h_kv) if with_plan else None
    out, lse = mla_decode_with_kvcache(g.q, g.blocked_k, g.block_table, g.cache_seqlens, D_V,
                                       w.softmax_scale, w.causal, metadata=meta,
                                       no_alloc=no_alloc)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


# (larger input, smaller input): wide kernel (128 and 256 rows) and narrow kernel (16, 32 rows)
PAIRS = [
    (Workload("na_wide", batch=6, s_q=1, h_q=128, causal=False, seqlens="fixed",
              fixed_seqlens=(3000, 70, 1500, 900, 4100, 1)),
     Workload("na_wide_small", batch=2, s_q=2, h_q=128, causal=True, seqlens="fixed",
              fixed_seqlens=(500, 64), pitch=640)),
    (Workload("na_narrow", batch=5, s_q=2, h_q=16, causal=True, seqlens="fixed",
              fixed_seqlens=(2000, 33, 700, 1, 1300)),
     Workload("na_narrow_small", batch=1, s_q=1, h_q=16, causal=False, seqlens="fixed",
              fixed_seqlens=(200,))),
]


@pytest.mark.parametrize("with_plan", [False, True], ids=["plan_inside", "plan_passed"])
@pytest.mark.parametrize("pair", PAIRS, ids=["wide", "narrow"])
def test_no_alloc_equals_workspace_call(pair, with_plan):
    inputs = [draw(w, seed=40 + i, poison=True).to("cuda:0") for i, w in enumerate(pair)]
    note(f"[no-alloc] {pair[0].name}: workspace calls")
    refs = [decode(g, False, with_plan) for g in inputs]
    note(f"[no-alloc] {pair[0].name}: two no-allocation calls in a row, the second smaller")
    got = [decode(g, True, with_plan) for g in inputs]
    for (ro, rl), (o, l), w in zip(refs, got, pair):
        assert torch.equal(o, ro), f"{w.name}: out differs from the workspace call"
        assert torch.equal(l, rl), f"{w.name}: lse differs from the workspace call"


def test_no_alloc_fp8_equals_workspace_call():
    """The same with an fp8 cache (the 128-row kernel with its staging area)."""
    pair = [Workload("na_fp8", batch=4, s_q=1, h_q=128, causal=False, seqlens="fixed",
                     fixed_seqlens=(2500, 90, 1200, 1), kv_format="fp8_e4m3", kv_scale=1 / 64),
            Workload("na_fp8_small", batch=1, s_q=2, h_q=64, causal=True, seqlens="fixed",
                     fixed_seqlens=(300,), kv_format="fp8_e4m3", kv_scale=1 / 64)]
    inputs = [draw(w, seed=60 + i, poison=True).to("cuda:0") for i, w in enumerate(pair)]

    def run(g, no_alloc):
        w = g.workload
        out, lse = mla_decode_with_kvcache(g.q, g.blocked_k, g.block_table, g.cache_seqlens, D_V,
                                           w.softmax_scale, w.causal, no_alloc=no_alloc,
                                           kv_scale=w.kv_scale)
        torch.cuda.synchronize()
        return out.cpu(), lse.cpu()

    note("[no-alloc] fp8: workspace calls, then two no-allocation calls")
    refs = [run(g, False) for g in inputs]
    got = [run(g, True) for g in inputs]
    for (ro, rl), (o, l), w in zip(refs, got, pair):
        assert torch.equal(o, ro) and torch.equal(l, rl), w.name


def test_no_alloc_rejects_a_call_beyond_its_scratch():
    """16384 sequences of 1024 rows need far more than the static scratch: the
    call returns MLA_ERR_SCRATCH_TOO_SMALL before enqueueing anything."""
    lib = _lib.load()
    q = torch.zeros(16, dtype=torch.bfloat16, device="cuda:0")
    i32 = torch.zeros(16, dtype=torch.int32, device="cuda:0")
    f32 = torch.zeros(16, dtype=torch.float32, device="cuda:0")
    p = _lib.DecodeParams()
    p.q, p.k_cache, p.out = q.data_ptr(), q.data_ptr(), q.data_ptr()
    p.block_table, p.cache_seqlens, p.lse = i32.data_ptr(), i32.data_ptr(), f32.data_ptr()
    p.batch, p.s_q, p.h_q = 16384, 8, 128
    p.q_batch_stride, p.q_seq_stride, p.q_head_stride = 8 * 128 * 576, 128 * 576, 576
    p.out_batch_stride, p.out_seq_stride, p.out_head_stride = 8 * 128 * 512, 128 * 512, 512
    p.lse_batch_stride, p.lse_seq_stride, p.lse_head_stride = 8 * 128, 128, 1
    p.k_block_stride, p.k_row_stride, p.k_head_stride = 64 * 576, 576, 576
    p.num_blocks, p.block_size, p.h_kv, p.d = 1, 64, 1, 576
    p.block_table_stride, p.max_blocks_per_seq = 1, 1
    p.dv, p.softmax_scale, p.causal = 512, 0.0721688, 1
    st = lib.mla_decode_with_kvcache_noalloc(ctypes.byref(p), None)
    assert st == _lib.MLA_ERR_SCRATCH_TOO_SMALL
    assert "static scratch" in _lib.status_string(st)
