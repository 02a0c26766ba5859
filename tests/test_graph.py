"""The plan and the decode captured in a HIP graph (torch.cuda.CUDAGraph).

The library launches only kernels (no memset, copy or allocation), so a
serving loop can capture one decode step and replay it.  Each replay here is
checked bit for bit against an eager call on the same inputs, with eager work
(new queries written in place, an eager decode, synchronisations) between
the replays; the first one is also checked against the oracle.
"""

import numpy as np
import pytest
import torch

from conftest import bits
from oracle import mla_ref
from paged_mla_decode_04_amd import get_mla_metadata, mla_decode_with_kvcache, workspace_size
from paged_mla_decode_04_amd.workloads import D_V, Workload, draw

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("h_q,s_q,parts", [(128, 2, 7), (16, 1, 5)])
def test_graph_replays_match_eager(h_q, s_q, parts):
    w = Workload("graph", batch=3, s_q=s_q, h_q=h_q, causal=s_q > 1, seqlens="fixed",
                 fixed_seqlens=(700, 64, 1300))
    host = draw(w, seed=11)
    g = host.to("cuda:0")
    rows = s_q * h_q
    out = torch.empty((3, s_q, h_q, D_V), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((3, s_q, h_q), dtype=torch.float32, device="cuda:0")
    ws = torch.empty((workspace_size(3, s_q, h_q, 1, D_V, parts),), dtype=torch.uint8, device="cuda:0")

    def step(o, l):
        meta = get_mla_metadata(g.cache_seqlens, rows, 1, num_parts=parts)
        mla_decode_with_kvcache(g.q, g.blocked_k, g.block_table, g.cache_seqlens, D_V,
                                w.softmax_scale, w.causal, metadata=meta, out=o, lse=l, workspace=ws)

    print(f"[graph] h_q={h_q} s_q={s_q} parts={parts}: eager warm-up", flush=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out, lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(out, lse)
    torch.cuda.synchronize()

    gen = torch.Generator(device="cpu")
    gen.manual_seed(5)
    for rep in range(3):
        if rep > 0:  # eager work between replays: new queries, in place
            g.q.copy_(torch.randn(g.q.shape, generator=gen).to(torch.bfloat16).to("cuda:0"))
        e_out = torch.empty_like(out)
        e_lse = torch.empty_like(lse)
        step(e_out, e_lse)
        torch.cuda.synchronize()
        print(f"[graph] replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, e_out), f"replay {rep}: out differs from the eager call"
        assert torch.equal(lse, e_lse), f"replay {rep}: lse differs from the eager call"
        if rep == 0:
            ref_out, ref_lse = mla_ref.mla_decode_ref(bits(host.q), bits(host.k_storage),
                                                      host.block_table.numpy(), host.cache_seqlens.numpy(),
                                                      w.softmax_scale, w.causal)
            o = out.cpu().float().numpy().astype(np.float64)
            assert np.all(np.abs(o - ref_out) <= 1e-2 * np.maximum(1.0, np.abs(ref_out)))
            assert np.all(np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse) <= 2e-3)
