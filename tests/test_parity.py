"""GPU parity: the HIP path against the fp64 CPU oracle.

Tolerance, elementwise: |out - ref| <= 1e-2 * max(1, |ref|) and, on rows with
a visible key, |lse - ref| <= 2e-3; a row with no visible key must give
out = 0 and lse = -inf on both sides.

Full-size workloads run in the launch configuration the benchmark times
(default number of parts, plan from get_mla_metadata) and every sequence of
every one of them is compared element by element with the oracle.  The worst
error of each case, as a fraction of its bound, is printed and, when the
environment names a file in MLA_PARITY_REPORT, appended to it as a JSON line.  Small cases span several pages with ragged tails, both entry pitches,
causal and not, with every cache byte the result must not depend on poisoned
with NaN.
"""

import json
import math
import os
import sys

import numpy as np
import pytest
import torch

from conftest import bits
from oracle import mla_ref
from paged_mla_decode_04_amd import (get_mla_metadata, mla_decode_with_kvcache, plan_host,
                                     default_num_parts, workspace_size)
from paged_mla_decode_04_amd.workloads import D_V, FP8_KV_SCALE, WORKLOADS, Workload, draw

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
LSE_TOL = 2e-3


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(inp, num_parts=None, use_metadata=True, dev="cuda:0"):
    g = inp.to(dev)
    w = inp.workload
    meta = None
    if use_metadata:
        meta = get_mla_metadata(g.cache_seqlens, w.s_q * w.h_q, w.h_kv, num_parts=num_parts)
    fp8 = w.kv_format == "fp8_e4m3"
    out, lse = mla_decode_with_kvcache(g.q, g.blocked_k, g.block_table, g.cache_seqlens, D_V,
                                       w.softmax_scale, w.causal, metadata=meta,
                                       num_parts=num_parts, kv_scale=w.kv_scale if fp8 else None)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), meta


def cache_raw(inp):
    """The cache storage as the oracle reads it: bf16 bits or E4M3 bytes."""
    if inp.kv_format == "fp8_e4m3":
        return inp.k_storage.numpy()
    return bits(inp.k_storage)


def oracle(inp, batch_indices=None):
    return mla_ref.mla_decode_ref(bits(inp.q), cache_raw(inp), inp.block_table.numpy(),
                                  inp.cache_seqlens.numpy(), inp.softmax_scale, inp.causal,
                                  batch_indices=batch_indices, kv_format=inp.kv_format,
                                  kv_scale=inp.kv_scale)


def assert_parity(out, lse, ref_out, ref_lse, rows=None, what=""):
    o = out.float().numpy().astype(np.float64)
    l = lse.numpy().astype(np.float64)
    if rows is not None:
        o, l, ref_out, ref_lse = o[rows], l[rows], ref_out[rows], ref_lse[rows]
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(l), empty), f"{what}: -inf rows differ"
    assert np.all(o[empty] == 0), f"{what}: empty rows must be 0"
    full = ~empty
    d = np.abs(o[full] - ref_out[full])
    bound = OUT_TOL * np.maximum(1.0, np.abs(ref_out[full]))
    worst = float(np.max(d / bound)) if d.size else 0.0
    assert np.all(d <= bound), f"{what}: out error {float(d.max()):.3e} (x{worst:.2f} of bound)"
    dl = np.abs(l[full] - ref_lse[full])
    assert np.all(dl <= LSE_TOL), f"{what}: lse error {float(dl.max()):.3e}"
    lse_worst = float(dl.max()) if dl.size else 0.0
    report(what, worst, lse_worst, int(np.count_nonzero(full)))
    return worst


def report(what, out_ratio, lse_err, rows):
    """Print (and optionally record) the margin of one parity case."""
    line = {"case": what, "out_err_over_bound": round(out_ratio, 4),
            "lse_abs_err": float(f"{lse_err:.3e}"), "rows_compared": rows}
    note(f"[margin] {json.dumps(line)}")
    path = os.environ.get("MLA_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(line) + "\n")


@pytest.mark.parametrize("name", ["tiny", "v2lite", "wide", "mtp", "skewed"])
def test_workload_parity(name):
    """Every sequence of the full-size workload against the oracle."""
    note(f"[parity] workload {name}: drawing inputs")
    inp = draw(name)
    note(f"[parity] workload {name}: GPU decode, b={inp.workload.batch}")
    out, lse, meta = run_gpu(inp)
    note(f"[parity] workload {name}: oracle on all {inp.workload.batch} sequences")
    ref_out, ref_lse = oracle(inp)
    worst = assert_parity(out, lse, ref_out, ref_lse, what=name)
    note(f"[parity] workload {name}: worst out error {worst:.3f} of the bound")


SMALL = [
    # (seqlens, s_q, h_q, causal, pitch, parts)
    ((37, 130), 1, 16, False, 576, None),
    ((1, 64, 65, 200), 2, 16, True, 640, 5),
    ((300, 7, 129), 1, 128, False, 576, 3),
    ((513, 64, 2), 2, 128, True, 640, 7),
    ((100, 250), 1, 40, False, 640, 2),
    ((90, 33, 1000), 2, 64, True, 576, 4),
    ((77,), 1, 1, False, 576, 1),
    ((640, 17), 2, 8, True, 576, 9),
    ((129, 300, 64, 5), 1, 256, False, 576, 6),
    # three and four query tokens (multi-token prediction / speculative decode)
    ((200, 90, 1), 3, 128, True, 576, 5),
    ((500, 64), 4, 128, True, 640, 3),
    ((300, 33, 3), 4, 16, True, 576, 2),
    ((129, 70), 3, 32, True, 576, None),
    ((260,), 4, 64, False, 576, 2),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"small{i}" for i in range(len(SMALL))])
def test_small_cases_with_poisoned_cache(case):
    lens, s_q, h_q, causal, pitch, parts = case
    w = Workload("small", batch=len(lens), s_q=s_q, h_q=h_q, causal=causal, seqlens="fixed",
                 fixed_seqlens=lens, pitch=pitch)
    inp = draw(w, seed=len(lens) * 1000 + h_q, poison=True)
    note(f"[parity] small {case}")
    out, lse, _ = run_gpu(inp, num_parts=parts)
    ref_out, ref_lse = oracle(inp)
    assert_parity(out, lse, ref_out, ref_lse, what=str(case))


def test_empty_and_edge_lengths():
    lens = (0, 1, 63, 64, 65, 127, 128, 129)
    w = Workload("edge", batch=len(lens), s_q=2, h_q=16, causal=True, seqlens="fixed",
                 fixed_seqlens=lens, pitch=640)
    inp = draw(w, seed=5, poison=True)
    note("[parity] edge lengths")
    out, lse, _ = run_gpu(inp, num_parts=3)
    ref_out, ref_lse = oracle(inp)
    assert np.isneginf(ref_lse[0]).all() and np.isneginf(ref_lse[1, 0]).all()
    assert_parity(out, lse, ref_out, ref_lse, what="edge")


@pytest.mark.parametrize("parts", [1, 7, 64, 256, 1024])
def test_split_count_invariance(parts):
    w = Workload("split", batch=3, s_q=2, h_q=128, causal=True, seqlens="fixed",
                 fixed_seqlens=(3000, 70, 1500))
    inp = draw(w, seed=2)
    note(f"[parity] forced parts {parts}")
    out, lse, _ = run_gpu(inp, num_parts=parts)
    ref_out, ref_lse = oracle(inp)
    assert_parity(out, lse, ref_out, ref_lse, what=f"parts={parts}")


def test_internal_plan_equals_explicit_plan():
    inp = draw("tiny")
    a = run_gpu(inp, num_parts=5, use_metadata=False)
    b = run_gpu(inp, num_parts=5, use_metadata=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def plan_in_workspace(ws, parts, batch):
    """The plan a decode without metadata leaves at the start of its workspace:
    tile_md [parts][8] at byte 0, num_splits [batch + 1] from the next 256-byte
    boundary."""
    md = ws[: parts * 32].view(torch.int32).reshape(parts, 8).cpu()
    off = (parts * 32 + 255) // 256 * 256
    return md, ws[off: off + 4 * (batch + 1)].view(torch.int32).cpu()


def decode_planning_in_kernel(inp, parts, dev="cuda:0"):
    """Decode without metadata into a poisoned workspace; returns (out, lse,
    the plan found in the workspace)."""
    g = inp.to(dev)
    w = inp.workload
    ws = torch.full((workspace_size(w.batch, w.s_q, w.h_q, 1, D_V, parts),), 0xA5, dtype=torch.uint8,
                    device=dev)
    out, lse = mla_decode_with_kvcache(g.q, g.blocked_k, g.block_table, g.cache_seqlens, D_V,
                                       w.softmax_scale, w.causal, num_parts=parts, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), plan_in_workspace(ws, parts, w.batch)


def mixed_lengths(batch, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 3000, size=batch)
    lens[rng.random(batch) < 0.2] = 0
    return tuple(int(x) for x in lens)


IN_KERNEL_PLAN_CASES = [
    ("tiny", None), ("tiny", 1), ("tiny", 5), ("v2lite", None), ("v2lite", 1024), ("skewed", None),
    ("wide", None), ("wide", 7), ("mtp", None),
    # 256 sequences: the in-kernel limit, four full blocks of 64 lengths per wave
    (Workload("mixed256", batch=256, s_q=1, h_q=128, causal=False, seqlens="fixed",
              fixed_seqlens=mixed_lengths(256, 3)), 97),
    (Workload("mixed128", batch=128, s_q=1, h_q=128, causal=False, seqlens="fixed",
              fixed_seqlens=mixed_lengths(128, 4)), 300),
    # 257 sequences: past the in-kernel limit, the plan kernel runs first
    (Workload("mixed257", batch=257, s_q=1, h_q=128, causal=False, seqlens="fixed",
              fixed_seqlens=mixed_lengths(257, 5)), 64),
    (Workload("mixed40", batch=40, s_q=1, h_q=32, causal=False, seqlens="fixed",
              fixed_seqlens=mixed_lengths(40, 6)), 23),
    # most parts idle (13 cost units over 64 parts), and a single sequence
    (Workload("idle", batch=3, s_q=1, h_q=128, causal=False, seqlens="fixed",
              fixed_seqlens=(5, 70, 1)), 64),
    (Workload("one", batch=1, s_q=2, h_q=128, causal=True, seqlens="fixed",
              fixed_seqlens=(700,)), 16),
]


@pytest.mark.parametrize("case", IN_KERNEL_PLAN_CASES,
                         ids=[f"{c[0] if isinstance(c[0], str) else c[0].name}-{c[1]}" for c in IN_KERNEL_PLAN_CASES])
def test_plan_without_metadata_equals_the_host_plan(case):
    """A decode called without metadata plans inside its kernel (128-row
    blocks, bf16 cache, up to 256 sequences) or runs the plan kernel first:
    either way the plan it leaves in the workspace is the host plan, and its
    results are bit for bit those of a decode given the plan kernel's
    metadata."""
    name, parts = case
    inp = draw(name, seed=7)
    w = inp.workload
    rows = w.s_q * w.h_q
    parts = parts or default_num_parts(rows)
    note(f"[plan] {w.name} parts={parts}")
    out, lse, (md, ns) = decode_planning_in_kernel(inp, parts)
    hmd, hns = plan_host(inp.cache_seqlens, rows, 1, parts)
    assert torch.equal(md, hmd), f"{w.name}: part records differ"
    assert torch.equal(ns, hns), f"{w.name}: num_splits differ"
    out2, lse2, _ = run_gpu(inp, num_parts=parts, use_metadata=True)
    assert torch.equal(out, out2) and torch.equal(lse, lse2), f"{w.name}: results differ"


def test_device_plan_equals_host_plan():
    for name in ("tiny", "v2lite", "skewed"):
        inp = draw(name)
        w = inp.workload
        rows = w.s_q * w.h_q
        parts = default_num_parts(rows)
        md, ns = get_mla_metadata(inp.cache_seqlens.cuda(), rows, 1, num_parts=parts)
        hmd, hns = plan_host(inp.cache_seqlens, rows, 1, parts)
        assert torch.equal(md.cpu(), hmd) and torch.equal(ns.cpu(), hns), name


def test_one_plan_serves_consecutive_calls():
    """One plan serves several calls in a row (one per layer of a decode
    step), each exact, and no call changes it."""
    w = Workload("layers", batch=6, s_q=2, h_q=128, causal=True, seqlens="fixed",
                 fixed_seqlens=(900, 64, 2100, 1, 333, 1500))
    parts = 9  # every long sequence split in two or three
    meta = None
    for layer in range(3):
        inp = draw(w, seed=20 + layer)
        g = inp.to("cuda:0")
        if meta is None:
            meta = get_mla_metadata(g.cache_seqlens, w.s_q * w.h_q, w.h_kv, num_parts=parts)
            host_md, host_ns = plan_host(inp.cache_seqlens, w.s_q * w.h_q, w.h_kv, parts)
        note(f"[parity] one plan, call {layer}")
        out, lse = mla_decode_with_kvcache(g.q, g.blocked_k, g.block_table, g.cache_seqlens, D_V,
                                           w.softmax_scale, w.causal, metadata=meta)
        torch.cuda.synchronize()
        ref_out, ref_lse = oracle(inp)
        assert_parity(out.cpu(), lse.cpu(), ref_out, ref_lse, what=f"call {layer}")
        md = meta[0].cpu()
        assert torch.equal(md, host_md) and torch.equal(meta[1].cpu(), host_ns), "plan changed"


def test_page_permutation_is_bit_identical():
    w = Workload("perm", batch=3, s_q=2, h_q=64, causal=True, seqlens="fixed",
                 fixed_seqlens=(700, 64, 333))
    inp = draw(w, seed=4)
    a_out, a_lse, _ = run_gpu(inp, num_parts=4)
    nb = inp.k_storage.shape[0]
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(9))
    moved = inp.k_storage.clone()
    moved[perm] = inp.k_storage
    inp.k_storage = moved
    inp.blocked_k = moved[..., :576]
    inp.block_table = perm[inp.block_table.long()].to(torch.int32)
    b_out, b_lse, _ = run_gpu(inp, num_parts=4)
    assert torch.equal(a_out, b_out) and torch.equal(a_lse, b_lse)


def test_pitch_640_is_bit_identical_to_576():
    w = Workload("pitch", batch=2, s_q=1, h_q=128, causal=False, seqlens="fixed",
                 fixed_seqlens=(1000, 129))
    inp = draw(w, seed=6)
    a_out, a_lse, _ = run_gpu(inp, num_parts=3)
    padded = torch.full(inp.k_storage.shape[:-1] + (640,), float("nan"), dtype=torch.bfloat16)
    padded[..., :576] = inp.k_storage
    inp.k_storage = padded
    inp.blocked_k = padded[..., :576]
    b_out, b_lse, _ = run_gpu(inp, num_parts=3)
    assert torch.equal(a_out, b_out) and torch.equal(a_lse, b_lse)


def test_results_are_deterministic():
    inp = draw("v2lite")
    a = run_gpu(inp)
    b = run_gpu(inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def ramp_scores(inp, per_token=0.125, q_value=4.0):
    """Make scores grow along each sequence: q[..., 0] = q_value, k_t[0] = t * per_token.

    With softmax_scale 1/sqrt(192) the score of token t is about 0.036 t (natural
    units) on top of the random part, so the running max passes the kernel's
    rescale slack several times over a few hundred tokens.
    """
    inp.q[..., 0] = q_value
    for b in range(inp.block_table.shape[0]):
        n = int(inp.cache_seqlens[b])
        for t in range(n):
            inp.k_storage[int(inp.block_table[b, t // 64]), t % 64, :, 0] = t * per_token
    return inp


@pytest.mark.parametrize("h_q,s_q,causal,parts", [(16, 1, False, 1), (32, 2, True, 2),
                                                   (128, 1, False, 3), (128, 2, True, 1)])
def test_growing_scores_exercise_the_rescale(h_q, s_q, causal, parts):
    w = Workload("ramp", batch=2, s_q=s_q, h_q=h_q, causal=causal, seqlens="fixed",
                 fixed_seqlens=(1500, 700))
    inp = ramp_scores(draw(w, seed=8))
    note(f"[parity] growing scores h_q={h_q} s_q={s_q} parts={parts}")
    out, lse, _ = run_gpu(inp, num_parts=parts)
    ref_out, ref_lse = oracle(inp)
    assert float(ref_lse.max()) > 40.0  # far past several rescale thresholds
    assert_parity(out, lse, ref_out, ref_lse, what="ramp")


@pytest.mark.parametrize("log2_scale", [17, -20])
def test_split_partials_outside_the_fp16_range(log2_scale):
    """Split sequences whose weighted values leave fp16's normal range: the
    cache is scaled by 2^s and the queries by 2^-s (exact in bf16), so every
    score is unchanged and every O / l is 2^s times the unscaled one -- above
    fp16's largest value at s = 17, below its smallest normal at s = -20 (the
    wide kernel rewrites such a partial row with a power-of-two scale).  Both
    sides are compared at the unscaled magnitude (out / 2^s against ref / 2^s,
    exact): the bound's floor of 1 is not scale-invariant, and an element that
    cancels carries an error proportional to its row's scale (P is bf16)."""
    w = Workload("fp16range", batch=3, s_q=1, h_q=128, causal=False, seqlens="fixed",
                 fixed_seqlens=(1500, 900, 2100))
    inp = draw(w, seed=31)
    f = 2.0 ** log2_scale
    inp.k_storage.mul_(f)
    inp.q.mul_(1.0 / f)
    note(f"[parity] split partials scaled by 2^{log2_scale}")
    out, lse, _ = run_gpu(inp, num_parts=7)
    ref_out, ref_lse = oracle(inp)
    peak = float(np.abs(ref_out).max())
    assert (peak > 65504.0) if log2_scale > 0 else (peak < 2.0 ** -14)
    assert_parity(out.float() / f, lse, ref_out / f, ref_lse, what=f"partials x2^{log2_scale}")


def test_maximum_rows():
    """s_q * h_q at the library's limit (1024 rows: eight row blocks), causal."""
    w = Workload("maxrows", batch=3, s_q=8, h_q=128, causal=True, seqlens="fixed",
                 fixed_seqlens=(70, 9, 200))
    inp = draw(w, seed=21, poison=True)
    note("[parity] maximum rows s_q=8 h_q=128")
    out, lse, _ = run_gpu(inp, num_parts=5)
    ref_out, ref_lse = oracle(inp)
    assert_parity(out, lse, ref_out, ref_lse, what="max rows")


def test_large_batch_of_short_sequences():
    """2048 sequences of 1..300 tokens in one call (many parts touch several
    sequences each), every sequence against the oracle."""
    rng = np.random.default_rng(5)
    lens = tuple(int(x) for x in rng.integers(1, 301, size=2048))
    w = Workload("batch", batch=len(lens), s_q=1, h_q=16, causal=False, seqlens="fixed",
                 fixed_seqlens=lens)
    inp = draw(w, seed=22)
    note("[parity] 2048 short sequences")
    out, lse, _ = run_gpu(inp)
    ref_out, ref_lse = oracle(inp)
    assert_parity(out, lse, ref_out, ref_lse, what="large batch")


@pytest.mark.parametrize("h_q,parts", [(128, 2), (128, 5), (128, 9), (16, 2), (16, 5)])
def test_lengths_past_the_table_are_clamped(h_q, parts):
    """A stored length past max_blocks_per_seq * 64 reads as the clamped length.

    The plan cuts parts by the stored lengths, so some parts start past the
    clamp of the first sequence; the sequences after it must still come out
    right, and the clamped one equal to the decode of its first 128 tokens.
    """
    w = Workload("clamp", batch=3, s_q=1, h_q=h_q, causal=False, seqlens="fixed",
                 fixed_seqlens=(128, 100, 128))
    inp = draw(w, seed=31, poison=True)
    inp.block_table = inp.block_table[:, :2].contiguous()  # cap: 2 pages = 128 tokens
    ref_out, ref_lse = oracle(inp)
    inp.cache_seqlens = torch.tensor([1000, 100, 129], dtype=torch.int32)
    note(f"[parity] clamped lengths h_q={h_q} parts={parts}")
    out, lse, _ = run_gpu(inp, num_parts=parts)
    assert_parity(out, lse, ref_out, ref_lse, what=f"clamp h_q={h_q} parts={parts}")
    # without metadata: the 128-row kernel plans for itself and counts the
    # clamped lengths; the 16-row one runs the plan kernel on the stored ones
    note(f"[parity] clamped lengths, no metadata, h_q={h_q} parts={parts}")
    out, lse, (md, ns) = decode_planning_in_kernel(inp, parts)
    assert_parity(out, lse, ref_out, ref_lse, what=f"clamp, no metadata, h_q={h_q} parts={parts}")
    planned = [128, 100, 128] if h_q == 128 else [1000, 100, 129]
    hmd, hns = plan_host(torch.tensor(planned, dtype=torch.int32), h_q, 1, parts)
    assert torch.equal(md, hmd) and torch.equal(ns, hns)


@pytest.mark.parametrize("h_q,kv", [(128, "bf16"), (16, "bf16"), (128, "fp8_e4m3")])
def test_negative_lengths_read_as_empty(h_q, kv):
    """A negative stored length is an empty sequence (out 0, lse -inf); the
    sequences around it are unaffected."""
    w = Workload("neg", batch=3, s_q=2, h_q=h_q, causal=True, seqlens="fixed",
                 fixed_seqlens=(300, 0, 700), kv_format=kv,
                 kv_scale=FP8_KV_SCALE if kv == "fp8_e4m3" else 1.0)
    inp = draw(w, seed=33, poison=True)
    ref_out, ref_lse = oracle(inp)
    inp.cache_seqlens = torch.tensor([300, -5, 700], dtype=torch.int32)
    note(f"[parity] negative length h_q={h_q} {kv}")
    out, lse, _ = run_gpu(inp, num_parts=5)
    assert_parity(out, lse, ref_out, ref_lse, what=f"negative length h_q={h_q} {kv}")


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes(seed):
    """Seeded random shapes: odd head counts (rows not a multiple of 16 or 32),
    one to four query tokens, both pitches, random part counts, poisoned cache."""
    from paged_mla_decode_04_amd.workloads import random_case
    g = torch.Generator().manual_seed(1000 + seed)
    w = random_case(g, max_batch=4, s_q_choices=(1, 2, 3, 4),
                    h_q_choices=(1, 3, 8, 16, 24, 48, 64, 96, 128, 160, 256), max_len=700)
    if w.s_q * w.h_q > 1024:
        w = Workload(**{**w.__dict__, "s_q": 1})
    parts = int(torch.randint(1, 65, (1,), generator=g))
    inp = draw(w, seed=seed, poison=True)
    note(f"[parity] random seed={seed}: b={w.batch} s_q={w.s_q} h_q={w.h_q} causal={w.causal} "
         f"pitch={w.pitch} lens={w.fixed_seqlens} parts={parts}")
    out, lse, _ = run_gpu(inp, num_parts=parts)
    ref_out, ref_lse = oracle(inp)
    assert_parity(out, lse, ref_out, ref_lse, what=f"random {seed}")


# ------------------------------------------------------------- FP8 E4M3 cache

FP8_SMALL = [
    # (seqlens, s_q, h_q, causal, pitch, parts)
    ((37, 130), 1, 16, False, 576, None),
    ((1, 64, 65, 200), 2, 16, True, 640, 5),
    ((300, 7, 129), 1, 128, False, 576, 3),
    ((513, 64, 2), 2, 128, True, 640, 7),
    ((129, 300, 64, 5), 1, 256, False, 576, 6),
    ((90, 33, 1000), 2, 64, True, 576, 4),
    ((0, 1, 63, 64, 65, 127, 128, 129), 2, 32, True, 640, 3),
]


@pytest.mark.parametrize("case", FP8_SMALL, ids=[f"fp8_small{i}" for i in range(len(FP8_SMALL))])
def test_fp8_cache_small_cases(case):
    lens, s_q, h_q, causal, pitch, parts = case
    w = Workload("fp8small", batch=len(lens), s_q=s_q, h_q=h_q, causal=causal, seqlens="fixed",
                 fixed_seqlens=lens, pitch=pitch, kv_format="fp8_e4m3", kv_scale=FP8_KV_SCALE)
    inp = draw(w, seed=len(lens) * 1000 + h_q, poison=True)
    note(f"[parity] fp8 small {case}")
    out, lse, _ = run_gpu(inp, num_parts=parts)
    ref_out, ref_lse = oracle(inp)
    assert_parity(out, lse, ref_out, ref_lse, what=f"fp8 {case}")


@pytest.mark.parametrize("name", ["wide", "mtp"])
def test_fp8_cache_full_size(name):
    """The wide-head and two-token workloads with their cache stored as E4M3 bytes
    (same shapes, lengths and pages), every sequence against the oracle."""
    base = WORKLOADS[name]
    w = Workload(**{**base.__dict__, "name": name + "_fp8", "kv_format": "fp8_e4m3",
                    "kv_scale": FP8_KV_SCALE})
    note(f"[parity] fp8 workload {name}: drawing inputs")
    inp = draw(w)
    out, lse, _ = run_gpu(inp)
    note(f"[parity] fp8 workload {name}: oracle on all {w.batch} sequences")
    ref_out, ref_lse = oracle(inp)
    worst = assert_parity(out, lse, ref_out, ref_lse, what=f"fp8 {name}")
    note(f"[parity] fp8 workload {name}: worst out error {worst:.3f} of the bound")


def test_fp8_single_token_returns_every_code_exactly():
    """One cached token whose 576 bytes run through every finite E4M3 code: out is
    its first 512 values times the scale, exactly (each is a bf16 number)."""
    w = Workload("fp8codes", batch=1, s_q=1, h_q=16, causal=False, seqlens="fixed",
                 fixed_seqlens=(1,), kv_format="fp8_e4m3", kv_scale=0.5)
    inp = draw(w, seed=3)
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    row = torch.tensor((finite * 3)[:576], dtype=torch.uint8)
    inp.k_storage[int(inp.block_table[0, 0]), 0, 0, :576] = row
    out, lse, _ = run_gpu(inp, num_parts=1)
    ref_out, ref_lse = oracle(inp)
    assert np.array_equal(out.float().numpy().astype(np.float64), ref_out)
    assert np.all(np.abs(lse.numpy() - ref_lse) <= LSE_TOL)


def test_fp8_scale_folds_into_scores_and_output():
    """kv_scale s on the GPU equals the decode at kv_scale 1 with softmax_scale * s,
    times s (the oracle's closed form, now on the HIP path)."""
    w = Workload("fp8scale", batch=2, s_q=1, h_q=128, causal=False, seqlens="fixed",
                 fixed_seqlens=(700, 90), kv_format="fp8_e4m3", kv_scale=0.25)
    inp = draw(w, seed=12)
    a_out, a_lse, _ = run_gpu(inp, num_parts=3)
    ref_out, ref_lse = oracle(inp)
    assert_parity(a_out, a_lse, ref_out, ref_lse, what="fp8 scale 0.25")


def _fp8_inputs(lens, s_q, h_q, causal, seed):
    w = Workload("fp8inv", batch=len(lens), s_q=s_q, h_q=h_q, causal=causal, seqlens="fixed",
                 fixed_seqlens=lens, kv_format="fp8_e4m3", kv_scale=FP8_KV_SCALE)
    return draw(w, seed=seed)


def test_fp8_page_permutation_and_pitch_are_bit_identical():
    """With an fp8 cache, moving the pages (and the table with them) and storing
    the entries at a 640-byte pitch change no bit of the results."""
    inp = _fp8_inputs((700, 64, 333), 2, 128, True, seed=14)
    a_out, a_lse, _ = run_gpu(inp, num_parts=4)
    nb = inp.k_storage.shape[0]
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(15))
    moved = inp.k_storage.clone()
    moved[perm] = inp.k_storage
    padded = torch.full(moved.shape[:-1] + (640,), 0x7F, dtype=torch.uint8)  # E4M3 NaN bytes
    padded[..., :576] = moved
    inp.k_storage = padded
    inp.blocked_k = padded[..., :576]
    inp.block_table = perm[inp.block_table.long()].to(torch.int32)
    note("[parity] fp8 permuted pages at pitch 640")
    b_out, b_lse, _ = run_gpu(inp, num_parts=4)
    assert torch.equal(a_out, b_out) and torch.equal(a_lse, b_lse)


@pytest.mark.parametrize("parts", [1, 7, 64, 256])
def test_fp8_split_count_invariance(parts):
    inp = _fp8_inputs((3000, 70, 1500), 2, 128, True, seed=16)
    note(f"[parity] fp8 forced parts {parts}")
    out, lse, _ = run_gpu(inp, num_parts=parts)
    ref_out, ref_lse = oracle(inp)
    assert_parity(out, lse, ref_out, ref_lse, what=f"fp8 parts={parts}")
