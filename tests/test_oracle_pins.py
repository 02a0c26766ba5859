"""Pins of the CPU oracle against things other than itself.

Each check ties oracle.mla_ref to something independent: the scalar brute
force, closed forms of the softmax average, invariants of paging, layout,
causal alignment and key splitting, and torch's own fp64
scaled_dot_product_attention / logsumexp on gathered tensors.  The last test
plants plausible mistakes in the oracle and shows that each one trips at
least one pin.
"""

import math

import numpy as np
import pytest
import torch

from conftest import bits, f64
from oracle import mla_ref
from oracle.brute import brute_decode
from paged_mla_decode_04_amd.workloads import (D_QK, D_V, BLOCK_SIZE, Workload, draw,
                                               random_case)

TIGHT = 1e-12


def run_oracle(inp, **kw):
    return mla_ref.mla_decode_ref(bits(inp.q), bits(inp.k_storage), inp.block_table.numpy(),
                                  inp.cache_seqlens.numpy(), inp.softmax_scale, inp.causal, **kw)


def case(lens, *, s_q=1, h_q=2, causal=False, pitch=576, h_kv=1, table="randperm", seed=0,
         scale=1.0 / math.sqrt(192.0)):
    w = Workload("case", batch=len(lens), s_q=s_q, h_q=h_q, causal=causal, seqlens="fixed",
                 fixed_seqlens=tuple(lens), pitch=pitch, table=table, h_kv=h_kv,
                 softmax_scale=scale)
    return draw(w, seed=seed)


def close(a, b, tol=TIGHT):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    same_inf = (np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b)))
    diff = np.where(same_inf, 0.0, np.abs(a - b))
    return bool(np.all(diff <= tol * np.maximum(1.0, np.abs(np.where(same_inf, 0, b)))))


def brute_of(inp):
    return brute_decode(bits(inp.q), bits(inp.k_storage), inp.block_table.numpy(),
                        inp.cache_seqlens.numpy(), inp.softmax_scale, inp.causal)


# ---------------------------------------------------------------- brute force

def test_tiny_workload_matches_brute_force():
    inp = draw("tiny")
    out, lse = run_oracle(inp)
    bo, bl = brute_of(inp)
    assert close(out, np.array(bo))
    assert close(lse, np.array(bl))


@pytest.mark.parametrize("seed", range(10))
def test_random_small_cases_match_brute_force(seed):
    w = random_case(seed, max_batch=3, h_q_choices=(1, 2, 4), max_len=70)
    inp = draw(w, seed=seed)
    out, lse = run_oracle(inp)
    bo, bl = brute_of(inp)
    assert close(out, np.array(bo)), w
    assert close(lse, np.array(bl)), w


def test_grouped_kv_heads_match_brute_force():
    inp = case([5, 66], s_q=2, h_q=4, h_kv=2, causal=True, pitch=640)
    out, lse = run_oracle(inp)
    bo, bl = brute_of(inp)
    assert close(out, np.array(bo)) and close(lse, np.array(bl))


# --------------------------------------------------------------- closed forms

def test_single_token_returns_its_value_row():
    inp = case([1, 1, 1], h_q=3)
    out, lse = run_oracle(inp)
    for b in range(3):
        phys = int(inp.block_table[b, 0])
        k = f64(inp.blocked_k[phys, 0, 0])
        for h in range(3):
            assert np.array_equal(out[b, 0, h], k[:D_V])
            s = inp.softmax_scale * float(np.dot(f64(inp.q[b, 0, h]), k))
            assert abs(lse[b, 0, h] - s) <= 1e-13 * max(1, abs(s))


@pytest.mark.parametrize("n", [2, 63, 64, 65, 200])
def test_equal_scores_give_mean_value_and_score_plus_log_n(n):
    inp = case([n], h_q=2)
    inp.q[..., :D_V] = 0
    rope = torch.randn(D_QK - D_V, generator=torch.Generator().manual_seed(n)).to(torch.bfloat16)
    inp.k_storage[..., D_V:D_QK] = rope
    out, lse = run_oracle(inp)
    table = inp.block_table[0]
    V = np.stack([f64(inp.blocked_k[int(table[t // BLOCK_SIZE]), t % BLOCK_SIZE, 0, :D_V])
                  for t in range(n)])
    for h in range(2):
        s = inp.softmax_scale * float(np.dot(f64(inp.q[0, 0, h, D_V:]), f64(rope)))
        assert close(lse[0, 0, h], s + math.log(n))
        assert close(out[0, 0, h], V.mean(axis=0))


def test_zero_query_gives_log_n():
    inp = case([17, 130], h_q=2)
    inp.q.zero_()
    out, lse = run_oracle(inp)
    for b, n in enumerate([17, 130]):
        assert close(lse[b], np.full((1, 2), math.log(n)))


def test_no_visible_key_gives_zero_and_minus_inf():
    inp = case([0, 1, 5], s_q=2, h_q=2, causal=True)
    out, lse = run_oracle(inp)
    assert np.all(lse[0] == -np.inf) and np.all(out[0] == 0)
    assert np.all(lse[1, 0] == -np.inf) and np.all(out[1, 0] == 0)
    assert np.all(np.isfinite(lse[1, 1])) and np.all(np.isfinite(lse[2]))


# ----------------------------------------------------------------- invariants

def test_physical_page_permutation_is_invisible():
    inp = case([37, 130, 64], h_q=4, s_q=2, causal=True)
    out, lse = run_oracle(inp)
    nb = inp.k_storage.shape[0]
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(7))
    moved = inp.k_storage.clone()
    moved[perm] = inp.k_storage
    inp.k_storage = moved
    inp.blocked_k = moved[..., :D_QK]
    inp.block_table = perm[inp.block_table.long()].to(torch.int32)
    out2, lse2 = run_oracle(inp)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_entry_pitch_640_matches_576():
    a = case([37, 130], h_q=4, pitch=576)
    out, lse = run_oracle(a)
    padded = torch.full(a.k_storage.shape[:-1] + (640,), float("nan"), dtype=torch.bfloat16)
    padded[..., :D_QK] = a.k_storage
    a.k_storage = padded
    a.blocked_k = padded[..., :D_QK]
    out2, lse2 = run_oracle(a)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("n", [1, 2, 64, 65, 300])
def test_causal_two_token_rows_reduce_to_single_token(n):
    two = case([n], s_q=2, h_q=4, causal=True, seed=n)
    out2, lse2 = run_oracle(two)
    for row, (cut, ) in enumerate([(n - 1,), (n,)]):
        one = case([n], s_q=1, h_q=4, causal=False, seed=n)
        one.q = two.q[:, row:row + 1].clone()
        one.k_storage, one.blocked_k, one.block_table = two.k_storage, two.blocked_k, two.block_table
        one.cache_seqlens = torch.tensor([cut], dtype=torch.int32)
        out1, lse1 = run_oracle(one)
        assert np.array_equal(out2[:, row], out1[:, 0]), row
        assert np.array_equal(lse2[:, row], lse1[:, 0]), row


@pytest.mark.parametrize("cuts", [(0, 37, 130), (0, 64, 128, 130), (0, 1, 1, 129, 130), (0, 130)])
def test_key_splits_merge_to_the_whole(cuts):
    inp = case([130], h_q=4, s_q=2, causal=True, seed=3)
    out, lse = run_oracle(inp)
    parts = [run_oracle(inp, token_range=(lo, hi)) for lo, hi in zip(cuts[:-1], cuts[1:])]
    mo, ml = mla_ref.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    assert close(mo, out) and close(ml, lse)


def test_merge_of_only_empty_partials_is_empty():
    o = np.ones((3, 4))
    l = np.full(3, -np.inf)
    mo, ml = mla_ref.merge_partials([o, o], [l, l])
    assert np.all(ml == -np.inf) and np.all(mo == 0)


def test_sequences_are_independent():
    inp = case([37, 130, 70], h_q=2)
    out, lse = run_oracle(inp)
    for b in range(3):
        one = case([int(inp.cache_seqlens[b])], h_q=2)
        one.q = inp.q[b:b + 1].clone()
        one.k_storage, one.blocked_k = inp.k_storage, inp.blocked_k
        one.block_table = inp.block_table[b:b + 1].clone()
        o1, l1 = run_oracle(one)
        assert np.array_equal(o1[0], out[b]) and np.array_equal(l1[0], lse[b])


def test_head_permutation_permutes_rows():
    inp = case([90], h_q=8)
    out, lse = run_oracle(inp)
    perm = torch.randperm(8, generator=torch.Generator().manual_seed(1))
    inp.q = inp.q[:, :, perm].clone()
    out2, lse2 = run_oracle(inp)
    assert np.array_equal(out2, out[:, :, perm.numpy()])
    assert np.array_equal(lse2, lse[:, :, perm.numpy()])


# ------------------------------------------------------ library special case

@pytest.mark.parametrize("s_q,causal", [(1, False), (2, True), (2, False)])
def test_matches_torch_sdpa_on_gathered_tensors(s_q, causal):
    inp = case([37, 130, 200], s_q=s_q, h_q=4, causal=causal, seed=5)
    out, lse = run_oracle(inp)
    for b in range(3):
        n = int(inp.cache_seqlens[b])
        pages = inp.block_table[b, :(n + 63) // 64].long()
        K = inp.blocked_k[pages].reshape(-1, D_QK)[:n].to(torch.float64)
        V = K[:, :D_V]
        Q = inp.q[b].to(torch.float64).reshape(s_q * 4, D_QK)
        tok = torch.arange(s_q).repeat_interleave(4)
        vis = (n - (s_q - 1 - tok)) if causal else torch.full_like(tok, n)
        mask = torch.arange(n)[None, :] < vis[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[None], K[None], V[None], attn_mask=mask[None], scale=inp.softmax_scale)[0]
        scores = inp.softmax_scale * Q @ K.T
        ref_lse = torch.logsumexp(scores.masked_fill(~mask, -math.inf), dim=-1)
        assert close(out[b].reshape(s_q * 4, D_V), ref.numpy(), 1e-11)
        assert close(lse[b].reshape(-1), ref_lse.numpy(), 1e-12)


# ------------------------------------------------ planted mistakes are caught

def _pin_failures():
    """A compact run of the pins above; returns the names of those that fail."""
    failed = []
    try:
        inp = case([5, 70], s_q=2, h_q=2, causal=True, pitch=640, seed=11)
        out, lse = run_oracle(inp)
        bo, bl = brute_of(inp)
        if not (close(out, np.array(bo)) and close(lse, np.array(bl))):
            failed.append("brute")
    except Exception:
        failed.append("brute-crash")
    try:
        test_single_token_returns_its_value_row()
    except Exception:
        failed.append("single")
    try:
        test_equal_scores_give_mean_value_and_score_plus_log_n(65)
    except Exception:
        failed.append("equal")
    try:
        test_matches_torch_sdpa_on_gathered_tensors(2, True)
    except Exception:
        failed.append("sdpa")
    try:
        test_key_splits_merge_to_the_whole((0, 64, 128, 130))
    except Exception:
        failed.append("split")
    return failed


def _mut_drop_rope(orig):
    def f(*a, **k):
        K = orig(*a, **k).copy()
        K[:, D_V:] = 0
        return K
    return f


def _mut_v_tail(orig):
    def f(q_rows, K, counts, scale, dv=D_V, t_begin=0):
        R = q_rows.shape[0]
        out, lse = np.zeros((R, dv)), np.full(R, -np.inf)
        scores = scale * (q_rows @ K.T) if K.shape[0] else np.zeros((R, 0))
        V = K[:, K.shape[1] - dv:]
        for r in range(R):
            hi = int(counts[r])
            out[r], lse[r] = mla_ref.softmax_average(scores[r, t_begin:hi], V[t_begin:hi])
        return out, lse
    return f


def _mut_causal_off_by_one(orig):
    return lambda n, s_q, i, causal: max(0, n - (s_q - i)) if causal else max(0, n)


def _mut_no_scale(orig):
    return lambda q_rows, K, counts, scale, dv=D_V, t_begin=0: orig(q_rows, K, counts, 1.0, dv, t_begin)


def _mut_lse_base2(orig):
    def f(scores, values):
        o, l = orig(scores, values)
        return o, l / math.log(2) if np.isfinite(l) else l
    return f


def _mut_page_row_swap(orig):
    def f(k_bits, table_row, n, kv_head, block_size=BLOCK_SIZE, d=D_QK):
        t = np.arange(n)
        phys = np.asarray(table_row)[np.minimum(t % block_size, len(table_row) - 1)]
        return mla_ref.bf16_bits_to_f64(k_bits[phys, t // block_size, kv_head, :d])
    return f


def _mut_bf16_decode(orig):
    def f(b):
        u = np.asarray(b).astype(np.uint16).astype(np.uint32) << np.uint32(15)
        return u.view(np.float32).astype(np.float64)
    return f


def _mut_unshifted_exp(orig):
    def f(scores, values):
        if scores.shape[0] == 0:
            return np.zeros(values.shape[1]), -np.inf
        m = scores.max()
        w = np.exp(scores - m)
        lse = m + np.log(w.sum())
        return (w @ values) / len(scores), lse
    return f


MUTATIONS = {
    "drop_rope": ("gather_tokens", _mut_drop_rope),
    "v_from_tail": ("attend_rows", _mut_v_tail),
    "causal_off_by_one": ("visible_keys", _mut_causal_off_by_one),
    "no_scale": ("attend_rows", _mut_no_scale),
    "lse_base2": ("softmax_average", _mut_lse_base2),
    "page_row_swap": ("gather_tokens", _mut_page_row_swap),
    "bf16_decode": ("bf16_bits_to_f64", _mut_bf16_decode),
    "mean_not_softmax": ("softmax_average", _mut_unshifted_exp),
}


def test_pins_pass_on_the_oracle():
    assert _pin_failures() == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_each_planted_mistake_trips_a_pin(name, monkeypatch):
    attr, make = MUTATIONS[name]
    monkeypatch.setattr(mla_ref, attr, make(getattr(mla_ref, attr)))
    assert _pin_failures() != [], name
