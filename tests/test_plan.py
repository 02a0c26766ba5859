"""Invariants of the split-KV plan (host mirror; the GPU plan must equal it).

A plan is valid when, over the flattened (sequence, page) order with one
(possibly empty) unit for a sequence of no tokens, the parts cover every unit
exactly once, in order, as contiguous ranges; num_splits holds the prefix sums
of the number of parts touching each sequence; and each part's first-sequence
split index counts the earlier parts touching that sequence.  Plans are not
unique -- any such cover is correct -- so the balance is checked as a bound.
"""

import random

import pytest
import torch

from paged_mla_decode_04_amd import _lib, plan_host


@pytest.fixture(scope="module", autouse=True)
def lib():
    import os
    if not os.path.exists(_lib.LIB_PATH):
        from paged_mla_decode_04_amd import build
        build.build()
    return _lib.load()


def units(n):
    return max(1, -(-int(n) // 64))


def seg_cost(q_rows):
    r = 16 if q_rows <= 16 else 32 if q_rows <= 32 else 64 if q_rows <= 64 else 128
    return 3 if r == 128 else max(1, (r + 27) // 28)


def check_plan(seqlens, q_rows, num_parts, md, ns):
    b = len(seqlens)
    md = md.tolist()
    ns = ns.tolist()
    assert ns[0] == 0
    flat = [(s, p) for s in range(b) for p in range(units(seqlens[s]))]
    covered = []
    touches = [0] * b
    for part in md:
        sb, pb, sl, pe, first = part[:5]
        assert part[5:] == [0, 0, 0]
        if sb == b:
            assert (pb, sl, pe, first) == (0, b, 0, 0)
            continue
        assert 0 <= sb <= sl < b
        assert first == touches[sb]
        for s in range(sb, sl + 1):
            lo = pb if s == sb else 0
            hi = pe if s == sl else units(seqlens[s])
            assert 0 <= lo < hi <= units(seqlens[s]), (part, s)
            covered += [(s, p) for p in range(lo, hi)]
            touches[s] += 1
    assert covered == flat
    for s in range(b):
        assert ns[s + 1] - ns[s] == touches[s]
    # idle parts only after the busy ones
    busy = [p[0] < b for p in md]
    assert busy == sorted(busy, reverse=True)
    return md


def part_cost(part, seqlens, c):
    sb, pb, sl, pe = part[:4]
    if sb == len(seqlens):
        return 0
    cost = 0
    for s in range(sb, sl + 1):
        lo = pb if s == sb else 0
        hi = pe if s == sl else units(seqlens[s])
        cost += hi - lo + c
    return cost


CASES = [
    ([37, 130], 16, 256),
    ([37, 130], 16, 1),
    ([37, 130], 16, 2),
    ([0], 16, 4),
    ([0, 0, 5], 128, 3),
    ([64, 65, 1, 128], 128, 5),
    ([32768] + [1] * 15, 128, 128),
    (list(range(1, 300, 7)), 256, 64),
    ([4096] * 128, 128, 128),
]


@pytest.mark.parametrize("seqlens,q_rows,parts", CASES)
def test_plan_covers_each_unit_once(seqlens, q_rows, parts):
    md, ns = plan_host(seqlens, q_rows, 1, parts)
    check_plan(seqlens, q_rows, parts, md, ns)


@pytest.mark.parametrize("seed", range(40))
def test_random_plans_are_valid_and_balanced(seed):
    rng = random.Random(seed)
    b = rng.randint(1, 200)
    kind = rng.choice(["uniform", "skew", "tiny", "zeros"])
    if kind == "uniform":
        seqlens = [rng.randint(1, 8192) for _ in range(b)]
    elif kind == "skew":
        seqlens = [int(2 ** rng.uniform(0, 15)) for _ in range(b)]
    elif kind == "tiny":
        seqlens = [rng.randint(0, 70) for _ in range(b)]
    else:
        seqlens = [rng.choice([0, 0, 1, 64, 4096]) for _ in range(b)]
    q_rows = rng.choice([16, 32, 64, 128, 256])
    parts = rng.choice([1, 2, 7, 64, 128, 256, 1024])
    md, ns = plan_host(seqlens, q_rows, 1, parts)
    md = check_plan(seqlens, q_rows, parts, md, ns)
    c = seg_cost(q_rows)
    total = sum(units(n) + c for n in seqlens)
    stride = max(c + 1, -(-total // parts))
    costs = [part_cost(p, seqlens, c) for p in md]
    busy = [x for x, p in zip(costs, md) if p[0] < b]
    # each part owns `stride` cost positions; one that starts inside a sequence
    # pays one more segment overhead
    assert all(x <= stride + c for x in busy), (busy, stride)
    # and no part is idle while work remains for it
    assert len(busy) == min(parts, -(-total // stride))


def test_grouped_rows_divide_by_kv_heads():
    a = plan_host([100, 900], 32, 2, 8)
    b = plan_host([100, 900], 16, 1, 8)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_plan_rejects_bad_arguments():
    with pytest.raises(ValueError):
        plan_host([1, 2], 16, 1, 0)
    with pytest.raises(ValueError):
        plan_host([1, 2], 4096, 1, 4)


# ---- the plan the decode kernels derive for themselves (no metadata passed)
#
# Each wave finds its part from two passes over the lengths, 64 at a time,
# and starts the split bookkeeping from closed forms instead of the full
# scan of touch counts.  This restates that procedure in Python and checks it
# against the host mirror: the part records, num_splits at each part's first
# sequence, and the per-part lists (and which part publishes each entry).

def in_kernel_part(seqlens, c, P, p):
    """One wave's part record and (prefix, num_splits) at its first sequence."""
    B = len(seqlens)
    u = [c + units(n) for n in seqlens]
    W = sum(u)
    T = max(c + 1, -(-W // P))
    x, xn = p * T, p * T + T
    if x >= W:
        return [B, 0, B, 0, 0, 0, 0, 0], None
    carry, b, nb, K, u_prev_last = 0, None, None, 0, None
    for base in range(0, B, 64):
        lanes = range(base, min(B, base + 64))
        excl = {}
        for i in lanes:
            excl[i] = carry
            carry += u[i]
        # sequences j >= 1 whose window [prefix[j], prefix[j] + c] holds a multiple of T
        window = [i for i in lanes if i >= 1 and (excl[i] % T == 0 or excl[i] % T >= T - c)]
        hx = [i for i in lanes if excl[i] <= x < excl[i] + u[i]]
        if b is None:
            if hx:
                b, pre_b = hx[0], excl[hx[0]]
                K += sum(1 for i in window if i < b)
            else:
                K += len(window)
        hn = [i for i in lanes if excl[i] <= xn < excl[i] + u[i]]
        if hn:
            nb, pre_nb = hn[0], excl[hn[0]]
            u_nbm1 = u[nb - 1] if nb - 1 >= base else u_prev_last
        u_prev_last = u[lanes[-1]]
    pg = max(0, x - pre_b - c)
    if xn >= W:
        eb, epg = B - 1, u[B - 1] - c
    elif xn - pre_nb - c > 0:
        eb, epg = nb, xn - pre_nb - c
    else:
        eb, epg = nb - 1, u_nbm1 - c
    first = p - (pre_b + c) // T if pg > 0 else 0
    ns_b = 0 if b == 0 else b + (pre_b - 1) // T - K
    return [b, pg, eb, epg, first, 0, 0, 0], (pre_b, ns_b, T)


@pytest.mark.parametrize("seed", range(300))
def test_in_kernel_plan_closed_forms_match_the_host_plan(seed):
    rng = random.Random(1000 + seed)
    b = rng.choice([1, 2, 3, 16, 63, 64, 65, 128, 129, 256])
    pick = rng.random()
    if pick < 0.3:
        seqlens = [rng.randint(0, 200) for _ in range(b)]
    elif pick < 0.6:
        seqlens = [rng.randint(0, 9000) for _ in range(b)]
    else:
        seqlens = [rng.choice([0, 1, 63, 64, 65, 4096, 32768]) for _ in range(b)]
    q_rows = rng.choice([16, 32, 128, 256])
    parts = rng.choice([1, 2, 7, 64, 256, 1024])
    c = seg_cost(q_rows)
    md, ns = plan_host(torch.tensor(seqlens, dtype=torch.int32), q_rows, 1, parts)
    md, ns = md.tolist(), ns.tolist()
    published = [0] + [None] * b
    for p in range(parts):
        rec, start = in_kernel_part(seqlens, c, parts, p)
        assert rec == md[p], (p, rec, md[p])
        if start is None:
            continue
        pre, nsc, T = start
        assert nsc == ns[rec[0]]
        for s in range(rec[0], rec[2] + 1):  # the part's list, built forward
            nxt = pre + c + units(seqlens[s])
            touch = (nxt - 1) // T - (pre + c) // T + 1
            assert (nsc, nsc + touch) == (ns[s], ns[s + 1])
            if (nxt - 1) // T == p:  # the part holding s's last unit publishes it
                assert published[s + 1] is None
                published[s + 1] = nsc + touch
            pre, nsc = nxt, nsc + touch
    assert published == ns
