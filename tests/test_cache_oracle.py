"""Pins of the cache-write oracle (CPU): what appending and copying must leave
in a cache, checked against constructions that do not go through it."""

import numpy as np

from oracle import mla_ref
from oracle.mla_cache_ref import ENTRY, append_ref, copy_blocks_ref

NAN = 0x7FC0


def rand_bits(rng, shape):
    return rng.integers(0, 0x7F00, size=shape, dtype=np.uint16)  # finite bf16 patterns


def test_appending_a_sequence_builds_the_cache_the_decode_reads():
    """Tokens appended one slot at a time through a block table give, for the
    decode oracle, the same result as that cache written directly row by row."""
    rng = np.random.default_rng(0)
    n, pitch, nblocks = 150, 640, 5
    table = np.array([[3, 0, 4]], dtype=np.int32)
    rows = rand_bits(rng, (n, ENTRY)) & 0x3FFF        # modest magnitudes
    direct = np.full((nblocks, 64, 1, pitch), NAN, dtype=np.uint16)
    for t in range(n):
        direct[table[0, t // 64], t % 64, 0, :ENTRY] = rows[t]
    slots = np.array([table[0, t // 64] * 64 + t % 64 for t in range(n)])
    start = np.full((nblocks, 64, 1, pitch), NAN, dtype=np.uint16)
    built = append_ref(start, rows[:, :512], rows[:, 512:], slots)
    assert np.array_equal(built, direct)
    q = rand_bits(rng, (1, 1, 8, ENTRY)) & 0x3FFF
    seqlens = np.array([n], dtype=np.int32)
    a = mla_ref.mla_decode_ref(q, built, table, seqlens, 0.07, False)
    b = mla_ref.mla_decode_ref(q, direct, table, seqlens, 0.07, False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_append_skips_padding_tokens_and_slots_past_the_pool():
    rng = np.random.default_rng(1)
    cache = rand_bits(rng, (2, 64, 1, 576))
    kv_c, k_pe = rand_bits(rng, (3, 512)), rand_bits(rng, (3, 64))
    out = append_ref(cache, kv_c, k_pe, [-1, 128, 5])
    assert np.array_equal(out[0, 5, 0], np.concatenate([kv_c[2], k_pe[2]]))
    mask = np.ones(cache.shape, dtype=bool)
    mask[0, 5] = False
    assert np.array_equal(out[mask], cache[mask])


def test_append_leaves_the_pad_alone():
    rng = np.random.default_rng(2)
    cache = np.full((1, 64, 1, 640), NAN, dtype=np.uint16)
    out = append_ref(cache, rand_bits(rng, (64, 512)), rand_bits(rng, (64, 64)), np.arange(64))
    assert np.all(out[..., ENTRY:] == NAN) and not np.any(out[..., :ENTRY] == NAN)


def test_copy_round_trip_between_pitches():
    rng = np.random.default_rng(3)
    dense = rand_bits(rng, (6, 64, 1, 576))
    padded = np.full((4, 64, 1, 640), NAN, dtype=np.uint16)
    m = np.array([[5, 0], [2, 3], [0, 1]])
    padded = copy_blocks_ref(dense, padded, m)
    assert np.array_equal(padded[0, :, :, :ENTRY], dense[5, :, :, :])
    assert np.all(padded[..., ENTRY:] == NAN) and np.all(padded[2] == NAN)
    back = copy_blocks_ref(padded, np.zeros_like(dense), m[:, ::-1])
    for a, b in m:
        assert np.array_equal(back[a], dense[a])


def test_copy_within_one_cache_and_skipped_pairs():
    rng = np.random.default_rng(4)
    c = rand_bits(rng, (4, 64, 1, 576))
    out = copy_blocks_ref(c, c, [[1, 3], [2, 2], [7, 0], [0, -1]])
    assert np.array_equal(out[3], c[1]) and np.array_equal(out[:3], c[:3])
