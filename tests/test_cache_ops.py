"""GPU: the cache writes (append at a slot mapping, page copy) against the
oracle, bit for bit over the whole storage (pad elements included), and a
decode of a cache built by appends."""

import numpy as np
import pytest
import torch

from conftest import bits
from oracle import mla_ref
from oracle.mla_cache_ref import ENTRY, append_ref, copy_blocks_ref
from paged_mla_decode_04_amd import append_kv, copy_blocks, mla_decode_with_kvcache
from paged_mla_decode_04_amd.workloads import D_V

pytestmark = pytest.mark.gpu

NAN = 0x7FC0


def to_bf16(a: np.ndarray, dev="cuda:0") -> torch.Tensor:
    return torch.from_numpy(a.astype(np.int16)).view(torch.bfloat16).to(dev)


def rand_bits(rng, shape):
    return rng.integers(0, 0x4000, size=shape, dtype=np.uint16)


def storage(nblocks, pitch, fill=NAN):
    return np.full((nblocks, 64, 1, pitch), fill, dtype=np.uint16)


@pytest.mark.parametrize("pitch", [576, 640])
def test_append_matches_the_oracle(pitch):
    rng = np.random.default_rng(pitch)
    nblocks, T = 9, 300
    cache = storage(nblocks, pitch)
    cache[..., :ENTRY] = rand_bits(rng, (nblocks, 64, 1, ENTRY))
    # strided token rows: kv_c and k_pe are column slices of wider arrays
    wide_c = rand_bits(rng, (T, 520))
    wide_pe = rand_bits(rng, (T, 72))
    slots = rng.permutation(nblocks * 64)[:T].astype(np.int64)
    slots[::37] = -1                      # padding tokens
    slots[5] = nblocks * 64 + 3           # past the pool
    ref = append_ref(cache, wide_c[:, :512], wide_pe[:, :64], slots)
    print(f"[cache] append pitch={pitch} T={T}", flush=True)
    k = to_bf16(cache)
    append_kv(to_bf16(wide_c)[:, :512], to_bf16(wide_pe)[:, :64],
              torch.from_numpy(slots).to("cuda:0"), k[..., :ENTRY])
    torch.cuda.synchronize()
    assert np.array_equal(bits(k.cpu()), ref)


@pytest.mark.parametrize("src_pitch,dst_pitch", [(576, 640), (640, 576), (640, 640)])
def test_copy_blocks_matches_the_oracle(src_pitch, dst_pitch):
    rng = np.random.default_rng(src_pitch + 7 * dst_pitch)
    src = storage(7, src_pitch)
    src[..., :ENTRY] = rand_bits(rng, (7, 64, 1, ENTRY))
    dst = storage(5, dst_pitch, fill=0x1234)
    m = np.array([[6, 0], [2, 4], [0, 1], [9, 2], [3, -1]], dtype=np.int64)  # last two skipped
    ref = copy_blocks_ref(src, dst, m)
    print(f"[cache] copy {src_pitch}->{dst_pitch}", flush=True)
    ks, kd = to_bf16(src), to_bf16(dst)
    copy_blocks(ks[..., :ENTRY], kd[..., :ENTRY], torch.from_numpy(m).to("cuda:0"))
    torch.cuda.synchronize()
    assert np.array_equal(bits(kd.cpu()), ref)
    assert np.array_equal(bits(ks.cpu()), src)


def test_copy_blocks_within_one_cache():
    rng = np.random.default_rng(3)
    c = storage(6, 640)
    c[..., :ENTRY] = rand_bits(rng, (6, 64, 1, ENTRY))
    m = np.array([[0, 5], [1, 4]], dtype=np.int64)
    ref = copy_blocks_ref(c, c, m)
    k = to_bf16(c)
    copy_blocks(k[..., :ENTRY], k[..., :ENTRY], torch.from_numpy(m).to("cuda:0"))
    torch.cuda.synchronize()
    assert np.array_equal(bits(k.cpu()), ref)


def test_decode_of_an_appended_cache():
    """Sequences written token by token with append_kv decode like the oracle on
    the oracle's own appended cache."""
    rng = np.random.default_rng(9)
    lens = [130, 64, 257]
    table = np.array([[4, 1, 7, -1, -1], [0, -1, -1, -1, -1], [2, 6, 3, 5, 8]], dtype=np.int32)
    nblocks, pitch, h_q = 9, 640, 64
    rows = [rng.standard_normal((n, ENTRY)).astype(np.float32) for n in lens]
    kv_bits = [bits(torch.from_numpy(r).to(torch.bfloat16)) for r in rows]
    slots = np.concatenate([[table[b, t // 64] * 64 + t % 64 for t in range(n)] for b, n in enumerate(lens)])
    allrows = np.concatenate(kv_bits)
    ref_cache = append_ref(storage(nblocks, pitch), allrows[:, :512], allrows[:, 512:], slots)
    k = to_bf16(storage(nblocks, pitch))
    print("[cache] decode after append", flush=True)
    append_kv(to_bf16(allrows[:, :512].copy()), to_bf16(allrows[:, 512:].copy()),
              torch.from_numpy(slots.astype(np.int64)).to("cuda:0"), k[..., :ENTRY])
    torch.cuda.synchronize()
    assert np.array_equal(bits(k.cpu()), ref_cache)
    q = torch.randn((3, 1, h_q, ENTRY), generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    seqlens = np.array(lens, dtype=np.int32)
    out, lse = mla_decode_with_kvcache(q.to("cuda:0"), k[..., :ENTRY], torch.from_numpy(table).to("cuda:0"),
                                       torch.from_numpy(seqlens).to("cuda:0"), D_V, 0.0721688, False)
    torch.cuda.synchronize()
    ref_out, ref_lse = mla_ref.mla_decode_ref(bits(q), ref_cache, table, seqlens, 0.0721688, False)
    o = out.cpu().float().numpy().astype(np.float64)
    assert np.all(np.abs(o - ref_out) <= 1e-2 * np.maximum(1.0, np.abs(ref_out)))
    assert np.all(np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse) <= 2e-3)
