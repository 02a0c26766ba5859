"""Plain CPU oracle of the paged-cache writes (append at a slot mapping, page copy).

TEST INFRASTRUCTURE ONLY.  Only the test suite may import this module; it
shares no code with the HIP path.

What it computes, on the raw bf16 bits (uint16 arrays, so equality is exact):

  append:  for token t with slot s = slot_mapping[t] >= 0 (and inside the
           pool), cache[s // 64, s % 64, 0, 0:512] = kv_c[t] and
           cache[s // 64, s % 64, 0, 512:576] = k_pe[t]; nothing else changes.
  copy:    for each pair (a, b) of block_mapping, dst[b, :, 0, 0:576] =
           src[a, :, 0, 0:576]; nothing else changes (the pad elements of a
           640-element pitch are not part of an entry).

Sources.  vLLM pull request "[Perf] Mem align KV caches for CUDA devices (MLA
perf improvement) #12676": the cache-engine diff allocates each entry padded
to 256 bytes and views its first 576 elements; the pull request adds a
copy_blocks_mla operation over a block mapping and a block swap, because the
padded layout can no longer be copied as a dense tensor.  The append's
definition (the latent part then the rope part of one token into one slot)
is how the 576-element entry the decode reads is formed; the pages state the
entry, not the write, so this is the plain reading.
"""

from __future__ import annotations

import numpy as np

LATENT = 512
ROPE = 64
ENTRY = LATENT + ROPE
PAGE = 64


def append_ref(cache: np.ndarray, kv_c: np.ndarray, k_pe: np.ndarray, slot_mapping) -> np.ndarray:
    """A copy of cache ([num_blocks, 64, 1, pitch] uint16) with the tokens written."""
    out = cache.copy()
    pool = cache.shape[0] * PAGE
    for t, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0 or s >= pool:
            continue
        page, row = divmod(int(s), PAGE)
        out[page, row, 0, 0:LATENT] = kv_c[t]
        out[page, row, 0, LATENT:ENTRY] = k_pe[t]
    return out


def copy_blocks_ref(src: np.ndarray, dst: np.ndarray, block_mapping) -> np.ndarray:
    """A copy of dst with each mapped page's 64 entries taken from src."""
    out = dst.copy()
    for a, b in np.asarray(block_mapping).reshape(-1, 2).tolist():
        if 0 <= a < src.shape[0] and 0 <= b < dst.shape[0]:
            out[b, :, 0, 0:ENTRY] = src[a, :, 0, 0:ENTRY]
    return out
