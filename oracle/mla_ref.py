"""Plain fp64 CPU oracle for paged MLA decode.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check of the graft entry
point and the benchmark's CPU-baseline leg use it.  It shares no code with the
HIP path; the two are fed from the same seeded input generator and nothing
else.

What it computes (the plain definition the decode kernel must reach up to
rounding order):

  For every sequence b with n = cache_seqlens[b] cached tokens, every query
  token i < s_q and every query head h (kv head g = h // (h_q / h_kv)):

    k_t = blocked_k[block_table[b, t // 64], t % 64, g, 0:576]   t < n
    v_t = k_t[0:512]
    J   = {t < n}, or {t < n - (s_q - 1 - i)} when causal
    s_t = softmax_scale * <q[b, i, h, :], k_t>
    lse = log(sum_{t in J} exp(s_t))            (natural log)
    out = sum_{t in J} exp(s_t - lse) * v_t
    an empty J gives out = 0 and lse = -inf.

Sources.  The pages state the pieces, not the formula:
  * [PAI] PAI FlashMLA tutorial (segmentfault, "云上玩转DeepSeek系列之五：实测优化16%,
    体验FlashMLA加速DeepSeek-V2-Lite推理"), section 二.4: the benchmark's inputs
    (q [b, s_q, h_q, d], a paged cache [num_blocks, 64, h_kv, d] addressed
    through an int32 block table) and its cost formulas: FLOPs count (d + dv)
    multiply-adds per query-key pair, bytes count the cache once per token
    with d elements only -- so V is read out of the same row as K.  Every
    implementation returns (out, lse).
  * [PR12676] vLLM pull request "[Perf] Mem align KV caches for CUDA devices
    (MLA perf improvement) #12676", description and cache-engine diff: an MLA
    entry is 576 elements, possibly stored at a 640-element pitch whose tail
    is never viewed.
  * [HN] Hacker News discussion of the FlashMLA release: Flash-Decoding splits
    the key/value length and merges the pieces, which must reproduce the
    unsplit result exactly (merge_partials below).
The split 576 = 512 latent + 64 rope, V = the first 512 elements, the
bottom-right causal alignment and the natural-log lse are the statement of
the problem the library implements; the pages leave them implicit.

Every floating-point step is fp64.  bf16 inputs are decoded from their raw
bits (bf16 -> fp32 -> fp64 is exact), so the oracle is indifferent to the
cache pitch and never touches a cache element outside J x [0, 576).
"""

from __future__ import annotations

import numpy as np

D_QK = 576
D_V = 512
BLOCK_SIZE = 64


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode raw bf16 bit patterns (uint16/int16) exactly into float64."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def e4m3_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode raw FP8 E4M3 bytes (the OCP "fn" variant) exactly into float64.

    One sign bit, four exponent bits with bias 7, three mantissa bits, no
    infinities:
      exponent 0:        (-1)^s * 2^-6 * m / 8          (zero and subnormals)
      exponent 1..15:    (-1)^s * 2^(e - 7) * (1 + m / 8)
      exponent 15, m 7:  NaN (the format's only non-finite code, 0x7F / 0xFF)
    The largest finite magnitude is 448 (0x7E), the smallest 2^-9 (0x01).
    Reading of the FP8 latent cache (see fp8 cache in mla_decode_ref).
    """
    b = np.asarray(bits).astype(np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = sign * mag
    return np.where((e == 15) & (b & 0x7 == 7), np.nan, val)


def visible_keys(n: int, s_q: int, i: int, causal: bool) -> int:
    """How many leading keys query token i of s_q sees in an n-token cache.

    The s_q query tokens are the last s_q positions of the sequence (the
    bottom-right alignment), so with causal masking token i sees
    n - (s_q - 1 - i) keys.  Without causal masking every token sees all n.
    """
    if causal:
        return max(0, n - (s_q - 1 - i))
    return max(0, n)


def gather_tokens(k_bits: np.ndarray, table_row: np.ndarray, n: int, kv_head: int,
                  block_size: int = BLOCK_SIZE, d: int = D_QK, kv_format: str = "bf16",
                  kv_scale: float = 1.0) -> np.ndarray:
    """Logical tokens 0..n-1 of one sequence as an (n, d) fp64 matrix.

    Token t lives in physical page table_row[t // block_size], row
    t % block_size ([PAI] section 二.4: the cache is blocked by pages that the
    block table maps).  Only the first d elements of each entry are read
    ([PR12676]: the padded tail is never viewed).  An fp8 cache
    (kv_format "fp8_e4m3") holds one E4M3 byte per element; its value is the
    decoded byte times the cache's scale kv_scale.
    """
    t = np.arange(n)
    phys = np.asarray(table_row)[t // block_size].astype(np.int64)
    rows = t % block_size
    raw = k_bits[phys, rows, kv_head, :d]
    if kv_format == "bf16":
        return bf16_bits_to_f64(raw)
    if kv_format == "fp8_e4m3":
        return e4m3_bits_to_f64(raw) * float(kv_scale)
    raise ValueError(f"unknown cache format {kv_format!r}")


def softmax_average(scores: np.ndarray, values: np.ndarray):
    """lse and softmax-weighted average of values for one row of scores.

    scores: (c,) fp64, values: (c, dv) fp64.  An empty row gives (0, -inf).
    """
    if scores.shape[0] == 0:
        return np.zeros(values.shape[1]), -np.inf
    m = scores.max()
    w = np.exp(scores - m)
    lse = m + np.log(w.sum())
    out = np.exp(scores - lse) @ values
    return out, lse


def attend_rows(q_rows: np.ndarray, K: np.ndarray, counts, softmax_scale: float,
                dv: int = D_V, t_begin: int = 0):
    """Attention of query rows over keys K[t_begin : counts[r]].

    q_rows: (R, d) fp64; K: (n, d) fp64 with V = K[:, :dv]; counts[r] is the
    number of leading keys row r may see.  Restricting to t >= t_begin gives
    the partial result of one key range, as one split of Flash-Decoding sees.
    """
    R = q_rows.shape[0]
    out = np.zeros((R, dv))
    lse = np.full(R, -np.inf)
    scores = softmax_scale * (q_rows @ K.T) if K.shape[0] else np.zeros((R, 0))
    V = K[:, :dv]
    for r in range(R):
        hi = int(counts[r])
        out[r], lse[r] = softmax_average(scores[r, t_begin:hi], V[t_begin:hi])
    return out, lse


def mla_decode_ref(q_bits: np.ndarray, k_bits: np.ndarray, block_table: np.ndarray,
                   cache_seqlens: np.ndarray, softmax_scale: float, causal: bool,
                   dv: int = D_V, batch_indices=None, block_size: int = BLOCK_SIZE,
                   token_range=None, kv_format: str = "bf16", kv_scale: float = 1.0):
    """The oracle.

    q_bits:   uint16 [b, s_q, h_q, d]       raw bf16 bits of the queries
    k_bits:   [num_blocks, block_size, h_kv, pitch >= d] raw cache elements:
              uint16 bf16 bits, or (kv_format "fp8_e4m3") uint8 E4M3 bytes
              whose values are scaled by kv_scale
    block_table: int [b, max_blocks_per_seq]
    cache_seqlens: int [b]
    batch_indices: optional subset of sequences to compute (others stay 0 / -inf)
    token_range: optional (begin, end) to restrict every row to keys in
                 [begin, end) -- the partial result of one key split.

    The fp8 cache is our reading of the FP8 latent cache the Hacker News
    discussion of the FlashMLA release links to (vLLM's MLA and FP8 work):
    the whole 576-element entry stored as E4M3 bytes with one scale per
    cache; K and V are the dequantised values, so the definition above is
    unchanged.

    Returns fp64 out [b, s_q, h_q, dv] and lse [b, s_q, h_q].
    """
    b, s_q, h_q, d = q_bits.shape
    h_kv = k_bits.shape[2]
    if h_q % h_kv:
        raise ValueError("h_q must be a multiple of h_kv")
    group = h_q // h_kv
    out = np.zeros((b, s_q, h_q, dv))
    lse = np.full((b, s_q, h_q), -np.inf)
    todo = range(b) if batch_indices is None else batch_indices
    for bi in todo:
        n = int(cache_seqlens[bi])
        for g in range(h_kv):
            K = gather_tokens(k_bits, block_table[bi], n, g, block_size, d, kv_format, kv_scale)
            heads = np.arange(g * group, (g + 1) * group)
            q_rows = bf16_bits_to_f64(q_bits[bi][:, heads, :]).reshape(s_q * group, d)
            counts = np.repeat([visible_keys(n, s_q, i, causal) for i in range(s_q)], group)
            t_begin = 0
            if token_range is not None:
                t_begin = token_range[0]
                counts = np.minimum(counts, token_range[1])
            o, l = attend_rows(q_rows, K, counts, softmax_scale, dv, t_begin)
            out[bi][:, heads, :] = o.reshape(s_q, group, dv)
            lse[bi][:, heads] = l.reshape(s_q, group)
    return out, lse


def merge_partials(outs, lses):
    """Merge partial results of disjoint key ranges by their lse.

    With L = log(sum_i exp(lse_i)), the whole-range result is
    out = sum_i exp(lse_i - L) * out_i and lse = L.  Ranges whose lse is -inf
    saw no key and carry weight 0; if every range is empty the merge is empty
    (out = 0, lse = -inf).  This is how Flash-Decoding reassembles its
    key-length splits ([HN], the Flash-Decoding description).

    outs: list of arrays [..., dv]; lses: list of arrays [...].
    """
    lses = np.stack([np.asarray(x, dtype=np.float64) for x in lses])
    outs = np.stack([np.asarray(x, dtype=np.float64) for x in outs])
    m = np.max(lses, axis=0)
    finite = np.isfinite(m)
    safe_m = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - safe_m), 0.0)
    tot = w.sum(axis=0)
    L = np.where(finite, safe_m + np.log(np.where(finite, tot, 1.0)), -np.inf)
    scale = np.where(finite, 1.0, 0.0)[None] * np.where(
        np.isfinite(lses), np.exp(lses - np.where(finite, L, 0.0)[None]), 0.0)
    out = (scale[..., None] * outs).sum(axis=0)
    return out, L
