"""Cost model of one paged MLA decode call, as FlashMLA's benchmark counts it.

PAI FlashMLA tutorial (segmentfault, "云上玩转DeepSeek系列之五：实测优化16%,
体验FlashMLA加速DeepSeek-V2-Lite推理"), section 二.4:
  * FLOPs = s_q * sum(seqlens) * h_q * (d + dv) * 2
  * bytes = (sum(seqlens) * h_kv * d + b * s_q * h_q * d + b * s_q * h_q * dv)
            * bytes per element
  * TFLOPS = FLOPs / 1e9 / ms and GB/s = bytes / 1e6 / ms (decimal units,
    time in milliseconds).
The byte count reads every cached token once, with d elements: K and V come
out of the same row.  It always uses d = 576, also when entries are stored at
a 640-element pitch: the pad is not algorithmic traffic.

vLLM pull request "[Perf] Mem align KV caches for CUDA devices (MLA perf
improvement) #12676", description and cache-engine diff: an entry is padded
up to the next 256-byte boundary (576 bf16 -> 640 elements, 1152 -> 1280 B),
which shrinks the number of cache blocks that fit by 576/640.
"""

from __future__ import annotations

D_QK = 576
D_V = 512


def decode_flops(s_q: int, total_seqlens: int, h_q: int, d: int = D_QK, dv: int = D_V) -> int:
    return int(s_q) * int(total_seqlens) * int(h_q) * (int(d) + int(dv)) * 2


def decode_bytes(total_seqlens: int, b: int, s_q: int, h_q: int, h_kv: int = 1,
                 d: int = D_QK, dv: int = D_V, elem_bytes: int = 2) -> int:
    return (int(total_seqlens) * h_kv * d + b * s_q * h_q * d + b * s_q * h_q * dv) * elem_bytes


def tflops(flops: float, ms: float) -> float:
    return flops / 1e9 / ms


def gbps(nbytes: float, ms: float) -> float:
    return nbytes / 1e6 / ms


def aligned_entry_elems(entry_elems: int, elem_bytes: int = 2, align_bytes: int = 256) -> int:
    """Elements allocated per cache entry when entries start on align_bytes boundaries."""
    nbytes = entry_elems * elem_bytes
    padded = (nbytes + align_bytes - 1) // align_bytes * align_bytes
    return padded // elem_bytes


def blocks_after_alignment(blocks: int, entry_elems: int = D_QK, elem_bytes: int = 2,
                           align_bytes: int = 256) -> int:
    """Cache blocks that fit in the same memory once entries are padded."""
    padded = aligned_entry_elems(entry_elems, elem_bytes, align_bytes)
    return blocks * entry_elems // padded


def workload_cost(seqlens, b: int, s_q: int, h_q: int, h_kv: int = 1, cache_elem_bytes: int = 2):
    """FLOPs and bytes of one call.  With an fp8 cache (cache_elem_bytes 1) the
    cache term counts one byte per element and the query and output terms stay
    bf16: the same formula with each term at its own element size."""
    total = int(sum(int(x) for x in seqlens))
    qo = decode_bytes(0, b, s_q, h_q, h_kv)
    return {
        "total_seqlens": total,
        "flops": decode_flops(s_q, total, h_q),
        "bytes": qo + int(total) * h_kv * D_QK * int(cache_elem_bytes),
    }
