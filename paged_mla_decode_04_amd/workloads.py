"""Seeded synthetic inputs for paged MLA decode.

This module only draws inputs: it holds none of the attention arithmetic, so
both the HIP path and the CPU oracle can be fed from it without sharing any
computation.

The shapes and value distributions follow FlashMLA's built-in benchmark as the
PAI FlashMLA tutorial runs it (segmentfault, "云上玩转DeepSeek系列之五：实测优化16%,
体验FlashMLA加速DeepSeek-V2-Lite推理", section 二.4): bf16 N(0,1) queries and a
paged latent cache with 64-token pages, the longest sequence padded up to a
multiple of 256 tokens, a block table with one row of that padded width per
sequence, and a pool of exactly batch * width pages, seeded with 0.  The
640-element entry pitch follows the vLLM pull request "[Perf] Mem align KV
caches for CUDA devices (MLA perf improvement) #12676" (the cache-engine diff):
allocate the padded entry, then view its first 576 elements.

Draw order from one CPU torch.Generator: seqlens, q, blocked_k, block_table.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

D_QK = 576          # 512 latent + 64 rope elements per cached token
D_V = 512           # V is the first 512 elements of the same row
BLOCK_SIZE = 64     # tokens per page
DEFAULT_SCALE = 1.0 / math.sqrt(192.0)

BF16_QUIET_NAN_BITS = 0x7FC0
E4M3_NAN_BYTE = 0x7F
FP8_KV_SCALE = 1.0 / 64.0    # a power of two: N(0,1) values / scale stay inside +-448


@dataclass(frozen=True)
class Workload:
    """One decode workload: shapes, length recipe and cache layout."""

    name: str
    batch: int
    s_q: int
    h_q: int
    causal: bool
    seqlens: str                 # recipe name, see _draw_seqlens
    pitch: int = D_QK            # elements between consecutive cached tokens
    table: str = "randperm"      # "randperm" | "arange"
    h_kv: int = 1
    softmax_scale: float = DEFAULT_SCALE
    fixed_seqlens: Optional[tuple] = None
    description: str = ""
    kv_format: str = "bf16"      # "bf16" | "fp8_e4m3" (one E4M3 byte per element)
    kv_scale: float = 1.0        # value of an fp8 element = decoded byte * kv_scale


# The five workloads: a tiny one, a DeepSeek-V2-Lite-shaped one (16 heads),
# the wide-head b=128/h_q=128/seqlen~4096 shape of the tutorial's bandwidth
# plot, a two-token causal one with 640-element entries, and a skewed
# long-context one that exercises split-KV.
WORKLOADS = {
    "tiny": Workload(
        "tiny", batch=2, s_q=1, h_q=16, causal=False, seqlens="fixed",
        fixed_seqlens=(37, 130),
        description="b=2 s_q=1 h_q=16, seqlens [37,130], permuted 8-page pool"),
    "v2lite": Workload(
        "v2lite", batch=32, s_q=1, h_q=16, causal=False, seqlens="uniform_1024_4096",
        description="b=32 s_q=1 h_q=16, seqlens uniform in [1024,4096], shuffled table"),
    "wide": Workload(
        "wide", batch=128, s_q=1, h_q=128, causal=False, seqlens="normal_4096_1024",
        table="arange",
        description="b=128 s_q=1 h_q=128, seqlens ~ N(4096,1024) clipped to [1,8192], "
                    "identity table"),
    "mtp": Workload(
        "mtp", batch=64, s_q=2, h_q=128, causal=True, seqlens="uniform_4096_12288",
        pitch=640,
        description="b=64 s_q=2 causal h_q=128, seqlens uniform in [4096,12288], "
                    "640-element entry pitch"),
    "skewed": Workload(
        "skewed", batch=16, s_q=1, h_q=128, causal=False, seqlens="loguniform_32768",
        description="b=16 s_q=1 h_q=128, seqlens log-uniform in [1,32768], one forced "
                    "to 32768, scattered pages"),
}


@dataclass
class DecodeInputs:
    """Host (CPU) tensors of one drawn workload."""

    workload: Workload
    cache_seqlens: torch.Tensor      # int32 [b]
    q: torch.Tensor                  # bf16 [b, s_q, h_q, 576]
    blocked_k: torch.Tensor          # bf16 [num_blocks, 64, h_kv, 576] (maybe a strided view)
    block_table: torch.Tensor        # int32 [b, max_blocks_per_seq]
    k_storage: torch.Tensor          # the allocation blocked_k views ([..., pitch])
    meta: dict = field(default_factory=dict)

    @property
    def softmax_scale(self) -> float:
        return self.workload.softmax_scale

    @property
    def causal(self) -> bool:
        return self.workload.causal

    @property
    def kv_format(self) -> str:
        return self.workload.kv_format

    @property
    def kv_scale(self) -> float:
        return self.workload.kv_scale

    def to(self, device) -> "DecodeInputs":
        """Copy to a device, keeping the cache's pitch (the padded storage moves whole)."""
        storage = self.k_storage.to(device)
        view = storage[..., :D_QK]
        return DecodeInputs(self.workload, self.cache_seqlens.to(device), self.q.to(device),
                            view, self.block_table.to(device), storage, dict(self.meta))


def _draw_seqlens(w: Workload, gen: torch.Generator) -> torch.Tensor:
    b = w.batch
    if w.seqlens == "fixed":
        s = torch.tensor(w.fixed_seqlens, dtype=torch.int64)
    elif w.seqlens.startswith("uniform_"):
        _, lo, hi = w.seqlens.split("_")
        s = torch.randint(int(lo), int(hi) + 1, (b,), generator=gen, dtype=torch.int64)
    elif w.seqlens.startswith("normal_"):
        _, mean, sd = w.seqlens.split("_")
        x = torch.randn(b, generator=gen, dtype=torch.float64) * float(sd) + float(mean)
        s = torch.round(x).clamp(1, 2 * int(mean)).to(torch.int64)
    elif w.seqlens.startswith("loguniform_"):
        top = int(w.seqlens.split("_")[1])
        u = torch.rand(b, generator=gen, dtype=torch.float64) * math.log(top)
        s = torch.floor(torch.exp(u)).clamp(1, top).to(torch.int64)
        forced = int(torch.randint(0, b, (1,), generator=gen).item())
        s[forced] = top
    else:
        raise ValueError(f"unknown seqlen recipe {w.seqlens!r}")
    return s.to(torch.int32)


def padded_max_seqlen(cache_seqlens: torch.Tensor) -> int:
    """Longest sequence rounded up to a multiple of 256 tokens, as the benchmark pads it."""
    mx = int(cache_seqlens.max().item()) if cache_seqlens.numel() else 0
    return max(256, ((mx + 255) // 256) * 256)


def draw(w: Workload | str, seed: int = 0, *, seqlens_override=None,
         poison: bool = False) -> DecodeInputs:
    """Draw one workload's inputs on the CPU.

    seqlens_override replaces the recipe (same draw order afterwards).
    poison=True fills every cache byte the result must not depend on (pad
    columns, rows past each sequence's length, pages no sequence uses) with
    NaN (bf16 NaN bits, or the E4M3 NaN byte 0x7F of an fp8 cache), and the
    block-table entries past each sequence's last page with
    -1.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    if seqlens_override is not None:
        seqlens = torch.as_tensor(seqlens_override, dtype=torch.int32).clone()
        if seqlens.numel() != w.batch:
            w = Workload(**{**w.__dict__, "batch": int(seqlens.numel())})
    else:
        seqlens = _draw_seqlens(w, gen)
    b = w.batch
    max_pad = padded_max_seqlen(seqlens)
    width = max_pad // BLOCK_SIZE
    num_blocks = b * width

    q = torch.randn(b, w.s_q, w.h_q, D_QK, generator=gen, dtype=torch.float32).to(torch.bfloat16)
    k_storage = torch.randn(num_blocks, BLOCK_SIZE, w.h_kv, w.pitch, generator=gen,
                            dtype=torch.float32)
    if w.kv_format == "fp8_e4m3":
        # the same N(0,1) values stored as E4M3 bytes of x / kv_scale (torch's
        # round-to-nearest conversion, inside the format's +-448)
        k_storage = (k_storage / w.kv_scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        k_storage = k_storage.view(torch.uint8)
    else:
        k_storage = k_storage.to(torch.bfloat16)
    if w.table == "arange":
        table = torch.arange(num_blocks, dtype=torch.int32).view(b, width)
    else:
        table = torch.randperm(num_blocks, generator=gen).to(torch.int32).view(b, width)
    table = table.contiguous()

    if poison:
        _poison(k_storage, table, seqlens)
    blocked_k = k_storage[..., :D_QK]
    return DecodeInputs(w, seqlens, q, blocked_k, table, k_storage,
                        {"seed": seed, "max_seqlen_pad": max_pad, "poison": poison})


def _poison(k_storage: torch.Tensor, table: torch.Tensor, seqlens: torch.Tensor) -> None:
    if k_storage.dtype == torch.uint8:  # fp8 cache: 0x7F is E4M3's NaN
        bits = k_storage
        nan = torch.tensor(E4M3_NAN_BYTE, dtype=torch.uint8)
    else:
        bits = k_storage.view(torch.int16)
        nan = torch.tensor(BF16_QUIET_NAN_BITS, dtype=torch.int16)
    if k_storage.shape[-1] > D_QK:
        bits[..., D_QK:] = nan
    used = torch.zeros(k_storage.shape[0], dtype=torch.bool)
    for bi in range(table.shape[0]):
        n = int(seqlens[bi])
        pages = (n + BLOCK_SIZE - 1) // BLOCK_SIZE
        for p in range(pages):
            phys = int(table[bi, p])
            used[phys] = True
            if p == pages - 1 and n % BLOCK_SIZE:
                bits[phys, n % BLOCK_SIZE:] = nan
        table[bi, pages:] = -1
    bits[~used] = nan


def random_case(rng: "torch.Generator | int", *, max_batch=3, s_q_choices=(1, 2),
                h_q_choices=(1, 2, 16), max_len=200, h_kv=1, pitch_choices=(576, 640)):
    """A small random workload description for brute-force style tests."""
    if isinstance(rng, int):
        g = torch.Generator().manual_seed(rng)
    else:
        g = rng

    def pick(seq):
        return seq[int(torch.randint(0, len(seq), (1,), generator=g))]

    b = int(torch.randint(1, max_batch + 1, (1,), generator=g))
    lens = tuple(int(x) for x in torch.randint(1, max_len + 1, (b,), generator=g))
    h_q = pick(h_q_choices)
    h_q = max(h_q, h_kv) // h_kv * h_kv
    return Workload("random", batch=b, s_q=pick(s_q_choices), h_q=h_q,
                    causal=bool(torch.randint(0, 2, (1,), generator=g)),
                    seqlens="fixed", fixed_seqlens=lens, pitch=pick(pitch_choices),
                    h_kv=h_kv)
