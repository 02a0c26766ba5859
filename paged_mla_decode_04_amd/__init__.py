"""Paged MLA decode on MI355X (gfx950): Python binding of libmla_decode.so.

Two calls, as a serving engine makes them (the PAI FlashMLA tutorial on
segmentfault, "云上玩转DeepSeek系列之五", section 二.2: metadata once per decode
step, the forward once per layer):

    tile_md, num_splits = get_mla_metadata(cache_seqlens, s_q * h_q, h_kv)
    out, lse = mla_decode_with_kvcache(q, blocked_k, block_table, cache_seqlens,
                                       dv, softmax_scale, causal,
                                       metadata=(tile_md, num_splits))

This module only marshals arguments: torch provides device memory and the
current stream, and every step of the computation runs in the library's HIP
kernels.  Importing it does not load the library; the first call does, and
raises if the library has not been built.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import MLAError, TILE_MD_INTS

__all__ = ["get_mla_metadata", "mla_decode_with_kvcache", "plan_host", "default_num_parts",
           "workspace_size", "append_kv", "copy_blocks", "MLAError", "TILE_MD_INTS"]

D_QK = 576
D_V = 512
BLOCK_SIZE = 64


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def default_num_parts(q_rows: int, h_kv: int = 1, device: int = 0) -> int:
    n = ctypes.c_int32(0)
    _lib.check(_lib.load().mla_default_num_parts(int(device), int(q_rows), int(h_kv),
                                                 ctypes.byref(n)), "mla_default_num_parts")
    return n.value


def workspace_size(batch: int, s_q: int, h_q: int, h_kv: int = 1, dv: int = D_V,
                   num_parts: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().mla_workspace_size(batch, s_q, h_q, h_kv, dv, num_parts, ctypes.byref(n)),
               "mla_workspace_size")
    return n.value


def plan_host(cache_seqlens, q_rows: int, h_kv: int, num_parts: int):
    """The plan computed on the host (int32 CPU tensors), identical to get_mla_metadata's."""
    sl = torch.as_tensor(cache_seqlens, dtype=torch.int32).contiguous().cpu()
    b = sl.numel()
    md = torch.empty((num_parts, TILE_MD_INTS), dtype=torch.int32)
    ns = torch.empty((b + 1,), dtype=torch.int32)
    _lib.check(_lib.load().mla_plan_host(_ptr(sl) if b else None, b, int(q_rows), int(h_kv),
                                         int(num_parts), _ptr(md), _ptr(ns)), "mla_plan_host")
    return md, ns


def get_mla_metadata(cache_seqlens: torch.Tensor, q_rows: int, h_kv: int,
                     num_parts: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Plan the split-KV work for one decode step (enqueued on the current stream).

    cache_seqlens: int32 [b] on the GPU; q_rows = s_q * h_q.
    Returns (tile_md int32 [num_parts, 8], num_splits int32 [b + 1]) on the same device.
    """
    if cache_seqlens.dtype != torch.int32 or not cache_seqlens.is_cuda:
        raise ValueError("cache_seqlens must be an int32 GPU tensor")
    sl = cache_seqlens.contiguous()
    dev = sl.device
    if num_parts is None:
        num_parts = default_num_parts(q_rows, h_kv, dev.index or 0)
    b = sl.numel()
    md = torch.empty((num_parts, TILE_MD_INTS), dtype=torch.int32, device=dev)
    ns = torch.empty((b + 1,), dtype=torch.int32, device=dev)
    _lib.check(_lib.load().mla_get_metadata(_ptr(sl), b, int(q_rows), int(h_kv), int(num_parts),
                                            _ptr(md), _ptr(ns), _stream(dev)), "mla_get_metadata")
    return md, ns


def mla_decode_with_kvcache(q: torch.Tensor, blocked_k: torch.Tensor, block_table: torch.Tensor,
                            cache_seqlens: torch.Tensor, dv: int, softmax_scale: float,
                            causal: bool, *, metadata=None, num_parts: Optional[int] = None,
                            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, no_alloc: bool = False,
                            kv_scale: Optional[float] = None):
    """Paged MLA decode.

    q           bf16 [b, s_q, h_q, 576], last dim contiguous
    blocked_k   bf16 [num_blocks, 64, h_kv, 576] (any strided view with unit last-dim
                stride, e.g. the first 576 elements of a [num_blocks, 64, h_kv, 640] cache),
                or an fp8 cache of the same shape: uint8 or float8_e4m3fn E4M3 bytes whose
                values are times kv_scale (required then)
    block_table int32 [b, max_blocks_per_seq]
    cache_seqlens int32 [b]
    metadata    optional (tile_md, num_splits) from get_mla_metadata for these seqlens;
                without it the call plans for itself (inside the decode kernel, with
                no separate plan launch, for a bf16 cache, more than 64 query rows per
                kv head and at most 256 sequences)
    no_alloc    use mla_decode_with_kvcache_noalloc: the library's static scratch
                instead of a workspace (none is allocated; `workspace` is ignored)
    Returns (out bf16 [b, s_q, h_q, dv], lse fp32 [b, s_q, h_q]).
    """
    if q.dim() != 4 or blocked_k.dim() != 4 or block_table.dim() != 2:
        raise ValueError("q and blocked_k must be 4-D, block_table 2-D")
    fp8 = blocked_k.dtype in (torch.uint8, torch.float8_e4m3fn)
    if q.dtype != torch.bfloat16 or not (fp8 or blocked_k.dtype == torch.bfloat16):
        raise ValueError("q must be bfloat16 and blocked_k bfloat16 or E4M3 bytes")
    if fp8 and kv_scale is None:
        raise ValueError("an fp8 cache needs its kv_scale")
    if block_table.dtype != torch.int32 or cache_seqlens.dtype != torch.int32:
        raise ValueError("block_table and cache_seqlens must be int32")
    dev = q.device
    for t in (q, blocked_k, block_table, cache_seqlens):
        if not t.is_cuda or t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
    if q.stride(-1) != 1 or blocked_k.stride(-1) != 1 or block_table.stride(-1) != 1:
        raise ValueError("the last dimension of q, blocked_k and block_table must be contiguous")
    b, s_q, h_q, d = q.shape
    num_blocks, block_size, h_kv, dk = blocked_k.shape
    if dk != d:
        raise ValueError("q and blocked_k disagree on the head size")
    if block_table.shape[0] != b or cache_seqlens.numel() != b:
        raise ValueError("block_table / cache_seqlens batch mismatch")
    seqlens = cache_seqlens.contiguous()
    if out is None:
        out = torch.empty((b, s_q, h_q, dv), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((b, s_q, h_q), dtype=torch.float32, device=dev)
    tile_md = num_splits = None
    if metadata is not None:
        tile_md, num_splits = metadata
        num_parts = tile_md.shape[0]
    parts = 0 if num_parts is None else int(num_parts)
    if not no_alloc:
        need = workspace_size(b, s_q, h_q, h_kv, dv, parts) if b else 256
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    p = _lib.DecodeParams()
    p.q = q.data_ptr()
    p.q_batch_stride, p.q_seq_stride, p.q_head_stride = q.stride(0), q.stride(1), q.stride(2)
    p.batch, p.s_q, p.h_q = b, s_q, h_q
    p.k_cache = blocked_k.data_ptr()
    p.k_block_stride, p.k_row_stride, p.k_head_stride = (blocked_k.stride(0), blocked_k.stride(1),
                                                         blocked_k.stride(2))
    p.num_blocks, p.block_size, p.h_kv, p.d = num_blocks, block_size, h_kv, d
    p.block_table = block_table.data_ptr()
    p.block_table_stride = block_table.stride(0)
    p.max_blocks_per_seq = block_table.shape[1]
    p.cache_seqlens = seqlens.data_ptr()
    p.dv = int(dv)
    p.softmax_scale = float(softmax_scale)
    p.causal = 1 if causal else 0
    p.tile_md = None if tile_md is None else tile_md.data_ptr()
    p.num_splits = None if num_splits is None else num_splits.data_ptr()
    p.num_parts = parts
    p.workspace = None if no_alloc else workspace.data_ptr()
    p.workspace_bytes = 0 if no_alloc else workspace.numel()
    p.out = out.data_ptr()
    p.out_batch_stride, p.out_seq_stride, p.out_head_stride = out.stride(0), out.stride(1), out.stride(2)
    p.lse = lse.data_ptr()
    p.lse_batch_stride, p.lse_seq_stride, p.lse_head_stride = lse.stride(0), lse.stride(1), lse.stride(2)
    p.kv_dtype = _lib.KV_FP8_E4M3 if fp8 else _lib.KV_BF16
    p.kv_scale = float(kv_scale) if fp8 else 1.0
    entry = "mla_decode_with_kvcache_noalloc" if no_alloc else "mla_decode_with_kvcache"
    _lib.check(getattr(_lib.load(), entry)(ctypes.byref(p), _stream(dev)), entry)
    return out, lse


def _cache_view(blocked_k: torch.Tensor, what: str):
    """(num_blocks, block_stride, row_stride) of a [num_blocks, 64, 1, 576] bf16 cache view."""
    if blocked_k.dim() != 4 or tuple(blocked_k.shape[1:]) != (BLOCK_SIZE, 1, D_QK):
        raise ValueError(f"{what} must be [num_blocks, 64, 1, 576]")
    if blocked_k.dtype != torch.bfloat16 or not blocked_k.is_cuda or blocked_k.stride(-1) != 1:
        raise ValueError(f"{what} must be a bf16 GPU tensor with a contiguous last dimension")
    return blocked_k.shape[0], blocked_k.stride(0), blocked_k.stride(1)


def append_kv(kv_c: torch.Tensor, k_pe: torch.Tensor, slot_mapping: torch.Tensor,
              blocked_k: torch.Tensor) -> None:
    """Write token t's entry (kv_c[t] then k_pe[t]) to cache slot slot_mapping[t].

    kv_c bf16 [T, 512], k_pe bf16 [T, 64] (rows may be strided), slot_mapping
    int64 [T] (negative = skip), blocked_k the cache view the decode reads
    ([num_blocks, 64, 1, 576], either entry pitch).  Enqueued on the current
    stream.
    """
    if kv_c.dim() != 2 or kv_c.shape[1] != D_V or k_pe.dim() != 2 or k_pe.shape[1] != D_QK - D_V:
        raise ValueError("kv_c must be [T, 512] and k_pe [T, 64]")
    if kv_c.dtype != torch.bfloat16 or k_pe.dtype != torch.bfloat16:
        raise ValueError("kv_c and k_pe must be bfloat16")
    if slot_mapping.dtype != torch.int64 or slot_mapping.dim() != 1:
        raise ValueError("slot_mapping must be a 1-D int64 tensor")
    t = kv_c.shape[0]
    if k_pe.shape[0] != t or slot_mapping.numel() != t:
        raise ValueError("kv_c, k_pe and slot_mapping disagree on the token count")
    dev = blocked_k.device
    for x in (kv_c, k_pe, slot_mapping):
        if not x.is_cuda or x.device != dev:
            raise ValueError("all tensors must be on the cache's GPU")
    if kv_c.stride(1) != 1 or k_pe.stride(1) != 1:
        raise ValueError("kv_c and k_pe rows must be contiguous")
    nb, bs, rs = _cache_view(blocked_k, "blocked_k")
    slots = slot_mapping.contiguous()
    _lib.check(_lib.load().mla_append_kv(_ptr(kv_c), kv_c.stride(0), _ptr(k_pe), k_pe.stride(0), _ptr(slots),
                                         t, _ptr(blocked_k), nb, bs, rs, _stream(dev)), "mla_append_kv")


def copy_blocks(src_k: torch.Tensor, dst_k: torch.Tensor, block_mapping: torch.Tensor) -> None:
    """Copy page block_mapping[k, 0] of src_k to page block_mapping[k, 1] of dst_k, for every k.

    src_k and dst_k are cache views ([num_blocks, 64, 1, 576], either entry
    pitch; the same tensor for an in-place block copy); block_mapping is int64
    [num_pairs, 2] on the GPU.  Enqueued on the current stream.
    """
    if block_mapping.dtype != torch.int64 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be an int64 [num_pairs, 2] tensor")
    dev = dst_k.device
    if src_k.device != dev or block_mapping.device != dev:
        raise ValueError("all tensors must be on the same GPU")
    sn, sbs, srs = _cache_view(src_k, "src_k")
    dn, dbs, drs = _cache_view(dst_k, "dst_k")
    m = block_mapping.contiguous()
    _lib.check(_lib.load().mla_copy_blocks(_ptr(src_k), sn, sbs, srs, _ptr(dst_k), dn, dbs, drs, _ptr(m),
                                           m.shape[0], _stream(dev)), "mla_copy_blocks")
