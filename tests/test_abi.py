"""The C ABI: the library loads, exports what the header declares, and rejects
bad arguments with the documented status before touching any device.

None of these tests makes a HIP call: every case fails host-side validation.
"""

import ctypes
import os
import re

import pytest

from paged_mla_decode_04_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from paged_mla_decode_04_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_params_struct_layout_matches(lib):
    assert lib.mla_decode_params_size() == ctypes.sizeof(_lib.DecodeParams)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (MLA_[A-Z0-9_]+) (\d+)", text))
    assert int(consts["MLA_TILE_MD_INTS"]) == _lib.TILE_MD_INTS
    assert int(consts["MLA_ROWS_PER_WORKGROUP"]) == _lib.ROWS_PER_WORKGROUP
    assert int(consts["MLA_MAX_ROWS"]) == _lib.MAX_ROWS
    assert int(consts["MLA_KV_BF16"]) == _lib.KV_BF16
    assert int(consts["MLA_KV_FP8_E4M3"]) == _lib.KV_FP8_E4M3
    codes = dict(re.findall(r"(MLA_(?:OK|ERR_[A-Z_]+)) = (\d+)", text))
    for k, v in codes.items():
        assert getattr(_lib, k) == int(v), k


def test_status_strings(lib):
    for s in range(9):
        assert lib.mla_status_string(s)
    assert lib.mla_status_string(99) == b"unknown status"


# A valid-looking parameter block with fake (never dereferenced) pointers.
FAKE = 0x10000


def good_params(**over):
    p = _lib.DecodeParams()
    vals = dict(q=FAKE, q_batch_stride=576, q_seq_stride=576, q_head_stride=576, batch=2, s_q=1, h_q=16,
                k_cache=FAKE, k_block_stride=64 * 576, k_row_stride=576, k_head_stride=576,
                num_blocks=8, block_size=64, h_kv=1, d=576, block_table=FAKE, block_table_stride=4,
                max_blocks_per_seq=4, cache_seqlens=FAKE, dv=512, softmax_scale=0.07, causal=0,
                tile_md=FAKE, num_splits=FAKE, num_parts=4, workspace=FAKE, workspace_bytes=1 << 30,
                out=FAKE, out_batch_stride=512 * 16, out_seq_stride=512 * 16, out_head_stride=512,
                lse=FAKE, lse_batch_stride=16, lse_seq_stride=16, lse_head_stride=1)
    vals.update(over)
    for k, v in vals.items():
        setattr(p, k, v)
    return p


BAD = [
    ("null q", dict(q=None), _lib.MLA_ERR_NULL_POINTER),
    ("null cache", dict(k_cache=None), _lib.MLA_ERR_NULL_POINTER),
    ("null table", dict(block_table=None), _lib.MLA_ERR_NULL_POINTER),
    ("null seqlens", dict(cache_seqlens=None), _lib.MLA_ERR_NULL_POINTER),
    ("null out", dict(out=None), _lib.MLA_ERR_NULL_POINTER),
    ("null lse", dict(lse=None), _lib.MLA_ERR_NULL_POINTER),
    ("null workspace", dict(workspace=None), _lib.MLA_ERR_NULL_POINTER),
    ("half a plan", dict(num_splits=None), _lib.MLA_ERR_NULL_POINTER),
    ("negative batch", dict(batch=-1), _lib.MLA_ERR_BAD_SHAPE),
    ("zero s_q", dict(s_q=0), _lib.MLA_ERR_BAD_SHAPE),
    ("zero heads", dict(h_q=0), _lib.MLA_ERR_BAD_SHAPE),
    ("d 512", dict(d=512), _lib.MLA_ERR_UNSUPPORTED),
    ("dv 576", dict(dv=576), _lib.MLA_ERR_UNSUPPORTED),
    ("block 16", dict(block_size=16), _lib.MLA_ERR_UNSUPPORTED),
    ("two kv heads", dict(h_kv=2, h_q=16), _lib.MLA_ERR_UNSUPPORTED),
    ("too many rows", dict(h_q=1025), _lib.MLA_ERR_UNSUPPORTED),
    ("nan scale", dict(softmax_scale=float("nan")), _lib.MLA_ERR_BAD_ARGUMENT),
    ("inf scale", dict(softmax_scale=float("inf")), _lib.MLA_ERR_BAD_ARGUMENT),
    ("misaligned q", dict(q=FAKE + 8), _lib.MLA_ERR_BAD_STRIDE),
    ("misaligned cache", dict(k_cache=FAKE + 2), _lib.MLA_ERR_BAD_STRIDE),
    ("misaligned out", dict(out=FAKE + 4), _lib.MLA_ERR_BAD_STRIDE),
    ("misaligned workspace", dict(workspace=FAKE + 16), _lib.MLA_ERR_BAD_STRIDE),
    ("odd q stride", dict(q_head_stride=580), _lib.MLA_ERR_BAD_STRIDE),
    ("pitch < d", dict(k_row_stride=568), _lib.MLA_ERR_BAD_STRIDE),
    ("odd pitch", dict(k_row_stride=577), _lib.MLA_ERR_BAD_STRIDE),
    ("odd out stride", dict(out_head_stride=514), _lib.MLA_ERR_BAD_STRIDE),
    ("negative lse stride", dict(lse_head_stride=-1), _lib.MLA_ERR_BAD_STRIDE),
    ("table stride", dict(block_table_stride=3), _lib.MLA_ERR_BAD_STRIDE),
    ("blocks overlap", dict(k_block_stride=63 * 576), _lib.MLA_ERR_BAD_STRIDE),
    ("plan without parts", dict(num_parts=0), _lib.MLA_ERR_BAD_SHAPE),
    ("workspace too small", dict(workspace_bytes=1024), _lib.MLA_ERR_WORKSPACE_TOO_SMALL),
    ("unknown cache type", dict(kv_dtype=2), _lib.MLA_ERR_BAD_ARGUMENT),
    ("fp8 without a scale", dict(kv_dtype=_lib.KV_FP8_E4M3, kv_scale=0.0), _lib.MLA_ERR_BAD_ARGUMENT),
    ("fp8 negative scale", dict(kv_dtype=_lib.KV_FP8_E4M3, kv_scale=-1.0), _lib.MLA_ERR_BAD_ARGUMENT),
    ("fp8 nan scale", dict(kv_dtype=_lib.KV_FP8_E4M3, kv_scale=float("nan")), _lib.MLA_ERR_BAD_ARGUMENT),
    ("fp8 inf scale", dict(kv_dtype=_lib.KV_FP8_E4M3, kv_scale=float("inf")), _lib.MLA_ERR_BAD_ARGUMENT),
    # an fp8 row is 1 byte per element: the pitch must be a multiple of 16 bytes
    ("fp8 pitch 584", dict(kv_dtype=_lib.KV_FP8_E4M3, kv_scale=0.5, k_row_stride=584,
                            k_block_stride=64 * 584), _lib.MLA_ERR_BAD_STRIDE),
    ("fp8 block stride", dict(kv_dtype=_lib.KV_FP8_E4M3, kv_scale=0.5, k_block_stride=64 * 576 + 8),
     _lib.MLA_ERR_BAD_STRIDE),
]


@pytest.mark.parametrize("name,over,status", BAD, ids=[b[0] for b in BAD])
def test_decode_rejects_bad_arguments(lib, name, over, status):
    p = good_params(**over)
    assert lib.mla_decode_with_kvcache(ctypes.byref(p), None) == status


def test_decode_rejects_null_params(lib):
    assert lib.mla_decode_with_kvcache(None, None) == _lib.MLA_ERR_NULL_POINTER


def test_batch_past_the_device_plan_needs_metadata(lib):
    # without metadata the library plans on the device, which holds at most
    # 16384 sequences; with metadata any batch is accepted
    p = good_params(batch=16385, tile_md=None, num_splits=None, num_parts=4)
    assert lib.mla_decode_with_kvcache(ctypes.byref(p), None) == _lib.MLA_ERR_UNSUPPORTED


def test_empty_batch_is_a_no_op(lib):
    p = good_params(batch=0, q=None, out=None)
    assert lib.mla_decode_with_kvcache(ctypes.byref(p), None) == _lib.MLA_OK


def test_metadata_rejects_bad_arguments(lib):
    buf = (ctypes.c_int32 * 64)()
    f = lib.mla_get_metadata
    assert f(None, 2, 16, 1, 4, buf, buf, None) == _lib.MLA_ERR_NULL_POINTER
    assert f(buf, 2, 16, 1, 4, None, buf, None) == _lib.MLA_ERR_NULL_POINTER
    assert f(buf, 2, 16, 1, 0, buf, buf, None) == _lib.MLA_ERR_BAD_SHAPE
    assert f(buf, -1, 16, 1, 4, buf, buf, None) == _lib.MLA_ERR_BAD_SHAPE
    assert f(buf, 2, 15, 2, 4, buf, buf, None) == _lib.MLA_ERR_BAD_SHAPE
    assert f(buf, 2, 4096, 1, 4, buf, buf, None) == _lib.MLA_ERR_UNSUPPORTED


def test_workspace_size_formula(lib):
    n = ctypes.c_size_t()

    def a256(x):
        return (x + 255) // 256 * 256

    for b, s_q, h_q, parts in [(2, 1, 16, 7), (128, 1, 128, 128), (64, 2, 128, 64)]:
        assert lib.mla_workspace_size(b, s_q, h_q, 1, 512, parts, ctypes.byref(n)) == _lib.MLA_OK
        rows = s_q * h_q
        slots = b + parts
        # plan, partial lse, partial row scales, partial O
        want = (a256(parts * 8 * 4) + a256((b + 1) * 4) + 2 * a256(slots * rows * 4)
                + a256(slots * rows * 512 * 4))
        assert n.value == want
    assert lib.mla_workspace_size(2, 1, 16, 1, 512, 4, None) == _lib.MLA_ERR_NULL_POINTER
    assert lib.mla_workspace_size(2, 0, 16, 1, 512, 4, ctypes.byref(n)) == _lib.MLA_ERR_BAD_SHAPE


def append_args(**over):
    vals = dict(kv_c=FAKE, kv_c_stride=512, k_pe=FAKE, k_pe_stride=64, slots=FAKE, num_tokens=4, cache=FAKE,
                num_blocks=8, block_stride=64 * 640, row_stride=640, stream=None)
    vals.update(over)
    return [vals[k] for k in ("kv_c", "kv_c_stride", "k_pe", "k_pe_stride", "slots", "num_tokens", "cache",
                              "num_blocks", "block_stride", "row_stride", "stream")]


APPEND_BAD = [
    ("null kv_c", dict(kv_c=None), _lib.MLA_ERR_NULL_POINTER),
    ("null k_pe", dict(k_pe=None), _lib.MLA_ERR_NULL_POINTER),
    ("null slots", dict(slots=None), _lib.MLA_ERR_NULL_POINTER),
    ("null cache", dict(cache=None), _lib.MLA_ERR_NULL_POINTER),
    ("negative tokens", dict(num_tokens=-1), _lib.MLA_ERR_BAD_SHAPE),
    ("negative blocks", dict(num_blocks=-1), _lib.MLA_ERR_BAD_SHAPE),
    ("misaligned cache", dict(cache=FAKE + 8), _lib.MLA_ERR_BAD_STRIDE),
    ("misaligned kv_c", dict(kv_c=FAKE + 2), _lib.MLA_ERR_BAD_STRIDE),
    ("short kv_c rows", dict(kv_c_stride=504), _lib.MLA_ERR_BAD_STRIDE),
    ("odd k_pe rows", dict(k_pe_stride=68), _lib.MLA_ERR_BAD_STRIDE),
    ("pitch < 576", dict(row_stride=568, block_stride=64 * 568), _lib.MLA_ERR_BAD_STRIDE),
    ("odd pitch", dict(row_stride=580, block_stride=64 * 580), _lib.MLA_ERR_BAD_STRIDE),
    ("pages overlap", dict(block_stride=63 * 640), _lib.MLA_ERR_BAD_STRIDE),
]


@pytest.mark.parametrize("name,over,status", APPEND_BAD, ids=[b[0] for b in APPEND_BAD])
def test_append_rejects_bad_arguments(lib, name, over, status):
    assert lib.mla_append_kv(*append_args(**over)) == status


def test_append_of_no_tokens_is_a_no_op(lib):
    assert lib.mla_append_kv(*append_args(num_tokens=0, kv_c=None, cache=None)) == _lib.MLA_OK


def test_copy_blocks_rejects_bad_arguments(lib):
    f = lib.mla_copy_blocks
    ok = (FAKE, 8, 64 * 576, 576, FAKE, 8, 64 * 640, 640, FAKE, 2, None)

    def call(**over):
        names = ("src", "sn", "sbs", "srs", "dst", "dn", "dbs", "drs", "map", "pairs", "stream")
        args = dict(zip(names, ok))
        args.update(over)
        return f(*[args[n] for n in names])

    assert call(src=None) == _lib.MLA_ERR_NULL_POINTER
    assert call(dst=None) == _lib.MLA_ERR_NULL_POINTER
    assert call(map=None) == _lib.MLA_ERR_NULL_POINTER
    assert call(pairs=-1) == _lib.MLA_ERR_BAD_SHAPE
    assert call(pairs=0, src=None, map=None) == _lib.MLA_OK
    assert call(sn=-2) == _lib.MLA_ERR_BAD_SHAPE
    assert call(srs=570) == _lib.MLA_ERR_BAD_STRIDE
    assert call(dbs=63 * 640) == _lib.MLA_ERR_BAD_STRIDE
    assert call(dst=FAKE + 4) == _lib.MLA_ERR_BAD_STRIDE
