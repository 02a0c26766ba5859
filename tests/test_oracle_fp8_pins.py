"""Pins of the oracle's FP8 latent cache against things other than itself.

The FP8 cache is our reading of the FP8 work the Hacker News discussion of
the FlashMLA release links to: every 576-element entry stored as OCP E4M3
bytes (one per element) with one fp32 scale per cache, K and V being the
decoded bytes times the scale.  The pins:

* the byte decode against the format's definition written another way
  (oracle.brute), against torch's float8_e4m3fn, and at the format's
  landmark codes (zero, smallest subnormal and normal, one, largest, NaN);
* attention over an fp8 cache against the scalar brute force on tiny inputs;
* an fp8 cache against the bf16 oracle (pinned in test_oracle_pins.py) on a
  bf16 cache holding exactly the same values;
* the closed form of the scale: scaling the cache by s is the same as
  scaling the scores by s and the output by s;
* planted mistakes in the decode and the scale, each tripping a pin.
"""

import math

import numpy as np
import pytest
import torch

from conftest import bits
from oracle import mla_ref
from oracle.brute import brute_decode, e4m3_to_float
from paged_mla_decode_04_amd.workloads import FP8_KV_SCALE, Workload, draw

TIGHT = 1e-12


def fp8_case(lens, *, s_q=1, h_q=2, causal=False, pitch=576, seed=0, kv_scale=FP8_KV_SCALE,
             poison=False):
    w = Workload("fp8case", batch=len(lens), s_q=s_q, h_q=h_q, causal=causal, seqlens="fixed",
                 fixed_seqlens=tuple(lens), pitch=pitch, kv_format="fp8_e4m3", kv_scale=kv_scale)
    return draw(w, seed=seed, poison=poison)


def run_fp8(inp, **kw):
    kw.setdefault("kv_scale", inp.kv_scale)
    kw.setdefault("softmax_scale", inp.softmax_scale)
    return mla_ref.mla_decode_ref(bits(inp.q), inp.k_storage.numpy(), inp.block_table.numpy(),
                                  inp.cache_seqlens.numpy(), kw.pop("softmax_scale"), inp.causal,
                                  kv_format="fp8_e4m3", **kw)


def close(a, b, tol=TIGHT):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    diff = np.where(same_inf, 0.0, np.abs(a - b))
    return bool(np.all(diff <= tol * np.maximum(1.0, np.abs(np.where(same_inf, 0, b)))))


# ------------------------------------------------------------- the byte decode

def test_decode_matches_the_format_definition_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = mla_ref.e4m3_bits_to_f64(codes)
    theirs = np.array([e4m3_to_float(c) for c in range(256)])
    assert np.array_equal(np.isnan(ours), np.isnan(theirs))
    ok = ~np.isnan(theirs)
    assert np.array_equal(ours[ok], theirs[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(theirs[ok]))


def test_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = mla_ref.e4m3_bits_to_f64(codes.numpy())
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(ours[ok], lib[ok])


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0),
    (0x39, 1.125), (0x40, 2.0), (0x7E, 448.0), (0xFE, -448.0), (0xB8, -1.0), (0x80, -0.0)])
def test_landmark_codes(code, value):
    got = float(mla_ref.e4m3_bits_to_f64(np.array([code], dtype=np.uint8))[0])
    assert got == value and math.copysign(1.0, got) == math.copysign(1.0, value)


def test_only_the_two_all_ones_codes_are_nan():
    v = mla_ref.e4m3_bits_to_f64(np.arange(256, dtype=np.uint8))
    assert sorted(np.flatnonzero(np.isnan(v)).tolist()) == [0x7F, 0xFF]
    assert np.all(np.isfinite(v[~np.isnan(v)]))


# ------------------------------------------------------- attention over bytes

@pytest.mark.parametrize("seed", range(4))
def test_fp8_cache_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(1, 90, size=2)]
    inp = fp8_case(lens, s_q=2, h_q=2, causal=bool(seed % 2), pitch=(576, 640)[seed % 2], seed=seed)
    out, lse = run_fp8(inp)
    bo, bl = brute_decode(bits(inp.q), inp.k_storage.numpy(), inp.block_table.numpy(),
                          inp.cache_seqlens.numpy(), inp.softmax_scale, inp.causal,
                          kv_format="fp8_e4m3", kv_scale=inp.kv_scale)
    assert close(out, np.array(bo)) and close(lse, np.array(bl))


def _bf16_copy_of(inp):
    """A bf16 cache holding exactly the fp8 cache's values (decoded byte times a
    power-of-two scale is exact in bf16: 4 significant bits, exponents far
    inside bf16's range)."""
    vals = mla_ref.e4m3_bits_to_f64(inp.k_storage.numpy()) * inp.kv_scale
    t = torch.from_numpy(vals).to(torch.bfloat16)
    assert np.array_equal(t.to(torch.float64).numpy(), vals, equal_nan=True)
    return t


@pytest.mark.parametrize("kv_scale", [FP8_KV_SCALE, 1.0, 0.5])
def test_fp8_cache_equals_the_bf16_cache_of_its_values(kv_scale):
    inp = fp8_case([70, 129, 5], s_q=2, h_q=4, causal=True, pitch=640, seed=3, kv_scale=kv_scale)
    out, lse = run_fp8(inp)
    k16 = _bf16_copy_of(inp)
    ro, rl = mla_ref.mla_decode_ref(bits(inp.q), bits(k16), inp.block_table.numpy(),
                                    inp.cache_seqlens.numpy(), inp.softmax_scale, inp.causal)
    assert close(out, ro) and close(lse, rl)


@pytest.mark.parametrize("s", [0.25, 3.0, 1.0 / 64.0])
def test_scale_is_a_score_scale_and_an_output_scale(s):
    """Values k = s * e(byte): scores are (softmax_scale * s) * q.e and the
    output is s * sum_t p_t e_t, so decoding with kv_scale s equals decoding
    with kv_scale 1 and softmax_scale * s, times s."""
    inp = fp8_case([50, 100], s_q=1, h_q=3, seed=5)
    out_s, lse_s = run_fp8(inp, kv_scale=s)
    out_1, lse_1 = run_fp8(inp, kv_scale=1.0, softmax_scale=inp.softmax_scale * s)
    assert close(out_s, s * out_1, 1e-11) and close(lse_s, lse_1, 1e-11)


def test_poisoned_bytes_outside_the_sequences_do_not_matter():
    clean = fp8_case([37, 130], h_q=2, pitch=640, seed=9)
    dirty = fp8_case([37, 130], h_q=2, pitch=640, seed=9, poison=True)
    a = run_fp8(clean)
    b = run_fp8(dirty)
    assert close(a[0], b[0], 0.0) and close(a[1], b[1], 0.0)


# ------------------------------------------------ planted mistakes are caught

def _fp8_pin_failures():
    failed = []
    try:
        test_decode_matches_the_format_definition_on_every_code()
    except Exception:
        failed.append("definition")
    try:
        test_fp8_cache_matches_brute_force(1)
    except Exception:
        failed.append("brute")
    try:
        test_fp8_cache_equals_the_bf16_cache_of_its_values(FP8_KV_SCALE)
    except Exception:
        failed.append("bf16")
    try:
        test_scale_is_a_score_scale_and_an_output_scale(3.0)
    except Exception:
        failed.append("scale")
    return failed


def _mut_bias8(orig):
    def f(b):
        b = np.asarray(b).astype(np.uint8).astype(np.int64)
        sign = np.where(b & 0x80, -1.0, 1.0)
        e, m = (b >> 3) & 0xF, (b & 7).astype(np.float64)
        return sign * np.where(e == 0, np.ldexp(m / 8, -6), np.ldexp(1 + m / 8, e - 8))
    return f


def _mut_subnormal_as_normal(orig):
    def f(b):
        b = np.asarray(b).astype(np.uint8).astype(np.int64)
        sign = np.where(b & 0x80, -1.0, 1.0)
        e, m = (b >> 3) & 0xF, (b & 7).astype(np.float64)
        return sign * np.where((e == 0) & (m == 0), 0.0, np.ldexp(1 + m / 8, e - 7))
    return f


def _mut_scale_on_keys_only(orig):
    def f(k_bits, table_row, n, kv_head, block_size=64, d=576, kv_format="bf16", kv_scale=1.0):
        K = orig(k_bits, table_row, n, kv_head, block_size, d, kv_format, 1.0)
        if kv_format == "fp8_e4m3":
            K = K.copy()
            K[:, 512:] *= kv_scale  # only the rope part (K-only columns) scaled
        return K
    return f


FP8_MUTATIONS = {
    "exponent_bias_8": ("e4m3_bits_to_f64", _mut_bias8),
    "subnormal_as_normal": ("e4m3_bits_to_f64", _mut_subnormal_as_normal),
    "scale_on_keys_only": ("gather_tokens", _mut_scale_on_keys_only),
}


def test_fp8_pins_pass_on_the_oracle():
    assert _fp8_pin_failures() == []


@pytest.mark.parametrize("name", sorted(FP8_MUTATIONS))
def test_each_planted_fp8_mistake_trips_a_pin(name, monkeypatch):
    attr, make = FP8_MUTATIONS[name]
    monkeypatch.setattr(mla_ref, attr, make(getattr(mla_ref, attr)))
    assert _fp8_pin_failures() != [], name
