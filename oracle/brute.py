"""Scalar brute-force paged MLA decode, for tiny inputs.

TEST INFRASTRUCTURE ONLY (same rule as mla_ref: only tests, the smoke check
and the benchmark's CPU-baseline leg may use anything under oracle/).

A second, deliberately naive statement of the same definition as
mla_ref.mla_decode_ref, written without NumPy and without any of mla_ref's
helpers: triple loops over tokens, heads and elements, exactly rounded sums
(math.fsum), and its own bf16 decode through struct.  The NumPy oracle is
trusted only because it agrees with this one on small cases.

Definition (see mla_ref for the sources): for query token i of s_q, head h,
kv head g = h // (h_q // h_kv), the visible keys are the first n tokens, or
the first n - (s_q - 1 - i) with causal masking; score s_t = scale * q . k_t
over all 576 elements; out = sum_t softmax(s)_t * k_t[0:512]; lse is the
natural log of sum_t exp(s_t); no visible key gives out = 0, lse = -inf.
"""

from __future__ import annotations

import math
import struct


def bf16_to_float(bits: int) -> float:
    """A bf16 bit pattern is the top half of an IEEE single."""
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def e4m3_to_float(byte: int) -> float:
    """An FP8 E4M3 byte (OCP "fn" variant) from its fields, written as an
    integer significand times a power of two: 8 + m for a normal number
    (exponent field e > 0), m for a subnormal, scaled by 2^(max(e, 1) - 10);
    the code with every exponent and mantissa bit set is NaN."""
    byte = int(byte) & 0xFF
    e, m = (byte >> 3) & 0xF, byte & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    sig = (8 + m) if e > 0 else m
    val = math.ldexp(sig, max(e, 1) - 10)
    return -val if byte & 0x80 else val


def brute_decode(q_bits, k_bits, block_table, cache_seqlens, softmax_scale, causal,
                 d=576, dv=512, block_size=64, kv_format="bf16", kv_scale=1.0):
    """q_bits[b][i][h][c], k_bits[page][row][g][c]: nested sequences (or arrays)
    of raw bf16 bits, or for kv_format "fp8_e4m3" raw E4M3 cache bytes whose
    values are times kv_scale.  Returns nested lists out[b][i][h][c] and
    lse[b][i][h]."""
    if kv_format == "bf16":
        kdec = bf16_to_float
    elif kv_format == "fp8_e4m3":
        def kdec(x):
            return e4m3_to_float(x) * kv_scale
    else:
        raise ValueError(kv_format)
    B = len(q_bits)
    out, lse = [], []
    for b in range(B):
        s_q = len(q_bits[b])
        h_q = len(q_bits[b][0])
        h_kv = len(k_bits[0][0])
        n = int(cache_seqlens[b])
        ob, lb = [], []
        for i in range(s_q):
            oi, li = [], []
            if causal:
                visible = n - (s_q - 1 - i)
            else:
                visible = n
            for h in range(h_q):
                g = h // (h_q // h_kv)
                qs = [bf16_to_float(q_bits[b][i][h][c]) for c in range(d)]
                scores, vrows = [], []
                for t in range(max(visible, 0)):
                    page = int(block_table[b][t // block_size])
                    row = t % block_size
                    kt = [kdec(k_bits[page][row][g][c]) for c in range(d)]
                    scores.append(softmax_scale * math.fsum(qs[c] * kt[c] for c in range(d)))
                    vrows.append(kt[:dv])
                if not scores:
                    oi.append([0.0] * dv)
                    li.append(-math.inf)
                    continue
                top = max(scores)
                total = math.fsum(math.exp(s - top) for s in scores)
                lse_h = top + math.log(total)
                weights = [math.exp(s - lse_h) for s in scores]
                oi.append([math.fsum(weights[t] * vrows[t][c] for t in range(len(vrows)))
                           for c in range(dv)])
                li.append(lse_h)
            ob.append(oi)
            lb.append(li)
        out.append(ob)
        lse.append(lb)
    return out, lse
