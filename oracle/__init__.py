"""CPU oracle for paged MLA decode -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the graft entry point's smoke check and the benchmark's
CPU-baseline leg may import anything from this package.  The product path
(the HIP library and its Python binding) never does, and fails loudly when
its native library is missing instead of falling back to this code.

Modules:
  mla_ref -- the fp64 NumPy definition (mla_decode_ref, over a bf16 or an
             FP8 E4M3 cache) and the lse merge of key-range partials
             (merge_partials).
  brute   -- a scalar pure-Python statement of the same definition, used to
             pin mla_ref on tiny inputs.

Parity status: every function here is pinned by tests/test_oracle_pins.py
(brute force, closed forms, invariants, a library special case).  The pages
print no out/lse values, so agreement with any published implementation is
not pinned.
"""

from .mla_ref import (bf16_bits_to_f64, e4m3_bits_to_f64, visible_keys, gather_tokens,
                      softmax_average, attend_rows, mla_decode_ref, merge_partials)

__all__ = ["bf16_bits_to_f64", "e4m3_bits_to_f64", "visible_keys", "gather_tokens",
           "softmax_average", "attend_rows", "mla_decode_ref", "merge_partials"]
