"""fp64 CPU oracle for the fused attention forward pass - TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package. The HIP library and its Python binding never do,
and this package imports nothing from them.

Parity status of each function (what pins it, all in ``tests/test_oracle.py``):
  attention         pinned: closed forms (Q = 0 means of V, single dominant
                    logit, causal row 0), softmax invariants, hand-worked
                    example in ``tests/golden/``, brute-force agreement with
                    ``attention_online``, torch CPU fp64 SDPA cross-check.
  attention_online  pinned against ``attention`` and the same closed forms.
  allowed_mask      pinned by brute-force loops over i, j.
  checker.check     pinned by planted mistakes (NaN, wrong -inf, out of band).
"""
from .attention import allowed_mask, attention, attention_online, bf16_bits_to_f64  # noqa: F401
from .checker import check, CheckResult  # noqa: F401
