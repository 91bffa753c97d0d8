"""fp64 CPU oracle for the attention forward and backward passes - TEST INFRASTRUCTURE.

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
  attention_bwd     pinned (tests/test_oracle_bwd.py): central finite
                    differences of ``attention``, zero-sum of dK over keys,
                    zero gradients for dO = 0 and for V with equal rows, the
                    Q = 0 closed form of dV, torch CPU fp64 autograd cross-check.
  check_grads       pinned by planted mistakes (NaN, out of band).
  e4m3_decode       pinned (tests/test_oracle_fp8.py): the format's defining
                    values, monotonicity, torch float8_e4m3fn cross-check.
  attention_fp8     pinned: pure-Python brute force on tiny inputs, closed
                    forms (Q = 0, equal V rows), descale invariances.
"""
from .attention import (allowed_mask, attention, attention_online, bf16_bits_to_f64, causal_offset,  # noqa: F401
                        expand_block_mask)
from .backward import attention_bwd  # noqa: F401
from .fp8 import attention_fp8, e4m3_decode  # noqa: F401
from .checker import check, check_grads, merge, CheckResult, GradCheckResult  # noqa: F401
