"""Host-side accounting of bench.py (CPU only): the effective flops of a
masked workload equal 4*d times the allowed (query, key) pairs counted one by
one from the oracle's explicit mask."""
import numpy as np

import bench
from oracle import allowed_mask
from workloads import Inputs, Workload


def brute_pairs(w, seqlens, qstart):
    n = 0
    for b in range(w.B):
        kv = None if seqlens is None else int(seqlens[b])
        qs = None if qstart is None else int(qstart[b])
        n += int(allowed_mask(w.N_q, w.N_k, w.causal, kv, qs).sum())
    return n * w.H


def test_effective_flops_match_brute_force():
    for causal in (False, True):
        w = Workload("t", B=4, H=3, N_q=50, N_k=50, d=64, causal=causal, seed=0, seqlens_range=(0, 50))
        seqlens = np.array([0, 17, 50, 99], np.int32)     # 99 is clamped to N_k
        qstart = np.array([0, 5, 49, -3], np.int32)      # -3 is clamped to 0
        inp = Inputs(q=None, k=None, v=None, seqlens_k=seqlens, q_start=qstart, scale=w.scale, causal=causal)
        assert bench.effective_flops(w, inp) == 4.0 * w.d * brute_pairs(w, seqlens, qstart)


def test_effective_flops_without_masks_is_the_square_or_triangle():
    w = Workload("t", B=2, H=2, N_q=64, N_k=64, d=128, causal=False, seed=0)
    inp = Inputs(q=None, k=None, v=None, seqlens_k=None, q_start=None, scale=w.scale, causal=False)
    assert bench.effective_flops(w, inp) == w.flops()
    wc = Workload("t", B=2, H=2, N_q=64, N_k=64, d=128, causal=True, seed=0)
    assert bench.effective_flops(wc, inp) == 4.0 * 128 * 2 * 2 * (64 * 65 // 2)


def test_every_workload_has_its_own_metric():
    from workloads import HEADLINE, WORKLOADS
    names = {bench.metric_of(w) for w in WORKLOADS.values()}
    assert len(names) == len(WORKLOADS)
    assert bench.metric_of(WORKLOADS[HEADLINE]) == bench.METRIC


def test_every_fp8_workload_has_its_own_metric():
    from workloads import HEADLINE, WORKLOADS
    fixed = [w for w in WORKLOADS.values() if w.seqlens_range is None]
    names = {bench.fp8_metric_of(w) for w in fixed}
    assert len(names) == len(fixed)
    assert bench.fp8_metric_of(WORKLOADS[HEADLINE]) == bench.FP8_METRIC
    assert "non-causal" in bench.fp8_metric_of(WORKLOADS["noncausal_n4096_d128"])


def test_every_backward_workload_has_its_own_metric():
    from workloads import HEADLINE, WORKLOADS
    names = {bench.bwd_metric_of(w) for w in WORKLOADS.values()}
    assert len(names) == len(WORKLOADS)
    assert bench.bwd_metric_of(WORKLOADS[HEADLINE]) == bench.BWD_METRIC
