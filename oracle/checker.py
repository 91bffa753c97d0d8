"""Tolerance checker comparing a tested O / LSE with the fp64 oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/attention.py``).

Bars (element by element, over every compared row):
  * O (bfloat16 result expanded to float64): max |dO| <= 2e-2 and mean |dO| <= 2e-3;
    any NaN or Inf fails; a row the oracle marks fully masked must be exactly 0.
  * LSE (float32 result): |dLSE| <= 1e-3 on rows with a finite oracle value;
    a fully masked row must be exactly -inf; any NaN fails.
Why these bars hold for a correct bf16 kernel: O is a convex combination of V
rows, so |O| <= max|V| and its final bf16 rounding is at most half an ulp
(2**-7 for |O| < 4); the fp32 running state adds far less.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3


@dataclass
class CheckResult:
    ok: bool
    o_max_abs: float
    o_mean_abs: float
    lse_max_abs: float
    reasons: list
    o_abs_sum: float = 0.0     # sum of |dO| over the compared elements (for merging slices)
    o_count: int = 0           # number of compared O elements

    def __str__(self) -> str:
        state = "PASS" if self.ok else "FAIL"
        return (f"{state} O max|d|={self.o_max_abs:.3e} mean|d|={self.o_mean_abs:.3e} "
                f"LSE max|d|={self.lse_max_abs:.3e} {'; '.join(self.reasons)}")


def check(o_test: np.ndarray, o_ref: np.ndarray, lse_test: Optional[np.ndarray] = None,
          lse_ref: Optional[np.ndarray] = None, mean_bar: bool = True) -> CheckResult:
    """Compare float64 views of the tested outputs with the oracle's.

    ``o_test``/``o_ref``: [..., R, d]; ``lse_test``/``lse_ref``: [..., R].
    A row is fully masked when its oracle LSE is -inf (the oracle's O is 0 there).
    ``mean_bar=False`` leaves the mean-abs bar to ``merge`` (one slice of a
    larger output, whose mean is taken over all slices together).
    """
    o_test = np.asarray(o_test, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    reasons = []
    if o_test.shape != o_ref.shape:
        return CheckResult(False, np.inf, np.inf, np.inf, [f"O shape {o_test.shape} != {o_ref.shape}"])
    if not np.all(np.isfinite(o_test)):
        reasons.append(f"O has {int(np.sum(~np.isfinite(o_test)))} non-finite values")
    diff = np.abs(o_test - o_ref)
    diff = np.where(np.isfinite(diff), diff, np.inf)
    o_max = float(diff.max()) if diff.size else 0.0
    o_mean = float(diff.mean()) if diff.size else 0.0
    if o_max > O_MAX_ABS:
        reasons.append(f"O max abs {o_max:.3e} > {O_MAX_ABS}")
    if mean_bar and o_mean > O_MEAN_ABS:
        reasons.append(f"O mean abs {o_mean:.3e} > {O_MEAN_ABS}")
    o_sum = float(diff.sum()) if diff.size else 0.0
    lse_max = 0.0
    if lse_ref is not None:
        lse_ref = np.asarray(lse_ref, dtype=np.float64)
        dead = np.isneginf(lse_ref)
        if np.any(dead):
            rows_nonzero = np.any(o_test[dead] != 0.0, axis=-1) if o_test[dead].size else np.zeros(0, bool)
            if np.any(rows_nonzero):
                reasons.append(f"{int(rows_nonzero.sum())} fully masked rows have nonzero O")
        if lse_test is not None:
            lse_test = np.asarray(lse_test, dtype=np.float64)
            if lse_test.shape != lse_ref.shape:
                return CheckResult(False, o_max, o_mean, np.inf, [f"LSE shape {lse_test.shape} != {lse_ref.shape}"])
            if np.any(np.isnan(lse_test)):
                reasons.append(f"LSE has {int(np.isnan(lse_test).sum())} NaN values")
            if np.any(dead) and not np.all(np.isneginf(lse_test[dead])):
                reasons.append("fully masked rows have LSE != -inf")
            live = ~dead
            if np.any(live):
                d = np.abs(lse_test[live] - lse_ref[live])
                d = np.where(np.isfinite(d), d, np.inf)
                lse_max = float(d.max())
                if lse_max > LSE_MAX_ABS:
                    reasons.append(f"LSE max abs {lse_max:.3e} > {LSE_MAX_ABS}")
    return CheckResult(not reasons, o_max, o_mean, lse_max, reasons, o_sum, int(diff.size))


def merge(parts) -> CheckResult:
    """One verdict for a whole output checked slice by slice (``check(...,
    mean_bar=False)`` on each): the max bars are the slices' maxima, the
    mean-abs bar is applied to the mean over every element of every slice."""
    parts = list(parts)
    reasons = [r for p in parts for r in p.reasons]
    o_max = max((p.o_max_abs for p in parts), default=0.0)
    lse_max = max((p.lse_max_abs for p in parts), default=0.0)
    total = sum(p.o_abs_sum for p in parts)
    count = sum(p.o_count for p in parts)
    o_mean = total / count if count else 0.0
    if o_mean > O_MEAN_ABS:
        reasons.append(f"O mean abs {o_mean:.3e} > {O_MEAN_ABS} over {count} elements")
    return CheckResult(not reasons, o_max, o_mean, lse_max, reasons, total, count)


# Gradients (the backward pass). The benchmark statement fixes no tolerance for
# them, so the bars are derived from bf16's 8-bit significand, relative to each
# tensor's size. A bf16 result carries a rounding error of at most 2**-9 of its
# magnitude (about 2**-10.5 on average), and the bf16 rounding of the
# recomputed probabilities and score gradients that feed the matrix products
# adds errors of the same relative size; in rows where a few keys dominate they
# do not cancel, so the mean error is a few times 2**-10 of the mean magnitude.
# Bars: the max against the forward's 2e-2 scaled by the largest magnitude, the
# mean against 1 % of the mean magnitude (about 3x the expected error; a wrong
# index, sign or term gives errors of the order of the values themselves).
GRAD_MAX_REL = 2e-2     # max |d| <= GRAD_MAX_REL * max(1, max |ref|)
GRAD_MEAN_REL = 1e-2    # mean |d| <= GRAD_MEAN_REL * mean |ref| + GRAD_MEAN_FLOOR
GRAD_MEAN_FLOOR = 1e-6


@dataclass
class GradCheckResult:
    ok: bool
    stats: dict
    reasons: list

    def __str__(self) -> str:
        state = "PASS" if self.ok else "FAIL"
        parts = [f"{n} max|d|={s[0]:.3e} (bar {s[1]:.2e}) mean|d|={s[2]:.3e} (bar {s[3]:.2e})"
                 for n, s in self.stats.items()]
        return f"{state} " + "; ".join(parts) + ("" if self.ok else " :: " + "; ".join(self.reasons))


def check_grads(test: dict, ref: dict) -> GradCheckResult:
    """Compare tested gradients with the oracle's, tensor by tensor.

    ``test`` and ``ref`` map names ("dq", "dk", "dv") to float64 views of
    equal shape. Any NaN or Inf in a tested tensor fails.
    """
    reasons, stats = [], {}
    for name, r in ref.items():
        r = np.asarray(r, dtype=np.float64)
        t = np.asarray(test[name], dtype=np.float64)
        if t.shape != r.shape:
            reasons.append(f"{name} shape {t.shape} != {r.shape}")
            continue
        if not np.all(np.isfinite(t)):
            reasons.append(f"{name} has {int(np.sum(~np.isfinite(t)))} non-finite values")
        d = np.abs(t - r)
        d = np.where(np.isfinite(d), d, np.inf)
        mx = float(d.max()) if d.size else 0.0
        mn = float(d.mean()) if d.size else 0.0
        bar_max = GRAD_MAX_REL * max(1.0, float(np.abs(r).max()) if r.size else 0.0)
        bar_mean = GRAD_MEAN_REL * (float(np.abs(r).mean()) if r.size else 0.0) + GRAD_MEAN_FLOOR
        stats[name] = (mx, bar_max, mn, bar_mean)
        if mx > bar_max:
            reasons.append(f"{name} max abs {mx:.3e} > {bar_max:.3e}")
        if mn > bar_mean:
            reasons.append(f"{name} mean abs {mn:.3e} > {bar_mean:.3e}")
    return GradCheckResult(not reasons, stats, reasons)
