"""Per-group learning-rate schedules in fp64.

TEST INFRASTRUCTURE ONLY (imported by tests/, never by the product library).

The SomaSpeed landing page (paragraph 8) requires that every parameter group
keeps its own learning-rate schedule through the fused step; the workloads
name two shapes, a linear warm-up over the first updates and a cosine decay
over the run.  No formula is printed, so the textbook forms are written out
here, for update t = 1, 2, ... (the group's update count):

* linear warm-up over W updates:  lr_t = peak * min(t, W) / W;
* cosine annealing (Loshchilov & Hutter, without restarts) over T updates:
  lr_t = floor + (peak - floor) * (1 + cos(pi * k / T)) / 2 with
  k = min(t - 1, T), so the first update uses the peak and every update from
  T + 1 on uses the floor;
* warm-up then cosine: the warm-up for t <= W, then the cosine over the
  remaining T - W updates starting again from k = 0 at t = W + 1.

Pins: tests/test_schedule_oracle.py (exact rational values of the warm-up,
cosine end points, symmetry, the closed-form sum of one half period, and the
configurations' own schedules).
"""
from __future__ import annotations

import math

NONE, LINEAR_WARMUP, COSINE, WARMUP_COSINE = 0, 1, 2, 3


def warmup_lr(t: int, peak: float, warmup: int) -> float:
    """Linear rise to the peak over `warmup` updates, then the peak."""
    return peak * min(t, warmup) / warmup


def cosine_lr(k: int, peak: float, floor: float, period: int) -> float:
    """Half a cosine period from peak (k = 0) to floor (k = period), held after."""
    k = min(max(k, 0), period)
    return floor + (peak - floor) * 0.5 * (1.0 + math.cos(math.pi * k / period))


def scheduled_lr(kind: int, t: int, lr: float = 0.0, peak: float = 0.0, floor: float = 0.0,
                 warmup: int = 0, total: int = 0) -> float:
    """Learning rate of update t; `lr` is the group's own value for NONE."""
    if kind == NONE:
        return lr
    if kind == LINEAR_WARMUP:
        return warmup_lr(t, peak, warmup)
    if kind == COSINE:
        return cosine_lr(t - 1, peak, floor, total)
    if kind == WARMUP_COSINE:
        if t <= warmup:
            return warmup_lr(t, peak, warmup)
        return cosine_lr(t - warmup - 1, peak, floor, total - warmup)
    raise ValueError(f"unknown schedule kind {kind}")
