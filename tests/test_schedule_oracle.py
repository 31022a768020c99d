"""Pins of the oracle's learning-rate schedules (oracle/schedule_fp64.py).

Each pin comes from the mathematics, not from re-typing the formula: exact
rational values of the warm-up, the cosine's end points and its symmetry about
the half-period, and the closed form of one half period's sum,
sum_{k=0}^{T-1} cos(pi k / T) = 1 (so a schedule that starts at k = 1 instead
of k = 0 is off by peak - floor).  Planted mistakes must each fail a pin.
"""
import math
from fractions import Fraction

import pytest

from oracle import schedule_fp64 as S

PEAK, FLOOR = 5e-6, 4e-7


def ulps(x, y):
    return abs(x - y) / math.ulp(max(abs(x), abs(y), 1e-300))


def pins(lr_fn):
    """Return the names of the pins that the schedule function `lr_fn(kind, t, peak, floor, W, T)` fails."""
    bad = []
    W, T = 10, 16
    # warm-up: exact fractions peak * t / W (two roundings at most) and the peak after W
    for t in range(1, 3 * W):
        exact = Fraction(PEAK) * min(t, W) / W
        if ulps(lr_fn(S.LINEAR_WARMUP, t, PEAK, 0.0, W, 0), float(exact)) > 1.0:
            bad.append(f"warmup t={t}")
            break
    # cosine end points: the peak at t = 1, the floor from t = T + 1 on
    if ulps(lr_fn(S.COSINE, 1, PEAK, FLOOR, 0, T), PEAK) > 1.0:
        bad.append("cosine start")
    for t in (T + 1, T + 2, 3 * T):
        if lr_fn(S.COSINE, t, PEAK, FLOOR, 0, T) != FLOOR:
            bad.append(f"cosine floor t={t}")
            break
    # half period: the mean of peak and floor at t = T / 2 + 1
    if abs(lr_fn(S.COSINE, T // 2 + 1, PEAK, FLOOR, 0, T) - (PEAK + FLOOR) / 2) > 1e-15 * PEAK:
        bad.append("cosine half period")
    # symmetry: lr(t) + lr(T + 2 - t) = peak + floor (cos(pi - x) = -cos x)
    for t in range(1, T + 2):
        s = lr_fn(S.COSINE, t, PEAK, FLOOR, 0, T) + lr_fn(S.COSINE, T + 2 - t, PEAK, FLOOR, 0, T)
        if abs(s - (PEAK + FLOOR)) > 1e-15 * PEAK:
            bad.append(f"cosine symmetry t={t}")
            break
    # sum over one half period: T floor + (peak - floor)(T + 1) / 2
    total = math.fsum(lr_fn(S.COSINE, t, PEAK, FLOOR, 0, T) for t in range(1, T + 1))
    if abs(total - (T * FLOOR + (PEAK - FLOOR) * (T + 1) / 2)) > 1e-14 * PEAK * T:
        bad.append("cosine sum")
    # monotone: non-decreasing warm-up, non-increasing cosine
    c = [lr_fn(S.COSINE, t, PEAK, FLOOR, 0, T) for t in range(1, T + 3)]
    if any(b > a for a, b in zip(c, c[1:])):
        bad.append("cosine monotone")
    # warm-up then cosine: the warm-up up to W, the peak again at W + 1, the floor at T + 1
    Wc, Tc = 4, 14
    if lr_fn(S.WARMUP_COSINE, 2, PEAK, FLOOR, Wc, Tc) != lr_fn(S.LINEAR_WARMUP, 2, PEAK, 0.0, Wc, 0):
        bad.append("warmup-cosine rise")
    if ulps(lr_fn(S.WARMUP_COSINE, Wc + 1, PEAK, FLOOR, Wc, Tc), PEAK) > 1.0:
        bad.append("warmup-cosine restart")
    if lr_fn(S.WARMUP_COSINE, Tc + 1, PEAK, FLOOR, Wc, Tc) != FLOOR:
        bad.append("warmup-cosine floor")
    return bad


def oracle_fn(kind, t, peak, floor, w, total):
    return S.scheduled_lr(kind, t, peak=peak, floor=floor, warmup=w, total=total)


def test_oracle_schedules_pass_every_pin():
    assert pins(oracle_fn) == []


def test_none_returns_the_groups_lr():
    assert S.scheduled_lr(S.NONE, 7, lr=3.25e-5) == 3.25e-5


def _mutant(change):
    def fn(kind, t, peak, floor, w, total):
        if change == "k_from_t":            # cosine indexed from t instead of t - 1
            if kind == S.COSINE:
                return S.cosine_lr(t, peak, floor, total)
        if change == "no_half":             # (1 + cos) not halved
            if kind == S.COSINE:
                k = min(max(t - 1, 0), total)
                return floor + (peak - floor) * (1.0 + math.cos(math.pi * k / total))
        if change == "floor_dropped":       # decays to zero instead of the floor
            if kind == S.COSINE:
                return S.cosine_lr(t - 1, peak - floor, 0.0, total)
        if change == "warmup_from_zero":    # warm-up uses t - 1
            if kind == S.LINEAR_WARMUP:
                return peak * min(t - 1, w) / w
        if change == "no_restart":          # warm-up-cosine continues the cosine from t
            if kind == S.WARMUP_COSINE and t > w:
                return S.cosine_lr(t - 1, peak, floor, total)
        if change == "unclamped":           # the cosine rises again after T
            if kind == S.COSINE:
                return floor + (peak - floor) * 0.5 * (1.0 + math.cos(math.pi * (t - 1) / total))
        return oracle_fn(kind, t, peak, floor, w, total)
    return fn


@pytest.mark.parametrize("change", ["k_from_t", "no_half", "floor_dropped", "warmup_from_zero",
                                    "no_restart", "unclamped"])
def test_planted_mistakes_fail_a_pin(change):
    assert pins(_mutant(change)), f"mutant {change} passes every pin"


def test_configurations_schedules_are_these_forms():
    """The launch-bound configuration warms up linearly over its 10 updates and
    the sharded 7B configuration decays along a cosine to zero over 10."""
    from tensor_optimizer_step_amd import workloads as W
    lb = W.launch_bound(n_tensors=30)
    for k in range(1, 11):
        want = [S.scheduled_lr(S.LINEAR_WARMUP, k, peak=g.lr, warmup=lb.steps) for g in lb.groups]
        assert lb.lrs_for_step(k) == want
    groups = [W.GroupHP(5e-6, 0.01), W.GroupHP(5e-6, 0.0)]
    cos_wl = W.Workload("cos", 5, [W.TensorSpec("t", 8, 0, W.F32)], groups, 1.0, 1.0, steps=10,
                        schedule="cosine")
    for k in range(1, 11):
        want = [S.scheduled_lr(S.COSINE, k, peak=g.lr, floor=0.0, total=10) for g in groups]
        got = cos_wl.lrs_for_step(k)
        assert all(ulps(a, b) <= 1.0 for a, b in zip(got, want)), (k, got, want)
