"""fp64 CPU oracle for the fused clip + AdamW optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP library: it is the plain definition written out
in NumPy float64, slow and obviously correct.

What it computes (one optimizer step after backward), following the SomaSpeed
landing page, prose paragraphs 7 and 8 (numbered in page order after the
title; they name the post-backward work and its fused form):

1. normalize every trainable gradient for the effective batch (divide by D);
2. measure one global L2 norm over the normalized gradients, in which every
   owned element counts once (every gradient shard enters exactly once);
3. take one global clipping decision c = min(1, max_norm / (norm + 1e-6)),
   the torch ``clip_grad_norm_`` rule the veRL page calls with max_norm=1.0
   ("Phase 4: Actor Update", section 4.2 "PPO Update": the gradient clip and
   optimizer step that follow the accumulated micro-batches);
4. update weights and both running moments with decoupled-weight-decay AdamW
   from the original gradients, per parameter group, with fp32 states widened
   to fp64 (RLinf page, "Retaining Low-Precision Gradients": gradients are
   converted for the update and optimizer states are kept in fp32).

Gradient buffers are never written, and frozen tensors are never read or
written (landing page, paragraph 8).

Readings where the pages are silent (each also listed in the design notes):
* AdamW is the textbook decoupled form (Loshchilov & Hutter) in torch's
  parameterization: decay lr*wd applied to the pre-update weight, bias
  corrections 1 - beta^t, eps added to sqrt(v_hat).
* The norm is measured after the effective-batch division.
* The step counter t is per group and is 1 on the first update.
* A non-finite sum of squares is not skipped: c is computed literally (NaN
  propagates) and a non-finite flag is raised.

Pins: every function here is pinned by tests/test_oracle_pins.py against
closed forms, exact decimal brute force, invariants, and torch's CPU float64
``clip_grad_norm_`` + ``AdamW`` as a library special case.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

CLIP_EPS = 1e-6  # added to the norm in the clip coefficient (torch clip_grad_norm_ rule)


def widen_grad(g: np.ndarray) -> np.ndarray:
    """Exact widening of a gradient buffer to float64.

    ``g`` is float32 values, float16 values, or uint16 bf16 bit patterns; bf16
    is the top half of an IEEE float32, so shifting the bits left by 16 is
    exact.  (RLinf page, "Retaining Low-Precision Gradients": gradients kept in
    the compute dtype are converted to fp32 for the update.)
    """
    g = np.asarray(g)
    if g.dtype == np.uint16:
        return (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if g.dtype in (np.float16, np.float32, np.float64):
        return g.astype(np.float64)
    raise TypeError(f"unsupported gradient dtype {g.dtype}")


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 working copy of fp32 master weights: round to nearest, ties to even.

    RLinf page, "Retaining Low-Precision Gradients": bf16/fp16 parameters keep
    an fp32 master copy; the working copy is the master rounded to bf16.  The
    rounding decision is taken from the fp32 value, as the master is fp32.
    Returns uint16 bit patterns; NaN maps to a quiet NaN.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + keep_lsb) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    return np.where(nan, np.uint16(0x7FC0), rounded)


def round_to_f16(x: np.ndarray) -> np.ndarray:
    """fp16 working copy of fp32 master weights (IEEE round to nearest even;
    values beyond the fp16 range become infinities)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16)


def normalized_sumsq(grads: Sequence[np.ndarray], owned: Sequence[bool], divisor: float) -> float:
    """Sum over owned tensors of the squared effective-batch-normalized gradient.

    Landing page, paragraph 7: the gradients are normalized for the effective
    batch before their overall magnitude is measured; paragraph 8: under
    distributed ownership every shard enters once.  Tensors are summed in list
    order.
    """
    total = 0.0
    for g, own in zip(grads, owned):
        if not own:
            continue
        x = widen_grad(g) / divisor
        total += float(np.sum(x * x))
    return total


def global_norm(grads: Sequence[np.ndarray], owned: Sequence[bool], divisor: float) -> float:
    """L2 norm of all owned, normalized gradients."""
    return float(np.sqrt(normalized_sumsq(grads, owned, divisor)))


def clip_coefficient(norm: float, max_norm: float) -> float:
    """c = min(1, max_norm / (norm + 1e-6)); NaN propagates (no clamp on NaN)."""
    raw = max_norm / (norm + CLIP_EPS)
    return raw if not (raw > 1.0) else 1.0


def adamw_update(p: np.ndarray, m: np.ndarray, v: np.ndarray, g_hat: np.ndarray,
                 lr: float, weight_decay: float, beta1: float, beta2: float,
                 eps: float, t: int):
    """One decoupled-weight-decay AdamW update on float64 arrays.

    ``g_hat`` is the normalized, clipped gradient.  Returns new (p, m, v).
    Elementwise, so it is exact on any subset of elements.
    """
    p = p * (1.0 - lr * weight_decay)
    m = beta1 * m + (1.0 - beta1) * g_hat
    v = beta2 * v + (1.0 - beta2) * (g_hat * g_hat)
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v


@dataclass
class StepStats:
    sumsq: float        # owned sum of squares of the normalized gradients
    norm: float         # sqrt(sumsq): the global norm that clipping tests
    coef: float         # clip coefficient
    nonfinite: bool     # sumsq is NaN or infinite


@dataclass
class Group:
    lr: float
    weight_decay: float
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8


class Oracle:
    """Holds fp64 weights and moments of the trainable tensors across steps.

    ``params`` are the initial fp32 weights (any float array); moments start at
    zero.  Frozen tensors keep ``None`` state and are never touched.
    """

    def __init__(self, params: Sequence[Optional[np.ndarray]], trainable: Sequence[bool],
                 owner: Sequence[bool], group: Sequence[int], groups: Sequence[Group],
                 max_norm: float, grad_divisor: float,
                 exp_avg: Optional[Sequence[np.ndarray]] = None,
                 exp_avg_sq: Optional[Sequence[np.ndarray]] = None,
                 initial_step: int = 0):
        self.trainable = [bool(x) for x in trainable]
        self.owner = [bool(x) for x in owner]
        self.group = [int(x) for x in group]
        self.groups = [Group(g.lr, g.weight_decay, g.beta1, g.beta2, g.eps) for g in groups]
        self.max_norm = float(max_norm)
        self.grad_divisor = float(grad_divisor)
        self.p: List[Optional[np.ndarray]] = []
        self.m: List[Optional[np.ndarray]] = []
        self.v: List[Optional[np.ndarray]] = []
        for i, tr in enumerate(self.trainable):
            if not tr:
                self.p.append(None)
                self.m.append(None)
                self.v.append(None)
                continue
            p = np.asarray(params[i], dtype=np.float64).copy()
            self.p.append(p)
            self.m.append(np.zeros_like(p) if exp_avg is None
                          else np.asarray(exp_avg[i], dtype=np.float64).copy())
            self.v.append(np.zeros_like(p) if exp_avg_sq is None
                          else np.asarray(exp_avg_sq[i], dtype=np.float64).copy())
        self.t = [int(initial_step)] * len(self.groups)

    def set_lrs(self, lrs: Sequence[float]) -> None:
        for k, lr in enumerate(lrs):
            self.groups[k].lr = float(lr)

    def measure(self, grads: Sequence[Optional[np.ndarray]]) -> StepStats:
        """Pass 1 semantics: norm and clip decision from owned trainable grads."""
        use = [g for g, tr in zip(grads, self.trainable) if tr]
        own = [o for o, tr in zip(self.owner, self.trainable) if tr]
        s = normalized_sumsq(use, own, self.grad_divisor)
        n = float(np.sqrt(s))
        return StepStats(sumsq=s, norm=n, coef=clip_coefficient(n, self.max_norm),
                         nonfinite=not np.isfinite(s))

    def step(self, grads: Sequence[Optional[np.ndarray]],
             lrs: Optional[Sequence[float]] = None) -> StepStats:
        """One full optimizer step; returns the statistics it used."""
        if lrs is not None:
            self.set_lrs(lrs)
        stats = self.measure(grads)
        for k in range(len(self.groups)):
            self.t[k] += 1
        for i, tr in enumerate(self.trainable):
            if not tr:
                continue
            grp = self.groups[self.group[i]]
            g_hat = (widen_grad(grads[i]) / self.grad_divisor) * stats.coef
            self.p[i], self.m[i], self.v[i] = adamw_update(
                self.p[i], self.m[i], self.v[i], g_hat, grp.lr, grp.weight_decay,
                grp.beta1, grp.beta2, grp.eps, self.t[self.group[i]])
        return stats


def update_elements(p: np.ndarray, m: np.ndarray, v: np.ndarray, g: np.ndarray,
                    coef: float, grad_divisor: float, grp: Group, t: int):
    """Per-element update for a sampled subset (the update is elementwise).

    Used where the full state is too large for host memory: the caller computes
    ``coef`` from the full gradient with :func:`normalized_sumsq` and then
    follows the chosen elements only.
    """
    g_hat = (widen_grad(g) / grad_divisor) * coef
    return adamw_update(np.asarray(p, np.float64), np.asarray(m, np.float64),
                        np.asarray(v, np.float64), g_hat, grp.lr, grp.weight_decay,
                        grp.beta1, grp.beta2, grp.eps, t)

