"""CPU oracle of the gradient-arrival epilogue with the norm pass fused in.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).  It
shares no code with the HIP library.

The step before the optimizer path (SomaSpeed landing page, paragraphs 1 and
8, prose paragraphs numbered in page order after the title): with sharded
state every GPU receives its already-reduced gradient shard after backward and
adds it into the gradient shard it holds (or stores it, for the first
contribution of a step); the fused optimizer then starts with the owned sum of
squares of those gradients.  Computing that sum in the arrival pass removes
the norm pass's separate read of every gradient.

Reading taken (the pages do not spell the arithmetic out): the new gradient is
the IEEE fp32 sum of the held and the arriving value, both widened exactly
from the storage dtype, rounded once to the storage dtype to nearest with ties
to even (a no-op for fp32 storage); with accumulation off it is the arriving
value, unchanged.  The statistics are exactly those of the norm pass on the
new gradients (`normalized_sumsq` in adamw_fp64).  The rounding decision is
taken in fp32, the precision the kernel adds in, so the new gradient is
compared bit for bit.

Pinned in tests/test_oracle_pins.py: exact rational rounding of random pairs
(an independent fp32-then-storage rounding written with fractions), tie cases
worked by hand, copy and identity cases.
"""
from __future__ import annotations

import numpy as np

from .adamw_fp64 import round_to_bf16_bits


def _widen32(g: np.ndarray) -> np.ndarray:
    """Exact fp32 value of a stored gradient (uint16 bf16 bits, fp16 or fp32)."""
    g = np.asarray(g)
    if g.dtype == np.uint16:
        return (g.astype(np.uint32) << 16).view(np.float32)
    if g.dtype in (np.float16, np.float32):
        return g.astype(np.float32)
    raise TypeError(f"unsupported gradient dtype {g.dtype}")


def accumulate_gradient(held: np.ndarray, incoming: np.ndarray, accumulate: bool) -> np.ndarray:
    """New contents of a gradient buffer, in its storage dtype.

    ``held`` and ``incoming`` have the same storage dtype: uint16 arrays are bf16
    bit patterns, float16 and float32 arrays hold the values themselves.
    """
    held, incoming = np.asarray(held), np.asarray(incoming)
    if held.dtype != incoming.dtype or held.shape != incoming.shape:
        raise ValueError("held and incoming gradients differ in dtype or shape")
    if not accumulate:
        return incoming.copy()
    with np.errstate(over="ignore", invalid="ignore"):
        s = _widen32(held) + _widen32(incoming)          # one IEEE fp32 rounding
        if held.dtype == np.uint16:
            return round_to_bf16_bits(s)
        if held.dtype == np.float16:
            return s.astype(np.float16)                   # IEEE fp32 -> fp16, nearest even
        return s
