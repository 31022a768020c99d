"""fp64 CPU oracle for tiled attention over frozen and trainable keys.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).  It
shares no code with the HIP library.

SomaSpeed landing page, paragraph 5 (prose paragraphs numbered in page order
after the title): queries come from the trainable action computation, keys
and values identify and carry the context; the kernel reads keys and values
tile by tile, never stores the full score matrix and does no gradient work for
frozen inputs.  Paragraph 6: the context keys/values are frozen (backbone
features or a frozen prefix) while the action stream may add trainable
keys/values.

Reading taken (the pages print no formula): textbook scaled dot-product
attention per (batch, head), no mask,
    S = scale * Q K^T,  P = softmax_rows(S),  O = P V,  LSE = log sum_j exp(S_ij)
and its gradient with the usual saved activations O and LSE,
    D_i = sum_c dO_ic O_ic,  dP = dO V^T,  dS = P * (dP - D),
    dQ = scale * dS K,  dK = scale * dS^T Q,  dV = P^T dO,
where the first ``lk_frozen`` keys are frozen: their dK and dV are not
produced.  Pinned in tests/test_attention_oracle.py against torch CPU float64
autograd and closed forms.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:       # bf16 bit patterns
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def attention_forward(q, k, v, scale: float):
    """q: [..., Lq, d], k, v: [..., Lk, d] -> (O [..., Lq, d], LSE [..., Lq])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    s = scale * (q @ np.swapaxes(k, -1, -2))
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    p = e / z
    o = p @ v
    lse = (m + np.log(z))[..., 0]
    return o, lse


def attention_probs(q, k, lse, scale: float) -> np.ndarray:
    """P recomputed from the saved log-sum-exp (as a tiled backward does)."""
    q, k = _f64(q), _f64(k)
    s = scale * (q @ np.swapaxes(k, -1, -2))
    return np.exp(s - _f64(lse)[..., None])


def attention_backward(q, k, v, o, lse, d_o, scale: float, lk_frozen: int):
    """Gradients from the saved activations O and LSE.

    Returns (dQ [..., Lq, d], dK [..., Lk - lk_frozen, d], dV [...]) for the
    trainable keys only; frozen keys get no gradient.
    """
    q, k, v, o, d_o = _f64(q), _f64(k), _f64(v), _f64(o), _f64(d_o)
    p = attention_probs(q, k, lse, scale)
    dp = d_o @ np.swapaxes(v, -1, -2)
    delta = (d_o * o).sum(axis=-1, keepdims=True)
    ds = p * (dp - delta)
    dq = scale * (ds @ k)
    dk = scale * (np.swapaxes(ds, -1, -2) @ q)
    dv = np.swapaxes(p, -1, -2) @ d_o
    return dq, dk[..., lk_frozen:, :], dv[..., lk_frozen:, :]


def error_budget_forward(q, k, v, lse, scale: float, unit: float = 2.0 ** -8):
    """Per-element bound for O computed with P rounded once to bf16 and fp32
    accumulation: unit * sum_j P_ij |V_jc| (plus a tiny absolute floor)."""
    p = attention_probs(q, k, lse, scale)
    return unit * (p @ np.abs(_f64(v))) + 1e-6


def error_budget_backward(q, k, v, o, lse, d_o, scale: float, lk_frozen: int,
                          unit: float = 2.0 ** -8, unit32: float = 2.0 ** -18):
    """Per-element bounds for dQ, dK, dV when P and dS are rounded once to bf16
    before their products and everything else runs in fp32: ``unit`` times the
    magnitude of the rounded operand's contribution, plus ``unit32`` times the
    magnitude of dP and D feeding the (possibly cancelling) difference dP - D."""
    q, k, v, o, d_o = _f64(q), _f64(k), _f64(v), _f64(o), _f64(d_o)
    p = attention_probs(q, k, lse, scale)
    dp = d_o @ np.swapaxes(v, -1, -2)
    delta = (d_o * o).sum(axis=-1, keepdims=True)
    ds_abs = np.abs(p * (dp - delta)) * unit + p * (np.abs(dp) + np.abs(delta)) * unit32
    bq = scale * (ds_abs @ np.abs(k)) + 1e-6
    bk = scale * (np.swapaxes(ds_abs, -1, -2) @ np.abs(q)) + 1e-6
    bv = unit * (np.swapaxes(p, -1, -2) @ np.abs(d_o)) + 1e-6
    return bq, bk[..., lk_frozen:, :], bv[..., lk_frozen:, :]
