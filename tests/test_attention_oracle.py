"""Pins of the fp64 attention oracle (frozen and trainable keys).

Library special case: torch CPU float64 autograd of softmax attention, with the
frozen keys/values outside autograd.  Closed forms: zero queries give uniform
weights; identical value rows make every gradient vanish; a common shift of all
keys leaves the weights unchanged.  Planted mistakes must fail a pin.
"""
import math

import numpy as np
import pytest

from oracle import attention_fp64 as A

torch = pytest.importorskip("torch")


def _case(seed, b=2, h=3, lq=7, lk=11, d=8, lf=6):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(b, h, lq, d))
    k = rng.normal(size=(b, h, lk, d))
    v = rng.normal(size=(b, h, lk, d))
    do = rng.normal(size=(b, h, lq, d))
    return q, k, v, do, lf, 1.0 / math.sqrt(d)


def pin_forward_against_torch():
    q, k, v, do, lf, s = _case(1)
    o, lse = A.attention_forward(q, k, v, s)
    tq, tk, tv = (torch.tensor(x) for x in (q, k, v))
    w = torch.softmax(s * tq @ tk.transpose(-1, -2), dim=-1)
    assert np.allclose(o, (w @ tv).numpy(), rtol=1e-13, atol=1e-14)
    assert np.allclose(lse, torch.logsumexp(s * tq @ tk.transpose(-1, -2), dim=-1).numpy(), rtol=1e-13)


def pin_backward_against_torch_autograd():
    q, k, v, do, lf, s = _case(2)
    o, lse = A.attention_forward(q, k, v, s)
    dq, dk, dv = A.attention_backward(q, k, v, o, lse, do, s, lf)
    tq = torch.tensor(q, requires_grad=True)
    k_fr, k_tr = torch.tensor(k[..., :lf, :]), torch.tensor(k[..., lf:, :], requires_grad=True)
    v_fr, v_tr = torch.tensor(v[..., :lf, :]), torch.tensor(v[..., lf:, :], requires_grad=True)
    tk, tv = torch.cat([k_fr, k_tr], dim=-2), torch.cat([v_fr, v_tr], dim=-2)
    out = torch.softmax(s * tq @ tk.transpose(-1, -2), dim=-1) @ tv
    (out * torch.tensor(do)).sum().backward()
    assert k_fr.grad is None and v_fr.grad is None
    assert np.allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-13)
    assert np.allclose(dk, k_tr.grad.numpy(), rtol=1e-11, atol=1e-13)
    assert np.allclose(dv, v_tr.grad.numpy(), rtol=1e-11, atol=1e-13)
    assert dk.shape[-2] == k.shape[-2] - lf


def pin_zero_queries_uniform_weights():
    q, k, v, do, lf, s = _case(3)
    q = np.zeros_like(q)
    o, lse = A.attention_forward(q, k, v, s)
    assert np.allclose(o, v.mean(axis=-2, keepdims=True).repeat(q.shape[-2], axis=-2), rtol=1e-13)
    assert np.allclose(lse, math.log(k.shape[-2]), rtol=1e-14)


def pin_identical_values_zero_gradients():
    q, k, v, do, lf, s = _case(4)
    v = np.broadcast_to(v[..., :1, :], v.shape).copy()
    o, lse = A.attention_forward(q, k, v, s)
    assert np.allclose(o, np.broadcast_to(v[..., :1, :], o.shape), rtol=1e-13)
    dq, dk, dv = A.attention_backward(q, k, v, o, lse, do, s, lf)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    # dV still carries the attention weights
    assert np.abs(dv).max() > 1e-3


def pin_key_shift_invariance():
    q, k, v, do, lf, s = _case(5)
    o1, lse1 = A.attention_forward(q, k, v, s)
    c = np.random.default_rng(6).normal(size=k.shape[-1])
    o2, lse2 = A.attention_forward(q, k + c, v, s)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse2 - lse1, s * (q @ c), rtol=1e-12, atol=1e-12)


def pin_key_permutation_invariance():
    q, k, v, do, lf, s = _case(7)
    perm = np.random.default_rng(8).permutation(k.shape[-2])
    o1, lse1 = A.attention_forward(q, k, v, s)
    o2, lse2 = A.attention_forward(q, k[..., perm, :], v[..., perm, :], s)
    assert np.allclose(o1, o2, rtol=1e-12) and np.allclose(lse1, lse2, rtol=1e-13)


def pin_frozen_only_drops_outputs():
    q, k, v, do, lf, s = _case(9)
    o, lse = A.attention_forward(q, k, v, s)
    full = A.attention_backward(q, k, v, o, lse, do, s, 0)
    part = A.attention_backward(q, k, v, o, lse, do, s, lf)
    assert np.array_equal(full[0], part[0])
    assert np.array_equal(full[1][..., lf:, :], part[1]) and np.array_equal(full[2][..., lf:, :], part[2])


PINS = [pin_forward_against_torch, pin_backward_against_torch_autograd,
        pin_zero_queries_uniform_weights, pin_identical_values_zero_gradients,
        pin_key_shift_invariance, pin_key_permutation_invariance, pin_frozen_only_drops_outputs]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_attention_pin(pin):
    pin()


_REAL_BWD = A.attention_backward
_REAL_PROBS = A.attention_probs


def _bwd_no_delta(q, k, v, o, lse, d_o, scale, lk_frozen):
    return _REAL_BWD(q, k, v, np.zeros_like(np.asarray(o, np.float64)), lse, d_o, scale, lk_frozen)


def _bwd_no_scale(q, k, v, o, lse, d_o, scale, lk_frozen):
    dq, dk, dv = _REAL_BWD(q, k, v, o, lse, d_o, scale, lk_frozen)
    return dq / scale, dk / scale, dv


def _probs_unnormalized(q, k, lse, scale):
    return _REAL_PROBS(q, k, np.zeros_like(np.asarray(lse, np.float64)), scale)


def _fwd_no_scale(q, k, v, scale):
    return _REAL_FWD(q, k, v, 1.0)


_REAL_FWD = A.attention_forward

MUTANTS = {"delta_dropped": ("attention_backward", _bwd_no_delta),
           "grad_scale_dropped": ("attention_backward", _bwd_no_scale),
           "probs_not_normalised": ("attention_probs", _probs_unnormalized),
           "forward_scale_dropped": ("attention_forward", _fwd_no_scale)}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_attention_mutants_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
