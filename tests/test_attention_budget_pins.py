"""Pins of the attention oracle's per-element error budgets.

The GPU attention tests accept an output element when its distance from the
exact fp64 oracle is within ``error_budget_forward`` / ``error_budget_backward``.
Those budgets model the kernels' one deliberate loss of precision: the
probabilities P (before O = P V and dV = P^T dO) and the score gradients
dS = P * (dP - D) (before dQ = scale dS K and dK = scale dS^T Q) are rounded
once to bf16 for the matrix-core products; everything else is fp32.

The pins check the budget functions against an independent simulation of
those numerics in fp64 (round P and dS once to bf16 with round-to-nearest-
even, every other step exact):
  * validity: the simulated error never exceeds the budget, over many seeded
    shapes and value scales;
  * tightness: inputs built so that every rounding lands just short of a
    rounding midpoint, with the signs aligned, reach at least 0.9 of each
    budget, so a budget looser by a small factor fails;
  * sensitivity: plausible kernel mistakes simulated the same way (the
    row term D dropped, the score scale dropped, O not divided by the softmax
    sum, P rounded to a format 4x coarser) exceed the budget;
  * planted mistakes in the budget functions themselves fail a pin.
"""
import math

import numpy as np
import pytest

from oracle import attention_fp64 as A

U = 2.0 ** -8          # unit roundoff of bf16 (8 significant bits, nearest even)


def round_bf16(x, bits=8):
    """Exact round-to-nearest-even of fp64 values to ``bits`` significant bits
    (bf16: 8).  frexp gives x = m 2^e with 0.5 <= |m| < 1; m 2^bits is rounded
    to an integer with ties to even (np.rint), so the result is a single
    rounding of the exact value (no detour through float32)."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, bits)), e - bits)


def simulate(q, k, v, d_o, scale, lk_frozen, mistake=None, bits=8):
    """The kernels' numerics in fp64: P and dS rounded once (``bits``
    significant bits), everything else exact.  Returns (O, dQ, dK, dV); the
    backward is fed the exact O and LSE, as the GPU tests feed the oracle the
    kernel's own saved activations."""
    o_exact, lse = A.attention_forward(q, k, v, scale)
    s = (1.0 if mistake == "scale_dropped" else scale) * (q @ np.swapaxes(k, -1, -2))
    if mistake == "not_renormalized":
        p = np.exp(s - s.max(axis=-1, keepdims=True))
    else:
        p = np.exp(s - lse[..., None])
    pr = round_bf16(p, bits)
    o = pr @ v
    dp = d_o @ np.swapaxes(v, -1, -2)
    delta = 0.0 if mistake == "delta_dropped" else (d_o * o_exact).sum(-1, keepdims=True)
    dsr = round_bf16(p * (dp - delta), bits)
    sc = 1.0 if mistake == "scale_dropped" else scale
    dq = sc * (dsr @ k)
    dk = sc * (np.swapaxes(dsr, -1, -2) @ q)
    dv = np.swapaxes(pr, -1, -2) @ d_o
    return o, dq, dk[..., lk_frozen:, :], dv[..., lk_frozen:, :]


def worst_ratios(q, k, v, d_o, scale, lk_frozen, **kw):
    """max |simulated - exact| / budget for O, dQ, dK, dV."""
    o_ref, lse = A.attention_forward(q, k, v, scale)
    dq_ref, dk_ref, dv_ref = A.attention_backward(q, k, v, o_ref, lse, d_o, scale, lk_frozen)
    bo = A.error_budget_forward(q, k, v, lse, scale)
    bq, bk, bv = A.error_budget_backward(q, k, v, o_ref, lse, d_o, scale, lk_frozen)
    o, dq, dk, dv = simulate(q, k, v, d_o, scale, lk_frozen, **kw)

    def r(got, want, bud):
        return float((np.abs(got - want) / bud).max()) if want.size else 0.0
    return dict(O=r(o, o_ref, bo), dQ=r(dq, dq_ref, bq), dK=r(dk, dk_ref, bk), dV=r(dv, dv_ref, bv))


def random_case(seed):
    """Seeded shapes and value scales: several query and key counts, head
    dimensions, frozen prefixes, and score spreads from flat to peaked."""
    rng = np.random.default_rng(seed)
    b, h = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    lq, lk = int(rng.integers(1, 40)), int(rng.integers(1, 90))
    d = int(rng.choice([8, 16, 64]))
    lf = int(rng.integers(0, lk + 1))
    spread = float(rng.choice([0.3, 1.0, 3.0]))
    q = rng.normal(0, spread, (b, h, lq, d))
    k = rng.normal(0, 1.0, (b, h, lk, d))
    v = rng.normal(0, 1.0, (b, h, lk, d))
    do = rng.normal(0, 1.0, (b, h, lq, d))
    return q, k, v, do, 1.0 / math.sqrt(d), lf


SEEDS = range(40)


# ----------------------------------------------------------------- constructions

def _just_below_midpoint(x0):
    """The value just below the midpoint between bf16 x0 (a power of two) and
    the next bf16 value up: it rounds down to x0 with an error of almost half
    a unit in the last place, i.e. almost U relative to x0."""
    return x0 * (1.0 + U - 2.0 ** -24)


def tight_forward():
    """O with one key holding P just below the rounding midpoint above 1/2 and
    value 1, the other key (value 0) taking the rest: the rounding error of O
    is almost U * P * |V|, the whole budget."""
    p0 = _just_below_midpoint(0.5)
    k = np.log(np.array([p0, 1.0 - p0]))[None, None, :, None]      # scores = log P (q = 1, d = 1)
    q = np.ones((1, 1, 1, 1))
    v = np.array([1.0, 0.0])[None, None, :, None]
    return q, k, v, np.zeros_like(q), 1.0, 0


def tight_dv():
    """dV of key 0 summed over 8 queries that all give it the same P (just
    below a midpoint) and all have dO = 1: the eight rounding errors add."""
    p0 = _just_below_midpoint(0.5)
    k = np.log(np.array([p0, 1.0 - p0]))[None, None, :, None]
    q = np.ones((1, 1, 8, 1))
    v = np.zeros((1, 1, 2, 1))
    return q, k, v, np.ones((1, 1, 8, 1)), 1.0, 0


def tight_dq():
    """dQ from two keys of equal score whose dS are +a and -a with a just below
    a midpoint: rounding moves both towards zero, and key components +1 / -1
    in a second dimension (which does not touch the scores, q = (1, 0)) make
    the two errors add.  dS = P (dP - D) with dO = (1, 0): V chosen so that
    dP_j = +-2a and D = 0.  A score scale of 1/2 (the scores are 0 whatever
    it is) makes a budget that forgets the scale fail."""
    a = _just_below_midpoint(2.0 ** -4)
    q = np.array([1.0, 0.0])[None, None, None, :]
    k = np.array([[0.0, 1.0], [0.0, -1.0]])[None, None]
    v = np.array([[2 * a, 0.0], [-2 * a, 0.0]])[None, None]
    do = np.array([1.0, 0.0])[None, None, None, :]
    return q, k, v, do, 0.5, 0


def tight_dk():
    """dK of key 0 over two queries whose rows both give dS = +a (just below a
    midpoint) for key 0 and -a for key 1; the queries' second components are
    +1 and the keys' are 0, so the scores stay equal and the errors add."""
    a = _just_below_midpoint(2.0 ** -4)
    q = np.array([[0.0, 1.0], [0.0, 1.0]])[None, None]
    k = np.zeros((1, 1, 2, 2))
    v = np.array([[2 * a, 0.0], [-2 * a, 0.0]])[None, None]
    do = np.array([[1.0, 0.0], [1.0, 0.0]])[None, None]
    return q, k, v, do, 0.5, 0


TIGHT = {"O": tight_forward, "dV": tight_dv, "dQ": tight_dq, "dK": tight_dk}


# --------------------------------------------------------------------------- pins

def pin_round_bf16_is_nearest_even():
    # exact representable values stay; halfway cases go to the even neighbour
    assert round_bf16(1.0) == 1.0 and round_bf16(-0.375) == -0.375
    assert round_bf16(1.0 + 2.0 ** -8) == 1.0                    # tie -> even (1.0)
    assert round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6     # tie -> even (...10)
    assert round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    # against float32 -> bf16 bit rounding on values that are exact in float32
    rng = np.random.default_rng(5)
    x = rng.normal(0, 10, 2000).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    assert np.array_equal(round_bf16(x.astype(np.float64)), bits.view(np.float32).astype(np.float64))


def pin_budgets_bound_the_simulated_error():
    worst = {n: 0.0 for n in ("O", "dQ", "dK", "dV")}
    for seed in SEEDS:
        r = worst_ratios(*random_case(seed))
        for n in worst:
            worst[n] = max(worst[n], r[n])
    assert all(x <= 1.0 for x in worst.values()), worst
    # the tight constructions stay within their budgets too
    for name, make in TIGHT.items():
        assert worst_ratios(*make())[name] <= 1.0, name


def pin_budgets_are_tight():
    for name, make in TIGHT.items():
        r = worst_ratios(*make())[name]
        assert r >= 0.9, f"{name}: a worst-case rounding reaches only {r:.3f} of the budget"


@pytest.mark.parametrize("mistake", ["delta_dropped", "scale_dropped", "not_renormalized", "coarse_rounding"])
def test_kernel_mistakes_exceed_the_budget(mistake):
    """A kernel that made one of these mistakes would fail the GPU tests."""
    worst = {n: 0.0 for n in ("O", "dQ", "dK", "dV")}
    cases = [random_case(s) for s in SEEDS] + [make() for make in TIGHT.values()]
    for c in cases:
        kw = dict(bits=6) if mistake == "coarse_rounding" else dict(mistake=mistake)
        r = worst_ratios(*c, **kw)
        for n in worst:
            worst[n] = max(worst[n], r[n])
    assert max(worst.values()) > 1.0, (mistake, worst)


PINS = [pin_round_bf16_is_nearest_even, pin_budgets_bound_the_simulated_error, pin_budgets_are_tight]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_budget_pin(pin):
    pin()


# ------------------------------------------------- planted mistakes in the budgets

_REAL_F, _REAL_B = A.error_budget_forward, A.error_budget_backward


def _fwd_4x_loose(q, k, v, lse, scale, unit=2.0 ** -8):
    return _REAL_F(q, k, v, lse, scale, unit=4 * unit)


def _fwd_signed_values(q, k, v, lse, scale, unit=2.0 ** -8):
    p = A.attention_probs(q, k, lse, scale)
    return unit * np.abs(p @ A._f64(v)) + 1e-6


def _bwd_4x_loose(q, k, v, o, lse, d_o, scale, lk_frozen, unit=2.0 ** -8, unit32=2.0 ** -18):
    return _REAL_B(q, k, v, o, lse, d_o, scale, lk_frozen, unit=4 * unit, unit32=unit32)


def _bwd_no_scale(q, k, v, o, lse, d_o, scale, lk_frozen, unit=2.0 ** -8, unit32=2.0 ** -18):
    bq, bk, bv = _REAL_B(q, k, v, o, lse, d_o, scale, lk_frozen, unit, unit32)
    return bq / scale, bk / scale, bv


def _bwd_dv_from_ds(q, k, v, o, lse, d_o, scale, lk_frozen, unit=2.0 ** -8, unit32=2.0 ** -18):
    bq, bk, bv = _REAL_B(q, k, v, o, lse, d_o, scale, lk_frozen, unit, unit32)
    return bq, bk, np.full_like(bv, 1e-6)


BUDGET_MUTANTS = {
    "forward_4x_loose": ("error_budget_forward", _fwd_4x_loose),
    "forward_signed_values": ("error_budget_forward", _fwd_signed_values),
    "backward_4x_loose": ("error_budget_backward", _bwd_4x_loose),
    "backward_scale_dropped": ("error_budget_backward", _bwd_no_scale),
    "backward_dv_budget_missing": ("error_budget_backward", _bwd_dv_from_ds),
}


@pytest.mark.parametrize("name", sorted(BUDGET_MUTANTS))
def test_budget_mutants_are_caught(name, monkeypatch):
    attr, fn = BUDGET_MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
