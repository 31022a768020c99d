"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Each ``pin_*`` function checks the oracle against something independent of it:
exact decimal brute force, a closed form derived by hand from the AdamW
recurrences, an invariant of the definition (reordering, sharding with an
owner mask), or a library special case (torch CPU float64 ``clip_grad_norm_``
followed by ``torch.optim.AdamW``, the unfused sequence the veRL page shows in
section 4.2).  ``test_mutants_are_caught`` plants plausible mistakes in the
oracle (on the CPU) and checks that at least one pin rejects each of them.
"""
import math
from decimal import Decimal, localcontext

import numpy as np
import pytest

import oracle
from oracle import adamw_fp64 as OA

# Large hyperparameters make second-order mistakes visible in fp64.
LR, WD, B1, B2, EPS = 1e-2, 0.1, 0.9, 0.999, 1e-8


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16_bits_from_f32(x):
    """Round-to-nearest-even float32 -> bf16 bit patterns (test input helper)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    return ((u + rounding) >> 16).astype(np.uint16)


def _decimal_norm(grads, divisor, prec=60):
    """Exact-ish brute force: every fp value is a finite binary fraction."""
    with localcontext() as ctx:
        ctx.prec = prec
        d = Decimal(float(divisor))
        s = Decimal(0)
        for g in grads:
            g = np.asarray(g)
            if g.dtype == np.uint16:
                vals = [float(np.array([int(b) << 16], np.uint32).view(np.float32)[0]) for b in g]
            else:
                vals = [float(x) for x in g]
            for x in vals:
                q = Decimal(x) / d
                s += q * q
        return s.sqrt()


# --------------------------------------------------------------------------- pins

def pin_norm_exact_example():
    # g = [3, 4] with effective-batch divisor 4: the normalized gradient is
    # [0.75, 1.0] and its L2 norm is exactly 1.25.
    g = [np.array([3.0, 4.0], np.float32)]
    assert OA.global_norm(g, [True], 4.0) == 1.25
    ora = OA.Oracle([np.zeros(2, np.float32)], [True], [True], [0], [OA.Group(LR, WD)],
                    max_norm=1.0, grad_divisor=4.0)
    st = ora.measure(g)
    assert st.norm == 1.25
    assert st.sumsq == 1.5625


def pin_norm_decimal_bruteforce():
    rng = _rng(11)
    for trial in range(20):
        grads = []
        for k in range(rng.integers(1, 5)):
            n = int(rng.integers(1, 8))
            x = rng.normal(0, 10.0 ** rng.integers(-4, 3), size=n).astype(np.float32)
            grads.append(_bf16_bits_from_f32(x) if k % 2 else x)
        divisor = float(rng.choice([1.0, 3.0, 4.0, 7.0, 16.0]))
        got = OA.global_norm(grads, [True] * len(grads), divisor)
        want = float(_decimal_norm(grads, divisor))
        assert abs(got - want) <= 4e-16 * want, (trial, got, want)


def pin_norm_reorder_invariance():
    rng = _rng(12)
    grads = [rng.normal(0, 0.05, size=int(rng.integers(1, 3000))).astype(np.float32)
             for _ in range(40)]
    base = OA.global_norm(grads, [True] * 40, 4.0)
    for s in range(5):
        perm = _rng(100 + s).permutation(40)
        got = OA.global_norm([grads[i] for i in perm], [True] * 40, 4.0)
        assert abs(got - base) <= 1e-13 * base


def pin_norm_owner_shards():
    """Cut tensors into shard pieces, replicate small ones, flag one owner."""
    rng = _rng(13)
    mats = [rng.normal(0, 0.1, size=int(rng.integers(50, 500))).astype(np.float32)
            for _ in range(6)]
    norms = [rng.normal(0, 0.1, size=16).astype(np.float32) for _ in range(3)]
    whole = OA.normalized_sumsq(mats + norms, [True] * 9, 2.0)
    flat = np.concatenate(mats)
    cuts = np.linspace(0, flat.size, 4).astype(int)
    pieces, owned = [], []
    for s in range(3):
        seg = flat[cuts[s]:cuts[s + 1]]
        pieces.append(seg)
        owned.append(True)
        for r in norms:
            pieces.append(r.copy())
            owned.append(s == 0)
    sharded = OA.normalized_sumsq(pieces, owned, 2.0)
    assert abs(sharded - whole) <= 1e-13 * whole
    # counting replicas more than once must change the answer
    assert OA.normalized_sumsq(pieces, [True] * len(pieces), 2.0) > whole * (1 + 1e-9)


def pin_clip_coefficient():
    # below the threshold: no clipping at all, exactly
    for n in (0.0, 1e-9, 0.5, 0.999):
        assert OA.clip_coefficient(n, 1.0) == 1.0
    # above it, c * (n + 1e-6) recovers max_norm to rounding, and c < 1
    for n in (1.0, 1.5, 5.0, 1738.0, 1e6):
        c = OA.clip_coefficient(n, 1.0)
        assert c < 1.0
        assert abs(c * (n + 1e-6) - 1.0) <= 2e-16
    # monotone non-increasing in the norm
    ns = np.linspace(0, 10, 1001)
    cs = [OA.clip_coefficient(float(n), 2.0) for n in ns]
    assert all(a >= b for a, b in zip(cs, cs[1:]))
    # clipped gradient norm never exceeds max_norm (+ tiny slack)
    for n in (0.3, 3.0, 30.0):
        assert n * OA.clip_coefficient(n, 1.0) <= 1.0 + 1e-12


def pin_step1_closed_form():
    # With m = v = 0, the bias-corrected moments after one step are g_hat and
    # g_hat^2, so p1 = p0 - lr*g_hat/(|g_hat| + eps) - lr*wd*p0.
    rng = _rng(14)
    p0 = rng.normal(0, 0.02, size=257).astype(np.float32)
    g = rng.normal(0, 0.05, size=257).astype(np.float32)
    D, M = 4.0, 1.0
    ora = OA.Oracle([p0], [True], [True], [0], [OA.Group(LR, WD, B1, B2, EPS)], M, D)
    st = ora.step([g])
    gh = g.astype(np.float64) / D * st.coef
    want_p = p0 - LR * gh / (np.abs(gh) + EPS) - LR * WD * p0.astype(np.float64)
    assert np.allclose(ora.p[0], want_p, rtol=1e-13, atol=0)
    assert np.allclose(ora.m[0], (1 - B1) * gh, rtol=1e-15, atol=0)
    assert np.allclose(ora.v[0], (1 - B2) * gh * gh, rtol=1e-15, atol=0)


def pin_two_step_moments():
    # m2 = b1 (1-b1) g1 + (1-b1) g2 and v2 likewise, from the recurrences.
    rng = _rng(15)
    p0 = rng.normal(0, 0.02, size=64).astype(np.float32)
    g1 = rng.normal(0, 0.05, size=64).astype(np.float32)
    g2 = rng.normal(0, 0.05, size=64).astype(np.float32)
    ora = OA.Oracle([p0], [True], [True], [0], [OA.Group(LR, WD, B1, B2, EPS)], 1e9, 1.0)
    ora.step([g1])
    ora.step([g2])
    a, b = g1.astype(np.float64), g2.astype(np.float64)
    assert np.allclose(ora.m[0], B1 * (1 - B1) * a + (1 - B1) * b, rtol=1e-14, atol=0)
    assert np.allclose(ora.v[0], B2 * (1 - B2) * a * a + (1 - B2) * b * b, rtol=1e-14, atol=0)
    assert ora.t == [2]


def pin_constant_gradient_closed_form():
    # Constant g_hat makes m_hat = g_hat and v_hat = g_hat^2 exactly at every t,
    # so each step is p <- a p - u with a = 1 - lr wd, u = lr g/(|g| + eps):
    # p_T = a^T p0 - u (1 - a^T) / (1 - a).
    rng = _rng(16)
    p0 = rng.normal(0, 0.02, size=100).astype(np.float32)
    g = rng.normal(0, 0.05, size=100).astype(np.float32)
    T = 10
    ora = OA.Oracle([p0], [True], [True], [0], [OA.Group(LR, WD, B1, B2, EPS)], 1e9, 2.0)
    for _ in range(T):
        st = ora.step([g])
        assert st.coef == 1.0
    gh = g.astype(np.float64) / 2.0
    a = 1 - LR * WD
    u = LR * gh / (np.abs(gh) + EPS)
    want = a ** T * p0.astype(np.float64) - u * (1 - a ** T) / (1 - a)
    assert np.allclose(ora.p[0], want, rtol=1e-12, atol=1e-17)
    # wd = 0: p_T = p0 - T u
    ora = OA.Oracle([p0], [True], [True], [0], [OA.Group(LR, 0.0, B1, B2, EPS)], 1e9, 2.0)
    for _ in range(T):
        ora.step([g])
    assert np.allclose(ora.p[0], p0.astype(np.float64) - T * u, rtol=1e-12, atol=1e-17)


def pin_pure_decay():
    # Zero gradient: moments stay 0, the Adam term is 0/(0+eps) = 0, and the
    # weight only decays: p_T = (1 - lr wd)^T p0.
    rng = _rng(17)
    p0 = rng.normal(0, 0.02, size=50).astype(np.float32)
    ora = OA.Oracle([p0], [True], [True], [0], [OA.Group(LR, WD, B1, B2, EPS)], 1.0, 1.0)
    for _ in range(7):
        ora.step([np.zeros(50, np.float32)])
    assert np.allclose(ora.p[0], (1 - LR * WD) ** 7 * p0.astype(np.float64), rtol=1e-14, atol=0)
    assert not np.any(ora.m[0]) and not np.any(ora.v[0])


def pin_lr_zero_is_identity():
    rng = _rng(18)
    p0 = rng.normal(0, 0.02, size=33).astype(np.float32)
    ora = OA.Oracle([p0], [True], [True], [0], [OA.Group(0.0, WD, B1, B2, EPS)], 1.0, 1.0)
    for _ in range(3):
        ora.step([rng.normal(0, 1, size=33).astype(np.float32)])
    assert np.array_equal(ora.p[0], p0.astype(np.float64))


def pin_bf16_widening():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0xFF80, 0x8000, 0x3E80, 0x4049], np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, math.inf, -math.inf, -0.0, 0.25, 3.140625]
    got = OA.widen_grad(bits)
    assert got.dtype == np.float64
    for a, b in zip(got.tolist(), want):
        assert a == b and math.copysign(1, a) == math.copysign(1, b)
    nan = OA.widen_grad(np.array([0x7FC0], np.uint16))
    assert np.isnan(nan[0])


def pin_fp16_widening():
    vals = np.array([1.0, -2.5, 65504.0, 2.0 ** -24, -0.0, np.inf], np.float16)
    got = OA.widen_grad(vals)
    assert got.dtype == np.float64 and got.tolist() == [1.0, -2.5, 65504.0, 2.0 ** -24, -0.0, math.inf]


def pin_bf16_working_copy_rounding():
    """RNE fp32 -> bf16: exact ties, carries into the exponent, NaN; and the
    library special case torch .to(torch.bfloat16) on random values."""
    def f32(bits):
        return np.array([bits], np.uint32).view(np.float32)
    cases = {
        0x3F808000: 0x3F80,   # tie, even lower half kept
        0x3F818000: 0x3F82,   # tie, odd -> rounds up to even
        0x3F808001: 0x3F81,   # just above the tie
        0x3F807FFF: 0x3F80,   # just below the tie
        0x3FFF8000: 0x4000,   # tie that carries into the exponent
        0x7F7FFFFF: 0x7F80,   # largest finite rounds to infinity
        0x80000001: 0x8000,   # tiny negative subnormal -> -0
        0x7F800000: 0x7F80,   # +inf stays
    }
    for bits, want in cases.items():
        assert int(OA.round_to_bf16_bits(f32(bits))[0]) == want, hex(bits)
    assert int(OA.round_to_bf16_bits(np.array([np.nan], np.float32))[0]) == 0x7FC0
    torch = pytest.importorskip("torch")
    x = (_rng(22).standard_normal(100000) * 10.0 ** _rng(23).integers(-30, 30, 100000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(OA.round_to_bf16_bits(x), ref)
    # fp16 working copy: numpy's conversion agrees with torch's
    y = (x / 1e20).astype(np.float32)
    assert np.array_equal(OA.round_to_f16(y).view(np.uint16),
                          torch.from_numpy(y).to(torch.float16).numpy().view(np.uint16))


def pin_inputs_untouched_and_frozen_skipped():
    rng = _rng(19)
    ps = [rng.normal(0, 0.02, size=n).astype(np.float32) for n in (5, 7, 9)]
    gs = [rng.normal(0, 0.05, size=n).astype(np.float32) for n in (5, 7, 9)]
    gs[1] = np.full(7, np.nan, np.float32)          # frozen tensor: NaN never read
    for a in ps + gs:
        a.setflags(write=False)
    ora = OA.Oracle(ps, [True, False, True], [True] * 3, [0] * 3,
                    [OA.Group(LR, WD, B1, B2, EPS)], 1.0, 1.0)
    st = ora.step(gs)
    assert np.isfinite(st.norm)
    want = OA.global_norm([gs[0], gs[2]], [True, True], 1.0)
    assert st.norm == want
    assert ora.p[1] is None and ora.m[1] is None


def pin_nonfinite():
    ora = OA.Oracle([np.zeros(3, np.float32)], [True], [True], [0], [OA.Group(LR, WD)], 1.0, 1.0)
    st = ora.measure([np.array([1.0, np.inf, 0.0], np.float32)])
    assert st.nonfinite and st.coef == 0.0
    st = ora.measure([np.array([1.0, np.nan, 0.0], np.float32)])
    assert st.nonfinite and math.isnan(st.coef)
    st = ora.measure([np.array([1.0, 2.0, 0.0], np.float32)])
    assert not st.nonfinite


def pin_resume_equals_continuation():
    rng = _rng(20)
    p0 = rng.normal(0, 0.02, size=40).astype(np.float32)
    gs = [rng.normal(0, 0.05, size=40).astype(np.float32) for _ in range(6)]
    hp = [OA.Group(LR, WD, B1, B2, EPS)]
    a = OA.Oracle([p0], [True], [True], [0], hp, 1.0, 1.0)
    for g in gs:
        a.step([g])
    b = OA.Oracle([p0], [True], [True], [0], hp, 1.0, 1.0)
    for g in gs[:3]:
        b.step([g])
    c = OA.Oracle([b.p[0]], [True], [True], [0], hp, 1.0, 1.0,
                  exp_avg=[b.m[0]], exp_avg_sq=[b.v[0]], initial_step=3)
    for g in gs[3:]:
        c.step([g])
    assert np.array_equal(a.p[0], c.p[0]) and np.array_equal(a.v[0], c.v[0])


def pin_torch_cpu_float64():
    """Library special case: unsharded, all owned, fp32 grads.

    The unfused sequence (divide by D, clip_grad_norm_, AdamW.step) in torch
    CPU float64 must agree with the oracle over 10 steps, per group.
    """
    torch = pytest.importorskip("torch")
    rng = _rng(21)
    sizes = [3, 17, 64, 1, 300, 45]
    groups_of = [0, 1, 0, 2, 1, 0]
    hps = [OA.Group(LR, WD, B1, B2, EPS), OA.Group(2 * LR, 0.0, 0.8, 0.99, 1e-6),
           OA.Group(0.5 * LR, 0.05, 0.95, 0.9999, 1e-8)]
    D, M = 4.0, 1.0
    p0 = [rng.normal(0, 0.02, size=n).astype(np.float32) for n in sizes]
    tparams = [torch.tensor(p.astype(np.float64), requires_grad=True) for p in p0]
    opt = torch.optim.AdamW(
        [{"params": [tparams[i] for i in range(6) if groups_of[i] == k], "lr": h.lr,
          "weight_decay": h.weight_decay, "betas": (h.beta1, h.beta2), "eps": h.eps}
         for k, h in enumerate(hps)], foreach=False)
    ora = OA.Oracle(p0, [True] * 6, [True] * 6, groups_of, hps, M, D)
    for step in range(1, 11):
        scale = 0.5 if step % 2 else 8.0            # alternate below / above max_norm
        gs = [(rng.normal(0, 1, size=n) * scale / math.sqrt(sum(sizes))).astype(np.float32)
              for n in sizes]
        lrs = [h.lr * step / 10 for h in hps]
        for i, t in enumerate(tparams):
            t.grad = torch.tensor(gs[i].astype(np.float64)) / D
        total = torch.nn.utils.clip_grad_norm_(tparams, max_norm=M)
        for k, pg in enumerate(opt.param_groups):
            pg["lr"] = lrs[k]
        opt.step()
        st = ora.step(gs, lrs)
        assert abs(st.norm - float(total)) <= 1e-14 * st.norm
        for i, t in enumerate(tparams):
            s = opt.state[t]
            assert np.allclose(ora.p[i], t.detach().numpy(), rtol=1e-12, atol=1e-18)
            assert np.allclose(ora.m[i], s["exp_avg"].numpy(), rtol=1e-12, atol=1e-18)
            assert np.allclose(ora.v[i], s["exp_avg_sq"].numpy(), rtol=1e-12, atol=1e-24)


def pin_update_elements_matches_step():
    """update_elements, which the full-size tests use to follow sampled
    elements, equals Oracle.step on those elements bit for bit over 10 steps:
    divisors 3 and 16, three groups (one with eps as large as the normalized
    gradients, so every change of the gradient's scale shows), fp32 and bf16
    gradients, clipped and unclipped steps.  The clip coefficient given to it
    is the one computed from ALL gradients, as the full-size tests do."""
    rng = _rng(40)
    groups = [OA.Group(1e-2, 0.1, 0.9, 0.999, 1e-3), OA.Group(3e-3, 0.0, 0.8, 0.99, 5e-4),
              OA.Group(5e-3, 0.05, 0.9, 0.999, 1e-8)]
    for divisor in (3.0, 16.0):
        sizes = [int(rng.integers(40, 300)) for _ in range(7)]
        group = [i % 3 for i in range(7)]
        p0 = [rng.normal(0, 0.02, n).astype(np.float32) for n in sizes]
        ora = OA.Oracle(p0, [True] * 7, [True] * 7, group, groups, max_norm=1.0, grad_divisor=divisor)
        idx = [np.sort(rng.choice(n, size=17, replace=False)) for n in sizes]
        sp = [p.astype(np.float64)[ix] for p, ix in zip(p0, idx)]
        sm = [np.zeros(len(ix)) for ix in idx]
        sv = [np.zeros(len(ix)) for ix in idx]
        t = [0, 0, 0]
        clipped = []
        for k in range(1, 11):
            std = 0.002 * divisor if k % 2 else 0.2 * divisor      # norm ~0.03 or ~3
            grads = []
            for i, n in enumerate(sizes):
                x = rng.normal(0, std, n).astype(np.float32)
                grads.append(_bf16_bits_from_f32(x) if i % 2 else x)
            coef = OA.clip_coefficient(OA.global_norm(grads, [True] * 7, divisor), 1.0)
            st = ora.step(grads)
            assert coef == st.coef
            clipped.append(coef < 1.0)
            for j in range(3):
                t[j] += 1
            for i in range(7):
                sp[i], sm[i], sv[i] = OA.update_elements(sp[i], sm[i], sv[i], grads[i][idx[i]], coef, divisor,
                                                         groups[group[i]], t[group[i]])
                assert np.array_equal(sp[i], ora.p[i][idx[i]]), (divisor, k, i, "p")
                assert np.array_equal(sm[i], ora.m[i][idx[i]]), (divisor, k, i, "m")
                assert np.array_equal(sv[i], ora.v[i][idx[i]]), (divisor, k, i, "v")
        assert any(clipped) and not all(clipped)


PINS = [pin_norm_exact_example, pin_norm_decimal_bruteforce, pin_norm_reorder_invariance,
        pin_norm_owner_shards, pin_clip_coefficient, pin_step1_closed_form,
        pin_two_step_moments, pin_constant_gradient_closed_form, pin_pure_decay,
        pin_lr_zero_is_identity, pin_bf16_widening, pin_inputs_untouched_and_frozen_skipped,
        pin_nonfinite, pin_resume_equals_continuation, pin_torch_cpu_float64, pin_fp16_widening,
        pin_bf16_working_copy_rounding, pin_update_elements_matches_step]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin()


# ------------------------------------------------------------------ planted mistakes

def _adamw_decay_after(p, m, v, gh, lr, wd, b1, b2, eps, t):
    m = b1 * m + (1 - b1) * gh
    v = b2 * v + (1 - b2) * gh * gh
    p = p - lr * (m / (1 - b1 ** t)) / (np.sqrt(v / (1 - b2 ** t)) + eps)
    return p * (1 - lr * wd), m, v


def _adamw_eps_inside(p, m, v, gh, lr, wd, b1, b2, eps, t):
    p = p * (1 - lr * wd)
    m = b1 * m + (1 - b1) * gh
    v = b2 * v + (1 - b2) * gh * gh
    return p - lr * (m / (1 - b1 ** t)) / np.sqrt(v / (1 - b2 ** t) + eps), m, v


def _adamw_no_bias_correction(p, m, v, gh, lr, wd, b1, b2, eps, t):
    p = p * (1 - lr * wd)
    m = b1 * m + (1 - b1) * gh
    v = b2 * v + (1 - b2) * gh * gh
    return p - lr * m / (np.sqrt(v) + eps), m, v


def _adamw_decay_sign(p, m, v, gh, lr, wd, b1, b2, eps, t):
    return _REAL["adamw_update"](p * (1 + 2 * lr * wd), m, v, gh, lr, wd, b1, b2, eps, t)


def _adamw_betas_swapped(p, m, v, gh, lr, wd, b1, b2, eps, t):
    return _REAL["adamw_update"](p, m, v, gh, lr, wd, b2, b1, eps, t)


def _adamw_l2_not_decoupled(p, m, v, gh, lr, wd, b1, b2, eps, t):
    return _REAL["adamw_update"](p, m, v, gh + wd * p, lr, 0.0, b1, b2, eps, t)


def _adamw_bias_t_minus_1(p, m, v, gh, lr, wd, b1, b2, eps, t):
    return _REAL["adamw_update"](p, m, v, gh, lr, wd, b1, b2, eps, t + 1)


def _sumsq_no_divisor(grads, owned, divisor):
    return _REAL["normalized_sumsq"](grads, owned, 1.0)


def _sumsq_ignore_owner(grads, owned, divisor):
    return _REAL["normalized_sumsq"](grads, [True] * len(owned), divisor)


def _sumsq_abs_not_square(grads, owned, divisor):
    total = 0.0
    for g, own in zip(grads, owned):
        if own:
            total += float(np.sum(np.abs(OA.widen_grad(g) / divisor))) ** 2
    return total


def _clip_no_eps(norm, max_norm):
    raw = max_norm / norm if norm else math.inf
    return raw if not (raw > 1.0) else 1.0


def _clip_no_clamp(norm, max_norm):
    return max_norm / (norm + OA.CLIP_EPS)


def _widen_shift15(g):
    g = np.asarray(g)
    if g.dtype == np.uint16:
        return (g.astype(np.uint32) << 15).view(np.float32).astype(np.float64)
    return g.astype(np.float64)


def _update_no_divisor(p, m, v, g, coef, grad_divisor, grp, t):
    return _REAL["update_elements"](p, m, v, g, coef, 1.0, grp, t)


def _update_coef_twice(p, m, v, g, coef, grad_divisor, grp, t):
    return _REAL["update_elements"](p, m, v, g, coef * coef, grad_divisor, grp, t)


def _round_truncate(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _round_half_up(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x8000) >> 16).astype(np.uint16)


_REAL = {"normalized_sumsq": OA.normalized_sumsq, "adamw_update": OA.adamw_update,
         "update_elements": OA.update_elements}

MUTANTS = {
    "decay_after_update": ("adamw_update", _adamw_decay_after),
    "eps_inside_sqrt": ("adamw_update", _adamw_eps_inside),
    "no_bias_correction": ("adamw_update", _adamw_no_bias_correction),
    "decay_wrong_sign": ("adamw_update", _adamw_decay_sign),
    "betas_swapped": ("adamw_update", _adamw_betas_swapped),
    "l2_instead_of_decoupled": ("adamw_update", _adamw_l2_not_decoupled),
    "bias_correction_off_by_one": ("adamw_update", _adamw_bias_t_minus_1),
    "norm_before_divisor": ("normalized_sumsq", _sumsq_no_divisor),
    "owner_ignored": ("normalized_sumsq", _sumsq_ignore_owner),
    "l1_instead_of_l2": ("normalized_sumsq", _sumsq_abs_not_square),
    "clip_without_eps": ("clip_coefficient", _clip_no_eps),
    "clip_not_clamped": ("clip_coefficient", _clip_no_clamp),
    "bf16_widen_wrong_shift": ("widen_grad", _widen_shift15),
    "bf16_round_truncates": ("round_to_bf16_bits", _round_truncate),
    "bf16_round_half_up": ("round_to_bf16_bits", _round_half_up),
    "update_elements_divisor_dropped": ("update_elements", _update_no_divisor),
    "update_elements_coef_twice": ("update_elements", _update_coef_twice),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OA, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"


def test_package_exports():
    for name in ("Oracle", "Group", "adamw_update", "clip_coefficient", "normalized_sumsq",
                 "update_elements", "widen_grad"):
        assert hasattr(oracle, name)
