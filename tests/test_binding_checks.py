"""Host-only checks of the Python binding's tensor validation (no GPU needed).

The library addresses every buffer as ``numel`` contiguous elements of its
dtype starting at ``data_ptr()``, and its own range check only bounds a buffer
by the enclosing device allocation.  Under torch's caching allocator that
allocation also holds other tensors, so the binding refuses a wrong dtype, a
non-contiguous view, a shorter moment or gradient, or a buffer on another
device before any pointer is handed over.  These tests build CPU tensors: every
mismatch below is caught before the device check, and a table that is correct
except for living on the CPU is refused by the device check.
"""
import os

import pytest

torch = pytest.importorskip("torch")

from tensor_optimizer_step_amd import somaopt as S  # noqa: E402
from tensor_optimizer_step_amd.workloads import GroupHP  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(S.LIB_PATH),
                                reason="libsomaopt.so not built (python -m tensor_optimizer_step_amd.build)")

N = 40
GROUPS = [GroupHP(lr=1e-3, weight_decay=0.01)]


def row(**over):
    t = dict(p=torch.zeros(N), g=torch.zeros(N, dtype=torch.bfloat16), m=torch.zeros(N), v=torch.zeros(N),
             lp=None)
    t.update(over)
    return t


def build(t):
    return S.FusedAdamW([t["p"]], [t["g"]], [t["m"]], [t["v"]], [0], GROUPS, 1.0, 1.0,
                        params_lowp=[t["lp"]] if t["lp"] is not None else None)


@pytest.mark.parametrize("over,exc,match", [
    (dict(p=torch.zeros(N, dtype=torch.bfloat16)), TypeError, "param: dtype bfloat16"),
    (dict(m=torch.zeros(N, dtype=torch.float64)), TypeError, "exp_avg: dtype float64"),
    (dict(v=torch.zeros(N, dtype=torch.float16)), TypeError, "exp_avg_sq: dtype"),
    (dict(g=torch.zeros(N, dtype=torch.int16)), TypeError, "grad: dtype int16"),
    (dict(lp=torch.zeros(N)), TypeError, "param_lowp: dtype float32"),
    (dict(m=torch.zeros(N - 1)), ValueError, "exp_avg: 39 elements, the weight has 40"),
    (dict(v=torch.zeros(N + 8)), ValueError, "exp_avg_sq: 48 elements"),
    (dict(g=torch.zeros(N - 4, dtype=torch.bfloat16)), ValueError, "grad: 36 elements"),
    (dict(lp=torch.zeros(N // 2, dtype=torch.bfloat16)), ValueError, "param_lowp: 20 elements"),
    (dict(p=torch.zeros(2 * N)[::2]), ValueError, "param: not contiguous"),
    (dict(g=torch.zeros(N, 2, dtype=torch.bfloat16)[:, 0]), ValueError, "grad: not contiguous"),
    (dict(m=torch.zeros(8, 5).t()), ValueError, "exp_avg: not contiguous"),
    (dict(), ValueError, "param: on cpu, not on a GPU"),
])
def test_fused_adamw_refuses(over, exc, match):
    with pytest.raises(exc, match=match):
        build(row(**over))


def test_fused_adamw_refuses_mismatched_lists():
    t = row()
    with pytest.raises(ValueError, match="exp_avgs has 2 entries, params has 1"):
        S.FusedAdamW([t["p"]], [t["g"]], [t["m"], t["m"]], [t["v"]], [0], GROUPS, 1.0, 1.0)
    with pytest.raises(ValueError, match="params_lowp has 0 entries"):
        S.FusedAdamW([t["p"]], [t["g"]], [t["m"]], [t["v"]], [0], GROUPS, 1.0, 1.0, params_lowp=[])


def test_frozen_entries_are_not_checked():
    """A frozen tensor is never read or written: its entries may be anything
    (here None gradients and moments); the trainable one still is checked."""
    t = row()
    with pytest.raises(ValueError, match="tensor 1 param: on cpu"):
        S.FusedAdamW([torch.zeros(3), t["p"]], [None, t["g"]], [None, t["m"]], [None, t["v"]], [0, 0],
                     GROUPS, 1.0, 1.0, trainable=[False, True])


@pytest.mark.parametrize("name,val,exc,match", [
    ("k", lambda b, h, lk, d: torch.zeros(b, h, lk, d), TypeError, "k: dtype torch.float32"),
    ("o", lambda b, h, lk, d: torch.zeros(b, h, 9, d, dtype=torch.bfloat16), ValueError, "o: shape"),
    ("lse", lambda b, h, lk, d: torch.zeros(b, h, 16, 2)[..., 0], ValueError, "lse: not contiguous"),
    (None, None, ValueError, "q: on cpu"),
])
def test_attention_refuses(name, val, exc, match):
    b, h, lq, lk, d = 2, 3, 16, 40, 64
    bf = torch.bfloat16
    t = dict(q=torch.zeros(b, h, lq, d, dtype=bf), k=torch.zeros(b, h, lk, d, dtype=bf),
             v=torch.zeros(b, h, lk, d, dtype=bf), o=torch.zeros(b, h, lq, d, dtype=bf),
             lse=torch.zeros(b, h, lq))
    if name is not None:
        t[name] = val(b, h, lk, d)
    with pytest.raises(exc, match=match):
        S.attn_forward(t["q"], t["k"], t["v"], t["o"], t["lse"], lk_frozen=8)
