"""Shared helpers of the GPU parity tests: device buffers for a workload,
gradient refresh, and element-wise comparison with the fp64 oracle.

Tolerance (stated by the acceptance bar and used everywhere): an element passes
if |gpu - oracle| <= max(2e-6 * |oracle|, 1e-9).  The global norm must agree to
1e-5 relative; both sides accumulate in fp64, so the tests also hold it to
1e-11 (a few hundred fp64 roundings of positive terms).
"""
from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from tensor_optimizer_step_amd import workloads as W

RTOL = 2e-6
ATOL = 1e-9
NORM_RTOL = 1e-5
NORM_RTOL_FP64 = 1e-11
# Tensor-wise bound: max |gpu - oracle| <= 1e-5 * max |oracle| over a tensor.
# The per-element floor of 1e-9 is loose for first moments of size ~1e-6 and
# near their zero crossings; this bound still catches a wrong term there.  fp32
# state rounding over ten steps stays below ~1e-6 of the tensor's scale.
TENSOR_RTOL = 1e-5


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class DeviceState:
    p: list
    g: list
    m: list
    v: list


def allocate(wl: W.Workload, device="cuda") -> DeviceState:
    """One allocation per tensor: fp32 p (seeded), zero m and v, gradient buffers."""
    import torch
    p, g, m, v = [], [], [], []
    for i, t in enumerate(wl.tensors):
        p.append(W.param_values(wl, i, device))
        g.append(torch.empty(t.numel, dtype=W.torch_dtype(t.grad_dtype), device=device))
        m.append(torch.zeros(t.numel, dtype=torch.float32, device=device))
        v.append(torch.zeros(t.numel, dtype=torch.float32, device=device))
    return DeviceState(p, g, m, v)


def fill_grads(wl: W.Workload, st: DeviceState, step: int) -> None:
    """Write update ``step``'s seeded gradients into the existing buffers."""
    for i in range(wl.n_tensors):
        st.g[i].copy_(W.grad_values(wl, i, step, st.g[i].device))


def make_handle(wl: W.Workload, st: DeviceState, **kw):
    from tensor_optimizer_step_amd.somaopt import FusedAdamW
    trainable = [t.trainable for t in wl.tensors]
    return FusedAdamW(st.p, st.g, st.m, st.v, [t.group for t in wl.tensors], wl.groups,
                      kw.pop("max_norm", wl.max_norm), kw.pop("grad_divisor", wl.grad_divisor),
                      trainable=trainable, **kw)


def make_oracle(wl: W.Workload, p0: List[np.ndarray], owner=None, max_norm=None, divisor=None):
    import oracle as O
    groups = [O.Group(g.lr, g.weight_decay, g.beta1, g.beta2, g.eps) for g in wl.groups]
    n = wl.n_tensors
    return O.Oracle(p0, [t.trainable for t in wl.tensors], owner or [True] * n,
                    [t.group for t in wl.tensors], groups,
                    wl.max_norm if max_norm is None else max_norm,
                    wl.grad_divisor if divisor is None else divisor)


def host(t) -> np.ndarray:
    """Host copy of a device tensor (float32 values or bf16 bit patterns)."""
    return W.to_numpy_grad(t)


def assert_close(name: str, got: np.ndarray, want: np.ndarray, rtol=RTOL, atol=ATOL,
                 tensor_rtol=TENSOR_RTOL) -> float:
    """Element-wise acceptance bar plus the tensor-wise bound; returns the
    tensor-wise relative error max|err| / max|oracle|."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    if got.size == 0:
        return 0.0
    err = np.abs(got - want)
    bound = np.maximum(rtol * np.abs(want), atol)
    bad = err > bound
    if bad.any():
        k = int(np.argmax(bad))
        raise AssertionError(f"{name}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
                             f"first at {k}: gpu={got[k]!r} oracle={want[k]!r}")
    scale = float(np.abs(want).max())
    worst = float(err.max())
    if scale > 0:
        assert worst <= tensor_rtol * scale, (
            f"{name}: tensor-wise error {worst / scale:.3e} > {tensor_rtol} (max |oracle| {scale:.3e})")
        return worst / scale
    assert worst == 0.0, f"{name}: oracle is all zero but gpu differs by {worst}"
    return 0.0


def assert_norm(got: float, want: float, what="norm") -> None:
    rel = abs(got - want) / max(abs(want), 1e-300)
    assert rel <= NORM_RTOL, f"{what}: rel error {rel} > {NORM_RTOL}"
    assert rel <= NORM_RTOL_FP64, f"{what}: rel error {rel} > {NORM_RTOL_FP64} (fp64 accumulation)"
