"""Full-size parity in the launch configuration the benchmark times.

The whole step runs as the captured HIP graph with the default chunking.
Every step's global norm is computed by the oracle on the host from ALL owned
gradients.  Element comparisons cover every element:

* the 302,092,288-element action expert (arena layout): the oracle keeps the
  fp64 state of every element of every tensor and all of p, m and v are
  compared after 10 steps (the per-tensor layout and the working-copy run
  follow sampled windows);
* the 6,738,939,904-element 7B backbone and the same state cut into four
  shards with replicated RMSNorms: after steps 1 and 2, every element of every
  tensor (every piece and every replica) is compared with the oracle run on
  that tensor alone from its regenerated seeded inputs and the steps' global
  clip coefficients, streamed piece by piece; steps 3..10 follow sampled
  windows.  This covers the update pass's split into 13 launches and the cuts
  between shards element by element;
* one tensor of 2^32 + 3*2^20 + 5 elements: every element after step 1,
  windows across 2^31 and 2^32 elements after step 2.

Gradient buffers are checked unchanged on the device against a clone.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle as O
from tensor_optimizer_step_amd import workloads as W

from parity_util import assert_close, assert_norm, log

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(420)]

torch = pytest.importorskip("torch")

WINDOW = 2048
WORKERS = 16


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tensor_optimizer_step_amd import somaopt
    somaopt.load()
    torch.cuda.empty_cache()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def sample_indices(numel: int, rng) -> np.ndarray:
    """First and last windows plus two seeded windows (all elements if small)."""
    if numel <= 4 * WINDOW:
        return np.arange(numel)
    starts = [0, numel - WINDOW] + list(rng.integers(WINDOW, numel - 2 * WINDOW, size=2))
    idx = np.unique(np.concatenate([np.arange(s, s + WINDOW) for s in starts]))
    return idx


def host_sumsq_by_tensor(grads_dev, divisor):
    """Oracle norm input: every owned gradient copied to the host and summed by
    the oracle in tensor order (per-tensor sums run in a thread pool; the
    fixed-order accumulation is the oracle's own)."""
    def one(g):
        return O.normalized_sumsq([W.to_numpy_grad(g)], [True], divisor)
    with ThreadPoolExecutor(WORKERS) as ex:
        parts = list(ex.map(one, grads_dev))
    total = 0.0
    for x in parts:
        total += x
    return total


PIECE = 1 << 22


def host_sumsq(g_host, divisor):
    """As host_sumsq_by_tensor, from host copies already taken."""
    with ThreadPoolExecutor(WORKERS) as ex:
        parts = list(ex.map(lambda x: O.normalized_sumsq([x], [True], divisor), g_host))
    total = 0.0
    for x in parts:
        total += x
    return total


def _groups_at(wl, lrs):
    return [O.Group(lr, h.weight_decay, h.beta1, h.beta2, h.eps) for lr, h in zip(lrs, wl.groups)]


def stream_check(wl, k_done, coefs, lrs_per_step, locate, label):
    """Every element of every trainable tensor after update k_done, against the
    oracle run on that tensor alone: its seeded initial weights and gradients
    are regenerated, the oracle applies updates 1..k_done with the global clip
    coefficients ``coefs`` (from the full norm of each step) and the per-step
    learning rates, and the result is compared with the device state, in
    pieces of PIECE elements on a thread pool.  ``locate(i, a, b)`` returns the
    device (p, m, v) views holding logical elements [a, b) of tensor i as a
    list of (start, stop, p, m, v) covering the range (several when the range
    crosses a shard cut; every replica of a replicated tensor is listed)."""
    worst = [0.0, 0.0, 0.0]
    n_checked = 0
    with ThreadPoolExecutor(WORKERS) as ex:
        for i, t in enumerate(wl.tensors):
            if not t.trainable:
                continue
            p0 = W.param_values(wl, i, "cuda").cpu().numpy()
            gs = [W.to_numpy_grad(W.grad_values(wl, i, k, "cuda")) for k in range(1, k_done + 1)]
            grp = [_groups_at(wl, lrs_per_step[k])[t.group] for k in range(k_done)]

            def piece(ab, i=i, p0=p0, gs=gs, grp=grp):
                a, b = ab
                p = np.asarray(p0[a:b], np.float64)
                m = np.zeros(b - a)
                v = np.zeros(b - a)
                for k in range(k_done):
                    p, m, v = O.update_elements(p, m, v, gs[k][a:b], coefs[k], wl.grad_divisor, grp[k], k + 1)
                out = [0.0, 0.0, 0.0]
                for lo, hi, dp, dm, dv in locate(i, a, b):
                    for j, (dt, want) in enumerate(((dp, p), (dm, m), (dv, v))):
                        got = dt.cpu().numpy()
                        out[j] = max(out[j], assert_close(f"{label} step {k_done} {'pmv'[j]}[{i}][{lo}:{hi}]",
                                                          got, want[lo - a:hi - a]))
                return out

            for r in ex.map(piece, [(a, min(a + PIECE, t.numel)) for a in range(0, t.numel, PIECE)]):
                worst = [max(x, y) for x, y in zip(worst, r)]
            n_checked += t.numel
            if i % 40 == 0:
                log(f"[fullsize] {label}: step {k_done} checked through tensor {i} ({n_checked} elements)")
    log(f"[fullsize] {label}: every element after step {k_done} ({n_checked} per kind) within the bar; "
        f"tensor-wise rel err p={worst[0]:.2e} m={worst[1]:.2e} v={worst[2]:.2e}")


class FullOracle:
    """fp64 oracle state for every element of every trainable tensor, updated
    in pieces on a thread pool (the update is elementwise)."""

    def __init__(self, wl, p0_host):
        self.wl = wl
        self.p = [np.asarray(x, np.float64) for x in p0_host]
        self.m = [np.zeros_like(x) for x in self.p]
        self.v = [np.zeros_like(x) for x in self.p]
        self.t = [0] * len(wl.groups)

    def step(self, g_host, sumsq, lrs):
        norm = float(np.sqrt(sumsq))
        coef = O.clip_coefficient(norm, self.wl.max_norm)
        for k in range(len(self.t)):
            self.t[k] += 1
        groups = _groups_at(self.wl, lrs)
        jobs = [(i, a, min(a + PIECE, t.numel)) for i, t in enumerate(self.wl.tensors) for a in range(0, t.numel, PIECE)]

        def piece(job):
            i, a, b = job
            k = self.wl.tensors[i].group
            self.p[i][a:b], self.m[i][a:b], self.v[i][a:b] = O.update_elements(
                self.p[i][a:b], self.m[i][a:b], self.v[i][a:b], g_host[i][a:b], coef, self.wl.grad_divisor,
                groups[k], self.t[k])
        with ThreadPoolExecutor(WORKERS) as ex:
            list(ex.map(piece, jobs))
        return norm, coef


class SampledOracle:
    """fp64 oracle state for sampled elements of every trainable tensor."""

    def __init__(self, wl, p0_samples, idx):
        self.wl = wl
        self.idx = idx
        self.p = [np.asarray(x, np.float64) for x in p0_samples]
        self.m = [np.zeros_like(x) for x in self.p]
        self.v = [np.zeros_like(x) for x in self.p]
        self.t = [0] * len(wl.groups)
        self.groups = [O.Group(h.lr, h.weight_decay, h.beta1, h.beta2, h.eps) for h in wl.groups]

    def step(self, g_samples, sumsq, lrs):
        norm = float(np.sqrt(sumsq))
        coef = O.clip_coefficient(norm, self.wl.max_norm)
        for k in range(len(self.groups)):
            self.t[k] += 1
            self.groups[k].lr = lrs[k]
        for i, t in enumerate(self.wl.tensors):
            grp = self.groups[t.group]
            self.p[i], self.m[i], self.v[i] = O.update_elements(
                self.p[i], self.m[i], self.v[i], g_samples[i], coef, self.wl.grad_divisor, grp,
                self.t[t.group])
        return norm, coef


def _gather(t, idx):
    return t[torch.as_tensor(idx, device=t.device)].cpu()


def test_action_expert_full_size_every_element():
    """Arena layout (the bench's): the oracle follows every element and all of
    p, m and v are compared after 10 steps."""
    run_unsharded(W.action_expert(), layout="arena", full=True)


def test_action_expert_full_size_tensor_layout_sampled():
    run_unsharded(W.action_expert(), layout="tensor")


def test_backbone_7b_full_size():
    """Every element after steps 1 and 2 (streamed), sampled windows to 10."""
    run_unsharded(W.backbone_7b(), stream_after=(1, 2))


def test_action_expert_full_size_bf16_working_copy():
    """The bench's --lowp bf16 configuration at full size, three steps: sampled
    p/m/v against the oracle, and every element of every working copy equal to
    torch's round-to-nearest-even conversion of the kernel's fp32 master."""
    from dataclasses import replace
    run_unsharded(replace(W.action_expert(), steps=3), lowp=torch.bfloat16)


def _state(wl, dev, layout, lowp):
    """The bench's layouts: "arena" holds each kind (p, g, m, v, working copy)
    in buffers of at most 2^30 elements with every tensor at a 64-element
    boundary; "tensor" makes one allocation per tensor and kind."""
    if layout == "tensor":
        p, g, m, v = [], [], [], []
        for i, t in enumerate(wl.tensors):
            p.append(W.param_values(wl, i, dev))
            g.append(W.grad_values(wl, i, 1, dev))
            m.append(torch.zeros(t.numel, device=dev))
            v.append(torch.zeros(t.numel, device=dev))
        lp = [torch.empty(t.numel, dtype=lowp, device=dev) for t in wl.tensors] if lowp is not None else None
        return p, g, m, v, lp
    place, sizes = W.arena_layout(wl)
    gdt = W.torch_dtype(wl.tensors[0].grad_dtype)
    bufs = [[torch.empty(n, device=dev) for n in sizes], [torch.empty(n, dtype=gdt, device=dev) for n in sizes],
            [torch.zeros(n, device=dev) for n in sizes], [torch.zeros(n, device=dev) for n in sizes]]
    if lowp is not None:
        bufs.append([torch.empty(n, dtype=lowp, device=dev) for n in sizes])
    views = [[b[c][o:o + t.numel] for (c, o), t in zip(place, wl.tensors)] for b in bufs]
    for i in range(wl.n_tensors):
        views[0][i].copy_(W.param_values(wl, i, dev))
        views[1][i].copy_(W.grad_values(wl, i, 1, dev))
    return views[0], views[1], views[2], views[3], (views[4] if lowp is not None else None)


def run_unsharded(wl, lowp=None, layout="arena", full=False, stream_after=()):
    """``full``: the oracle follows every element and every element is compared
    at the end; else sampled windows, plus a streamed every-element check after
    each step in ``stream_after``."""
    from tensor_optimizer_step_amd.somaopt import FusedAdamW
    log(f"[fullsize] {wl.name}: {wl.n_tensors} tensors, {wl.trainable_numel} elements, {layout} layout")
    rng = np.random.default_rng(7)
    dev = "cuda"
    p, g, m, v, lp = _state(wl, dev, layout, lowp)
    idx = [sample_indices(t.numel, rng) for t in wl.tensors]
    if full:
        ora = FullOracle(wl, [x.cpu().numpy() for x in p])
    else:
        ora = SampledOracle(wl, [_gather(x, ix).numpy() for x, ix in zip(p, idx)], idx)
    opt = FusedAdamW(p, g, m, v, [t.group for t in wl.tensors], wl.groups, wl.max_norm,
                     wl.grad_divisor, params_lowp=lp)
    opt.capture()
    sumsq_cache = {}
    coefs, lrs_hist = [], []
    for k in range(1, wl.steps + 1):
        for i in range(wl.n_tensors):
            g[i].copy_(W.grad_values(wl, i, k, dev))
        key = k if not wl.grad_period else (1 + (k - 1) % wl.grad_period, wl.grad_std(k))
        g_host = [W.to_numpy_grad(x) for x in g] if full else None
        if key not in sumsq_cache:
            sumsq_cache[key] = (host_sumsq(g_host, wl.grad_divisor) if full
                                else host_sumsq_by_tensor(g, wl.grad_divisor))
        g_clone = [x.clone() for x in g] if k in (1, wl.steps) else None
        lrs = wl.lrs_for_step(k)
        opt.set_lrs(lrs)
        opt.replay()
        stats, steps = opt.read_stats()
        if full:
            norm, coef = ora.step(g_host, sumsq_cache[key], lrs)
            del g_host
        else:
            g_s = [W.to_numpy_grad(_gather(x, ix)) for x, ix in zip(g, idx)]
            norm, coef = ora.step(g_s, sumsq_cache[key], lrs)
        coefs.append(coef)
        lrs_hist.append(lrs)
        assert_norm(stats.norm, norm)
        assert stats.clip_coef == pytest.approx(coef, rel=1e-12)
        assert steps == [k] * len(wl.groups)
        if g_clone is not None:
            assert all(torch.equal(a, b) for a, b in zip(g, g_clone)), "a gradient buffer changed"
            del g_clone
        log(f"[fullsize] {wl.name} step {k}: norm {stats.norm:.6g} coef {stats.clip_coef:.6g}")
        if k in stream_after:
            torch.cuda.synchronize()
            stream_check(wl, k, coefs, lrs_hist, lambda i, a, b: [(a, b, p[i][a:b], m[i][a:b], v[i][a:b])],
                         wl.name)
    torch.cuda.synchronize()
    worst = [0.0, 0.0, 0.0]
    if full:
        jobs = [(i, a, min(a + PIECE, t.numel)) for i, t in enumerate(wl.tensors) for a in range(0, t.numel, PIECE)]

        def piece(job):
            i, a, b = job
            return [assert_close(f"{'pmv'[j]}[{i}][{a}:{b}]", dev_t[a:b].cpu().numpy(), want[a:b])
                    for j, (dev_t, want) in enumerate(((p[i], ora.p[i]), (m[i], ora.m[i]), (v[i], ora.v[i])))]
        with ThreadPoolExecutor(WORKERS) as ex:
            for r in ex.map(piece, jobs):
                worst = [max(x, y) for x, y in zip(worst, r)]
        log(f"[fullsize] {wl.name}: every element of p, m, v after {wl.steps} steps within the bar "
            f"({wl.trainable_numel} per kind)")
    else:
        for i in range(wl.n_tensors):
            for j, (dev_t, want) in enumerate(((p[i], ora.p[i]), (m[i], ora.m[i]), (v[i], ora.v[i]))):
                worst[j] = max(worst[j], assert_close(f"{'pmv'[j]}[{i}]", _gather(dev_t, idx[i]).numpy(), want))
    log(f"[fullsize] {wl.name}: tensor-wise rel err p={worst[0]:.2e} m={worst[1]:.2e} v={worst[2]:.2e}")
    if lp is not None:
        for i in range(wl.n_tensors):
            assert torch.equal(lp[i].view(torch.int16), p[i].to(lowp).view(torch.int16)), f"working copy {i}"
        log(f"[fullsize] {wl.name}: every working-copy element equals the rounding of its fp32 master")
    opt.close()
    del p, g, m, v, lp


def test_sharded_7b_full_size():
    """Four contiguous shards of the 7B matrices plus four RMSNorm replicas
    (owner = shard 0), one handle of 488 descriptors; compared with the oracle
    on the unsharded tensors, every replica included: every element of every
    piece and replica after steps 1 and 2 (streamed), sampled windows and the
    neighbourhoods of the cuts to step 10."""
    from tensor_optimizer_step_amd.somaopt import FusedAdamW
    lay = W.sharded_7b()
    wl = lay.base
    log(f"[fullsize] sharded_7b: {lay.n_descriptors} descriptors over {lay.n_shards} shards")
    dev = "cuda"
    S = lay.n_shards
    sp = [torch.empty(n, device=dev) for n in lay.shard_numel]
    sg = [torch.empty(n, dtype=torch.bfloat16, device=dev) for n in lay.shard_numel]
    sm = [torch.zeros(n, device=dev) for n in lay.shard_numel]
    sv = [torch.zeros(n, device=dev) for n in lay.shard_numel]
    by_tensor = {}
    for q in lay.pieces:
        by_tensor.setdefault(q.tensor, []).append(q)

    def scatter(dst, i, values):
        for q in by_tensor[i]:
            dst[q.shard][q.s_offset:q.s_offset + q.numel].copy_(values[q.t_offset:q.t_offset + q.numel])

    for i in range(wl.n_tensors):
        scatter(sp, i, W.param_values(wl, i, dev))
    rng = np.random.default_rng(11)
    idx = [sample_indices(t.numel, rng) for t in wl.tensors]
    # the pieces next to every cut are sampled too
    for i, qs in by_tensor.items():
        if len(qs) > 1 and wl.tensors[i].group == 0:
            cuts = [q.t_offset for q in qs if q.t_offset > 0]
            extra = [np.arange(max(c - 4096, 0), min(c + 4096, wl.tensors[i].numel)) for c in cuts]
            idx[i] = np.unique(np.concatenate([idx[i]] + extra))

    def logical(buf_list, i, ix):
        """Gather logical tensor i's sampled elements from the shard that owns
        each element (the first piece holding it; replicas: shard 0)."""
        out = np.empty(len(ix), dtype=np.float64)
        for q in by_tensor[i]:
            sel = (ix >= q.t_offset) & (ix < q.t_offset + q.numel)
            if q.shard != by_tensor[i][0].shard and wl.tensors[i].group == 1:
                continue
            if sel.any():
                src = buf_list[q.shard][q.s_offset:q.s_offset + q.numel]
                out[sel] = _gather(src, ix[sel] - q.t_offset).float().numpy()
        return out

    p0 = [logical(sp, i, idx[i]) for i in range(wl.n_tensors)]
    ora = SampledOracle(wl, p0, idx)
    descs_p, descs_g, descs_m, descs_v, groups_of, owner = [], [], [], [], [], []
    for q in lay.pieces:
        sl = slice(q.s_offset, q.s_offset + q.numel)
        descs_p.append(sp[q.shard][sl])
        descs_g.append(sg[q.shard][sl])
        descs_m.append(sm[q.shard][sl])
        descs_v.append(sv[q.shard][sl])
        groups_of.append(wl.tensors[q.tensor].group)
        owner.append(q.owner)
    opt = FusedAdamW(descs_p, descs_g, descs_m, descs_v, groups_of, wl.groups, wl.max_norm,
                     wl.grad_divisor, owner=owner)
    info = opt.plan_info()
    assert info.owned_numel == wl.trainable_numel
    assert info.trainable_numel == wl.trainable_numel + (S - 1) * sum(
        t.numel for t in wl.tensors if t.group == 1)
    opt.capture()

    def locate(i, a, b):
        """Device views of logical elements [a, b) of tensor i: the pieces
        covering them (a range may cross a shard cut) and every replica."""
        out = []
        for q in by_tensor[i]:
            lo, hi = max(a, q.t_offset), min(b, q.t_offset + q.numel)
            if lo < hi:
                s0 = q.s_offset + (lo - q.t_offset)
                sl = slice(s0, s0 + hi - lo)
                out.append((lo, hi, sp[q.shard][sl], sm[q.shard][sl], sv[q.shard][sl]))
        return out

    sumsq_cache = {}
    coefs, lrs_hist = [], []
    for k in range(1, wl.steps + 1):
        gl = []
        for i in range(wl.n_tensors):
            gi = W.grad_values(wl, i, k, dev)
            scatter(sg, i, gi)
            gl.append(gi)
        key = (1 + (k - 1) % wl.grad_period, wl.grad_std(k))
        if key not in sumsq_cache:
            sumsq_cache[key] = host_sumsq_by_tensor(gl, wl.grad_divisor)
        lrs = lay.base.lrs_for_step(k)
        opt.set_lrs(lrs)
        opt.replay()
        stats, steps = opt.read_stats()
        g_s = [W.to_numpy_grad(_gather(x, ix)) for x, ix in zip(gl, idx)]
        del gl
        norm, coef = ora.step(g_s, sumsq_cache[key], lrs)
        coefs.append(coef)
        lrs_hist.append(lrs)
        assert_norm(stats.norm, norm)
        assert stats.clip_coef == pytest.approx(coef, rel=1e-12)
        log(f"[fullsize] sharded_7b step {k}: norm {stats.norm:.6g} coef {stats.clip_coef:.6g}")
        if k in (1, 2):
            torch.cuda.synchronize()
            stream_check(wl, k, coefs, lrs_hist, locate, "sharded_7b")
    torch.cuda.synchronize()
    for i, t in enumerate(wl.tensors):
        for j, (bufs, want) in enumerate(((sp, ora.p[i]), (sm, ora.m[i]), (sv, ora.v[i]))):
            assert_close(f"{'pmv'[j]}[{i}]", logical(bufs, i, idx[i]), want)
        if t.group == 1:
            # every replica holds bit-identical values
            reps = [q for q in by_tensor[i]]
            assert len(reps) == S
            ref = sp[reps[0].shard][reps[0].s_offset:reps[0].s_offset + t.numel]
            for q in reps[1:]:
                other = sp[q.shard][q.s_offset:q.s_offset + t.numel]
                assert torch.equal(ref, other), f"replica of tensor {i} diverged"
    opt.close()


def test_action_expert_arrival_full_size():
    """The 302,092,288-element action expert fed by the arrival pass (the
    bench's --arrival configuration): three steps alternating accumulate and
    copy.  The new gradients are compared bit for bit in full against the
    oracle's accumulation of the host copies, the norm against the oracle's
    sum over all of them, and p, m, v on sampled windows."""
    import oracle as O
    from tensor_optimizer_step_amd.somaopt import FusedAdamW
    wl = W.action_expert()
    log(f"[fullsize] arrival {wl.name}: {wl.n_tensors} tensors, {wl.trainable_numel} elements")
    rng = np.random.default_rng(11)
    dev = "cuda"
    p, g, m, v, inc = [], [], [], [], []
    for i, t in enumerate(wl.tensors):
        p.append(W.param_values(wl, i, dev))
        g.append(W.grad_values(wl, i, 1, dev))
        m.append(torch.zeros(t.numel, device=dev))
        v.append(torch.zeros(t.numel, device=dev))
        inc.append(torch.empty_like(g[-1]))
    idx = [sample_indices(t.numel, rng) for t in wl.tensors]
    ora = SampledOracle(wl, [_gather(x, ix).numpy() for x, ix in zip(p, idx)], idx)
    opt = FusedAdamW(p, g, m, v, [t.group for t in wl.tensors], wl.groups, wl.max_norm, wl.grad_divisor)
    opt.register_arrival(inc)
    held = [W.to_numpy_grad(x) for x in g]
    for k, acc in ((1, True), (2, False), (3, True)):
        for i in range(wl.n_tensors):
            inc[i].copy_(W.grad_values(wl, i, 20 + k, dev))
        hin = [W.to_numpy_grad(x) for x in inc]
        lrs = wl.lrs_for_step(k)
        opt.set_lrs(lrs)
        opt.arrival_sqnorm(acc)
        opt.fused_adamw_step()
        stats, steps = opt.read_stats()
        with ThreadPoolExecutor(WORKERS) as ex:
            new = list(ex.map(lambda i: O.accumulate_gradient(held[i], hin[i], acc), range(wl.n_tensors)))
        for i in range(wl.n_tensors):
            assert np.array_equal(W.to_numpy_grad(g[i]), new[i]), f"step {k}: gradient {i} differs"
        with ThreadPoolExecutor(WORKERS) as ex:
            parts = list(ex.map(lambda x: O.normalized_sumsq([x], [True], wl.grad_divisor), new))
        sumsq = 0.0
        for x in parts:
            sumsq += x
        norm, coef = ora.step([x[ix] for x, ix in zip(new, idx)], sumsq, lrs)
        assert_norm(stats.norm, norm)
        assert stats.clip_coef == pytest.approx(coef, rel=1e-12)
        assert steps == [k] * len(wl.groups)
        log(f"[fullsize] arrival step {k} ({'accumulate' if acc else 'copy'}): norm {stats.norm:.6g}")
        held = new
    torch.cuda.synchronize()
    worst = [0.0, 0.0, 0.0]
    for i in range(wl.n_tensors):
        for j, (dev_t, want) in enumerate(((p[i], ora.p[i]), (m[i], ora.m[i]), (v[i], ora.v[i]))):
            worst[j] = max(worst[j], assert_close(f"{'pmv'[j]}[{i}]", _gather(dev_t, idx[i]).numpy(), want))
    log(f"[fullsize] arrival: tensor-wise rel err p={worst[0]:.2e} m={worst[1]:.2e} v={worst[2]:.2e}")
    opt.close()
    del p, g, m, v, inc


def test_single_tensor_past_two_to_the_32_elements():
    """One tensor of 2^32 + 3*2^20 + 5 elements (bf16 gradients, fp32 state:
    60 GB on the device), stepped as the captured graph: its segments, the
    update pass's launches and the byte offsets cross 2^31 and 2^32 elements,
    and the last segment ends in a ragged scalar tail.  The global norm comes
    from the oracle over every gradient on the host; after step 1 every element
    of p, m and v is compared with the oracle run on host copies of the initial
    weights and the gradients (streamed piece by piece), after step 2 (same
    gradients) windows at the start, across both boundaries and at the end;
    the gradients are compared bit for bit with their host copy at the end."""
    from tensor_optimizer_step_amd import somaopt
    n = (1 << 32) + 3 * (1 << 20) + 5
    lr, wd, max_norm, divisor = 5e-6, 0.01, 1.0, 2.0
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    p = torch.randn(n, generator=gen, device="cuda").mul_(0.02)
    g = torch.randn(n, generator=gen, device="cuda", dtype=torch.bfloat16).mul_(0.05)
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    torch.cuda.synchronize()
    log(f"[fullsize] single tensor: {n} elements allocated")
    p0 = p.cpu().numpy()
    g_host = W.to_numpy_grad(g)
    pieces = [(a, min(a + PIECE, n)) for a in range(0, n, PIECE)]
    total = host_sumsq([g_host[a:b] for a, b in pieces], divisor)
    coef = O.clip_coefficient(float(np.sqrt(total)), max_norm)
    assert coef < 1.0   # the step clips
    log(f"[fullsize] single tensor: host norm {np.sqrt(total):.6f}, coefficient {coef:.6e}")
    grp = O.Group(lr, wd, 0.9, 0.999, 1e-8)   # the same hyperparameters, for the oracle
    hp = {"lr": lr, "weight_decay": wd, "beta1": 0.9, "beta2": 0.999, "eps": 1e-8}
    opt = somaopt.FusedAdamW([p], [g], [m], [v], [0], [hp], max_norm, divisor)
    assert opt.plan_info().pass2_launches > 1
    opt.capture()
    opt.replay()
    torch.cuda.synchronize()
    stats, steps = opt.read_stats()
    assert steps == [1]
    assert_norm(stats.norm, float(np.sqrt(total)))

    def piece(ab):
        a, b = ab
        want = O.update_elements(p0[a:b], np.zeros(b - a), np.zeros(b - a), g_host[a:b], coef, divisor, grp, 1)
        return [assert_close(f"single tensor step 1 {k}[{a}:{b}]", dt[a:b].cpu().numpy(), w)
                for k, dt, w in zip("pmv", (p, m, v), want)]

    worst = [0.0, 0.0, 0.0]
    with ThreadPoolExecutor(WORKERS) as ex:
        for r in ex.map(piece, pieces):
            worst = [max(x, y) for x, y in zip(worst, r)]
    log(f"[fullsize] single tensor: every element after step 1 within the bar; tensor-wise rel err "
        f"p={worst[0]:.2e} m={worst[1]:.2e} v={worst[2]:.2e}")

    opt.replay()
    torch.cuda.synchronize()
    stats, steps = opt.read_stats()
    assert steps == [2]
    assert_norm(stats.norm, float(np.sqrt(total)))
    for a in (0, (1 << 31) - WINDOW // 2, (1 << 32) - WINDOW // 2, n - WINDOW):
        b = a + WINDOW
        st = (np.asarray(p0[a:b], np.float64), np.zeros(WINDOW), np.zeros(WINDOW))
        for k in (1, 2):
            st = O.update_elements(*st, g_host[a:b], coef, divisor, grp, k)
        for name, dt, w in zip("pmv", (p, m, v), st):
            assert_close(f"single tensor step 2 {name}[{a}:{b}]", dt[a:b].cpu().numpy(), w)
    assert np.array_equal(W.to_numpy_grad(g), g_host), "gradient buffer was written"
    log("[fullsize] single tensor: step-2 windows across 2^31 and 2^32 within the bar; gradients unchanged")
    opt.close()
