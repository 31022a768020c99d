"""GPU parity of the HIP path (through the C-ABI) against the fp64 oracle.

Inputs are seeded and synthetic (tensor_optimizer_step_amd.workloads), created
on the GPU with torch's generator and copied to the host for the oracle.
Sizes here finish in seconds on the oracle yet span many workgroups and ragged
tails; full-size workloads are in test_gpu_parity_fullsize.py.
"""
import math

import numpy as np
import pytest

import oracle as O
from tensor_optimizer_step_amd import workloads as W

from parity_util import (assert_close, assert_norm, allocate, fill_grads, host, log,
                         make_handle, make_oracle)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tensor_optimizer_step_amd import somaopt
    somaopt.load()          # fail loudly if the library is missing
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def schedule_lrs(wl, schedules, k):
    """The oracle's per-group lr of update k under on-device schedules."""
    return [O.scheduled_lr(sc[0], k, lr=g.lr, peak=sc[3], floor=sc[4], warmup=sc[1], total=sc[2])
            for sc, g in zip(schedules, wl.groups)]


def run_and_compare(wl, steps=None, graph=True, max_norm=None, divisor=None, check_every_step=True,
                    schedules=None):
    """Run ``steps`` updates on the GPU and the oracle; compare everything.
    With ``schedules`` the handle evaluates the lr schedules on the device
    (set once, no host call between steps) and the oracle follows its own
    schedule functions."""
    steps = wl.steps if steps is None else steps
    log(f"[parity] {wl.name}: {wl.n_tensors} tensors, {wl.trainable_numel} trainable, "
        f"{steps} steps, graph={graph}")
    st = allocate(wl)
    p0 = [host(x) for x in st.p]
    frozen_before = {i: (host(st.p[i]), host(st.m[i]), host(st.v[i]))
                     for i, t in enumerate(wl.tensors) if not t.trainable}
    kw = {}
    if max_norm is not None:
        kw["max_norm"] = max_norm
    if divisor is not None:
        kw["grad_divisor"] = divisor
    opt = make_handle(wl, st, **kw)
    if schedules is not None:
        opt.set_schedules(schedules)
    ora = make_oracle(wl, p0, max_norm=max_norm, divisor=divisor)
    if graph:
        opt.capture()
    for k in range(1, steps + 1):
        fill_grads(wl, st, k)
        grads = [host(g) for g in st.g]
        if schedules is None:
            lrs = wl.lrs_for_step(k)
            opt.set_lrs(lrs)
        else:
            lrs = schedule_lrs(wl, schedules, k)
        if graph:
            opt.replay()
        else:
            opt.step()
        stats, t = opt.read_stats()
        want = ora.step(grads, lrs)
        if check_every_step or k == steps:
            assert_norm(stats.norm, want.norm)
            assert stats.clip_coef == pytest.approx(want.coef, rel=1e-12)
            assert stats.nonfinite == 0
            assert t == [k] * len(wl.groups)
        # gradient buffers are never written
        for i, g in enumerate(st.g):
            assert np.array_equal(host(g).view(np.uint8), grads[i].view(np.uint8)), f"grad {i} changed"
    torch.cuda.synchronize()
    worst = {"p": 0.0, "m": 0.0, "v": 0.0}
    for i, t in enumerate(wl.tensors):
        if not t.trainable:
            fb = frozen_before[i]
            for name, a, b in zip("pmv", (st.p[i], st.m[i], st.v[i]), fb):
                assert np.array_equal(host(a).view(np.uint32), b.view(np.uint32)), f"frozen {name}{i}"
            continue
        worst["p"] = max(worst["p"], assert_close(f"p[{i}]", host(st.p[i]), ora.p[i]))
        worst["m"] = max(worst["m"], assert_close(f"m[{i}]", host(st.m[i]), ora.m[i]))
        worst["v"] = max(worst["v"], assert_close(f"v[{i}]", host(st.v[i]), ora.v[i]))
    log(f"[parity] {wl.name}: tensor-wise rel err p={worst['p']:.2e} m={worst['m']:.2e} v={worst['v']:.2e}")
    opt.close()
    return st, ora


def test_tiny_one_step_eager():
    run_and_compare(W.tiny(), graph=False)


def test_tiny_one_step_graph():
    run_and_compare(W.tiny(seed_offset=1), graph=True)


def test_tiny_micro_batch_divisor():
    # the veRL page's accumulation divisor: 128 // 8 = 16 micro-batches
    run_and_compare(W.tiny(seed_offset=2), steps=3, divisor=16.0)


def test_action_expert_scaled_bf16_ten_steps():
    wl = W.action_expert(blocks=2, d=256, mlp=1024, action_dim=32)
    run_and_compare(wl)


def test_launch_bound_full_ten_steps():
    # 20,000 tensors, 6,000 frozen with NaN gradients, warm-up schedule, 3 groups
    run_and_compare(W.launch_bound(), check_every_step=True)


def test_launch_bound_clipped_variant():
    run_and_compare(W.launch_bound(n_tensors=3000), steps=4, max_norm=1.0)


def test_launch_bound_device_warmup_schedule():
    # the launch-bound warm-up evaluated on the device, past its end
    from tensor_optimizer_step_amd import somaopt
    wl = W.launch_bound(n_tensors=3000)
    scheds = [(somaopt.SCHED_LINEAR_WARMUP, wl.steps, 0, g.lr, 0.0) for g in wl.groups]
    run_and_compare(wl, steps=wl.steps + 2, schedules=scheds)


def test_device_cosine_and_warmup_cosine_schedules():
    from tensor_optimizer_step_amd import somaopt
    wl = W.action_expert(blocks=1, d=128, mlp=512, action_dim=16)
    scheds = [(somaopt.SCHED_COSINE, 0, 6, 2e-4, 1e-5),
              (somaopt.SCHED_WARMUP_COSINE, 2, 6, 1e-4, 0.0)]
    run_and_compare(wl, steps=9, schedules=scheds)


def test_device_schedule_bitwise_equals_host_setter():
    """The device's linear warm-up takes the same fp64 operations as the host's
    schedule, so a replayed step with no host call matches eager steps fed by
    somaopt_set_groups bit for bit."""
    from tensor_optimizer_step_amd import somaopt
    wl = W.launch_bound(n_tensors=500)
    sts, opts = [], []
    for device_sched in (False, True):
        st = allocate(wl)
        opt = make_handle(wl, st)
        if device_sched:
            opt.set_schedules([(somaopt.SCHED_LINEAR_WARMUP, wl.steps, 0, g.lr, 0.0) for g in wl.groups])
            opt.capture()
        sts.append(st)
        opts.append(opt)
    for k in range(1, 6):
        for st in sts:
            fill_grads(wl, st, k)
        opts[0].set_lrs(wl.lrs_for_step(k))
        opts[0].step()
        opts[1].replay()
    torch.cuda.synchronize()
    for name in "pmv":
        for i, (a, b) in enumerate(zip(getattr(sts[0], name), getattr(sts[1], name))):
            assert np.array_equal(host(a).view(np.uint32), host(b).view(np.uint32)), f"{name}{i}"
    for o in opts:
        o.close()


def test_schedule_validation_and_reset():
    from tensor_optimizer_step_amd import somaopt
    wl = W.tiny(seed_offset=5)
    st = allocate(wl)
    opt = make_handle(wl, st)
    bad = [(7, 1, 1, 1e-3, 0.0), (somaopt.SCHED_LINEAR_WARMUP, 0, 0, 1e-3, 0.0),
           (somaopt.SCHED_COSINE, 0, 0, 1e-3, 0.0), (somaopt.SCHED_WARMUP_COSINE, 5, 5, 1e-3, 0.0),
           (somaopt.SCHED_COSINE, 0, 4, -1e-3, 0.0), (somaopt.SCHED_COSINE, 0, 4, math.nan, 0.0),
           (somaopt.SCHED_COSINE, 0, 4, 1e-3, math.inf)]
    for sc in bad:
        with pytest.raises(somaopt.SomaoptError):
            opt.set_schedules([sc])
    with pytest.raises(somaopt.SomaoptError):
        opt.set_schedules([(somaopt.SCHED_NONE, 0, 0, 0.0, 0.0)] * 2)   # wrong group count
    # a schedule, then back to none: the group's own lr applies again
    ora = make_oracle(wl, [host(x) for x in st.p])
    opt.set_schedules([(somaopt.SCHED_COSINE, 0, 3, 1e-4, 0.0)])
    fill_grads(wl, st, 1)
    opt.step()
    ora.step([host(g) for g in st.g], [O.scheduled_lr(O.schedule_fp64.COSINE, 1, peak=1e-4, total=3)])
    opt.set_schedules([(somaopt.SCHED_NONE, 0, 0, 0.0, 0.0)])
    fill_grads(wl, st, 2)
    opt.step()
    ora.step([host(g) for g in st.g], wl.lrs_for_step(2))
    torch.cuda.synchronize()
    for i, t in enumerate(wl.tensors):
        if t.trainable:
            assert_close(f"p[{i}]", host(st.p[i]), ora.p[i])
            assert_close(f"m[{i}]", host(st.m[i]), ora.m[i])
            assert_close(f"v[{i}]", host(st.v[i]), ora.v[i])
    opt.close()


def test_edge_sizes_and_empty_tensors():
    tensors = [W.TensorSpec(f"e{i}", n, i % 2, W.F32 if i % 3 else W.BF16)
               for i, n in enumerate([0, 1, 2, 3, 4, 5, 7, 8, 9, 255, 256, 257, 1023, 4095,
                                      8191, 8192, 8193, 0, 32767, 32768, 32769, 65537])]
    wl = W.Workload("edges", 1, tensors, [W.GroupHP(1e-3, 0.1), W.GroupHP(2e-3, 0.0)],
                    max_norm=1.0, grad_divisor=2.0, steps=3)
    run_and_compare(wl)


def test_no_owned_or_trainable_tensors():
    tensors = [W.TensorSpec(f"f{i}", 100, 0, W.F32, trainable=False) for i in range(3)]
    wl = W.Workload("all_frozen", 1, tensors, [W.GroupHP(1e-3, 0.1)], 1.0, 1.0, steps=2,
                    nan_frozen_grads=True)
    run_and_compare(wl)


def _arena_case(seed):
    """Tensors packed into shared arenas at odd element offsets, canaries in between.

    Half the tensors share one offset modulo 4 across p/m/v/g (vector path with
    a scalar head); the rest differ (scalar fallback).
    """
    rng = np.random.default_rng(seed)
    wl = W.tiny(seed_offset=seed, n_tensors=24, max_numel=9000)
    n = wl.n_tensors
    CANARY = 0x7FA5A5A5         # a NaN payload no computation produces
    offs = {k: [] for k in "pmvg"}
    pos = {k: 3 for k in "pmvg"}
    for i, t in enumerate(wl.tensors):
        common = int(rng.integers(0, 4))
        for k in "pmvg":
            sh = common if i % 2 == 0 else int(rng.integers(0, 4))
            pos[k] += 5 + sh
            offs[k].append(pos[k])
            pos[k] += t.numel
    arenas = {k: torch.full((pos[k] + 11,), 0, dtype=torch.int32, device="cuda").fill_(CANARY)
              .view(torch.float32) for k in "pmvg"}
    return wl, offs, arenas, CANARY


@pytest.mark.parametrize("seed", [0, 1])
def test_arena_odd_offsets_and_canaries(seed):
    from parity_util import DeviceState
    wl, offs, ar, canary = _arena_case(seed)
    log(f"[parity] arena seed={seed}")
    st = DeviceState([], [], [], [])
    for i, t in enumerate(wl.tensors):
        n = t.numel
        st.p.append(ar["p"][offs["p"][i]:offs["p"][i] + n])
        st.m.append(ar["m"][offs["m"][i]:offs["m"][i] + n])
        st.v.append(ar["v"][offs["v"][i]:offs["v"][i] + n])
        st.g.append(ar["g"][offs["g"][i]:offs["g"][i] + n])
        st.p[i].copy_(W.param_values(wl, i, "cuda"))
        st.m[i].zero_()
        st.v[i].zero_()
    masks = {}
    for k in "pmvg":
        msk = torch.ones(ar[k].numel(), dtype=torch.bool)
        for i, t in enumerate(wl.tensors):
            msk[offs[k][i]:offs[k][i] + t.numel] = False
        masks[k] = msk.numpy()
    p0 = [host(x) for x in st.p]
    opt = make_handle(wl, st)
    info = opt.plan_info()
    assert info.scalar_segments > 0       # both paths are exercised
    ora = make_oracle(wl, p0)
    for k in range(1, 3):
        fill_grads(wl, st, k)
        grads = [host(g) for g in st.g]
        opt.step()
        stats, _ = opt.read_stats()
        want = ora.step(grads)
        assert_norm(stats.norm, want.norm)
    for i in range(wl.n_tensors):
        assert_close(f"p[{i}]", host(st.p[i]), ora.p[i])
        assert_close(f"m[{i}]", host(st.m[i]), ora.m[i])
        assert_close(f"v[{i}]", host(st.v[i]), ora.v[i])
    for k in "pmvg":
        words = ar[k].view(torch.int32).cpu().numpy()
        assert (words[masks[k]] == canary).all(), f"canary overwritten in arena {k}"
    opt.close()


def _bits(st):
    return [host(x).view(np.uint32).copy() for x in st.p + st.m + st.v]


def _run_steps(wl, steps, graph, scale_pow2=0):
    st = allocate(wl)
    opt = make_handle(wl, st, grad_divisor=wl.grad_divisor * 2.0 ** scale_pow2)
    if graph:
        opt.capture()
    norms = []
    for k in range(1, steps + 1):
        fill_grads(wl, st, k)
        if scale_pow2:
            for g in st.g:
                g.mul_(2.0 ** scale_pow2)        # exact for a power of two
        opt.set_lrs(wl.lrs_for_step(k))
        opt.replay() if graph else opt.step()
        s, _ = opt.read_stats()
        norms.append((s.norm, s.clip_coef))
    torch.cuda.synchronize()
    out = _bits(st)
    opt.close()
    return out, norms


def test_graph_replay_equals_eager_bitwise():
    wl = W.launch_bound(n_tensors=2000)
    a, na = _run_steps(wl, 4, graph=False)
    b, nb = _run_steps(wl, 4, graph=True)
    assert na == nb
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_run_to_run_bitwise_determinism():
    wl = W.action_expert(blocks=1, d=512, mlp=2048)
    a, na = _run_steps(wl, 3, graph=True)
    b, nb = _run_steps(wl, 3, graph=True)
    assert na == nb
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_power_of_two_metamorphic():
    # scaling every gradient and the divisor by 2^j changes nothing, bit for bit
    wl = W.tiny(seed_offset=3)
    wl.steps = 2
    a, na = _run_steps(wl, 2, graph=True)
    b, nb = _run_steps(wl, 2, graph=True, scale_pow2=5)
    assert [x[0] for x in na] == [x[0] for x in nb]
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_resume_equals_continuation():
    wl = W.launch_bound(n_tensors=500)
    full, _ = _run_steps(wl, 6, graph=False)
    # 3 steps, then a fresh handle on the same state with initial_step=3
    st = allocate(wl)
    opt = make_handle(wl, st)
    for k in range(1, 4):
        fill_grads(wl, st, k)
        opt.set_lrs(wl.lrs_for_step(k))
        opt.step()
    opt.close()
    opt = make_handle(wl, st, initial_step=3)
    for k in range(4, 7):
        fill_grads(wl, st, k)
        opt.set_lrs(wl.lrs_for_step(k))
        opt.step()
    _, t = opt.read_stats()
    assert t == [6, 6, 6]
    torch.cuda.synchronize()
    assert all(np.array_equal(x, y) for x, y in zip(full, _bits(st)))
    opt.close()


def test_nonfinite_flag_and_remeasure():
    wl = W.tiny(seed_offset=4)
    st = allocate(wl)
    opt = make_handle(wl, st)
    fill_grads(wl, st, 1)
    st.g[5][0] = float("inf")
    opt.grad_sqnorm()
    s, t = opt.read_stats()
    assert s.nonfinite == 1 and s.clip_coef == 0.0 and t == [1]
    # measuring again before the update does not advance the step
    st.g[5][0] = 0.0
    opt.grad_sqnorm()
    s, t = opt.read_stats()
    assert s.nonfinite == 0 and math.isfinite(s.norm) and t == [1]
    opt.fused_adamw_step()
    opt.close()


def test_call_order_errors():
    from tensor_optimizer_step_amd.somaopt import SomaoptError, E_STATE, E_INVALID
    wl = W.tiny(seed_offset=5, n_tensors=4)
    st = allocate(wl)
    opt = make_handle(wl, st)
    with pytest.raises(SomaoptError) as e:
        opt.fused_adamw_step()
    assert e.value.code == E_STATE
    with pytest.raises(SomaoptError) as e:
        opt.replay()
    assert e.value.code == E_STATE          # not captured
    opt.capture()
    opt.grad_sqnorm()
    with pytest.raises(SomaoptError) as e:
        opt.replay()
    assert e.value.code == E_STATE          # eager norm pass pending
    opt.fused_adamw_step()
    opt.replay()
    with pytest.raises(SomaoptError) as e:
        opt.set_groups([W.GroupHP(1e-3, 0.0, beta1=1.0)])
    assert e.value.code == E_INVALID
    with pytest.raises(SomaoptError):
        opt.set_clip(0.0, 1.0)
    opt.close()


def _raw_init(rows, groups):
    """somaopt_init_tensor_table called through the C-ABI with raw pointers (no
    binding checks in between); returns the status and destroys any handle."""
    from tensor_optimizer_step_amd import somaopt as S
    lib = S.load()
    descs = S.make_descs(rows)
    grp = S.make_groups(groups)
    h = S.ctypes.c_void_p()
    rc = lib.somaopt_init_tensor_table(descs, len(rows), grp, len(groups), 1.0, 1.0, 0, None,
                                       S.ctypes.byref(h))
    if h.value:
        lib.somaopt_destroy(h)
    return rc, S.last_error()


def test_rejects_host_memory_and_out_of_range():
    """The library's own checks, reached through the raw C-ABI: host memory and
    a buffer that runs past the end of its allocation never reach a kernel.
    The binding refuses both earlier (a CPU tensor; a tensor whose size does
    not match the weight's)."""
    from tensor_optimizer_step_amd.somaopt import E_INVALID, FusedAdamW
    wl = W.tiny(seed_offset=6, n_tensors=2, max_numel=64)
    st = allocate(wl)
    bad = st.p[0].cpu()
    n = wl.tensors[0].numel
    rc, msg = _raw_init([(bad.data_ptr(), st.g[0].data_ptr(), st.m[0].data_ptr(), st.v[0].data_ptr(), n,
                          0, 0, 1, 1)], wl.groups)
    assert rc == E_INVALID and "device" in msg, msg
    from parity_util import DeviceState
    with pytest.raises(ValueError, match="not on a GPU"):
        make_handle(wl, DeviceState([bad] + st.p[1:], st.g, st.m, st.v))
    # a buffer whose declared size runs past the end of its allocation is
    # rejected before any kernel could touch it (64 MiB: its own allocation)
    torch.cuda.empty_cache()
    x = torch.zeros(1 << 24, device="cuda")
    rc, msg = _raw_init([(x[-50:].data_ptr(), x[200:300].data_ptr(), x[0:100].data_ptr(),
                          x[100:200].data_ptr(), 100, 0, 0, 1, 1)], wl.groups)
    assert rc == E_INVALID and "past the end" in msg, msg
    with pytest.raises(ValueError, match="grad: 100 elements, the weight has 50"):
        FusedAdamW([x[-50:]], [x[200:300]], [x[0:50]], [x[100:150]], [0], wl.groups, 1.0, 1.0)


@pytest.mark.parametrize("gdt,ldt", [(W.BF16, W.BF16), (W.F16, W.F16), (W.F32, W.BF16), (W.F16, W.BF16)])
def test_working_copy_and_gradient_dtypes(gdt, ldt):
    """bf16/fp16 working copies of the fp32 master (RLinf FP32MasterAdamW
    reading) and fp16 gradients.  The copy must equal the round-to-nearest-even
    of the kernel's own fp32 master bit for bit, and lie within one unit of the
    copy rounded from the oracle's weights."""
    import dataclasses
    import oracle as O
    from parity_util import DeviceState
    base = W.action_expert(blocks=1, d=256, mlp=512, steps=4)
    base.tensors = [dataclasses.replace(t, grad_dtype=gdt) for t in base.tensors]
    wl = base
    log(f"[parity] working copy grad={gdt} copy={ldt}")
    st = allocate(wl)
    ldtype = W.torch_dtype(ldt)
    lowp = [torch.full((t.numel,), float("nan"), dtype=ldtype, device="cuda") for t in wl.tensors]
    p0 = [host(x) for x in st.p]
    from tensor_optimizer_step_amd.somaopt import FusedAdamW
    opt = FusedAdamW(st.p, st.g, st.m, st.v, [t.group for t in wl.tensors], wl.groups, wl.max_norm,
                     wl.grad_divisor, params_lowp=lowp)
    ora = make_oracle(wl, p0)
    opt.capture()
    for k in range(1, wl.steps + 1):
        fill_grads(wl, st, k)
        grads = [host(g) for g in st.g]
        opt.replay()
        s, _ = opt.read_stats()
        want = ora.step(grads)
        assert_norm(s.norm, want.norm)
    torch.cuda.synchronize()
    for i in range(wl.n_tensors):
        gp = host(st.p[i])
        assert_close(f"p[{i}]", gp, ora.p[i])
        assert_close(f"m[{i}]", host(st.m[i]), ora.m[i])
        assert_close(f"v[{i}]", host(st.v[i]), ora.v[i])
        got = lowp[i].cpu().view(torch.int16).numpy().view(np.uint16)
        if ldt == W.BF16:
            mine = O.round_to_bf16_bits(gp)
            theirs = O.round_to_bf16_bits(ora.p[i].astype(np.float32))
        else:
            mine = O.round_to_f16(gp).view(np.uint16)
            theirs = O.round_to_f16(ora.p[i].astype(np.float32)).view(np.uint16)
        assert np.array_equal(got, mine), f"working copy {i} differs from RNE of the fp32 master"
        assert np.abs(got.astype(np.int32) - theirs.astype(np.int32)).max() <= 1
    opt.close()


@pytest.mark.parametrize("shift", [0, 4])
def test_working_copy_odd_vector_counts(shift):
    """bf16 working copies whose vector bodies hold odd numbers of 4-element
    vectors (the last vector has no partner for the paired 16-byte store), at
    a 16-byte-aligned start (shift 0) and at one only 8-byte aligned (shift 4
    elements: the per-lane 8-byte stores).  Guard elements on both sides of
    every copy must stay untouched."""
    import oracle as O
    from tensor_optimizer_step_amd.somaopt import FusedAdamW
    sizes = [1, 3, 4, 5, 7, 8, 12, 13, 20, 28, 36, 4092, 4096, 4100, 4104, 8196, 12292, 65540]
    tensors = [W.TensorSpec(f"w{i}", n, i % 2, W.BF16) for i, n in enumerate(sizes)]
    wl = W.Workload("lowp_edges", 1, tensors, [W.GroupHP(1e-3, 0.1), W.GroupHP(2e-3, 0.0)],
                    max_norm=1.0, grad_divisor=2.0, steps=3)
    log(f"[parity] working copy odd vector counts, shift={shift}")
    st = allocate(wl)
    guard = 8
    arenas = [torch.full((t.numel + shift + guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
              for t in tensors]
    lowp = [a[shift:shift + t.numel] for a, t in zip(arenas, tensors)]
    before = [a.cpu().view(torch.int16).numpy().copy() for a in arenas]
    p0 = [host(x) for x in st.p]
    opt = FusedAdamW(st.p, st.g, st.m, st.v, [t.group for t in tensors], wl.groups, wl.max_norm,
                     wl.grad_divisor, params_lowp=lowp)
    ora = make_oracle(wl, p0)
    opt.capture()
    for k in range(1, wl.steps + 1):
        fill_grads(wl, st, k)
        grads = [host(g) for g in st.g]
        opt.replay()
        ora.step(grads)
    torch.cuda.synchronize()
    for i, t in enumerate(tensors):
        gp = host(st.p[i])
        assert_close(f"p[{i}]", gp, ora.p[i])
        assert_close(f"m[{i}]", host(st.m[i]), ora.m[i])
        assert_close(f"v[{i}]", host(st.v[i]), ora.v[i])
        words = arenas[i].cpu().view(torch.int16).numpy()
        got = words[shift:shift + t.numel].view(np.uint16)
        assert np.array_equal(got, O.round_to_bf16_bits(gp)), f"working copy {i} (numel {t.numel})"
        assert np.array_equal(words[:shift], before[i][:shift]), f"guard before copy {i}"
        assert np.array_equal(words[shift + t.numel:], before[i][shift + t.numel:]), f"guard after copy {i}"
    opt.close()


def test_two_handles_on_two_streams_from_two_threads():
    """Handles share no state: two tables, each on its own stream, stepped
    from two host threads at once (the ABI asks only that one handle is used
    by one thread at a time), each matching its own oracle."""
    import threading
    wls = [W.tiny(seed_offset=11, n_tensors=12, max_numel=20000),
           W.tiny(seed_offset=12, n_tensors=9, max_numel=30000)]
    runs = []
    for wl in wls:
        st = allocate(wl)
        p0 = [host(x) for x in st.p]
        stream = torch.cuda.Stream()
        opt = make_handle(wl, st, stream=stream)
        opt.capture()
        runs.append((wl, st, opt, make_oracle(wl, p0), stream))
    # gradients of all three steps are drawn up front on the default stream
    grads = []
    for wl, st, _, _, _ in runs:
        per_step = []
        for k in range(1, 4):
            fill_grads(wl, st, k)
            per_step.append([g.clone() for g in st.g])
        grads.append(per_step)
    torch.cuda.synchronize()
    errors = []

    def worker(idx):
        try:
            wl, st, opt, _, stream = runs[idx]
            with torch.cuda.stream(stream):
                for k in range(3):
                    for dst, src in zip(st.g, grads[idx][k]):
                        dst.copy_(src)
                    opt.replay(stream)
            stream.synchronize()
        except Exception as e:      # reported on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for idx, (wl, st, opt, ora, _) in enumerate(runs):
        for k in range(3):
            ora.step([host(g) for g in grads[idx][k]])
        for i, t in enumerate(wl.tensors):
            if t.trainable:
                assert_close(f"h{idx} p[{i}]", host(st.p[i]), ora.p[i])
                assert_close(f"h{idx} m[{i}]", host(st.m[i]), ora.m[i])
                assert_close(f"h{idx} v[{i}]", host(st.v[i]), ora.v[i])
        _, steps = opt.read_stats()
        assert steps == [3] * len(wl.groups)
        opt.close()


def test_setters_mid_run_and_side_stream():
    """Change max_norm / divisor and the hyperparameters between steps, reset
    the step count on a live handle, and run everything on a non-default
    stream; the oracle follows the same settings."""
    import oracle as O
    wl = W.tiny(seed_offset=7, n_tensors=20, max_numel=30000)
    st = allocate(wl)
    p0 = [host(x) for x in st.p]
    side = torch.cuda.Stream()
    opt = make_handle(wl, st, stream=side)
    ora = make_oracle(wl, p0)
    opt.capture()
    plan = [  # (max_norm, divisor, lr, wd, beta1, beta2, eps, set_step)
        (1.0, 4.0, 5e-6, 0.01, 0.9, 0.999, 1e-8, None),
        (0.05, 4.0, 1e-4, 0.1, 0.9, 0.999, 1e-8, None),
        (10.0, 2.0, 1e-3, 0.0, 0.8, 0.99, 1e-6, None),
        (1.0, 16.0, 1e-3, 0.05, 0.95, 0.9999, 1e-8, 7),
        (0.5, 1.0, 2e-4, 0.01, 0.9, 0.999, 1e-8, 123456),
        (0.5, 1.0, 2e-4, 0.01, 0.9, 0.999, 1e-8, None),
    ]
    for k, (M, D, lr, wd, b1, b2, eps, reset) in enumerate(plan, start=1):
        fill_grads(wl, st, k)
        torch.cuda.synchronize()
        grads = [host(g) for g in st.g]
        with torch.cuda.stream(side):
            opt.set_clip(M, D, side)
            opt.set_groups([W.GroupHP(lr, wd, b1, b2, eps)], side)
            if reset is not None:
                opt.set_step(reset, side)
            opt.replay(side)
        s, t = opt.read_stats(side)
        ora.max_norm, ora.grad_divisor = M, D
        ora.groups[0] = O.Group(lr, wd, b1, b2, eps)
        if reset is not None:
            ora.t = [reset]
        want = ora.step(grads)
        assert_norm(s.norm, want.norm)
        assert s.clip_coef == pytest.approx(want.coef, rel=1e-12)
        assert t == ora.t
    torch.cuda.synchronize()
    for i in range(wl.n_tensors):
        assert_close(f"p[{i}]", host(st.p[i]), ora.p[i])
        assert_close(f"m[{i}]", host(st.m[i]), ora.m[i])
        assert_close(f"v[{i}]", host(st.v[i]), ora.v[i])
    opt.close()


@pytest.mark.parametrize("chunks", [(256, 256), (512, 4096), (65536, 1024)])
def test_other_chunkings_and_two_level_reduction(chunks, monkeypatch):
    """Other workgroup sizes (env tuning knobs), including the two-level
    reduction of norm partials (more than 8192 workgroups)."""
    monkeypatch.setenv("SOMAOPT_PASS1_CHUNK", str(chunks[0]))
    monkeypatch.setenv("SOMAOPT_PASS2_CHUNK", str(chunks[1]))
    wl = W.launch_bound(n_tensors=3000)
    wl.steps = 3
    st, ora = run_and_compare(wl)


@pytest.mark.parametrize("per_launch", [3, 100])
def test_update_pass_split_into_launches(per_launch, monkeypatch):
    """The update pass split into consecutive launches (the env knob, set far
    below its default so that a small table gets many launches) equals one
    launch bit for bit, eager and replayed."""
    wl = W.action_expert(blocks=1, d=512, mlp=2048)
    monkeypatch.setenv("SOMAOPT_PASS2_SLICE_BLOCKS", "0")
    one, n_one = _run_steps(wl, 3, graph=False)
    monkeypatch.setenv("SOMAOPT_PASS2_SLICE_BLOCKS", str(per_launch))
    probe = make_handle(wl, allocate(wl))
    info = probe.plan_info()
    probe.close()
    assert info.pass2_launches == -(-info.pass2_blocks // per_launch) > 1
    log(f"[split] {info.pass2_blocks} update workgroups in {info.pass2_launches} launches")
    for graph in (False, True):
        split, n_split = _run_steps(wl, 3, graph=graph)
        assert n_split == n_one
        assert all(np.array_equal(x, y) for x, y in zip(one, split)), f"graph={graph}"


def test_update_pass_split_matches_oracle(monkeypatch):
    monkeypatch.setenv("SOMAOPT_PASS2_SLICE_BLOCKS", "2")
    wl = W.tiny(seed_offset=5)
    wl.steps = 3
    run_and_compare(wl)
