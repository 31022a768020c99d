"""Handle lifetime: what somaopt_destroy waits for.

destroy issues no stream or device wait of its own, but it releases the
handle's device memory with hipFree, and the HIP runtime makes hipFree wait
until all work on the device has finished.  So destroy returns only once the
device is idle, including kernels on streams the handle never saw.  The test
measures that with a spin kernel of known duration on an unrelated stream
(the kernel ends normally on its own)."""
import time

import pytest

torch = pytest.importorskip("torch")

from tensor_optimizer_step_amd import workloads as W  # noqa: E402

from parity_util import allocate, fill_grads, log, make_handle  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _spin(stream, cycles):
    with torch.cuda.stream(stream):
        torch.cuda._sleep(cycles)


def test_destroy_returns_once_the_device_is_idle():
    from tensor_optimizer_step_amd import somaopt
    wl = W.tiny(seed_offset=9, n_tensors=8)
    st = allocate(wl)
    fill_grads(wl, st, 1)
    opt = make_handle(wl, st)
    opt.capture()
    opt.replay()
    torch.cuda.synchronize()
    other = torch.cuda.Stream()
    cycles = 1 << 27
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(other)
    _spin(other, cycles)
    e1.record(other)
    torch.cuda.synchronize()
    spin_ms = e0.elapsed_time(e1)
    assert spin_ms > 20.0, "the spin kernel is too short to tell waiting from not waiting"
    _spin(other, cycles)
    t0 = time.perf_counter()
    somaopt.load().somaopt_destroy(opt._h)      # the raw call: the binding's close() syncs its own streams first
    t1 = time.perf_counter()
    opt._h = None
    idle = other.query()
    torch.cuda.synchronize()
    ms = (t1 - t0) * 1e3
    log(f"[destroy] {ms:.2f} ms while a {spin_ms:.1f} ms kernel ran on another stream; that stream idle "
        f"after destroy: {idle}")
    assert idle, "destroy returned while a kernel on another stream was still running"
    assert ms > 0.5 * spin_ms


def test_close_waits_for_the_handles_streams_only_then_destroys():
    """The binding's close() first synchronizes every stream its calls were
    given, then destroys; a second close() is a no-op."""
    wl = W.tiny(seed_offset=10, n_tensors=4)
    st = allocate(wl)
    fill_grads(wl, st, 1)
    s = torch.cuda.Stream()
    opt = make_handle(wl, st)
    opt.step(stream=s)
    assert opt._streams == {s.cuda_stream}
    opt.close()
    assert s.query()
    opt.close()
