"""The plain-stream probe the benchmark measures the kernels against
(probe/libet_probe.so, built apart from the library): each stream shape reads
and writes what it says, in both store policies and both grid shapes (one
workgroup per tile, or a persistent grid stepping through the buffer), so
the ceiling it reports is the rate of real loads and stores of data.  Expected values are written out here from the probe's
stated outputs (XOR and sum of the 16-byte words read, per 32-bit lane)."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def probe():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import elementwise_transformer_amd  # noqa: F401  (same runtime as the library)
    lib = ctypes.CDLL(os.path.join(ROOT, "probe", "libet_probe.so"))
    f = lib.et_probe_stream
    vp = ctypes.c_void_p
    f.argtypes = [vp, vp, vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, vp]
    f.restype = ctypes.c_int
    return f


@pytest.mark.parametrize("nbytes", [16, 16 * 1000 + 16 * 37, 32 << 20])
@pytest.mark.parametrize("u", [4, 8])
@pytest.mark.parametrize("dev_scope", [0, 1])
@pytest.mark.parametrize("persist", [0, 3, 512])
def test_stream_probe_outputs(probe, nbytes, u, dev_scope, persist):
    g = np.random.default_rng([7070, nbytes, u])
    words = nbytes // 4
    a = g.integers(0, 2 ** 32, words, dtype=np.uint64).astype(np.uint32)
    b = g.integers(0, 2 ** 32, words, dtype=np.uint64).astype(np.uint32)
    at = torch.from_numpy(a.view(np.int32)).cuda()
    bt = torch.from_numpy(b.view(np.int32)).cuda()
    s = torch.cuda.current_stream().cuda_stream

    def run(nr, nw):
        y = torch.full((words,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
        h = torch.full((words,), 0x3C3C3C3C, dtype=torch.int32, device="cuda")
        assert probe(at.data_ptr(), bt.data_ptr(), y.data_ptr(), h.data_ptr(), nbytes, nr, nw, u,
                     dev_scope, persist, s) == 0
        torch.cuda.synchronize()
        return y.cpu().numpy().view(np.uint32), h.cpu().numpy().view(np.uint32)

    pattern = np.tile(np.array([0x11, 0x22, 0x33, 0x44], np.uint32), words // 4)
    y, h = run(2, 2)
    assert np.array_equal(y, a ^ b) and np.array_equal(h, a + b)
    y, h = run(2, 1)
    assert np.array_equal(y, a ^ b) and np.all(h == 0x3C3C3C3C)
    y, _ = run(1, 1)
    assert np.array_equal(y, a ^ pattern)
    y, _ = run(1, 0)
    assert np.all(y == 0x5A5A5A5A)                     # a pure read stores nothing for real data
    y, _ = run(0, 1)
    i = np.arange(words // 4, dtype=np.uint64)
    lane = np.stack([i.astype(np.uint32), np.full_like(i, 0x5bd1e995, dtype=np.uint32),
                     (i >> 7).astype(np.uint32), np.full_like(i, 0x1b873593, dtype=np.uint32)], axis=1)
    assert np.array_equal(y, (lane ^ np.array([0x11, 0x22, 0x33, 0x44], np.uint32)).ravel())


def test_probe_hold_keeps_the_stream_busy(probe):
    """The hold kernel occupies the stream for about the time asked (at least
    it, and well under the next power of ten) and then lets the work queued
    behind it run."""
    lib = ctypes.CDLL(os.path.join(ROOT, "probe", "libet_probe.so"))
    hold = lib.et_probe_hold
    hold.argtypes = [ctypes.c_int64, ctypes.c_void_p]
    hold.restype = ctypes.c_int
    s = torch.cuda.current_stream()
    x = torch.zeros(1024, device="cuda")
    # one untimed round: the first launch of each kernel loads its code object
    assert hold(1, ctypes.c_void_p(s.cuda_stream)) == 0
    x += 1.0
    torch.cuda.synchronize()
    for us in (200, 3000):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        assert hold(us, ctypes.c_void_p(s.cuda_stream)) == 0
        x += 1.0
        b.record(s)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        assert us * 1e-3 * 0.98 <= ms < us * 1e-2, (us, ms)
    assert float(x[0]) == 3.0
