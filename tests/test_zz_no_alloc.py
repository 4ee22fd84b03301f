"""The argmax entry point that allocates nothing (et_argmax_noalloc), through
the C ABI: its results equal et_argmax_*'s with a workspace (the existing
entry point whose split path it shares), bit for bit, on calls in a row --
each second call smaller than the first, so a stale key or counter left in
the library's scratch array would show -- for every storage type, on shapes
that take the split path (fewer than 1024 rows) and shapes that do not, with
planted ties, NaN rows, all -inf rows and +-0 maxima.  Also checked against
the oracle.  Runs alone in a fresh process and after the other tests."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import assert_bits, dev, host

pytestmark = pytest.mark.gpu

CODE = {"f32": 0, "bf16": 1, "f16": 2}


@pytest.fixture(scope="module")
def et():
    import elementwise_transformer_amd as m
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return m


def _rows(rows, n, key):
    g = np.random.default_rng([5151, rows, n, key])
    x = np.round(g.standard_normal((rows, n)) * 8).astype(np.float32)   # many exact ties
    if rows >= 5 and n >= 4:
        x[1, :] = np.nan
        x[2, :] = -np.inf
        x[3, :] = -1.0
        x[3, n // 3] = -0.0
        x[3, n - 2] = 0.0
        x[4, n - 1] = np.inf
        x[4, n // 2] = np.inf
    return x


def _noalloc(et, xt, dt):
    rows, n = xt.shape
    out = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    rc = et.lib.et_argmax_noalloc(CODE[dt], ctypes.c_void_p(xt.data_ptr()), rows, n,
                                  ctypes.c_void_p(out.data_ptr()),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, f"et_argmax_noalloc returned {rc}"
    return host(out)


PAIRS = [((7, 128256), (3, 50000)),        # both split
         ((200, 40000), (5, 17000)),       # both split, the second far smaller
         ((1100, 50000), (6, 128256)),     # one workgroup per row, then split
         ((1, 128256), (1, 2049)),         # one row: split, then a single chunk
         ((9, 300), (2, 5))]               # short rows: no split


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("pair", PAIRS)
def test_noalloc_matches_workspace_entry(et, orc, dt, pair):
    for k, (rows, n) in enumerate(pair):
        x = wl.store(_rows(rows, n, k), dt)
        xt = dev(x)
        ref = host(et.argmax(xt))                      # et_argmax_* with a workspace
        got = _noalloc(et, xt, dt)
        assert_bits(got, ref, f"{dt} {rows}x{n} call {k}")
        assert_bits(got, orc.argmax(x), f"{dt} {rows}x{n} call {k} vs oracle")


def test_noalloc_repeated_calls_and_streams(et):
    """Many calls back to back on one stream, then on a second stream after
    the first is drained: every result equals the workspace entry point's."""
    shapes = [(7, 128256), (3, 50000), (1023, 20000), (1, 128256), (4, 70000)] * 3
    xs = [dev(_rows(r, n, 10 + i)) for i, (r, n) in enumerate(shapes)]
    refs = [host(et.argmax(x)) for x in xs]
    outs = [_noalloc(et, x, "f32") for x in xs]
    for i, (a, b) in enumerate(zip(outs, refs)):
        assert_bits(a, b, f"call {i} {shapes[i]}")
    torch.cuda.synchronize()
    s2 = torch.cuda.Stream()
    with torch.cuda.stream(s2):
        outs2 = [_noalloc(et, x, "f32") for x in xs[:5]]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(outs2, refs[:5])):
        assert_bits(a, b, f"second stream call {i}")


def test_noalloc_degenerate_and_bad_arguments(et):
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = torch.full((3,), 5, dtype=torch.int32, device="cuda")
    x = torch.empty((3, 0), device="cuda")
    rc = et.lib.et_argmax_noalloc(0, ctypes.c_void_p(x.data_ptr()), 3, 0,
                                  ctypes.c_void_p(out.data_ptr()), s)
    assert rc == 0 and host(out).tolist() == [-1, -1, -1]
    y = torch.zeros((2, 8), device="cuda")
    for code in (-1, 3):
        assert et.lib.et_argmax_noalloc(code, ctypes.c_void_p(y.data_ptr()), 2, 8,
                                        ctypes.c_void_p(out.data_ptr()), s) == 3
    assert et.lib.et_argmax_noalloc(0, ctypes.c_void_p(y.data_ptr()), -1, 8,
                                    ctypes.c_void_p(out.data_ptr()), s) == 2
    assert et.lib.et_argmax_noalloc(0, None, 2, 8, ctypes.c_void_p(out.data_ptr()), s) == 1
    assert et.lib.et_argmax_noalloc(0, ctypes.c_void_p(y.data_ptr()), 2, 8, None, s) == 1
    assert et.lib.et_argmax_noalloc(0, ctypes.c_void_p(y.data_ptr()), 0, 8, None, s) == 0
