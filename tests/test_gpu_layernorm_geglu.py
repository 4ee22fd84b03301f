"""GPU parity of LayerNorm and the GELU-gated multiply (GeGLU) against the CPU
oracle, through the C ABI.

Tolerances, derived from the kernels' f32 arithmetic (u = 2^-24); the pages
give none for these ops:
  LayerNorm f32  |got - y| <= u inv |g| (|x| + 64 mean|x| + 64 |x - mu|)
                              + 2u (|b| + |y|) + 2^-140,
        inv = 1/sqrt(var + eps).  The mean carries at most 32 sequential
        additions per thread, a 6-level butterfly and 16 wave partials
        (< 64 u mean|x| absolute); x - mu adds u |x|; the variance, its square
        root and reciprocal < 64 u relative; the gain, bias and output
        roundings 2u.  The bound is absolute per element, because x - mu and
        + b cancel.
  LayerNorm bf16, f16  |got - y| <= (the f32 bound) + one ulp of y in the
        storage type.
  GeGLU f32  erf form:  |got - y| <= u (2 x^2 + 64) |y| + 2^-140: the
        argument -x/sqrt(2) carries 1.5 u, which erfc magnifies by up to
        2 z^2 = x^2 in the lower tail, plus the erfc fit (fractional error
        below 1.2e-7, 2u) and three products.
        tanh form: u (3 |v| + 64) |y| + 2^-140, v = -2u(x) the exponent,
        carrying 3 u (its polynomial), which exp turns into a relative error
        of up to 3 |v| u.
  GeGLU bf16, f16  1 ulp of the oracle's correctly rounded value.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import assert_bits, check_geglu, check_layernorm, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def et():
    import elementwise_transformer_amd as m
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return m


def _rng(*key):
    return np.random.default_rng([4444, *key])


def _misaligned(t):
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    v = flat[1:1 + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0
    return v


# ------------------------------------------------------------- LayerNorm

LN_SHAPES = [(1, 1), (3, 3), (5, 7), (4, 64), (33, 100), (7, 1000), (9, 4096), (6, 4100), (3, 8192),
             (2, 14336), (2, 40000), (2, 70001)]


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", LN_SHAPES)
def test_layernorm_matches_oracle(et, orc, dt, shape):
    rows, d = shape
    g = _rng(rows, d, 1)
    xs = wl.store((g.standard_normal(shape) * 2 + 0.5).astype(np.float32), dt)
    gs = wl.store(g.uniform(0.5, 1.5, d).astype(np.float32), dt)
    bs = wl.store(g.standard_normal(d).astype(np.float32), dt)
    for b in (bs, None):
        y, y64 = orc.layernorm(xs, gs, b, 1e-5)
        got = host(et.layernorm(dev(xs), dev(gs), None if b is None else dev(b), 1e-5))
        check_layernorm(got, xs, gs, b, 1e-5, y, y64, f"{dt} {shape} bias={b is not None}")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [7, 1000, 4100, 40003])
def test_layernorm_scalar_path_and_in_place(et, orc, dt, d):
    g = _rng(d, 2)
    xs = wl.store((g.standard_normal((3, d)) * 3).astype(np.float32), dt)
    gs = wl.store(g.uniform(0.5, 1.5, d).astype(np.float32), dt)
    bs = wl.store(g.standard_normal(d).astype(np.float32), dt)
    y, y64 = orc.layernorm(xs, gs, bs, 1e-6)
    got = host(et.layernorm(_misaligned(dev(xs)), dev(gs), dev(bs), 1e-6))
    check_layernorm(got, xs, gs, bs, 1e-6, y, y64, f"{dt} d={d} misaligned")
    xd = dev(xs)
    ref = host(et.layernorm(xd, dev(gs), dev(bs), 1e-6))
    et.layernorm(xd, dev(gs), dev(bs), 1e-6, out=xd)
    assert_bits(host(xd), ref, f"{dt} d={d} in place")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [64, 4096, 8192, 40000])
def test_layernorm_batch_invariance_and_constant_rows(et, dt, d):
    rows = 64 if d <= 4096 else 9
    g = _rng(d, 3)
    x = (g.standard_normal((rows, d)) * 2).astype(np.float32)
    x[1, :] = 1.75                                   # constant row: y is the bias
    xs = wl.store(x, dt)
    gs = wl.store(g.uniform(0.5, 1.5, d).astype(np.float32), dt)
    bs = wl.store(g.standard_normal(d).astype(np.float32), dt)
    full = host(et.layernorm(dev(xs), dev(gs), dev(bs), 1e-5))
    for r in (0, 1, rows - 1):
        one = host(et.layernorm(dev(np.ascontiguousarray(xs[r:r + 1])), dev(gs), dev(bs), 1e-5))
        assert_bits(one[0], full[r], f"{dt} d={d} row {r}")
    assert_bits(full[1], bs, f"{dt} d={d} constant row")


def test_layernorm_prefill_full_size(et, orc):
    """LayerNorm at the prefill size it is timed at, [4096, 4096] bf16 with
    gain and bias: sampled rows against the oracle."""
    g = np.random.default_rng([1002, 40])
    xs = wl.store(g.standard_normal((4096, 4096)).astype(np.float32), "bf16")
    gs = wl.store(g.uniform(0.5, 1.5, 4096).astype(np.float32), "bf16")
    bs = wl.store(g.standard_normal(4096).astype(np.float32), "bf16")
    got = host(et.layernorm(dev(xs), dev(gs), dev(bs), 1e-5))
    rows = [0, 1, 2047, 4095]
    sub = np.ascontiguousarray(xs[rows])
    y, y64 = orc.layernorm(sub, gs, bs, 1e-5)
    check_layernorm(got[rows], sub, gs, bs, 1e-5, y, y64, "prefill layernorm")


# ------------------------------------------------------------------ GeGLU

GEGLU_N = [1, 7, 100, 4099, (1 << 20) + 5]


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("form", [0, 1])
@pytest.mark.parametrize("n", GEGLU_N)
def test_geglu_matches_oracle(et, orc, dt, form, n):
    g = _rng(n, form, 4)
    gate = (g.standard_normal(n) * 2).astype(np.float32)
    if n >= 8:
        gate[:8] = [0.0, -0.0, 1e4, -1e4, 30.0, -30.0, 8.0, -8.0]
    if n >= 24:
        # the tail where x Phi(x) u is an f32 (and bf16) subnormal
        gate[8:24] = -np.linspace(12.9, 16.2, 16)
    up = g.standard_normal(n).astype(np.float32)
    gs, us = wl.store(gate, dt), wl.store(up, dt)
    y, y64 = orc.geglu(gs, us, form)
    got = host(et.geglu(dev(gs), dev(us), form))
    check_geglu(got, gs, form, y, y64, f"{dt} form={form} n={n}")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("form", [0, 1])
def test_geglu_large_up_and_deep_tail(et, orc, dt, form):
    """Gates from -40 to 0, and of magnitude up to the f32 limit, against ups
    near that limit and far below it: no intermediate may overflow where the
    product does not (x Phi(x) u for x = -4.46, u = 3e38 is -5.6e33; for x =
    -3e38 it is far below the smallest subnormal, a signed zero), and a GELU
    value below the f32 normal range still gives its product with a large up
    in full precision."""
    huge = [-1e20, -1e30, -2.0 ** 100, -2.0 ** 101, -1e37, -3e38, -3.4028235e38, 1e30, 3e38]
    gates = np.concatenate([-np.linspace(0.0, 40.0, 81), [-1e-3, -0.5, -4.456161, -13.3, -15.9], huge])
    ups = np.array([3e38, -3e38, 1e30, -1e30, 1.0, 1e-30], np.float64)
    gg, uu = np.meshgrid(gates, ups)
    gs, us = wl.store(gg.ravel().astype(np.float32), dt), wl.store(uu.ravel().astype(np.float32), dt)
    y, y64 = orc.geglu(gs, us, form)
    check_geglu(host(et.geglu(dev(gs), dev(us), form)), gs, form, y, y64, f"{dt} form={form} large up")
    g2 = _misaligned(dev(gs))
    check_geglu(host(et.geglu(g2, _misaligned(dev(us)), form)), gs, form, y, y64, f"{dt} form={form} scalar")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("form", [0, 1])
def test_geglu_special_values_in_place_and_scalar(et, orc, dt, form):
    x = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1.0, -1.0, 5.0] * 13, np.float32)
    u = np.array([1.0, 2.0, 0.5, np.nan, 3.0, -1.0, 1.0, np.inf] * 13, np.float32)
    gs, us = wl.store(x, dt), wl.store(u, dt)
    y, y64 = orc.geglu(gs, us, form)
    got = host(et.geglu(dev(gs), dev(us), form))
    check_geglu(got, gs, form, y, y64, f"{dt} form={form} special")
    g = (np.random.default_rng([4444, 5, form]).standard_normal(1001) * 2).astype(np.float32)
    gs2, us2 = wl.store(g, dt), wl.store(g[::-1].copy(), dt)
    y2, y64b = orc.geglu(gs2, us2, form)
    got2 = host(et.geglu(_misaligned(dev(gs2)), _misaligned(dev(us2)), form))
    check_geglu(got2, gs2, form, y2, y64b, f"{dt} form={form} misaligned")
    gd, ud = dev(gs2), dev(us2)
    ref = host(et.geglu(gd, ud, form))
    et.geglu(gd, ud, form, out=gd)
    assert_bits(host(gd), ref, f"{dt} form={form} in place (gate)")
    gd = dev(gs2)
    et.geglu(gd, ud, form, out=ud)
    assert_bits(host(ud), ref, f"{dt} form={form} in place (up)")


def test_geglu_prefill_full_size(et, orc):
    """GeGLU at the FFN size it is timed at, [4096, 14336] bf16, both forms:
    sampled slices against the oracle."""
    g = np.random.default_rng([1002, 41])
    gate = wl.store(g.standard_normal((4096, 14336)).astype(np.float32), "bf16")
    up = wl.store(g.standard_normal((4096, 14336)).astype(np.float32), "bf16")
    gd, ud = dev(gate), dev(up)
    for form in (0, 1):
        got = host(et.geglu(gd, ud, form))
        for r in (0, 2048, 4095):
            y, y64 = orc.geglu(np.ascontiguousarray(gate[r]), np.ascontiguousarray(up[r]), form)
            check_geglu(got[r], gate[r], form, y, y64, f"prefill geglu form={form} row {r}")
