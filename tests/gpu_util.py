"""Helpers for the GPU parity tests: moving storage-form numpy arrays to and
from the device, and the tolerance checks of the parity bar.

Tolerances (written out here, used by every parity test):
  EXACT     equal bits; NaN compared by class (embedding, add, argmax,
            fused h, RoPE pass-through entries).
  F32_REL   |got - y| <= 1e-6 |y| + 2^-140, y the oracle's unrounded f64
            value (RMSNorm, SiLU-mul in f32); where y is infinite or at least
            2^128 - 2^103 (f32 rounds it to infinity), got is that infinity.
  BF16_ULP  at most 1 ulp of the storage type (bf16 or f16) from the
            oracle's correctly rounded value, with +0 == -0 (RMSNorm,
            SiLU-mul, normalised tails in 2-byte storage).  For f16 this is
            tighter than the 1e-3 the op spec gives for F16.
  PAIR      RoPE outputs: error relative to the rotated pair's length,
            |got - y| <= 1e-6 * |(y_a, y_b)| in f32 (|(y_a, y_b)| = mu |(a, b)|,
            since rotation keeps the length); in bf16 or f16 either 1 ulp or
            |got - y| <= 2^-16 |(y_a, y_b)|.  Per-element relative error is
            unbounded under cancellation in a cos - b sin, the pair-relative
            one is not.
"""
from __future__ import annotations

import numpy as np
import torch

import functools

F32_REL = 1e-6
F32_FLOOR = 2.0 ** -140
BF16_PAIR = 2.0 ** -16


def _quiet(fn):
    """Run a check with numpy's invalid/overflow warnings off: with special
    values in the data, the tolerance arithmetic meets inf - inf and the
    like; NaN positions and infinities are compared on their own."""
    @functools.wraps(fn)
    def wrapped(*args, **kwargs):
        with np.errstate(invalid="ignore", over="ignore"):
            return fn(*args, **kwargs)
    return wrapped


def dev(a: np.ndarray) -> torch.Tensor:
    """Storage-form numpy (float32, float16, uint16 bf16 bits, int32) -> cuda."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """cuda tensor -> storage-form numpy."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def widen(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _isnan(a: np.ndarray) -> np.ndarray:
    return np.isnan(widen(a))


def assert_bits(got: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    gn, rn = _isnan(got), _isnan(ref)
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ ({gn.sum()} vs {rn.sum()})"
    g = got[~gn].view(np.uint16 if got.dtype.itemsize == 2 else np.uint32)
    r = ref[~rn].view(np.uint16 if ref.dtype.itemsize == 2 else np.uint32)
    bad = np.flatnonzero(g != r)
    assert bad.size == 0, f"{what}: {bad.size} elements differ in bits, first at {bad[:5]}"


F32_OVERFLOW = 2.0 ** 128 - 2.0 ** 103   # round-to-nearest f32 gives +-inf from here on


@_quiet
def assert_f32_rel(got: np.ndarray, y64: np.ndarray, what: str = "", rel: float = F32_REL,
                   abs_extra=None) -> None:
    """F32_REL; where y is infinite, or rounds to infinity in f32, got must be
    that infinity.  abs_extra (per element) widens the absolute floor: a
    product whose other factor went through an f32 subnormal carries that
    factor's rounding, up to 2^-150, times the other factor."""
    assert got.dtype == np.float32 and got.shape == y64.shape, what
    g = got.astype(np.float64)
    gn, rn = np.isnan(g), np.isnan(y64)
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ"
    with np.errstate(invalid="ignore"):
        big = ~rn & (np.abs(y64) >= F32_OVERFLOW)
    assert np.array_equal(g[big], np.copysign(np.inf, y64[big])), f"{what}: infinities differ"
    fin = ~rn & ~big
    err = np.abs(g[fin] - y64[fin])
    lim = rel * np.abs(y64[fin]) + F32_FLOOR
    if abs_extra is not None:
        lim = lim + np.broadcast_to(abs_extra, y64.shape)[fin]
    bad = np.flatnonzero(~(err <= lim))
    if bad.size:
        i = bad[np.argmax(err[bad] / lim[bad])]
        raise AssertionError(f"{what}: {bad.size} elements over 1e-6 rel; worst got={g[fin][i]!r} "
                             f"ref={y64[fin][i]!r} rel={err[i] / max(abs(y64[fin][i]), 1e-300):.3g}")


def bits16(a: np.ndarray) -> np.ndarray:
    """The 16-bit patterns of bf16 (uint16) or f16 (float16) storage."""
    return a.view(np.uint16) if a.dtype == np.float16 else a


def ulp16(v: np.ndarray, dtype) -> np.ndarray:
    """One ulp of the 2-byte storage type at each |v| (bf16: 8 significant
    bits, subnormal spacing 2^-133; f16: 11 bits, spacing 2^-24 below 2^-14)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    if np.dtype(dtype) == np.float16:
        return np.where(a >= 2.0 ** -14, 2.0 ** (e - 10), 2.0 ** -24)
    return np.where(a >= 2.0 ** -126, 2.0 ** (e - 7), 2.0 ** -133)


def bf16_key(bits: np.ndarray) -> np.ndarray:
    """Integer line of 2-byte float values (bf16 bits or float16): adjacent
    values differ by 1, +0 == -0."""
    b = bits16(bits).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def assert_bf16_ulp(got: np.ndarray, ref: np.ndarray, what: str = "", ulps: int = 1) -> None:
    """got, ref: bf16 bits or float16; ref is the oracle's correctly rounded
    output."""
    assert got.dtype == ref.dtype and got.dtype.itemsize == 2 and got.shape == ref.shape, what
    gn, rn = _isnan(got), _isnan(ref)
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ"
    d = np.abs(bf16_key(got[~gn]) - bf16_key(ref[~rn]))
    bad = np.flatnonzero(d > ulps)
    assert bad.size == 0, f"{what}: {bad.size} elements over {ulps} ulp (max {d.max()})"


def assert_close(got: np.ndarray, y64: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    """F32_REL for f32 storage, BF16_ULP for bf16 and f16 storage."""
    if got.dtype == np.float32:
        assert_f32_rel(got, y64, what)
    else:
        assert_bf16_ulp(got, ref, what)


def pair_norms(y64: np.ndarray, r: int, layout: int) -> np.ndarray:
    """|(y_a, y_b)| for every rotated entry of [..., D] (NaN elsewhere)."""
    out = np.full(y64.shape, np.nan)
    half = r // 2
    if half == 0:
        return out
    if layout == 0:
        a, b = y64[..., :half], y64[..., half:r]
        n = np.hypot(a, b)
        out[..., :half] = n
        out[..., half:r] = n
    else:
        a, b = y64[..., 0:r:2], y64[..., 1:r:2]
        n = np.hypot(a, b)
        out[..., 0:r:2] = n
        out[..., 1:r:2] = n
    return out


@_quiet
def assert_pair(got: np.ndarray, y64: np.ndarray, ref: np.ndarray, r: int, layout: int,
                what: str = "") -> None:
    """PAIR tolerance on the first r entries of each head row."""
    pn = pair_norms(y64, r, layout)[..., :r]
    g = widen(got[..., :r])
    y = y64[..., :r]
    err = np.abs(g - y)
    if got.dtype == np.float32:
        bad = np.flatnonzero(~(err <= F32_REL * pn + F32_FLOOR))
        if bad.size:
            i = bad[np.argmax((err / np.maximum(pn, 1e-300)).ravel()[bad])]
            raise AssertionError(f"{what}: {bad.size} rotated entries over 1e-6 of the pair length; "
                                 f"worst err/len={(err.ravel()[i] / pn.ravel()[i]):.3g}")
    else:
        ud = np.abs(bf16_key(got[..., :r]) - bf16_key(ref[..., :r]))
        bad = np.flatnonzero(~((ud <= 1) | (err <= BF16_PAIR * pn)))
        assert bad.size == 0, f"{what}: {bad.size} rotated 2-byte entries over 1 ulp and 2^-16 |pair|"


U = 2.0 ** -24


@_quiet
def check_softmax(got, x_store, t, y, y64, what=""):
    """Softmax bound: f32 derived relative bound, 2-byte 1 ulp; results
    below 2^-126 may come out as 0 (see the softmax tests)."""
    if got.dtype == np.float32:
        z = widen(x_store) / np.float64(np.float32(t))
        with np.errstate(invalid="ignore"):
            m = np.max(z, axis=-1, keepdims=True)
            tol = U * (2 * np.abs(z) + 3 * np.abs(m) + 3 * np.abs(z - m) + 128.0)
        g = got.astype(np.float64)
        gn, rn = np.isnan(g), np.isnan(y64)
        assert np.array_equal(gn, rn), f"{what}: NaN positions differ"
        fin = ~rn
        err = np.abs(g[fin] - y64[fin])
        # an exact 0 (the exponential of -inf) must come out as 0 (+ the floor)
        with np.errstate(invalid="ignore"):
            lim = np.where(y64[fin] == 0, 0.0, tol[fin] * np.abs(y64[fin])) + 2.0 ** -140
        flushed = (np.abs(y64[fin]) < 2.0 ** -126) & (g[fin] == 0)
        lim = np.where(flushed, np.inf, lim)
        bad = np.flatnonzero(~(err <= lim))
        if bad.size:
            i = bad[np.argmax(err[bad] / lim[bad])]
            raise AssertionError(f"{what}: {bad.size} over tolerance; worst got={g[fin][i]!r} "
                                 f"ref={y64[fin][i]!r} rel={err[i] / max(abs(y64[fin][i]), 1e-300):.3g} "
                                 f"tol={tol[fin][i]:.3g}")
    else:
        flushed = (np.abs(y64) < 2.0 ** -126) & (got == 0)
        g = np.where(flushed, y, got)
        assert_bf16_ulp(g, y, what)


@_quiet
def check_layernorm(got, xs, gs, bs, eps, y, y64, what=""):
    """LayerNorm absolute bound of the f32 arithmetic, plus one ulp in 2-byte
    storage (see the LayerNorm tests)."""
    x = widen(xs)
    g = widen(gs)
    b = np.zeros_like(g) if bs is None else widen(bs)
    mu = x.mean(axis=1, keepdims=True)
    c = x - mu
    inv = 1.0 / np.sqrt((c * c).mean(axis=1, keepdims=True) + float(np.float32(eps)))
    tol = U * inv * np.abs(g) * (np.abs(x) + 64 * np.abs(x).mean(axis=1, keepdims=True) + 64 * np.abs(c)) \
        + 2 * U * (np.abs(b) + np.abs(y64)) + 2.0 ** -140
    if got.dtype != np.float32:
        tol = tol + ulp16(y64, got.dtype)
    gw = widen(got)
    gn, rn = np.isnan(gw), np.isnan(y64)
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ"
    err = np.abs(gw - y64)
    bad = np.flatnonzero(~(err[~rn] <= tol[~rn]))
    if bad.size:
        i = bad[np.argmax((err[~rn] / tol[~rn])[bad])]
        raise AssertionError(f"{what}: {bad.size} over tolerance; worst got={gw[~rn][i]!r} "
                             f"ref={y64[~rn][i]!r} tol={tol[~rn][i]:.3g}")


@_quiet
def check_geglu(got, gate_s, form, y, y64, what="", abs_extra=None):
    """GeGLU: f32 relative bound of the form's arithmetic, 2-byte 1 ulp (see
    the GeGLU tests)."""
    if got.dtype != np.float32:
        assert_bf16_ulp(got, y, what)
        return
    x = widen(gate_s)
    with np.errstate(over="ignore", invalid="ignore"):
        if form == 0:
            rel = U * (2 * x * x + 64)
        else:
            v = 1.5957691216057308 * (x + 0.044715 * x ** 3)
            rel = U * (3 * np.abs(v) + 64)
    g = got.astype(np.float64)
    gn, rn = np.isnan(g), np.isnan(y64)
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ"
    with np.errstate(invalid="ignore"):
        fin = ~rn & (np.abs(y64) < F32_OVERFLOW)       # at or past it f32 gives an infinity
    assert np.array_equal(g[~rn & ~fin], np.copysign(np.inf, y64[~rn & ~fin])), f"{what}: infinities differ"
    err = np.abs(g[fin] - y64[fin])
    lim = rel[fin] * np.abs(y64[fin]) + 2.0 ** -140
    if abs_extra is not None:
        lim = lim + np.broadcast_to(abs_extra, y64.shape)[fin]
    bad = np.flatnonzero(~(err <= lim))
    if bad.size:
        i = bad[np.argmax(err[bad] / lim[bad])]
        raise AssertionError(f"{what}: {bad.size} over tolerance; worst got={g[fin][i]!r} "
                             f"ref={y64[fin][i]!r} x={x[fin][i]!r}")
