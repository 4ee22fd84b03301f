"""Pins that tie the CPU oracle to what the pages and the mathematics fix.

Every pin takes an ``oracle.Oracle`` (the real build, or a mutant build in
``test_oracle_mutants.py``) and raises ``AssertionError`` when the oracle
disagrees.  Sources are the two pages the ops come from:

  [OPS]  "Operations" (op spec): RmsNorm, Rope, Silu/SwiGlu, QK-norm,
         Sampling/Greedy, Fused ops.
  [ELT]  "Elementwise kernels in C: RMSNorm, RoPE, SiLU-mul, embedding, add,
         argmax": sections 2.1-2.4 (definitions), 3 (worked examples, stored in
         ``golden/worked_examples.txt``), 4 (test catalog), 5 (pitfalls).

A pin never compares the oracle with itself through the same formula: it
uses printed values, closed forms, invariants, library routines (numpy,
torch CPU casts and adds) or the brute-force evaluations in ``brute.py``.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction
from typing import Callable, Dict

import numpy as np

try:
    from . import brute
except ImportError:  # imported as a top-level module
    import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "worked_examples.txt")


def _golden():
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield json.loads(line)


def _f32(a):
    return np.array([float(v) for v in a], dtype=np.float32)


def _bf16(a: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _wide(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _pair_index(layout, r, i):
    return (i, i + r // 2) if layout == 0 else (2 * i, 2 * i + 1)


# ----------------------------------------------------------- worked examples

def pin_hand_example(orc):
    """[ELT] 3 and 4 (hand_example, rmsnorm_eps_is_inside_the_root,
    argmax_ties_nan_and_empty): printed values."""
    for case in _golden():
        op = case["op"]
        if op == "rmsnorm":
            x = _f32(case["x"])[None, :]
            y, y64 = orc.rmsnorm(x, _f32(case["w"]), case["eps"])
            exp = np.array(case["expect"])
            assert np.all(np.isfinite(y64)), case["cite"]
            assert np.max(np.abs(y64[0] - exp)) <= case["tol"], (case["cite"], y64)
            assert np.max(np.abs(y[0] - exp)) <= case["tol"] + 1e-7, (case["cite"], y)
        elif op == "rope":
            x = _f32(case["x"]).reshape(1, 1, case["D"])
            out, y64 = orc.rope(x, np.array([case["pos"]]), case["r"], _f32(case["inv_freq"]),
                                case["mu"], case["layout"])
            exp = np.array(case["expect"])
            assert np.max(np.abs(y64.ravel() - exp)) <= case["tol"], (case["cite"], y64)
        elif op == "silu_mul":
            y, y64 = orc.silu_mul(_f32(case["gate"]), _f32(case["up"]))
            assert np.max(np.abs(y64 - np.array(case["expect"]))) <= case["tol"], case["cite"]
        elif op == "argmax":
            x = _f32(case["x"]).reshape(1, -1)
            got = int(orc.argmax(x)[0])
            assert got == case["expect"], (case["cite"], got)
        else:
            raise AssertionError(f"unknown golden op {op}")


# ---------------------------------------------------------------- bf16 RNE

def pin_bf16_rounding(orc):
    """Rounding to bf16: agrees with torch's f32->bf16 cast on f32 values and
    with an exact neighbour search (brute.bf16_bits_exact) on f64 values that
    f32 cannot hold (no double rounding)."""
    g = np.random.default_rng(7)
    vals = np.concatenate([
        g.standard_normal(2000).astype(np.float32) * np.float32(10.0) ** g.integers(-30, 30, 2000).astype(np.float32),
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2 ** -130, 2 ** -133 * 1.5,
                  2 ** -149, 3.3895313e38, 3.3961775e38, -3.40282347e38, 0.0, -0.0], dtype=np.float32),
    ])
    vals = vals[np.isfinite(vals)]
    ref = _bf16(vals)
    for v, rb in zip(vals, ref):
        got = orc.bf16_from_f64(float(v))
        assert got == int(rb), (float(v), hex(got), hex(int(rb)))
    for v in [1.0 + 2 ** -8 + 2 ** -40, 1.0 + 2 ** -8 - 2 ** -40, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
              -(2.0 + 2 ** -7 + 2 ** -45), 2 ** -135 * 1.5, 2 ** -134, 2 ** 128 - 2 ** 119,
              2 ** 128 - 2 ** 120, 12345.6789, -1e-39]:
        assert orc.bf16_from_f64(v) == brute.bf16_bits_exact(v), (v, hex(orc.bf16_from_f64(v)))
    assert orc.bf16_from_f64(float("nan")) & 0x7FFF == 0x7FC0
    assert orc.bf16_from_f64(float("inf")) == 0x7F80
    assert orc.bf16_from_f64(-0.0) == 0x8000


# ----------------------------------------------------------------- RMSNorm

def pin_rmsnorm_eps_is_inside_the_root(orc):
    """[ELT] 2.1 and 4; [OPS] RmsNorm: eps inside the root; a zero row is 0,
    never NaN, in f32 and bf16."""
    y, y64 = orc.rmsnorm(_f32([1e-3, 1e-3])[None], _f32([1, 1]), 1e-6)
    assert abs(y64[0, 0] - 0.70710678) < 5e-5, y64       # outside the root: 0.9990
    for dt in ("f32", "bf16"):
        x = np.zeros((3, 16), np.float32)
        x[1] = 1.0
        w = np.linspace(0.5, 1.5, 16, dtype=np.float32)
        xs, ws = (x, w) if dt == "f32" else (_bf16(x), _bf16(w))
        y, y64 = orc.rmsnorm(xs, ws, 1e-5)
        assert np.all(y64[0] == 0.0) and np.all(y64[2] == 0.0)
        assert not np.any(np.isnan(y64))


def pin_rmsnorm_closed_forms(orc):
    """[OPS] RmsNorm definition: a constant row c gives c / sqrt(c^2 + eps) w;
    with eps = 0 the output is scale invariant and mean((y/w)^2) = 1."""
    for c, eps, d in [(2.0, 1e-5, 7), (0.003, 1e-6, 64), (-5.5, 0.0, 5)]:
        w = np.linspace(0.5, 1.5, d, dtype=np.float32)
        _, y64 = orc.rmsnorm(np.full((1, d), c, np.float32), w, eps)
        c = float(np.float32(c))
        expect = c / math.sqrt(c * c + float(np.float32(eps))) * w.astype(np.float64)
        assert np.allclose(y64[0], expect, rtol=1e-14, atol=0), (c, eps, d)
    g = np.random.default_rng(3)
    x = g.standard_normal((4, 33)).astype(np.float32)
    w = g.uniform(0.5, 1.5, 33).astype(np.float32)
    _, y1 = orc.rmsnorm(x, w, 0.0)
    _, y2 = orc.rmsnorm(x * np.float32(8.0), w, 0.0)
    assert np.allclose(y1, y2, rtol=1e-14, atol=0)
    assert np.allclose(np.mean((y1 / w.astype(np.float64)) ** 2, axis=1), 1.0, rtol=1e-13)


def pin_rmsnorm_brute(orc):
    """Brute force with the exact (Fraction) sum of squares on tiny rows."""
    g = np.random.default_rng(11)
    for d in (1, 2, 5, 16, 37):
        x = g.standard_normal((3, d)).astype(np.float32)
        w = g.uniform(0.5, 1.5, d).astype(np.float32)
        _, y64 = orc.rmsnorm(x, w, 1e-5)
        for r in range(3):
            ref = brute.rmsnorm_row([float(v) for v in x[r]], [float(v) for v in w], 1e-5)
            assert np.allclose(y64[r], ref, rtol=1e-13, atol=0), (d, r)


def pin_rmsnorm_rows_are_independent_and_in_place(orc):
    """[ELT] 2.1 and 4: every row alone equals the same row inside a batch of
    up to 12, bit for bit; y == x in place gives the same bits."""
    import ctypes
    g = np.random.default_rng(5)
    for dt in ("f32", "bf16"):
        x = g.standard_normal((12, 40)).astype(np.float32) * 3
        w = g.uniform(0.5, 1.5, 40).astype(np.float32)
        xs, ws = (x, w) if dt == "f32" else (_bf16(x), _bf16(w))
        for b in (1, 3, 12):
            yb, _ = orc.rmsnorm(xs[:b], ws, 1e-5)
            for r in range(b):
                y1, _ = orc.rmsnorm(xs[r:r + 1], ws, 1e-5)
                assert np.array_equal(y1[0].view(np.uint8), yb[r].view(np.uint8)), (dt, b, r)
        yb, _ = orc.rmsnorm(xs, ws, 1e-5)
        inplace = xs.copy()
        p = inplace.ctypes.data_as(ctypes.c_void_p)
        orc.lib.orc_rmsnorm(0 if dt == "f32" else 1, p, ws.ctypes.data_as(ctypes.c_void_p),
                            12, 40, ctypes.c_float(1e-5), None, p)
        assert np.array_equal(inplace.view(np.uint8), yb.view(np.uint8)), dt


def pin_add_rmsnorm_is_the_composition(orc):
    """[OPS] 10 Fused ops (FusedSkipNorm): h = x + skip exactly as the storage
    type adds (numpy f32 add, torch bf16 add), y = RmsNorm(h as stored) by
    brute force; in place (y over x, h over skip) gives the same bits."""
    import ctypes
    import torch
    g = np.random.default_rng(9)
    for dt in ("f32", "bf16"):
        x = g.standard_normal((5, 24)).astype(np.float32)
        s = (g.standard_normal((5, 24)) * 1e-2).astype(np.float32)
        w = g.uniform(0.5, 1.5, 24).astype(np.float32)
        if dt == "f32":
            xs, ss, ws = x, s, w
            h_ref = (x + s)
            hw = h_ref
        else:
            xs, ss, ws = _bf16(x), _bf16(s), _bf16(w)
            tx = torch.from_numpy(_wide(xs)).to(torch.bfloat16)
            ts = torch.from_numpy(_wide(ss)).to(torch.bfloat16)
            h_ref = (tx + ts).view(torch.int16).numpy().view(np.uint16)
            hw = _wide(h_ref)
        y, h, y64 = orc.add_rmsnorm(xs, ss, ws, 1e-5)
        assert np.array_equal(h.view(np.uint8), np.ascontiguousarray(h_ref).view(np.uint8)), dt
        wv = ws if dt == "f32" else _wide(ws)
        for r in range(5):
            ref = brute.rmsnorm_row([float(v) for v in hw[r]], [float(v) for v in wv], 1e-5)
            assert np.allclose(y64[r], ref, rtol=1e-13, atol=0), (dt, r)
        xi, si = xs.copy(), ss.copy()
        px, ps = xi.ctypes.data_as(ctypes.c_void_p), si.ctypes.data_as(ctypes.c_void_p)
        orc.lib.orc_add_rmsnorm(0 if dt == "f32" else 1, px, ps, ws.ctypes.data_as(ctypes.c_void_p),
                                5, 24, ctypes.c_float(1e-5), None, px, ps)
        assert np.array_equal(xi.view(np.uint8), y.view(np.uint8)), dt
        assert np.array_equal(si.view(np.uint8), h.view(np.uint8)), dt


# -------------------------------------------------------------------- RoPE

def pin_rope_angle_is_the_f32_product(orc):
    """[ELT] 2.2: the angle formed in f64 and rounded to f32 equals
    f32(p) * f32(w) (numpy's IEEE f32 multiply) for every |p| < 2^24."""
    g = np.random.default_rng(13)
    p = g.integers(0, 2 ** 24, 4000)
    w = np.power(1e4, -g.uniform(0, 1, 4000)).astype(np.float32)
    for pi, wi in zip(p, w):
        assert orc.rope_angle(int(pi), float(wi)) == np.float32(pi) * wi, (pi, wi)


def pin_rope_interleaved_layout_and_position_zero(orc):
    """[ELT] 4 (rope_interleaved_layout_and_position_zero) and [OPS] Rope edge
    cases: the interleaved worked example of [ELT] 3; position 0 is the
    identity rotation, bit for bit, both layouts."""
    for case in _golden():
        if case["op"] == "rope" and case["layout"] == 1:
            x = _f32(case["x"]).reshape(1, 1, case["D"])
            _, y64 = orc.rope(x, np.array([case["pos"]]), case["r"], _f32(case["inv_freq"]),
                              case["mu"], 1)
            assert np.max(np.abs(y64.ravel() - np.array(case["expect"]))) <= case["tol"], case["cite"]
    g = np.random.default_rng(17)
    for dt in ("f32", "bf16"):
        for layout in (0, 1):
            x = g.standard_normal((3, 2, 12)).astype(np.float32)
            xs = x if dt == "f32" else _bf16(x)
            out, _ = orc.rope(xs, np.zeros(3, np.int32), 8, np.array([1.0, 0.3, 0.1, 0.01, 0.5, 0.5],
                                                                      np.float32), 1.0, layout)
            assert np.array_equal(out.view(np.uint8), xs.view(np.uint8)), (dt, layout)


def pin_rope_partial_rotary_and_scaling(orc):
    """[ELT] 4 (rope_partial_rotary_and_scaling): the tail past r is untouched,
    mu = 2 doubles each pair, and [T, H, D] indexing (each head row equals the
    same row rotated alone with its token's position)."""
    g = np.random.default_rng(19)
    T, H, D, r = 4, 3, 10, 6
    inv = np.array([1.0, 0.1, 0.01, 7.0, 7.0], np.float32)     # r/2 used, rest unused
    pos = np.array([3, 0, 11, 250], np.int32)
    for dt in ("f32", "bf16"):
        for layout in (0, 1):
            x = g.standard_normal((T, H, D)).astype(np.float32)
            xs = x if dt == "f32" else _bf16(x)
            out1, y1 = orc.rope(xs, pos, r, inv, 1.0, layout)
            out2, y2 = orc.rope(xs, pos, r, inv, 2.0, layout)
            assert np.array_equal(out1[..., r:].view(np.uint8), xs[..., r:].view(np.uint8))
            assert np.array_equal(out2[..., r:].view(np.uint8), xs[..., r:].view(np.uint8))
            xw = (xs if dt == "f32" else _wide(xs)).astype(np.float64)
            assert np.array_equal(y1[..., r:], xw[..., r:]) and np.array_equal(y2[..., r:], xw[..., r:])
            assert np.allclose(y2[..., :r], 2.0 * y1[..., :r], rtol=1e-15, atol=0)
            for t in range(T):
                for h in range(H):
                    _, ys = orc.rope(np.ascontiguousarray(xs[t:t + 1, h:h + 1]), pos[t:t + 1], r, inv,
                                     1.0, layout)
                    assert np.array_equal(ys[0, 0], y1[t, h]), (dt, layout, t, h)


def pin_rope_is_a_rotation(orc):
    """[ELT] 2.2 and 4 (rope_is_a_rotation): every pair keeps its length times
    mu, for random shapes, positions and both layouts."""
    g = np.random.default_rng(23)
    for _ in range(12):
        T, H = int(g.integers(1, 5)), int(g.integers(1, 4))
        half = int(g.integers(1, 9))
        r = 2 * half
        D = r + int(g.integers(0, 5))
        layout = int(g.integers(0, 2))
        mu = float(np.float32(g.uniform(0.5, 2.0)))
        x = g.standard_normal((T, H, D)).astype(np.float32)
        pos = g.integers(0, 100000, T).astype(np.int32)
        inv = np.power(1e4, -np.arange(max(half, D // 2)) / half).astype(np.float32)
        _, y = orc.rope(x, pos, r, inv, mu, layout)
        for i in range(half):
            ia, ib = _pair_index(layout, r, i)
            n0 = np.hypot(x[..., ia].astype(np.float64), x[..., ib].astype(np.float64))
            n1 = np.hypot(y[..., ia], y[..., ib])
            assert np.allclose(n1, mu * n0, rtol=1e-13, atol=0), (T, H, D, r, layout, i)


def pin_rope_layouts_are_a_permutation(orc):
    """[ELT] 2.2: both layouts are the same rotation on a permuted vector:
    interleaved(P x) = P half(x), P sending i -> 2i and i + r/2 -> 2i + 1."""
    g = np.random.default_rng(29)
    T, H, D, r = 3, 2, 12, 8
    x = g.standard_normal((T, H, D)).astype(np.float32)
    pos = np.array([5, 77, 1234], np.int32)
    inv = np.array([1.0, 0.2, 0.03, 0.004, 9.0, 9.0], np.float32)
    perm = np.arange(D)
    for i in range(r // 2):
        perm[2 * i], perm[2 * i + 1] = i, i + r // 2        # (P x)[2i] = x[i]
    half, _ = orc.rope(x, pos, r, inv, 1.0, 0)
    inter, _ = orc.rope(np.ascontiguousarray(x[..., perm]), pos, r, inv, 1.0, 1)
    assert np.array_equal(inter.view(np.uint8), np.ascontiguousarray(half[..., perm]).view(np.uint8))


def pin_rope_brute_complex(orc):
    """Brute force: each pair as a complex number times mu e^{i theta}, with
    theta = f32(p) f32(w); both layouts, partial width, mu != 1."""
    g = np.random.default_rng(31)
    for layout in (0, 1):
        T, H, D, r = 3, 2, 14, 10
        mu = float(np.float32(1.1))
        x = g.standard_normal((T, H, D)).astype(np.float32)
        pos = np.array([0, 1, 1048575], np.int32)
        inv = np.power(np.float64(1e4), -2.0 * np.arange(D // 2) / r).astype(np.float32)
        _, y = orc.rope(x, pos, r, inv, mu, layout)
        for t in range(T):
            for h in range(H):
                ref = brute.rope_head([float(v) for v in x[t, h]], int(pos[t]), r, inv, mu, layout)
                nrm = float(np.linalg.norm(x[t, h].astype(np.float64)))
                assert np.max(np.abs(y[t, h] - np.array(ref))) <= 1e-13 * nrm, (layout, t, h)


def pin_rope_relative_position(orc):
    """[ELT] 2.2: the score of a rotated query and key depends only on the
    position difference (up to the f32 rounding of each angle)."""
    g = np.random.default_rng(37)
    D = r = 16
    q = g.standard_normal((1, 1, D)).astype(np.float32)
    k = g.standard_normal((1, 1, D)).astype(np.float32)
    inv = np.power(np.float64(1e4), -2.0 * np.arange(r // 2) / r).astype(np.float32)
    for layout in (0, 1):
        scores = []
        for pq, pk in [(5, 2), (13, 10), (103, 100), (3, 0)]:
            _, qy = orc.rope(q, np.array([pq], np.int32), r, inv, 1.0, layout)
            _, ky = orc.rope(k, np.array([pk], np.int32), r, inv, 1.0, layout)
            scores.append(float(np.dot(qy.ravel(), ky.ravel())))
        nq, nk = np.linalg.norm(q.astype(np.float64)), np.linalg.norm(k.astype(np.float64))
        assert max(scores) - min(scores) <= 1e-5 * nq * nk, (layout, scores)


# ------------------------------------------------------ fused RMSNorm+RoPE

def pin_qknorm_per_head_then_rope(orc):
    """[OPS] 5 QK-norm: RmsNorm per head over head_dim (not over heads x
    head_dim) with a [head_dim] gain, then Rope; brute force per head."""
    g = np.random.default_rng(41)
    for layout in (0, 1):
        T, H, D, r = 2, 3, 12, 8
        x = g.standard_normal((T, H, D)).astype(np.float32)
        x[:, 1] *= 50.0                       # one loud head must not leak into others
        gain = g.uniform(0.5, 1.5, D).astype(np.float32)
        pos = np.array([9, 40000], np.int32)
        inv = np.power(np.float64(5e5), -2.0 * np.arange(D // 2) / r).astype(np.float32)
        mu = float(np.float32(1.25))
        _, y = orc.rmsnorm_rope(x, gain, 1e-6, pos, r, inv, mu, layout)
        for t in range(T):
            for h in range(H):
                n = brute.rmsnorm_row([float(v) for v in x[t, h]], [float(v) for v in gain], 1e-6)
                ref = brute.rope_head(n, int(pos[t]), r, inv, mu, layout)
                assert np.allclose(y[t, h], ref, rtol=0, atol=1e-13 * max(1.0, max(map(abs, ref)))), \
                    (layout, t, h)


# ---------------------------------------------------------------- SiLU-mul

def pin_silu_mul_saturates_without_nan(orc):
    """[ELT] 2.3 and 4 (silu_mul_saturates_without_nan): g = +100 gives g u,
    g = -100 and -1e4 give -0 u (no NaN), g = 0 gives 0."""
    gate = np.array([100.0, -100.0, -1e4, 0.0, 1e4, -1e4], np.float32)
    up = np.array([3.0, 2.0, 5.0, 7.0, -2.0, -3.0], np.float32)
    for dt in ("f32", "bf16"):
        gs, us = (gate, up) if dt == "f32" else (_bf16(gate), _bf16(up))
        y, y64 = orc.silu_mul(gs, us)
        assert not np.any(np.isnan(y64))
        gw = (gs if dt == "f32" else _wide(gs)).astype(np.float64)
        uw = (us if dt == "f32" else _wide(us)).astype(np.float64)
        assert y64[0] == gw[0] * uw[0] and y64[4] == gw[4] * uw[4]
        assert y64[1] == 0.0 and math.copysign(1.0, y64[1]) < 0     # -0 * 2
        assert y64[2] == 0.0 and math.copysign(1.0, y64[2]) < 0     # -0 * 5
        assert y64[5] == 0.0 and math.copysign(1.0, y64[5]) > 0     # -0 * -3
        assert y64[3] == 0.0


def pin_silu_tanh_identity(orc):
    """silu(g) = g (1 + tanh(g/2)) / 2, an independent evaluation."""
    g = np.random.default_rng(43)
    gate = g.uniform(-30, 30, 500).astype(np.float32)
    up = g.standard_normal(500).astype(np.float32)
    _, y64 = orc.silu_mul(gate, up)
    ref = np.array([brute.silu_tanh(float(a)) * float(b) for a, b in zip(gate, up)])
    assert np.allclose(y64, ref, rtol=1e-13, atol=1e-300)


# ------------------------------------------------------- add, embedding

def pin_add_in_place(orc):
    """[ELT] 2.4 and 4 (add_in_place): y = a + b is IEEE addition in the
    storage type (numpy f32 add, torch bf16 add) and works with y == a."""
    import ctypes
    import torch
    g = np.random.default_rng(47)
    a = (g.standard_normal(999) * 10.0 ** g.integers(-3, 3, 999)).astype(np.float32)
    b = (g.standard_normal(999) * 10.0 ** g.integers(-3, 3, 999)).astype(np.float32)
    y = orc.add(a, b)
    assert np.array_equal(y.view(np.uint32), (a + b).view(np.uint32))
    ab, bb = _bf16(a), _bf16(b)
    yb = orc.add(ab, bb)
    ref = (torch.from_numpy(_wide(ab)).to(torch.bfloat16) + torch.from_numpy(_wide(bb)).to(torch.bfloat16))
    assert np.array_equal(yb, ref.view(torch.int16).numpy().view(np.uint16))
    inpl = a.copy()
    p = inpl.ctypes.data_as(ctypes.c_void_p)
    orc.lib.orc_add(0, p, b.ctypes.data_as(ctypes.c_void_p), 999, p)
    assert np.array_equal(inpl.view(np.uint32), y.view(np.uint32))


def pin_embedding_gathers_rows(orc):
    """[ELT] 2.4 and 4 (embedding_gathers_rows): repeated and out-of-order
    ids copy rows bit for bit (numpy fancy indexing); a bad id gives NaN."""
    g = np.random.default_rng(53)
    for dt in ("f32", "bf16"):
        table = g.standard_normal((9, 5)).astype(np.float32)
        ts = table if dt == "f32" else _bf16(table)
        ids = np.array([3, 3, 0, 8, 1, 3, 7, 0], np.int32)
        out = orc.embedding(ts, ids)
        assert np.array_equal(out.view(np.uint8), ts[ids].view(np.uint8)), dt
        bad = orc.embedding(ts, np.array([2, 9, -1], np.int32))
        wide = bad if dt == "f32" else _wide(bad)
        assert np.array_equal(bad[0].view(np.uint8), ts[2].view(np.uint8))
        assert np.all(np.isnan(wide[1])) and np.all(np.isnan(wide[2]))


# ------------------------------------------------------------------ argmax

def pin_argmax_ties_nan_and_empty(orc):
    """[ELT] 2.4 and 4 (argmax_ties_nan_and_empty) and [OPS] Greedy: ties to
    the lowest index, NaN skipped (also in first place), -1 when no number,
    all -inf gives 0, -0 ties +0, +inf wins."""
    nan, inf = float("nan"), float("inf")
    cases = [([1.0, 5.0, 5.0, 2.0], 1), ([nan, 1.0, 0.5], 1), ([nan] * 4, -1),
             ([-inf] * 3, 0), ([-1.0, -0.0, 0.0, -2.0], 1), ([-1.0, 0.0, -0.0], 1),
             ([1.0, inf, 3.0, inf], 1), ([nan, -inf], 1), ([3.0], 0), ([2.0, nan, 2.0], 0)]
    for dt in ("f32", "bf16"):
        for vals, expect in cases:
            x = _f32(vals)[None]
            xs = x if dt == "f32" else _bf16(x)
            assert int(orc.argmax(xs)[0]) == expect, (dt, vals)
        empty = np.zeros((3, 0), np.float32 if dt == "f32" else np.uint16)
        assert list(orc.argmax(empty)) == [-1, -1, -1]


def pin_argmax_matches_library(orc):
    """Rows with at least one number: numpy.nanargmax (first occurrence of the
    maximum) and the sorted-key brute force agree with the oracle."""
    g = np.random.default_rng(59)
    x = np.round(g.standard_normal((40, 300)) * 4).astype(np.float32)     # many ties
    x[g.random((40, 300)) < 0.05] = np.nan
    x[3, :] = np.nan
    got = orc.argmax(x)
    for r in range(40):
        if np.all(np.isnan(x[r])):
            assert got[r] == -1
        else:
            assert got[r] == np.nanargmax(x[r]), r
            assert got[r] == brute.argmax_sorted([float(v) for v in x[r]]), r
    xb = _bf16(x)
    gotb = orc.argmax(xb)
    wide = _wide(xb)
    for r in range(40):
        expect = -1 if np.all(np.isnan(wide[r])) else int(np.nanargmax(wide[r]))
        assert gotb[r] == expect, r


# ---------------------------------------------------------------- softmax

def pin_softmax_closed_forms(orc):
    """[OPS] Softmax: a constant row is uniform (1/n exactly, rounded once);
    two entries give the logistic function of their scaled difference;
    every row sums to 1."""
    for n in (1, 3, 7, 64):
        for dt in ("f32", "bf16"):
            x = np.full((2, n), 0.75, np.float32)
            xs = x if dt == "f32" else _bf16(x)
            y, y64 = orc.softmax(xs, 1.0)
            assert np.all(y64 == 1.0 / n), (n, dt)
            expect = np.float32(1.0 / n) if dt == "f32" else brute.bf16_bits_exact(Fraction(1, n))
            assert np.all(y == expect), (n, dt)
    for a, b, t in ((0.0, 1.0, 1.0), (2.5, -1.0, 0.5), (-3.0, -3.25, 4.0)):
        _, y64 = orc.softmax(_f32([a, b])[None], t)
        logistic = 0.5 * (1.0 + math.tanh((float(np.float32(a)) - float(np.float32(b))) / (2 * float(np.float32(t)))))
        assert abs(y64[0, 0] - logistic) <= 1e-15, (a, b, t)
        assert abs(y64[0, 0] + y64[0, 1] - 1.0) <= 1e-15
    g = np.random.default_rng(71)
    _, y64 = orc.softmax(g.standard_normal((5, 333)).astype(np.float32) * 3, 0.7)
    assert np.all(np.abs(y64.sum(axis=1) - 1.0) <= 1e-13)


def pin_softmax_max_is_subtracted(orc):
    """[OPS] Softmax: the max is subtracted so large logits stay finite --
    a shifted row gives the same result, and rows spanning a range wider than
    the exponential's gives 0 for the far entries, not NaN."""
    base = _f32([0.0, 1.0, 2.0])[None]
    y0, _ = orc.softmax(base, 1.0)
    for shift in (1000.0, -1000.0, 3.0e38 / 1.5):
        ys, _ = orc.softmax(base + np.float32(shift) if abs(shift) < 1e30 else _f32([shift, shift, shift])[None], 1.0)
        assert np.all(np.isfinite(ys)), shift
        if abs(shift) < 1e30:
            assert np.array_equal(ys.view(np.uint32), y0.view(np.uint32)), shift
    y, y64 = orc.softmax(_f32([-800.0, 0.0, -1.0e4])[None], 1.0)
    assert np.all(np.isfinite(y64)) and y64[0, 2] == 0.0
    assert abs(y64[0, 0] - math.exp(-800.0) / (1.0 + math.exp(-800.0))) <= 1e-320
    assert abs(y64[0, 1] - 1.0) <= 1e-15


def pin_softmax_temperature(orc):
    """[OPS] 8 Sampling / Temperature: probs = softmax(logits / t).  With t = 2
    the result equals t = 1 on the halved logits (exact in f32); a large t
    flattens the row towards uniform; brute force in 50-digit decimal."""
    g = np.random.default_rng(73)
    x = (g.standard_normal((4, 50)) * 4).astype(np.float32)
    y2, y2_64 = orc.softmax(x, 2.0)
    yh, yh_64 = orc.softmax(x * np.float32(0.5), 1.0)
    assert np.array_equal(y2.view(np.uint32), yh.view(np.uint32))
    assert np.array_equal(y2_64, yh_64)
    _, flat = orc.softmax(x, 1.0e6)
    assert np.all(np.abs(flat - 1.0 / 50) <= 1e-6)
    for t in (1.0, 0.3, 2.5):
        xs = (g.standard_normal(12) * 3).astype(np.float32)
        _, y64 = orc.softmax(xs[None], t)
        ref = brute.softmax_decimal([float(v) for v in xs], float(np.float32(t)))
        assert np.allclose(y64[0], ref, rtol=1e-14, atol=0.0), t


def pin_softmax_special_values(orc):
    """Special values follow the formula: a NaN anywhere makes the row NaN; a
    row of -inf (max -inf) or holding +inf is NaN (inf - inf); a single -inf
    among numbers gets 0; a quotient x/t beyond the f32 range is +-inf, as
    the single-precision division gives; rows are independent."""
    nan, inf = float("nan"), float("inf")
    x = _f32([1.0, 2.0, 3.0, 4.0] + [nan, 1.0, 2.0, 3.0] + [-inf] * 4 + [1.0, inf, 0.0, 2.0]
             + [0.0, -inf, 1.0, 2.0]).reshape(5, 4)
    for dt in ("f32", "bf16"):
        xs = x if dt == "f32" else _bf16(x)
        y, y64 = orc.softmax(xs, 1.0)
        assert np.all(np.isfinite(y64[0])) and abs(y64[0].sum() - 1.0) <= 1e-15
        assert np.all(np.isnan(y64[1:4])), dt
        assert y64[4, 1] == 0.0 and np.all(np.isfinite(y64[4]))
        wide = y if dt == "f32" else _wide(y)
        assert np.all(np.isnan(wide[1:4])) and wide[4, 1] == 0.0
        alone, _ = orc.softmax(np.ascontiguousarray(xs[4:5]), 1.0)
        assert np.array_equal(alone[0].view(np.uint8), y[4].view(np.uint8))
    _, y64 = orc.softmax(_f32([3.0, 4.0])[None], 1.0e-38)
    assert np.all(np.isnan(y64))
    _, y64 = orc.softmax(_f32([1.0, 2.0])[None], 1.0e-38)
    assert y64[0, 0] == 0.0 and y64[0, 1] == 1.0


def pin_softmax_matches_library(orc):
    """torch's CPU softmax in f64 on the same quotients (a library routine),
    for f32 and bf16 storage; the stored value is the f64 result rounded
    once."""
    import torch
    g = np.random.default_rng(79)
    x = (g.standard_normal((6, 1000)) * 3).astype(np.float32)
    for dt in ("f32", "bf16"):
        xs = x if dt == "f32" else _bf16(x)
        wide = xs if dt == "f32" else _wide(xs)
        t = np.float32(0.7)
        y, y64 = orc.softmax(xs, float(t))
        ref = torch.softmax(torch.from_numpy(wide.astype(np.float64)) / float(t), dim=1).numpy()
        assert np.allclose(y64, ref, rtol=1e-13, atol=1e-300)
        if dt == "f32":
            assert np.array_equal(y, ref.astype(np.float32))
        else:
            assert np.array_equal(y, _bf16(ref.astype(np.float32))) or \
                np.max(np.abs(y.astype(np.int32) - _bf16(ref.astype(np.float32)).astype(np.int32))) <= 1


# ------------------------------------------------------------ RoPE cache

def pin_rope_cache_values(orc):
    """[OPS] Rope, cos/sin cache: entry (p, i) is cos and sin of the f32 angle
    of [ELT] 2.2 rounded to f32 -- position 0 gives exactly (1, 0); against a
    decimal evaluation (pi by Machin's formula, Taylor series) for positions
    up to 2^20."""
    r = 64
    inv = np.power(np.float64(1e4), -2.0 * np.arange(r // 2) / r).astype(np.float32)
    c, s_ = orc.rope_cache(inv, 2000, r)
    assert np.all(c[0] == 1.0) and np.all(s_[0] == 0.0)
    assert np.all(np.abs(c.astype(np.float64) ** 2 + s_.astype(np.float64) ** 2 - 1.0) <= 2.0 ** -22)
    for p in (1, 7, 1999):
        for i in (0, 5, 31):
            ang = float(np.float32(np.float64(p) * np.float64(inv[i])))
            sd, cd = brute.sincos_decimal(ang)
            assert c[p, i] == np.float32(cd) and s_[p, i] == np.float32(sd), (p, i)
    big = np.array([1.0], np.float32)
    cb, sb = orc.rope_cache(big, 3, 2)
    for p in range(3):
        sd, cd = brute.sincos_decimal(float(p))
        assert cb[p, 0] == np.float32(cd) and sb[p, 0] == np.float32(sd)


def pin_rope_cached_rotation(orc):
    """The cached rotation is RoPE with (cos, sin) read instead of computed:
    with the cache built from the same angles it matches the computed oracle
    to the f32 rounding of cos and sin; a cache of quarter turns maps each
    pair (a, b) to mu (-b, a) in both layouts; a position outside the cache
    gives NaN in that token's rotated entries and leaves the rest."""
    g = np.random.default_rng(101)
    T, H, D, r = 6, 3, 16, 12
    x = g.standard_normal((T, H, D)).astype(np.float32)
    pos = np.array([0, 3, 9, 1, 9, 4], np.int32)
    inv = np.power(np.float64(500.0), -2.0 * np.arange(r // 2) / r).astype(np.float32)
    c, s_ = orc.rope_cache(inv, 10, r)
    for layout in (0, 1):
        _, y64 = orc.rope_cached(x, pos, r, c, s_, 1.3, layout)
        _, ref64 = orc.rope(x, pos, r, inv, 1.3, layout)
        pair = np.abs(x.astype(np.float64)).max()
        assert np.max(np.abs(y64 - ref64)) <= 1.3 * 2 * pair * 2.0 ** -24, layout
        q = np.zeros((10, r // 2), np.float32)
        one = np.ones((10, r // 2), np.float32)
        _, y64 = orc.rope_cached(x, pos, r, q, one, 1.25, layout)
        for i in range(r // 2):
            ia, ib = _pair_index(layout, r, i)
            assert np.array_equal(y64[..., ia], -1.25 * x[..., ib].astype(np.float64))
            assert np.array_equal(y64[..., ib], 1.25 * x[..., ia].astype(np.float64))
        bad = pos.copy()
        bad[2], bad[4] = 10, -1
        out, y64 = orc.rope_cached(x, bad, r, c, s_, 1.0, layout)
        for t in (2, 4):
            assert np.all(np.isnan(y64[t, :, :r])) and np.array_equal(y64[t, :, r:], x[t, :, r:])
        ok = [0, 1, 3, 5]
        _, good64 = orc.rope_cached(x, pos, r, c, s_, 1.0, layout)
        assert np.array_equal(y64[ok], good64[ok])


# ------------------------------------------------------- multi-axis RoPE

def _multi_brute(x, pos, dims, inv, mu, layout):
    """[OPS] Rope, multi-axis: the page's loop written out in Python floats --
    for each axis, its sub-range of the head is rotated as a whole head of
    dims[a] entries with that axis's position and frequencies (angles per
    [ELT] 2.2, the f64 product rounded to f32; sine and cosine in decimal)."""
    T, H, D = x.shape
    y = x.astype(np.float64)
    off, foff = 0, 0
    for a, da in enumerate(dims):
        for t in range(T):
            for j in range(da // 2):
                ang = float(np.float32(np.float64(int(pos[t, a])) * np.float64(inv[foff + j])))
                s, c = brute.sincos_decimal(ang, 30)
                ia, ib = _pair_index(layout, da, j)
                for h in range(H):
                    x1, x2 = y[t, h, off + ia], y[t, h, off + ib]
                    y[t, h, off + ia] = mu * (x1 * c - x2 * s)
                    y[t, h, off + ib] = mu * (x1 * s + x2 * c)
        off += da
        foff += da // 2
    return y


def pin_rope_multi_brute_force(orc):
    """[OPS] Rope, multi-axis (3D) RoPE on a tiny head: three axes of 4, 6
    and 4 entries in a head of 16 (the last 2 pass through), each axis with
    its own base, positions of both signs; both pairings.  Against the loop
    of the page written out independently (decimal sine and cosine)."""
    g = np.random.default_rng(303)
    T, H, D = 3, 2, 16
    dims = [4, 6, 4]
    x = g.standard_normal((T, H, D)).astype(np.float32)
    pos = np.array([[0, 5, -3], [7, 0, 2], [2, 9, 11]], np.int32)
    inv = np.concatenate([np.power(np.float64(b), -2.0 * np.arange(d // 2) / d)
                          for b, d in zip((10.0, 100.0, 1000.0), dims)]).astype(np.float32)
    for layout in (0, 1):
        out, y64 = orc.rope_multi(x, pos, dims, inv, 1.25, layout)
        ref = _multi_brute(x, pos, dims, inv, 1.25, layout)
        scale = np.abs(x.astype(np.float64)).max() * 1.25
        assert np.max(np.abs(y64 - ref)) <= 4 * scale * 2.0 ** -52, layout
        assert np.array_equal(out[..., 14:], x[..., 14:])
        assert np.array_equal(y64[..., 14:], x[..., 14:].astype(np.float64))


def pin_rope_multi_axes_decompose(orc):
    """Each axis is RoPE on its own sub-range: the multi-axis result, cut at
    the axis boundaries, equals the (separately pinned) single-axis RoPE of
    each slice with that axis's positions and frequencies, in f64 bits; one
    axis spanning r entries is partial RoPE with rotary width r; position
    vectors of zeros scale by mu only."""
    g = np.random.default_rng(304)
    T, H, D = 5, 3, 40
    dims = [8, 12, 16]
    x = g.standard_normal((T, H, D)).astype(np.float32)
    pos = g.integers(-5000, 5000, (T, 3)).astype(np.int32)
    inv = np.concatenate([np.power(np.float64(b), -2.0 * np.arange(d // 2) / d)
                          for b, d in zip((1e4, 5e3, 7e2), dims)]).astype(np.float32)
    for layout in (0, 1):
        _, y64 = orc.rope_multi(x, pos, dims, inv, 0.75, layout)
        off, foff = 0, 0
        for a, da in enumerate(dims):
            sl = np.ascontiguousarray(x[..., off:off + da])
            _, r64 = orc.rope(sl, pos[:, a].copy(), da, inv[foff:foff + da // 2].copy(), 0.75, layout)
            assert np.array_equal(y64[..., off:off + da], r64), (layout, a)
            off += da
            foff += da // 2
        _, one64 = orc.rope_multi(x, pos[:, 1:2], [24], inv[:12], 0.75, layout)
        _, p64 = orc.rope(x, pos[:, 1].copy(), 24, inv[:12].copy(), 0.75, layout)
        assert np.array_equal(one64, p64)
        _, z64 = orc.rope_multi(x, np.zeros((T, 3), np.int32), dims, inv, 0.75, layout)
        assert np.array_equal(z64[..., :36], 0.75 * x[..., :36].astype(np.float64))


# ------------------------------------------------------------ f16 storage

def _f16_all_finite():
    """Every non-negative finite binary16 value: bits and exact f64 values
    (numpy widens float16 exactly)."""
    bits = np.arange(0x7C00, dtype=np.uint16)
    return bits, bits.view(np.float16).astype(np.float64)


def pin_f16_rounding_exhaustive(orc):
    """[OPS] F16 storage: f64 -> binary16 rounds to nearest, ties to even,
    once.  Over every finite value: exact values map to themselves; the
    midpoint of each pair of neighbours goes to the one with an even
    significand, the doubles just below and above it to the lower and upper
    neighbour; 65520 (halfway past 65504) and above overflow to infinity;
    negatives mirror; NaN and infinity keep their class.  Then the library's
    float64 -> float16 cast (numpy) on values across the whole range."""
    bits, v = _f16_all_finite()
    assert np.array_equal(orc.round_to(v, "f16").view(np.uint16), bits)
    assert np.array_equal(orc.round_to(-v, "f16").view(np.uint16), bits | 0x8000)
    lo, hi = v[:-1], v[1:]
    mid = (lo + hi) / 2                                   # exact in f64
    even = np.where(bits[:-1] % 2 == 0, bits[:-1], bits[1:])
    assert np.array_equal(orc.round_to(mid, "f16").view(np.uint16), even)
    assert np.array_equal(orc.round_to(np.nextafter(mid, 0), "f16").view(np.uint16), bits[:-1])
    assert np.array_equal(orc.round_to(np.nextafter(mid, np.inf), "f16").view(np.uint16), bits[1:])
    top = orc.round_to(np.array([65519.999, 65520.0, 1e6, np.inf, -65520.0, -np.inf]), "f16")
    assert top.view(np.uint16).tolist() == [0x7BFF, 0x7C00, 0x7C00, 0x7C00, 0xFC00, 0xFC00]
    tiny = orc.round_to(np.array([2.0 ** -25, np.nextafter(2.0 ** -25, 1), 2.0 ** -26, -2.0 ** -25]), "f16")
    assert tiny.view(np.uint16).tolist() == [0x0000, 0x0001, 0x0000, 0x8000]
    n = orc.round_to(np.array([np.nan, -np.nan]), "f16").view(np.uint16)
    assert np.all((n & 0x7C00) == 0x7C00) and np.all((n & 0x03FF) != 0)
    g = np.random.default_rng(505)
    r = g.standard_normal(200000) * np.exp(g.uniform(-21, 12, 200000))
    with np.errstate(over="ignore"):
        ref = r.astype(np.float16)
    assert np.array_equal(orc.round_to(r, "f16").view(np.uint16), ref.view(np.uint16))


def pin_f16_storage_through_ops(orc):
    """Every op reads f16 storage exactly and rounds each result once: adding
    -0 returns every finite value, infinity and NaN as given; on f16
    inputs each op's f64 result equals its result on the same values held in
    f32 storage, and the stored output is that f64 result rounded by the
    library's float16 cast; the embedding copies bits; argmax picks the same
    index as on the f32 copy."""
    bits, v = _f16_all_finite()
    x = np.concatenate([bits, bits | 0x8000, [0x7C00, 0xFC00, 0x7E00]]).astype(np.uint16).view(np.float16)
    y = orc.add(x, np.full_like(x, -0.0))                  # x + (-0) == x for every x, signed zeros too
    assert np.array_equal(y.view(np.uint16)[:-1], x.view(np.uint16)[:-1])
    assert np.isnan(y[-1])
    g = np.random.default_rng(506)

    def h(shape, scale=1.0):
        return (g.standard_normal(shape) * scale).astype(np.float16)

    def same(out16, y16, y32, what):
        assert np.array_equal(y16, y32, equal_nan=True), f"{what}: f64 results differ"
        with np.errstate(over="ignore", invalid="ignore"):
            ref = y16.astype(np.float16)
        assert np.array_equal(out16.view(np.uint16), ref.view(np.uint16)), f"{what}: rounding"

    x16, w16, b16 = h((5, 96), 3), (g.uniform(0.5, 1.5, 96)).astype(np.float16), h(96)
    x16[0, :4] = [3e-6, -6e-8, 0, 6e4]                     # f16 subnormals and a large value
    f32 = lambda a: a.astype(np.float32)
    o, y1 = orc.rmsnorm(x16, w16, 1e-5)
    _, y2 = orc.rmsnorm(f32(x16), f32(w16), 1e-5)
    same(o, y1, y2, "rmsnorm")
    o, y1 = orc.layernorm(x16, w16, b16, 1e-5)
    _, y2 = orc.layernorm(f32(x16), f32(w16), f32(b16), 1e-5)
    same(o, y1, y2, "layernorm")
    o, y1 = orc.softmax(x16, 0.7)
    _, y2 = orc.softmax(f32(x16), 0.7)
    same(o, y1, y2, "softmax")
    u16 = h((5, 96))
    o, y1 = orc.silu_mul(x16, u16)
    _, y2 = orc.silu_mul(f32(x16), f32(u16))
    same(o, y1, y2, "silu_mul")
    for form in (0, 1):
        o, y1 = orc.geglu(x16, u16, form)
        _, y2 = orc.geglu(f32(x16), f32(u16), form)
        same(o, y1, y2, f"geglu {form}")
    q16 = h((4, 3, 32))
    pos = np.array([0, 5, 100, 4095], np.int32)
    inv = np.power(1e4, -2.0 * np.arange(16) / 32).astype(np.float32)
    for layout in (0, 1):
        o, y1 = orc.rope(q16, pos, 32, inv, 1.0, layout)
        _, y2 = orc.rope(f32(q16), pos, 32, inv, 1.0, layout)
        same(o, y1, y2, f"rope {layout}")
        o, y1 = orc.rope_multi(q16, np.stack([pos, pos + 1], 1), [16, 12], inv[:14], 1.0, layout)
        _, y2 = orc.rope_multi(f32(q16), np.stack([pos, pos + 1], 1), [16, 12], inv[:14], 1.0, layout)
        same(o, y1, y2, f"rope_multi {layout}")
    tab = h((50, 40))
    ids = np.array([3, 49, 0, 7, 50, -1], np.int32)
    e = orc.embedding(tab, ids)
    assert np.array_equal(e[:4].view(np.uint16), tab[ids[:4]].view(np.uint16))
    assert np.all(np.isnan(e[4:].astype(np.float32)))
    lg = h((6, 300), 3)
    lg[2, 7] = np.nan
    assert np.array_equal(orc.argmax(lg), orc.argmax(f32(lg)))


# -------------------------------------------------------------- LayerNorm

def pin_layernorm_closed_forms(orc):
    """[OPS] LayerNorm: a constant row gives exactly the bias (x - mu = 0), or
    0 without one; two entries give +-|a - c|/2 / sqrt(((a - c)/2)^2 + eps);
    eps is inside the root (the [ELT] 3 example's numbers: +-1e-3, eps 1e-6
    gives +-0.70711, not the 0.999 of eps outside)."""
    for dt in ("f32", "bf16"):
        cvt = (lambda a: a) if dt == "f32" else _bf16
        wide = (lambda a: a.astype(np.float64)) if dt == "f32" else (lambda a: _wide(a).astype(np.float64))
        x = cvt(np.full((3, 9), 1.75, np.float32))
        g = cvt(np.linspace(0.5, 1.5, 9).astype(np.float32))
        b = cvt(np.linspace(-1, 1, 9).astype(np.float32))
        y, y64 = orc.layernorm(x, g, b, 1e-5)
        assert np.array_equal(y64, np.broadcast_to(wide(b), (3, 9)))
        assert np.array_equal(y.view(np.uint8), np.broadcast_to(b, (3, 9)).view(np.uint8))
        _, y64 = orc.layernorm(x, g, None, 1e-5)
        assert np.all(y64 == 0.0)
    a, c, eps = 2.5, -1.0, 1e-3
    _, y64 = orc.layernorm(_f32([a, c])[None], _f32([1.0, 1.0]), None, eps)
    h = abs(a - c) / 2
    expect = h / math.sqrt(h * h + float(np.float32(eps)))
    assert abs(y64[0, 0] - expect) <= 1e-15 and abs(y64[0, 1] + expect) <= 1e-15
    _, y64 = orc.layernorm(_f32([1e-3, -1e-3])[None], _f32([1.0, 1.0]), None, 1e-6)
    assert abs(y64[0, 0] - 0.70711) < 1e-5 and abs(y64[0, 1] + 0.70711) < 1e-5


def pin_layernorm_invariants(orc):
    """Shifting a row by a constant changes nothing; with unit gain and zero
    bias the output has mean 0 and mean square var / (var + eps); the bias is
    added after the gain; a row's result does not depend on the others."""
    g = np.random.default_rng(83)
    x = np.round(g.standard_normal((5, 64)) * 8).astype(np.float32)    # integers: exact shifts
    one, zero = np.ones(64, np.float32), np.zeros(64, np.float32)
    y0, y64 = orc.layernorm(x, one, zero, 1e-5)
    ys, _ = orc.layernorm(x + np.float32(1024.0), one, zero, 1e-5)
    assert np.array_equal(y0.view(np.uint32), ys.view(np.uint32))
    xd = x.astype(np.float64)
    var = xd.var(axis=1)
    assert np.all(np.abs(y64.mean(axis=1)) < 1e-14)
    assert np.allclose((y64 ** 2).mean(axis=1), var / (var + float(np.float32(1e-5))), rtol=1e-13)
    gain = g.uniform(0.5, 1.5, 64).astype(np.float32)
    bias = g.standard_normal(64).astype(np.float32)
    _, yg = orc.layernorm(x, gain, bias, 1e-5)
    assert np.allclose(yg, y64 * gain.astype(np.float64) + bias.astype(np.float64), rtol=1e-14, atol=1e-14)
    alone, _ = orc.layernorm(np.ascontiguousarray(x[3:4]), gain, bias, 1e-5)
    full, _ = orc.layernorm(x, gain, bias, 1e-5)
    assert np.array_equal(alone[0].view(np.uint32), full[3].view(np.uint32))


def pin_layernorm_brute_and_library(orc):
    """Exact-fraction mean and variance with a 50-digit square root, and
    torch's f64 layer_norm, on random rows (with and without bias)."""
    import torch
    g = np.random.default_rng(89)
    x = (g.standard_normal((4, 37)) * 3 + 1).astype(np.float32)
    gain = g.uniform(0.5, 1.5, 37).astype(np.float32)
    bias = g.standard_normal(37).astype(np.float32)
    for b in (bias, None):
        _, y64 = orc.layernorm(x, gain, b, 1e-5)
        for r in range(4):
            ref = brute.layernorm_row_exact([float(v) for v in x[r]], [float(v) for v in gain],
                                            None if b is None else [float(v) for v in b], float(np.float32(1e-5)))
            assert np.allclose(y64[r], ref, rtol=1e-13, atol=1e-14), r
        lib = torch.nn.functional.layer_norm(torch.from_numpy(x.astype(np.float64)), (37,),
                                             torch.from_numpy(gain.astype(np.float64)),
                                             None if b is None else torch.from_numpy(b.astype(np.float64)),
                                             eps=float(np.float32(1e-5))).numpy()
        assert np.allclose(y64, lib, rtol=1e-12, atol=1e-13)
    xb, gb, bb = _bf16(x), _bf16(gain), _bf16(bias)
    y, y64 = orc.layernorm(xb, gb, bb, 1e-5)
    assert np.array_equal(y, np.array([brute.bf16_bits_exact(v) for v in y64.ravel()], np.uint16).reshape(y.shape))


def _page_rmsnorm_f32(x, w, eps):
    """[ELT] 2.1's routine in single precision: a float sum of squares in
    increasing i, then x * (1 / sqrt(ss / d + eps)) * w, every step in f32."""
    f = np.float32
    ss = f(0.0)
    with np.errstate(over="ignore", invalid="ignore"):
        for v in x:
            ss = f(ss + f(v) * f(v))
        inv = f(1.0) / np.sqrt(f(ss / f(len(x))) + f(eps))
        return np.array([f(f(v) * inv) * f(g) for v, g in zip(x, w)], np.float32)


def _page_layernorm_f32(x, g, b, eps):
    """[DNN] 7's two-pass statistics kept in f32: mean as a float sum / d,
    variance as a float sum of (x - mean)^2 / d, then
    (x - mean) * (1 / sqrt(var + eps)) * g + b, every step in f32."""
    f = np.float32
    with np.errstate(over="ignore", invalid="ignore"):
        s = f(0.0)
        for v in x:
            s = f(s + f(v))
        mu = f(s / f(len(x)))
        ss = f(0.0)
        for v in x:
            c = f(f(v) - mu)
            ss = f(ss + c * c)
        inv = f(1.0) / np.sqrt(f(ss / f(len(x))) + f(eps))
        return np.array([f(f(f(f(v) - mu) * inv) * f(gv)) + f(bv) for v, gv, bv in zip(x, g, b)],
                        np.float32)


def pin_norm_statistics_beyond_f32(orc):
    """The normalisation statistics are single-precision sums on the pages
    ([ELT] 2.1's float sum of squares, [DNN] 7's F32 statistics): a row
    whose sum of squares passes the f32 range normalises to x * 0 (signed
    zeros, NaN at an infinite entry), a LayerNorm row whose squared
    deviations pass it gives exactly the bias, and one whose (one-signed) sum
    passes it gives NaN.  Rows of the same shape that stay inside the range
    keep the f64 formula.  Checked bit for bit against the pages' routines
    run in numpy float32, in f32 and bf16 storage (all values here are bf16
    numbers)."""
    d = 16
    rms_rows = [
        [2.0 ** 65] * d,                             # every square already past the range
        [2.0 ** 63, -(2.0 ** 63)] * (d // 2),        # squares 2^126: the sum passes at the 4th term
        [2.0 ** 64] + [1.0] * (d - 1),               # one square of 2^128
        [float("inf")] + [3.0] * (d - 1),            # an infinite entry
    ]
    ln_rows = [
        [2.0 ** 65, -(2.0 ** 65)] * (d // 2),        # mean 0, squared deviations past the range
        [2.0 ** 126] * d,                            # a one-signed sum of 2^130
        [2.0 ** 120] * (d // 2) + [-(2.0 ** 120)] * (d // 2),  # mean 0, squares 2^240
    ]
    w = np.linspace(0.5, 1.5, d).astype(np.float32)
    b = np.linspace(-1.0, 1.0, d).astype(np.float32)
    for dt in ("f32", "bf16"):
        cvt = (lambda a: np.asarray(a, np.float32)) if dt == "f32" else (lambda a: _bf16(np.asarray(a, np.float32)))
        wide = (lambda a: a) if dt == "f32" else _wide
        ws, bs = cvt(w), cvt(b)
        x = cvt(np.array(rms_rows, np.float32))
        y, _ = orc.rmsnorm(x, ws, 1e-5)
        for r in range(len(rms_rows)):
            page = _page_rmsnorm_f32(wide(x[r]), wide(ws), 1e-5)
            assert np.array_equal(np.isnan(page), np.isnan(wide(y[r]))), (dt, r)
            ok = ~np.isnan(page)
            assert np.array_equal(np.signbit(page[ok]), np.signbit(wide(y[r])[ok])), (dt, r)
            assert np.all(page[ok] == 0) and np.all(wide(y[r])[ok] == 0), (dt, r)
        x = cvt(np.array(ln_rows, np.float32))
        y, _ = orc.layernorm(x, ws, bs, 1e-5)
        for r in range(len(ln_rows)):
            page = _page_layernorm_f32(wide(x[r]), wide(ws), wide(bs), 1e-5)
            got = wide(y[r])
            assert np.array_equal(np.isnan(page), np.isnan(got)), (dt, r)
            assert np.array_equal(page[~np.isnan(page)], got[~np.isnan(page)]), (dt, r)
        assert np.all(np.isnan(wide(y[1]))) and np.array_equal(wide(y[0]), wide(bs))
    # inside the range the f64 formula stands: squares summing to 2^126
    x = np.full((1, d), 2.0 ** 61, np.float32)
    _, y64 = orc.rmsnorm(x, np.ones(d, np.float32), 1e-5)
    assert np.allclose(y64, 1.0, rtol=1e-12)
    x = np.array([[2.0 ** 61, -(2.0 ** 61)] * (d // 2)], np.float32)
    _, y64 = orc.layernorm(x, np.ones(d, np.float32), None, 1e-5)
    assert np.allclose(np.abs(y64), 1.0, rtol=1e-12)


# ------------------------------------------------------------------ GeGLU

def pin_gelu_symmetry_and_limits(orc):
    """[OPS] Gelu, both forms: Gelu(x) - Gelu(-x) = x (erf and tanh are
    odd), Gelu(0) = 0, Gelu(x) -> x for large x and -> -0 far below zero; the
    up factor multiplies."""
    xs = _f32([0.25, 0.5, 1.0, 1.7, 2.5, 4.0, 6.0])
    for form in (0, 1):
        yp, yp64 = orc.geglu(xs, np.ones_like(xs), form)
        yn, yn64 = orc.geglu(-xs, np.ones_like(xs), form)
        assert np.allclose(yp64 - yn64, xs.astype(np.float64), rtol=1e-15, atol=0.0), form
        _, z64 = orc.geglu(_f32([0.0, 12.0, -60.0]), _f32([1.0, 1.0, 1.0]), form)
        assert z64[0] == 0.0 and z64[1] == 12.0 and z64[2] == 0.0 and math.copysign(1.0, z64[2]) < 0
        _, u64 = orc.geglu(xs, _f32([3.0] * 7), form)
        assert np.allclose(u64, 3.0 * yp64, rtol=1e-15, atol=0.0)
    # tanh form: e^(-2u) passes the f32 range between x = -10 and x = -10.5,
    # after which the value is -0, as for SiLU (x / inf)
    _, z64 = orc.geglu(_f32([-10.0, -10.5]), _f32([1.0, 1.0]), 1)
    assert z64[0] < 0 and abs(z64[0] - brute.gelu_tanh_decimal(-10.0)) <= 1e-13 * abs(z64[0])
    assert z64[1] == 0.0 and math.copysign(1.0, z64[1]) < 0
    # erf form with an infinite up: Phi(x) lies in (0, 1] for every finite x,
    # so the product is the infinity of sign(x) sign(up), however far below
    # zero x is (-60: x Phi(x) is below every float's range); Phi(0) x = 0 and
    # Phi(-inf) = 0 leave 0 * inf, NaN; Phi(+inf) = 1.  The tanh form, whose
    # value is -0 past the f32 limit above, gives NaN there.
    inf = float("inf")
    _, v64 = orc.geglu(_f32([-60.0, -60.0, -5.0, 3.0, 0.0, -inf, inf, -3e38]),
                       _f32([inf, -inf, inf, -inf, inf, inf, -inf, inf]), 0)
    assert list(v64[:4]) == [-inf, inf, -inf, -inf] and v64[6] == -inf and v64[7] == -inf
    assert math.isnan(v64[4]) and math.isnan(v64[5])
    _, w64 = orc.geglu(_f32([-60.0]), _f32([inf]), 1)
    assert math.isnan(w64[0])


def pin_gelu_brute(orc):
    """Both forms against high-precision decimal evaluations that take a
    different route: the erfc power series (with pi from Machin's formula) and
    tanh from decimal exponentials -- including x = -10, where 1 + erf(x/sqrt 2)
    cancels in f64 and only the exact identity keeps the 7.6e-23."""
    xs = [-10.0, -5.5, -2.0, -0.75, -0.1, 0.3, 1.0, 2.25, 4.5]
    x = _f32(xs)
    _, e64 = orc.geglu(x, np.ones_like(x), 0)
    _, t64 = orc.geglu(x, np.ones_like(x), 1)
    for i, v in enumerate(x):
        ref_e = brute.gelu_erf_decimal(float(v))
        ref_t = brute.gelu_tanh_decimal(float(v))
        assert abs(e64[i] - ref_e) <= 1e-13 * abs(ref_e) + 1e-300, (v, e64[i], ref_e)
        assert abs(t64[i] - ref_t) <= 1e-13 * abs(ref_t) + 1e-300, (v, t64[i], ref_t)


def pin_gelu_matches_library(orc):
    """torch's f64 gelu (approximate 'none' and 'tanh') on the same inputs,
    f32 and bf16 storage; the two forms stay within 1e-3 of each other but
    are not equal."""
    import torch
    g = np.random.default_rng(97)
    gate = (g.standard_normal(2000) * 2).astype(np.float32)
    up = g.standard_normal(2000).astype(np.float32)
    for dt in ("f32", "bf16"):
        gs, us = (gate, up) if dt == "f32" else (_bf16(gate), _bf16(up))
        gw = gs.astype(np.float64) if dt == "f32" else _wide(gs).astype(np.float64)
        uw = us.astype(np.float64) if dt == "f32" else _wide(us).astype(np.float64)
        for form, approx in ((0, "none"), (1, "tanh")):
            _, y64 = orc.geglu(gs, us, form)
            ref = torch.nn.functional.gelu(torch.from_numpy(gw), approximate=approx).numpy() * uw
            assert np.allclose(y64, ref, rtol=1e-12, atol=1e-15), (dt, form)
    _, e64 = orc.geglu(gate, np.ones_like(gate), 0)
    _, t64 = orc.geglu(gate, np.ones_like(gate), 1)
    d = np.abs(e64 - t64)
    assert d.max() < 1e-3 and d.max() > 1e-5


# ------------------------------------------------------- batch invariance

def pin_batch_invariance(orc):
    """[ELT] 2.1 (a row's bits never depend on its batch) extended to every
    row op: rows/tokens computed alone equal the same rows in a batch."""
    g = np.random.default_rng(61)
    for dt in ("f32", "bf16"):
        cvt = (lambda a: a) if dt == "f32" else _bf16
        x = cvt(g.standard_normal((6, 3, 16)).astype(np.float32))
        gain = cvt(g.uniform(0.5, 1.5, 16).astype(np.float32))
        pos = g.integers(0, 5000, 6).astype(np.int32)
        inv = np.power(np.float64(1e4), -2.0 * np.arange(8) / 16).astype(np.float32)
        full, _ = orc.rmsnorm_rope(x, gain, 1e-6, pos, 16, inv, 1.0, 0)
        full_r, _ = orc.rope(x, pos, 16, inv, 1.0, 1)
        res = cvt(g.standard_normal((6, 48)).astype(np.float32))
        w48 = cvt(g.uniform(0.5, 1.5, 48).astype(np.float32))
        yf, hf, _ = orc.add_rmsnorm(x.reshape(6, 48), res, w48, 1e-5)
        for t in range(6):
            one, _ = orc.rmsnorm_rope(np.ascontiguousarray(x[t:t + 1]), gain, 1e-6, pos[t:t + 1], 16, inv,
                                      1.0, 0)
            assert np.array_equal(one[0].view(np.uint8), full[t].view(np.uint8)), (dt, t)
            one_r, _ = orc.rope(np.ascontiguousarray(x[t:t + 1]), pos[t:t + 1], 16, inv, 1.0, 1)
            assert np.array_equal(one_r[0].view(np.uint8), full_r[t].view(np.uint8)), (dt, t)
            y1, h1, _ = orc.add_rmsnorm(np.ascontiguousarray(x[t].reshape(1, 48)), res[t:t + 1], w48, 1e-5)
            assert np.array_equal(y1[0].view(np.uint8), yf[t].view(np.uint8)), (dt, t)


PINS: Dict[str, Callable] = {name[4:]: fn for name, fn in sorted(globals().items())
                             if name.startswith("pin_") and callable(fn)}
