"""Tiny, independent evaluations used to pin the oracle (pure Python).

Each one reaches the op's result by a different route from ``oracle.c``:
exact rational sums (``fractions``), complex multiplication (``cmath``), the
tanh form of the logistic function, rounding by enumeration of neighbours.
Slow on purpose: only for a few hundred elements.
"""
from __future__ import annotations

import cmath
import math
import struct
from fractions import Fraction
from typing import List, Sequence, Tuple


def f32(v: float) -> float:
    """Round a Python float to the nearest f32 value (IEEE cast)."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def bf16_bits_exact(v) -> int:
    """bfloat16 bits nearest to the exact value v (Fraction or float), ties to
    even, found by comparing the two neighbouring bf16 values exactly."""
    if isinstance(v, float):
        if math.isnan(v):
            return 0x7FC0
        if math.isinf(v):
            return 0xFF80 if v < 0 else 0x7F80
        if v == 0.0:
            return 0x8000 if math.copysign(1.0, v) < 0 else 0
    v = Fraction(v)
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    if a == 0:
        return sign
    # binade e: 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    q = Fraction(2) ** (e - 7)
    k = a // q                      # lower neighbour = k*q
    rem = a - k * q
    if rem * 2 > q or (rem * 2 == q and k % 2 == 1):
        k += 1
    val = k * q
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    bits = struct.unpack("<I", struct.pack("<f", float(val)))[0] >> 16
    return sign | bits


def rmsnorm_row(x: Sequence[float], w: Sequence[float], eps: float) -> List[float]:
    """y_i = x_i w_i / sqrt(ss/d + eps) with the sum of squares exact."""
    d = len(x)
    ss = sum(Fraction(v) * Fraction(v) for v in x)
    ms = ss / d + Fraction(f32(eps))
    root = math.sqrt(ms)
    return [float(Fraction(xi) * Fraction(wi)) / root for xi, wi in zip(x, w)]


def rope_head(v: Sequence[float], pos: int, r: int, inv_freq: Sequence[float],
              mu: float, layout: int) -> List[float]:
    """Rotate one head row as complex numbers: (a + ib) mu e^{i theta}, with
    theta the f32 product f32(p) * f32(w) (exact for |p| < 2^24)."""
    out = list(v)
    half = r // 2
    for i in range(half):
        if layout == 0:
            ia, ib = i, i + half
        else:
            ia, ib = 2 * i, 2 * i + 1
        theta = f32(f32(float(pos)) * f32(inv_freq[i]))
        z = complex(v[ia], v[ib]) * f32(mu) * cmath.exp(1j * theta)
        out[ia], out[ib] = z.real, z.imag
    return out


def silu_tanh(g: float) -> float:
    """silu(g) = g * sigmoid(g), evaluated as g (1 + tanh(g/2)) / 2 for g >= 0
    and as g e^g / (1 + e^g) for g < 0 (where the tanh form cancels)."""
    if g >= 0:
        return g * (1.0 + math.tanh(g / 2.0)) / 2.0
    e = math.exp(g)
    return g * e / (1.0 + e)


def argmax_sorted(x: Sequence[float]) -> int:
    """Lowest index among the largest non-NaN values, by sorting keys."""
    keys: List[Tuple[float, int]] = [(-v, i) for i, v in enumerate(x) if not math.isnan(v)]
    if not keys:
        return -1
    keys.sort()
    return keys[0][1]


def softmax_decimal(x: Sequence[float], t: float, digits: int = 50) -> List[float]:
    """Softmax of x / t for finite inputs in 50-digit decimal arithmetic
    (``decimal``'s own exp, no libm), written as 1 / sum_j exp(z_j - z_i) --
    a different arrangement from the oracle's max-subtracted quotient."""
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = digits
        z = [Decimal(v) / Decimal(t) for v in x]
        out = []
        for zi in z:
            s = sum(((zj - zi).exp() for zj in z), Decimal(0))
            out.append(float(Decimal(1) / s))
        return out


def _dec_pi(ctx_prec: int):
    """pi in Decimal by Machin's formula, 16 * atan(1/5) - 4 * atan(1/239)."""
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = ctx_prec + 10

        def atan_inv(n):
            x = Decimal(1) / n
            x2 = x * x
            term, total, k = x, x, 1
            while True:
                term *= -x2
                k += 2
                add = term / k
                if add == 0 or abs(add) < Decimal(10) ** (-(ctx_prec + 8)):
                    break
                total += add
            return total
        return +(16 * atan_inv(5) - 4 * atan_inv(239))


def erfc_decimal(z: float, digits: int = 90):
    """erfc(z) = 1 - (2/sqrt(pi)) sum_n (-1)^n z^(2n+1) / (n! (2n+1)), summed in
    high-precision decimal (enough digits that 1 - erf keeps ~25 significant
    ones for |z| < 7.5).  Returns a Decimal."""
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = digits
        zz = Decimal(z)
        total, term, n = Decimal(0), zz, 0
        while True:
            add = term / (2 * n + 1)
            total += add
            n += 1
            term = -term * zz * zz / n
            if abs(add) < Decimal(10) ** (-(digits - 5)) and n > 5:
                break
        pi = _dec_pi(digits)
        return 1 - 2 * total / pi.sqrt()


def gelu_erf_decimal(x: float) -> float:
    """x * erfc(-x / sqrt 2) / 2 with erfc from the decimal series (the
    argument x / sqrt 2 is formed in 90-digit decimal and passed on as the
    nearest double, a relative change of 1e-16)."""
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = 90
        z = float(-Decimal(x) / Decimal(2).sqrt())
        return float(Decimal(x) * erfc_decimal(z) / 2)


def gelu_tanh_decimal(x: float) -> float:
    """0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3), with
    tanh(u) = (e^(2u) - 1) / (e^(2u) + 1) in 60-digit decimal."""
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = 60
        xx = Decimal(x)
        pi = _dec_pi(60)
        u = (2 / pi).sqrt() * (xx + Decimal("0.044715") * xx ** 3)
        e2 = (2 * u).exp()
        th = (e2 - 1) / (e2 + 1)
        return float(xx * (1 + th) / 2)


def layernorm_row_exact(x: Sequence[float], g: Sequence[float], b, eps: float) -> List[float]:
    """LayerNorm of one row with the mean and variance as exact fractions and
    the square root in 50-digit decimal."""
    from decimal import Decimal, localcontext
    d = len(x)
    fx = [Fraction(v) for v in x]
    mu = sum(fx) / d
    var = sum((v - mu) ** 2 for v in fx) / d
    with localcontext() as ctx:
        ctx.prec = 50
        den = (Decimal(var.numerator) / Decimal(var.denominator) + Decimal(eps)).sqrt()
        out = []
        for i, v in enumerate(fx):
            c = v - mu
            val = Decimal(c.numerator) / Decimal(c.denominator) / den * Decimal(g[i])
            if b is not None:
                val += Decimal(b[i])
            out.append(float(val))
        return out


def sincos_decimal(x: float, digits: int = 50):
    """(sin x, cos x) of a double x: reduction by pi/2 with pi from Machin's
    formula and the Taylor series, all in decimal."""
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = digits + 20
        pi = _dec_pi(digits + 20)
        xx = Decimal(x)
        k = (xx / (pi / 2)).to_integral_value()
        r = xx - k * (pi / 2)
        s, c = Decimal(0), Decimal(0)
        term, n = r, 1
        while abs(term) > Decimal(10) ** (-(digits + 5)):
            s += term
            term = -term * r * r / ((n + 1) * (n + 2))
            n += 2
        term, n = Decimal(1), 0
        while abs(term) > Decimal(10) ** (-(digits + 5)):
            c += term
            term = -term * r * r / ((n + 1) * (n + 2))
            n += 2
        q = int(k) % 4
        sv, cv = [(s, c), (c, -s), (-s, -c), (-c, s)][q]
        return float(sv), float(cv)
