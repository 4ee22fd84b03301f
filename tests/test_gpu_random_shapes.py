"""Seeded random shapes for every op, in every storage type, against the
CPU oracle through the C ABI.

The fixed-shape tests pick sizes around known launch boundaries; these draw
row lengths, row counts, head geometries, flat lengths and buffer alignment
at random (row lengths log-uniform up to about 140,000, half of them whole
16-byte vectors), so the launch-shape choices -- threads per row, vectors
per thread, long-row and chunked paths, ragged tails, the scalar path for
misaligned buffers -- are reached from points nobody picked.  Each result is
held to its op's own tolerance (gpu_util), and the ops whose kernels do no
reduction (add, embedding, argmax, RoPE pass-through, the fused sum h) to
equal bits.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import (BF16_PAIR, F32_FLOOR, F32_OVERFLOW, F32_REL, assert_bits, assert_close,
                      assert_f32_rel, assert_pair, bf16_key, check_geglu, check_layernorm, check_softmax,
                      dev, host, pair_norms, widen)

pytestmark = pytest.mark.gpu

DTS = ["f32", "bf16", "f16"]
SEEDS = range(8)


@pytest.fixture(scope="module")
def et():
    import elementwise_transformer_amd as m
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return m


def _length(g, lo, hi):
    """Log-uniform in [lo, hi]; half the draws rounded down to a multiple of 8."""
    n = int(np.exp(g.uniform(np.log(lo), np.log(hi + 1))))
    n = min(max(n, lo), hi)
    return max(lo, n - n % 8) if g.uniform() < 0.5 else n


def _rows(g, n, budget=1 << 21):
    """A row count from 1 to 40, capped so rows * n stays near the budget."""
    return int(max(1, min(int(g.integers(1, 41)), budget // max(n, 1))))


def _dev_maybe_misaligned(a, misalign):
    """To the device, at an address 16-byte aligned or (misalign) not."""
    t = dev(a)
    if not misalign:
        return t
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    v = flat[1:1 + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0
    return v


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("seed", SEEDS)
def test_random_norms(et, orc, dt, seed):
    g = np.random.default_rng([4848, seed, DTS.index(dt)])
    d = _length(g, 1, 70000)
    rows = _rows(g, d)
    mis = bool(g.uniform() < 0.25)
    x = wl.store((g.standard_normal((rows, d)) * 2).astype(np.float32), dt)
    r = wl.store(g.standard_normal((rows, d)).astype(np.float32), dt)
    w = wl.store(g.uniform(0.5, 1.5, d).astype(np.float32), dt)
    b = wl.store(g.standard_normal(d).astype(np.float32), dt)
    what = f"{dt} rows={rows} d={d} misaligned={mis}"
    xt = _dev_maybe_misaligned(x, mis)
    yr, y64 = orc.rmsnorm(x, w, 1e-5)
    assert_close(host(et.rmsnorm(xt, dev(w), 1e-5)), y64, yr, "rmsnorm " + what)
    yt, ht = et.add_rmsnorm(xt, dev(r), dev(w), 1e-5)
    oy, oh, oy64 = orc.add_rmsnorm(x, r, w, 1e-5)
    assert_bits(host(ht), oh, "add_rmsnorm h " + what)
    assert_close(host(yt), oy64, oy, "add_rmsnorm y " + what)
    y, ly64 = orc.layernorm(x, w, b, 1e-5)
    check_layernorm(host(et.layernorm(xt, dev(w), dev(b), 1e-5)), x, w, b, 1e-5, y, ly64,
                    "layernorm " + what)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("seed", SEEDS)
def test_random_softmax(et, orc, dt, seed):
    g = np.random.default_rng([4949, seed, DTS.index(dt)])
    n = _length(g, 1, 140000)
    rows = _rows(g, n)
    mis = bool(g.uniform() < 0.25)
    x = wl.store((g.standard_normal((rows, n)) * 3).astype(np.float32), dt)
    t = float(np.float32(g.choice([0.5, 0.7, 1.0, 1.7])))
    y, y64 = orc.softmax(x, t)
    got = host(et.softmax(_dev_maybe_misaligned(x, mis), t))
    check_softmax(got, x, t, y, y64, f"softmax {dt} rows={rows} n={n} t={t} misaligned={mis}")


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("seed", SEEDS)
def test_random_rope(et, orc, dt, seed):
    g = np.random.default_rng([5050, seed, DTS.index(dt)])
    D = int(2 * g.integers(1, 161))
    r = int(2 * g.integers(0, D // 2 + 1))
    T, Hq, Hk = int(g.integers(1, 50)), int(g.integers(1, 9)), int(g.integers(0, 5))
    layout = int(g.integers(0, 2))
    mu = float(np.float32(g.choice([1.0, 1.1, 0.5])))
    q = wl.store(g.standard_normal((T, Hq, D)).astype(np.float32), dt)
    k = wl.store(g.standard_normal((T, Hk, D)).astype(np.float32), dt) if Hk else None
    pos = g.integers(0, 1 << 20, T).astype(np.int32)
    inv = wl.inv_freq(1e4, r) if r else np.zeros(1, np.float32)
    gq = wl.store(g.uniform(0.5, 1.5, D).astype(np.float32), dt)
    gk = wl.store(g.uniform(0.5, 1.5, D).astype(np.float32), dt)
    what = f"{dt} T={T} Hq={Hq} Hk={Hk} D={D} r={r} layout={layout}"
    qt, kt = dev(q), (dev(k) if k is not None else None)
    et.rope_qk(qt, kt, dev(pos), dev(inv), d_rot=r, attn_scaling=mu, layout=layout)
    q2, k2 = dev(q), (dev(k) if k is not None else None)
    et.rmsnorm_rope_qk(q2, dev(gq), k2, dev(gk) if k is not None else None, 1e-6, dev(pos),
                       dev(inv), d_rot=r, attn_scaling=mu, layout=layout)
    for name, src, gain, t1, t2 in (("q", q, gq, qt, q2), ("k", k, gk, kt, k2)):
        if src is None:
            continue
        ref, y64 = orc.rope(src, pos, r, inv, mu, layout)
        got = host(t1)
        assert_pair(got, y64, ref, r, layout, f"rope {name} {what}")
        assert_bits(got[..., r:], src[..., r:], f"rope pass-through {name} {what}")
        ref, y64 = orc.rmsnorm_rope(src, gain, 1e-6, pos, r, inv, mu, layout)
        got = host(t2)
        assert_pair(got, y64, ref, r, layout, f"rmsnorm_rope {name} {what}")
        assert_close(got[..., r:], y64[..., r:], ref[..., r:], f"rmsnorm_rope tail {name} {what}")
    # the scalar path (misaligned q) gives the vector path's bits
    qm = _dev_maybe_misaligned(q, True)
    et.rope_qk(qm, None, dev(pos), dev(inv), d_rot=r, attn_scaling=mu, layout=layout)
    assert_bits(host(qm), host(qt), f"rope misaligned {what}")
    # the rotation read from the library's own cos/sin cache: the same bits,
    # on the vector and the scalar path
    if r:
        c, sn = et.rope_cache(dev(inv), int(pos.max()) + 1, r)
        qc, kc = dev(q), (dev(k) if k is not None else None)
        et.rope_qk_cached(qc, kc, dev(pos), c, sn, d_rot=r, attn_scaling=mu, layout=layout)
        assert_bits(host(qc), host(qt), f"cached rope q {what}")
        if k is not None:
            assert_bits(host(kc), host(kt), f"cached rope k {what}")
        qcm = _dev_maybe_misaligned(q, True)
        et.rope_qk_cached(qcm, None, dev(pos), c, sn, d_rot=r, attn_scaling=mu, layout=layout)
        assert_bits(host(qcm), host(qt), f"cached rope misaligned {what}")


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("seed", SEEDS)
def test_random_flat(et, orc, dt, seed):
    g = np.random.default_rng([5151, seed, DTS.index(dt)])
    n = _length(g, 1, 1 << 21)
    mis = bool(g.uniform() < 0.25)
    a = wl.store((g.standard_normal(n) * 3).astype(np.float32), dt)
    b = wl.store(g.standard_normal(n).astype(np.float32), dt)
    what = f"{dt} n={n} misaligned={mis}"
    at, bt = _dev_maybe_misaligned(a, mis), dev(b)
    assert_bits(host(et.add(at, bt)), orc.add(a, b), "add " + what)
    yr, y64 = orc.silu_mul(a, b)
    assert_close(host(et.silu_mul(at, bt)), y64, yr, "silu_mul " + what)
    for form in (0, 1):
        y, gy64 = orc.geglu(a, b, form)
        check_geglu(host(et.geglu(at, bt, form)), a, form, y, gy64, f"geglu form={form} {what}")


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("seed", SEEDS)
def test_random_embedding_argmax(et, orc, dt, seed):
    g = np.random.default_rng([5252, seed, DTS.index(dt)])
    V, d, nid = int(g.integers(1, 3000)), _length(g, 1, 9000), int(g.integers(1, 60))
    mis = bool(g.uniform() < 0.25)
    table = wl.store(g.standard_normal((V, d)).astype(np.float32), dt)
    ids = g.integers(-2, V + 2, nid).astype(np.int32)            # some out of range
    got = host(et.embedding(_dev_maybe_misaligned(table, mis), dev(ids)))
    assert_bits(got, orc.embedding(table, ids), f"embedding {dt} V={V} d={d} n={nid} misaligned={mis}")
    n = _length(g, 1, 140000)
    rows = _rows(g, n)
    # integer-valued logits: many ties, so the lowest-index rule is exercised
    x = wl.store(np.round(g.standard_normal((rows, n)) * 6).astype(np.float32), dt)
    ref = orc.argmax(x)
    for split in (True, False):
        got = host(et.argmax(_dev_maybe_misaligned(x, mis), split=split))
        assert_bits(got, ref, f"argmax {dt} rows={rows} n={n} split={split} misaligned={mis}")


# Special values planted at random positions: NaN, infinities, signed zeros,
# values whose sums or products leave the f32 range, subnormals, values
# beyond the f16 range (stored as infinities there).
SPECIALS = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 3e38, -3e38, 1e-40, -1e-40, 7e4, 1.0],
                    np.float32)


def _plant(g, a, frac=0.02):
    a = a.copy()
    flat = a.reshape(-1)
    m = max(1, int(flat.size * frac))
    idx = g.choice(flat.size, size=min(m, flat.size), replace=False)
    flat[idx] = g.choice(SPECIALS, size=idx.size)
    return a


@pytest.mark.parametrize("dt", DTS)
# seeds 8 and 10 plant a gate of -3e38 against an up of +-3e38 (f32 and bf16
# storage): x Phi(x) u is a signed zero there, with no overflow on the way
@pytest.mark.parametrize("seed", [*range(6), 8, 10])
def test_random_specials_flat(et, orc, dt, seed):
    """add (equal bits), SiLU-mul and both GeGLU forms (their tolerances,
    infinities exact) with special values planted in both operands."""
    g = np.random.default_rng([5353, seed, DTS.index(dt)])
    n = _length(g, 1, 300000)
    a = wl.store(_plant(g, (g.standard_normal(n) * 3).astype(np.float32)), dt)
    b = wl.store(_plant(g, g.standard_normal(n).astype(np.float32)), dt)
    what = f"{dt} n={n}"
    assert_bits(host(et.add(dev(a), dev(b))), orc.add(a, b), "add " + what)
    # f32: a subnormal gate makes the activation an f32 subnormal, rounded to
    # within 2^-150 in any single-precision order, and the product with up
    # scales that by |up| (up to 3e38 here)
    extra = 2.0 ** -149 * np.abs(b.astype(np.float64)) if dt == "f32" else None
    yr, y64 = orc.silu_mul(a, b)
    got = host(et.silu_mul(dev(a), dev(b)))
    if dt == "f32":
        assert_f32_rel(got, y64, "silu_mul " + what, abs_extra=extra)
    else:
        assert_close(got, y64, yr, "silu_mul " + what)
    for form in (0, 1):
        y, gy64 = orc.geglu(a, b, form)
        check_geglu(host(et.geglu(dev(a), dev(b), form)), a, form, y, gy64, f"geglu form={form} {what}",
                    abs_extra=extra)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("seed", range(6))
def test_random_specials_rows(et, orc, dt, seed):
    """RMSNorm, fused add+RMSNorm, LayerNorm, softmax and argmax over rows
    with special values planted in some of them (a NaN or an infinity
    spreads over its row as the formula says; the other rows are unaffected).
    Values whose sums overflow are kept to one sign per row here (R28 leaves
    mixed-sign overflow to the order of the partial sums)."""
    g = np.random.default_rng([5454, seed, DTS.index(dt)])
    d = _length(g, 1, 20000)
    rows = _rows(g, d, 1 << 19)
    base = (g.standard_normal((rows, d)) * 2).astype(np.float32)
    planted = _plant(g, base, frac=0.002)
    # no +-3e38 of both signs in a row
    for r in range(rows):
        row = planted[r]
        if np.any(row == np.float32(3e38)) and np.any(row == np.float32(-3e38)):
            row[row == np.float32(-3e38)] = np.float32(-1.0)
    x = wl.store(planted, dt)
    res = wl.store(g.standard_normal((rows, d)).astype(np.float32), dt)
    w = wl.store(g.uniform(0.5, 1.5, d).astype(np.float32), dt)
    bias = wl.store(g.standard_normal(d).astype(np.float32), dt)
    what = f"{dt} rows={rows} d={d}"
    yr, y64 = orc.rmsnorm(x, w, 1e-5)
    assert_close(host(et.rmsnorm(dev(x), dev(w), 1e-5)), y64, yr, "rmsnorm " + what)
    yt, ht = et.add_rmsnorm(dev(x), dev(res), dev(w), 1e-5)
    oy, oh, oy64 = orc.add_rmsnorm(x, res, w, 1e-5)
    assert_bits(host(ht), oh, "add_rmsnorm h " + what)
    assert_close(host(yt), oy64, oy, "add_rmsnorm y " + what)
    y, ly64 = orc.layernorm(x, w, bias, 1e-5)
    check_layernorm(host(et.layernorm(dev(x), dev(w), dev(bias), 1e-5)), x, w, bias, 1e-5, y, ly64,
                    "layernorm " + what)
    y, sy64 = orc.softmax(x, 0.7)
    check_softmax(host(et.softmax(dev(x), 0.7)), x, 0.7, y, sy64, "softmax " + what)
    assert_bits(host(et.argmax(dev(x))), orc.argmax(x), "argmax " + what)


def _assert_pair_special(got, y64, ref, r, layout, what):
    """The PAIR tolerance where a pair's two oracle values are finite; NaN
    and infinite entries elsewhere must match in position (and sign).  A
    pair of values near the f32 maximum can rotate past it (3e38 and -3e38
    at 45 degrees give 4.2e38): in f32 storage that entry is the infinity of
    its sign wherever the exact value lies within the tolerance of the
    overflow threshold or beyond it."""
    with np.errstate(invalid="ignore", over="ignore"):
        g, y = widen(got), y64
        assert np.array_equal(np.isnan(g), np.isnan(y)), f"{what}: NaN positions differ"
        inf = np.isinf(y)
        assert np.array_equal(g[inf], y[inf]), f"{what}: infinities differ"
        pn = pair_norms(np.where(np.isfinite(y), y, np.nan), r, layout)[..., :r]
        ok = np.isfinite(pn)
        err = np.abs(g[..., :r] - y[..., :r])
        if got.dtype == np.float32:
            yr = y[..., :r]
            rounds_inf = (g[..., :r] == np.copysign(np.inf, yr)) & \
                (np.abs(yr) + F32_REL * pn >= F32_OVERFLOW)
            bad = ok & ~((err <= F32_REL * pn + F32_FLOOR) | rounds_inf)
        else:
            ud = np.abs(bf16_key(got[..., :r]) - bf16_key(ref[..., :r]))
            bad = ok & ~((ud <= 1) | (err <= BF16_PAIR * pn))
    assert not bad.any(), f"{what}: {int(bad.sum())} rotated entries over the pair tolerance"


@pytest.mark.parametrize("dt", DTS)
# seeds 11 and 58 rotate a pair of +-3e38 past the f32 maximum
@pytest.mark.parametrize("seed", [*range(6), 11, 58])
def test_random_specials_rope(et, orc, dt, seed):
    """RoPE, fused RMSNorm+RoPE and multi-axis RoPE with special values
    planted in q and k (a NaN or infinity spreads to its pair partner, or
    through the norm to its head); pass-through entries keep their bits."""
    g = np.random.default_rng([5555, seed, DTS.index(dt)])
    D = int(2 * g.integers(4, 80))
    r = int(2 * g.integers(1, D // 2 + 1))
    T, Hq, Hk = int(g.integers(1, 30)), int(g.integers(1, 6)), int(g.integers(0, 4))
    layout, mu = int(g.integers(0, 2)), float(np.float32(g.choice([1.0, 0.9])))
    q = wl.store(_plant(g, g.standard_normal((T, Hq, D)).astype(np.float32), 0.01), dt)
    k = wl.store(_plant(g, g.standard_normal((T, Hk, D)).astype(np.float32), 0.01), dt) if Hk else None
    pos = g.integers(0, 1 << 16, T).astype(np.int32)
    pos[0] = 0                                          # the identity rotation (sin 0) included
    inv = wl.inv_freq(1e4, r)
    gq = wl.store(g.uniform(0.5, 1.5, D).astype(np.float32), dt)
    gk = wl.store(g.uniform(0.5, 1.5, D).astype(np.float32), dt)
    what = f"{dt} T={T} Hq={Hq} Hk={Hk} D={D} r={r} layout={layout}"
    qt, kt = dev(q), (dev(k) if k is not None else None)
    et.rope_qk(qt, kt, dev(pos), dev(inv), d_rot=r, attn_scaling=mu, layout=layout)
    for name, src, t in (("q", q, qt), ("k", k, kt)):
        if src is None:
            continue
        ref, y64 = orc.rope(src, pos, r, inv, mu, layout)
        got = host(t)
        _assert_pair_special(got, y64, ref, r, layout, f"rope {name} {what}")
        assert_bits(got[..., r:], src[..., r:], f"rope pass-through {name} {what}")
    # the rotation read from the library's cos/sin cache: the computed
    # rotation's bits, NaN and infinities included
    c, sn = et.rope_cache(dev(inv), int(pos.max()) + 1, r)
    qc, kc = dev(q), (dev(k) if k is not None else None)
    et.rope_qk_cached(qc, kc, dev(pos), c, sn, d_rot=r, attn_scaling=mu, layout=layout)
    assert_bits(host(qc), host(qt), f"cached rope q {what}")
    if k is not None:
        assert_bits(host(kc), host(kt), f"cached rope k {what}")
    q2, k2 = dev(q), (dev(k) if k is not None else None)
    et.rmsnorm_rope_qk(q2, dev(gq), k2, dev(gk) if k is not None else None, 1e-6, dev(pos), dev(inv),
                       d_rot=r, attn_scaling=mu, layout=layout)
    for name, src, gain, t in (("q", q, gq, q2), ("k", k, gk, k2)):
        if src is None:
            continue
        ref, y64 = orc.rmsnorm_rope(src, gain, 1e-6, pos, r, inv, mu, layout)
        _assert_pair_special(host(t), y64, ref, r, layout, f"rmsnorm_rope {name} {what}")
    dims = (r // 2 - (r // 2) % 2, r - (r // 2 - (r // 2) % 2))     # two even widths summing to r
    pm = np.stack([pos, pos[::-1]], axis=1).astype(np.int32)
    inv2 = wl.multi_inv_freq(dims, [1e4, 1e3])
    q3 = dev(q)
    et.rope_multi(q3, None, dev(pm), dims, dev(inv2), attn_scaling=mu, layout=layout)
    ref, y64 = orc.rope_multi(q, pm, dims, inv2, mu, layout)
    got = host(q3)
    o = 0
    for a, dw in enumerate(dims):
        if dw:
            _assert_pair_special(np.ascontiguousarray(got[..., o:o + dw]), np.ascontiguousarray(y64[..., o:o + dw]),
                                 np.ascontiguousarray(ref[..., o:o + dw]), dw, layout, f"multi axis {a} {what}")
        o += dw
    assert_bits(got[..., r:], q[..., r:], f"multi pass-through {what}")


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("seed", range(8))
def test_random_softmax_masks(et, orc, dt, seed):
    """Softmax of rows up to 140,000 entries under random masks: a stretch of
    -inf anywhere (whole 8192-entry chunks among them), top-k style rows
    with one to eight finite entries, rows entirely -inf (NaN rows), a NaN or
    a +inf planted (NaN rows); logits of scale 1 to 30 and temperatures from
    0.05 to 20; through a workspace, without one, and in place."""
    g = np.random.default_rng([5757, seed, DTS.index(dt)])
    n = _length(g, 1, 140000)
    rows = _rows(g, n, 1 << 20)
    x = (g.standard_normal((rows, n)) * g.choice([1.0, 3.0, 30.0])).astype(np.float32)
    for i in range(rows):
        kind = g.uniform()
        if kind < 0.4:
            a = int(g.integers(0, n))
            x[i, a:int(g.integers(a, n + 1))] = -np.inf
        elif kind < 0.6:
            keep = g.choice(n, size=min(n, int(g.integers(1, 9))), replace=False)
            row = np.full(n, -np.inf, np.float32)
            row[keep] = x[i, keep]
            x[i] = row
        elif kind < 0.65:
            x[i] = -np.inf
        elif kind < 0.7:
            x[i, int(g.integers(0, n))] = np.nan
        elif kind < 0.75:
            x[i, int(g.integers(0, n))] = np.inf
    xs = wl.store(x, dt)
    t = float(np.float32(g.choice([0.05, 0.7, 1.0, 20.0])))
    what = f"{dt} rows={rows} n={n} t={t}"
    y, y64 = orc.softmax(xs, t)
    check_softmax(host(et.softmax(dev(xs), t)), xs, t, y, y64, "softmax " + what)
    check_softmax(host(et.softmax(dev(xs), t, split=False)), xs, t, y, y64, "softmax no workspace " + what)
    xt = dev(xs)
    et.softmax(xt, t, out=xt)
    check_softmax(host(xt), xs, t, y, y64, "softmax in place " + what)


@pytest.mark.parametrize("seed", range(3))
def test_random_call_sequences_share_a_workspace(et, orc, seed):
    """A seeded sequence of argmax and softmax calls of random shapes and
    storage types, all through one caller-owned workspace sized for the
    largest: each result against the oracle, and the workspace zero-filled
    after every call (the contract that lets the next call reuse it)."""
    g = np.random.default_rng([5656, seed])
    shapes = []
    for _ in range(10):
        n = int(g.choice([_length(g, 2, 200000), (1024 * 8192) + int(g.integers(1, 9000))]))
        if n > 200000:
            rows = 1                                         # a row of more than 1024 chunks: two launches
        else:
            rows = _rows(g, n, 1 << 20)
        shapes.append((rows, n, DTS[int(g.integers(0, 3))], bool(g.uniform() < 0.5)))
    need = max(max(et.softmax_workspace_bytes(r, n), et.argmax_workspace_bytes(r, n)) for r, n, _, _ in shapes)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
    for i, (rows, n, dt, soft) in enumerate(shapes):
        x = wl.store(np.round(g.standard_normal((rows, n)) * 4).astype(np.float32), dt)
        xt = dev(x)
        what = f"call {i}: {'softmax' if soft else 'argmax'} {dt} {rows}x{n}"
        if soft:
            y, y64 = orc.softmax(x, 0.9)
            check_softmax(host(et.softmax(xt, 0.9, workspace=ws)), x, 0.9, y, y64, what)
        else:
            assert_bits(host(et.argmax(xt, workspace=ws)), orc.argmax(x), what)
        assert int(torch.count_nonzero(ws)) == 0, f"{what}: workspace not left zero-filled"
