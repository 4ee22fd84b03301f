"""GPU parity of RoPE with a precomputed cos/sin cache, through the C ABI.

Three claims, each its own test:
  * the cache the library builds (et_rope_cache_f32) is within 1.5e-7
    absolute of the oracle's correctly rounded cos and sin: the kernel's
    sine and cosine are accurate to 1e-7 absolute, the oracle's f32
    rounding adds at most 2^-25;
  * a rotation read from that cache gives the same bits as the computed
    rotation (et_rope_qk_*): same angles, same sine and cosine, same
    arithmetic after the table;
  * a rotation read from the ORACLE's cache matches the oracle's cached
    rotation within the PAIR tolerance of gpu_util (the cos/sin values are
    then exact inputs on both sides), and positions outside the cache give
    NaN in the rotated entries only.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import assert_bits, assert_pair, dev, host, widen

pytestmark = pytest.mark.gpu

DTS = ["f32", "bf16", "f16"]
CACHE_ABS = 1.5e-7


@pytest.fixture(scope="module")
def et():
    import elementwise_transformer_amd as m
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return m


def _rng(*key):
    return np.random.default_rng([4545, *key])


def _misaligned(t):
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    v = flat[1:1 + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0
    return v


@pytest.mark.parametrize("r,theta,max_pos", [(128, 5e5, 8192), (64, 1e4, 1 << 17), (6, 1e2, 100),
                                             (2, 1e4, 1), (128, 1e6, 4097)])
def test_rope_cache_matches_oracle(et, orc, r, theta, max_pos):
    inv = wl.inv_freq(theta, r)
    c, s = et.rope_cache(dev(inv), max_pos, r)
    oc, os_ = orc.rope_cache(inv, max_pos, r)
    for name, got, ref in (("cos", host(c), oc), ("sin", host(s), os_)):
        err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
        bad = np.flatnonzero(~(err <= CACHE_ABS))
        assert bad.size == 0, f"{name} r={r} max_pos={max_pos}: {bad.size} entries off by " \
                              f"up to {err.max():.3g}"
    # position 0: the angle is 0, cos 1 and sin 0 exactly
    assert np.all(host(c)[0] == 1.0) and np.all(host(s)[0] == 0.0)


def test_rope_cache_high_frequencies(et, orc):
    """Frequencies up to 1 rad per position at positions to 2^20: angles near
    1e6 rad still reduce accurately."""
    inv = np.array([1.0, 0.999, 0.5, 0.25, 1e-3, 1e-5, 3.3e-8, 0.7071], np.float32)
    c, s = et.rope_cache(dev(inv), 1 << 20, 16)
    oc, os_ = orc.rope_cache(inv, 1 << 20, 16)
    assert np.max(np.abs(host(c).astype(np.float64) - oc)) <= CACHE_ABS
    assert np.max(np.abs(host(s).astype(np.float64) - os_)) <= CACHE_ABS


ROPE_CASES = [
    # T, Hq, Hk, D, r, layout, mu, pos_hi
    (5, 3, 2, 128, 128, 0, 1.0, 4096),
    (5, 3, 2, 128, 128, 1, 1.0, 4096),
    (7, 4, 0, 128, 64, 1, 1.1, 1 << 20),
    (7, 4, 0, 128, 64, 0, 1.1, 1 << 20),
    (3, 2, 1, 10, 6, 0, 2.0, 100),        # scalar path (r not a multiple of 2V)
    (3, 2, 1, 10, 6, 1, 0.5, 100),
    (33, 32, 8, 128, 128, 0, 1.0, 8192),
    (9, 2, 2, 64, 0, 0, 1.0, 10),         # nothing rotates
    (1, 64, 8, 128, 128, 0, 1.0, 8191),
    (70, 5, 3, 32, 16, 0, 1.0, 70000),
    (300, 8, 2, 128, 128, 1, 1.0, 5000),  # many workgroups
]


def _inputs(case, dt, key):
    T, Hq, Hk, D, r, layout, mu, pos_hi = case
    g = _rng(key, DTS.index(dt))
    q = wl.store(g.standard_normal((T, Hq, D)).astype(np.float32), dt)
    k = wl.store(g.standard_normal((T, Hk, D)).astype(np.float32), dt) if Hk else None
    pos = g.integers(0, pos_hi, T).astype(np.int32)
    inv = wl.inv_freq(1e4, r) if r else np.zeros(1, np.float32)
    return q, k, pos, inv


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("ci", range(len(ROPE_CASES)))
def test_rope_cached_equals_computed(et, dt, ci):
    """The library's own cache reproduces the computed rotation bit for bit,
    on the vector and the scalar (misaligned) path."""
    case = ROPE_CASES[ci]
    T, Hq, Hk, D, r, layout, mu, pos_hi = case
    q, k, pos, inv = _inputs(case, dt, ci)
    mu = float(np.float32(mu))
    c, s = et.rope_cache(dev(inv), pos_hi, r)
    qa, ka = dev(q), (dev(k) if k is not None else None)
    et.rope_qk(qa, ka, dev(pos), dev(inv), d_rot=r, attn_scaling=mu, layout=layout)
    qb, kb = dev(q), (dev(k) if k is not None else None)
    et.rope_qk_cached(qb, kb, dev(pos), c, s, d_rot=r, attn_scaling=mu, layout=layout)
    assert_bits(host(qb), host(qa), f"{dt} case {ci} q")
    if k is not None:
        assert_bits(host(kb), host(ka), f"{dt} case {ci} k")
    qm = _misaligned(dev(q))
    et.rope_qk_cached(qm, None, dev(pos), c, s, d_rot=r, attn_scaling=mu, layout=layout)
    assert_bits(host(qm), host(qa), f"{dt} case {ci} misaligned")


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("ci", range(len(ROPE_CASES)))
def test_rope_cached_oracle_cache(et, orc, dt, ci):
    """With the oracle's cache as the input on both sides, the rotation
    matches the oracle's cached rotation within the PAIR tolerance, and the
    entries past d_rot are untouched."""
    case = ROPE_CASES[ci]
    T, Hq, Hk, D, r, layout, mu, pos_hi = case
    q, k, pos, inv = _inputs(case, dt, 50 + ci)
    mu = float(np.float32(mu))
    oc, os_ = orc.rope_cache(inv, pos_hi, r)
    qt, kt = dev(q), (dev(k) if k is not None else None)
    et.rope_qk_cached(qt, kt, dev(pos), dev(oc), dev(os_), d_rot=r, attn_scaling=mu, layout=layout)
    for name, src, t in (("q", q, qt), ("k", k, kt)):
        if src is None:
            continue
        ref, y64 = orc.rope_cached(src, pos, r, oc, os_, mu, layout)
        got = host(t)
        assert_pair(got, y64, ref, r, layout, f"cached {name} {dt} case {ci}")
        assert_bits(got[..., r:], src[..., r:], f"pass-through {name}")


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("layout", [0, 1])
def test_rope_cached_out_of_range_positions(et, orc, dt, layout):
    """Positions outside [0, max_pos) -- negative, max_pos itself, INT32_MAX
    -- rotate to NaN on the first d_rot entries of every head of that token;
    the other tokens and the pass-through entries are as computed."""
    g = _rng(90, layout, DTS.index(dt))
    T, Hq, Hk, D, r, max_pos = 40, 3, 2, 64, 48, 1000
    q = wl.store(g.standard_normal((T, Hq, D)).astype(np.float32), dt)
    k = wl.store(g.standard_normal((T, Hk, D)).astype(np.float32), dt)
    pos = g.integers(0, max_pos, T).astype(np.int32)
    bad = [0, 7, 19, 39]
    pos[bad] = [-1, max_pos, 2**31 - 1, -2**31]
    oc, os_ = orc.rope_cache(wl.inv_freq(1e4, r), max_pos, r)
    qt, kt = dev(q), dev(k)
    et.rope_qk_cached(qt, kt, dev(pos), dev(oc), dev(os_), d_rot=r, layout=layout)
    for name, src, t in (("q", q, qt), ("k", k, kt)):
        got = host(t)
        ref, y64 = orc.rope_cached(src, pos, r, oc, os_, 1.0, layout)
        assert np.all(np.isnan(widen(got[bad, :, :r]))), f"{name}: bad positions not NaN"
        assert np.array_equal(np.isnan(widen(got)), np.isnan(y64)), f"{name}: NaN positions"
        assert_bits(got[..., r:], src[..., r:], f"{name} pass-through")
        ok = np.setdiff1d(np.arange(T), bad)
        assert_pair(got[ok], y64[ok], ref[ok], r, layout, f"{name} in-range tokens")


@pytest.mark.parametrize("dt", DTS)
def test_rope_cached_empty_cache(et, dt):
    """max_pos == 0 with NULL caches: every token's rotated entries are NaN;
    T == 0 is a no-op."""
    g = _rng(91, DTS.index(dt))
    q = wl.store(g.standard_normal((4, 2, 16)).astype(np.float32), dt)
    qt = dev(q)
    e = torch.empty((0, 4), dtype=torch.float32, device="cuda")
    et.rope_qk_cached(qt, None, dev(np.arange(4, dtype=np.int32)), e, e, d_rot=8)
    got = host(qt)
    assert np.all(np.isnan(widen(got[..., :8])))
    assert_bits(got[..., 8:], q[..., 8:], "pass-through")
    z = torch.empty((0, 2, 16), dtype=qt.dtype, device="cuda")
    et.rope_qk_cached(z, None, torch.empty(0, dtype=torch.int32, device="cuda"), e, e, d_rot=8)


def test_rope_cached_prefill_full_size(et, orc):
    """The prefill rotation at its timed size, q [4096, 32, 128] and k
    [4096, 8, 128] bf16, positions 0..4095, theta 5e5, from the library's
    cache: bit-equal to the computed rotation; sampled tokens against the
    oracle's cached rotation with the oracle's cache."""
    w = wl.WORKLOADS[2]
    q, k, pos, inv = wl.gen_rope(w)
    s = w.rope
    c, sn = et.rope_cache(dev(inv), s.T, s.r)
    qa, ka = dev(q), dev(k)
    et.rope_qk(qa, ka, dev(pos), dev(inv), d_rot=s.r, attn_scaling=s.mu, layout=s.layout)
    qb, kb = dev(q), dev(k)
    et.rope_qk_cached(qb, kb, dev(pos), c, sn, d_rot=s.r, attn_scaling=s.mu, layout=s.layout)
    assert_bits(host(qb), host(qa), "prefill cached q")
    assert_bits(host(kb), host(ka), "prefill cached k")
    oc, os_ = orc.rope_cache(inv, s.T, s.r)
    qo = dev(q)
    et.rope_qk_cached(qo, None, dev(pos), dev(oc), dev(os_), d_rot=s.r, attn_scaling=s.mu,
                      layout=s.layout)
    toks = [0, 1, 2047, 4095]
    sub = np.ascontiguousarray(q[toks])
    ref, y64 = orc.rope_cached(sub, pos[toks], s.r, oc, os_, s.mu, s.layout)
    assert_pair(host(qo)[toks], y64, ref, s.r, s.layout, "prefill oracle cache")
