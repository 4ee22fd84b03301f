"""GPU parity of multi-axis (3D) RoPE against the CPU oracle, through the C ABI.

Tolerance: the PAIR tolerance of gpu_util, applied per axis (each axis's
sub-range is a head of its own width, paired inside it); entries past the
last sub-range must keep their bits.  Further claims, each its own test:
one axis of width r gives the bits of the single-axis RoPE entry point; the
scalar path (misaligned buffers) gives the vector path's bits; results do
not depend on the rows beside them.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import assert_bits, assert_pair, dev, host

pytestmark = pytest.mark.gpu

DTS = ["f32", "bf16", "f16"]


@pytest.fixture(scope="module")
def et():
    import elementwise_transformer_amd as m
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return m


def _rng(*key):
    return np.random.default_rng([4646, *key])


def _misaligned(t):
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    v = flat[1:1 + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0
    return v


def assert_multi(got, y64, ref, dims, layout, what):
    """PAIR tolerance per axis sub-range; bits kept past the last one."""
    o = 0
    for a, d in enumerate(dims):
        if d:
            assert_pair(np.ascontiguousarray(got[..., o:o + d]), np.ascontiguousarray(y64[..., o:o + d]),
                        np.ascontiguousarray(ref[..., o:o + d]), d, layout, f"{what} axis {a}")
        o += d
    assert_bits(np.ascontiguousarray(got[..., o:]), np.ascontiguousarray(ref[..., o:]), f"{what} tail")


CASES = [
    # T, Hq, Hk, D, dims, layout, mu, pos_hi
    (7, 4, 2, 128, (16, 56, 56), 0, 1.0, 64),          # halves of 28: not whole bf16 vectors
    (7, 4, 2, 128, (16, 56, 56), 1, 1.0, 64),
    (9, 3, 1, 128, (32, 48, 48), 0, 1.0, 100),         # halves on vector boundaries
    (6, 3, 0, 96, (32, 32, 16), 1, 1.1, 1000),         # partial: 80 of 96, no k
    (4, 2, 1, 10, (2, 4), 0, 2.0, 50),                 # scalar path (D not whole vectors)
    (300, 8, 2, 128, (44, 42, 42), 0, 1.0, 30000),     # many workgroups, odd half widths
    (3, 2, 2, 32, (8, 0, 24), 0, 1.0, 10),             # a zero-width axis
    (70, 5, 3, 64, (16, 16, 16, 16), 1, 0.5, 1 << 20), # four axes, large positions
    (1, 64, 8, 128, (16, 56, 56), 0, 1.0, 100),        # one token, many heads
    (33, 1, 0, 1024, (512, 256, 256), 0, 1.0, 5000),   # widest span, one head per token
    (5, 2, 3, 256, (2, 2, 2, 2, 2, 2, 2, 242), 1, 1.0, 7),  # eight axes
    (6, 3, 2, 512, (128, 192, 192), 0, 1.0, 500),      # a 2-byte head row of 64 vectors: one wave
    (9, 4, 1, 256, (64, 96, 96), 0, 1.0, 500),         # 32 vectors (2-byte), 64 (f32) per head row
]


def _inputs(case, dt, key):
    T, Hq, Hk, D, dims, layout, mu, pos_hi = case
    g = _rng(key, DTS.index(dt))
    q = wl.store(g.standard_normal((T, Hq, D)).astype(np.float32), dt)
    k = wl.store(g.standard_normal((T, Hk, D)).astype(np.float32), dt) if Hk else None
    pos = g.integers(-(pos_hi // 4), pos_hi, (T, len(dims))).astype(np.int32)
    thetas = [(1e4, 1e3, 5e2, 1e2)[a % 4] for a in range(len(dims))]
    inv = wl.multi_inv_freq(dims, thetas) if sum(dims) else np.zeros(1, np.float32)
    return q, k, pos, inv


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_rope_multi_matches_oracle(et, orc, dt, ci):
    case = CASES[ci]
    T, Hq, Hk, D, dims, layout, mu, _ = case
    q, k, pos, inv = _inputs(case, dt, ci)
    mu = float(np.float32(mu))
    qt, kt = dev(q), (dev(k) if k is not None else None)
    et.rope_multi(qt, kt, dev(pos), dims, dev(inv), attn_scaling=mu, layout=layout)
    for name, src, t in (("q", q, qt), ("k", k, kt)):
        if src is None:
            continue
        ref, y64 = orc.rope_multi(src, pos, dims, inv, mu, layout)
        assert_multi(host(t), y64, ref, dims, layout, f"multi {name} {dt} case {ci}")
    # the scalar path (misaligned q) gives the vector path's bits
    qm = _misaligned(dev(q))
    et.rope_multi(qm, None, dev(pos), dims, dev(inv), attn_scaling=mu, layout=layout)
    assert_bits(host(qm), host(qt), f"{dt} case {ci} misaligned")


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("D,r", [(128, 128), (128, 64), (64, 24), (10, 6)])
def test_rope_multi_single_axis_is_rope(et, dt, layout, D, r):
    """One axis of width r rotates as the RoPE entry point with d_rot = r,
    bit for bit."""
    g = _rng(70, D, r, layout, DTS.index(dt))
    T, Hq, Hk = 37, 6, 2
    q = wl.store(g.standard_normal((T, Hq, D)).astype(np.float32), dt)
    k = wl.store(g.standard_normal((T, Hk, D)).astype(np.float32), dt)
    pos = g.integers(0, 1 << 16, T).astype(np.int32)
    inv = wl.inv_freq(1e4, r)
    qa, ka = dev(q), dev(k)
    et.rope_qk(qa, ka, dev(pos), dev(inv), d_rot=r, attn_scaling=1.25, layout=layout)
    qb, kb = dev(q), dev(k)
    et.rope_multi(qb, kb, dev(pos.reshape(T, 1)), [r], dev(inv), attn_scaling=1.25, layout=layout)
    assert_bits(host(qb), host(qa), f"{dt} D={D} r={r} q")
    assert_bits(host(kb), host(ka), f"{dt} D={D} r={r} k")


@pytest.mark.parametrize("dt", DTS)
def test_rope_multi_rows_independent(et, dt):
    """A token's result does not depend on the other tokens of the call."""
    case = (200, 4, 2, 128, (16, 56, 56), 0, 1.0, 64)
    q, k, pos, inv = _inputs(case, dt, 80)
    qt, kt = dev(q), dev(k)
    et.rope_multi(qt, kt, dev(pos), case[4], dev(inv))
    full_q, full_k = host(qt), host(kt)
    for t in (0, 77, 199):
        q1, k1 = dev(np.ascontiguousarray(q[t:t + 1])), dev(np.ascontiguousarray(k[t:t + 1]))
        et.rope_multi(q1, k1, dev(np.ascontiguousarray(pos[t:t + 1])), case[4], dev(inv))
        assert_bits(host(q1)[0], full_q[t], f"{dt} token {t} q")
        assert_bits(host(k1)[0], full_k[t], f"{dt} token {t} k")


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("layout", [0, 1])
def test_rope_multi_wave_paths_agree(et, dt, layout):
    """With 24 query and 24 key heads every wave's 16 head rows lie in one
    token, so the kernel takes its batched path (one set of angles per lane,
    all partner reads issued together); with the 24 query heads alone the
    waves straddle tokens and take the per-slot path.  The query rows come
    out with the same bits either way."""
    case = (40, 24, 24, 128, (16, 56, 56), layout, 1.0, 64)
    q, k, pos, inv = _inputs(case, dt, 90 + layout)
    qa, ka = dev(q), dev(k)
    et.rope_multi(qa, ka, dev(pos), case[4], dev(inv), layout=layout)
    qb = dev(q)
    et.rope_multi(qb, None, dev(pos), case[4], dev(inv), layout=layout)
    assert_bits(host(qb), host(qa), f"{dt} layout {layout} q alone against q with k")


def test_rope_multi_degenerate(et):
    """T == 0, no heads and all-zero widths are no-ops; bad arguments raise."""
    z = torch.empty((0, 2, 16), device="cuda")
    et.rope_multi(z, None, torch.empty((0, 2), dtype=torch.int32, device="cuda"), [4, 4],
                  torch.zeros(4, device="cuda"))
    x = torch.randn((3, 2, 16), device="cuda")
    ref = x.clone()
    et.rope_multi(x, None, torch.zeros((3, 2), dtype=torch.int32, device="cuda"), [0, 0],
                  torch.zeros(1, device="cuda"))
    assert torch.equal(x, ref)
    with pytest.raises(Exception):
        et.rope_multi(x, None, torch.zeros((3, 2), dtype=torch.int32, device="cuda"), [4, 3],
                      torch.zeros(4, device="cuda"))


def test_rope_multi_video_full_size(et, orc):
    """The video DiT rotation at its timed size: q and k [19200, 24, 128]
    bf16 over a 16 x 30 x 40 latent grid, widths 16 / 56 / 56, base 256;
    sampled tokens (first, last, frame and row boundaries) against the
    oracle."""
    w = wl.WORKLOADS[6]
    s = w.rope_multi
    q, k, pos, inv = wl.gen_rope_multi(w)
    qt, kt = dev(q), dev(k)
    et.rope_multi(qt, kt, dev(pos), s.dims, dev(inv), attn_scaling=s.mu, layout=s.layout)
    toks = [0, 1, 39, 40, 1199, 1200, 9601, s.T - 1]
    for name, src, t in (("q", q, qt), ("k", k, kt)):
        sub = np.ascontiguousarray(src[toks])
        ref, y64 = orc.rope_multi(sub, pos[toks], s.dims, inv, s.mu, s.layout)
        assert_multi(host(t)[toks], y64, ref, s.dims, s.layout, f"video {name}")


def _random_case(g):
    """Random even widths (some zero, some narrower than a vector), a head
    at least as wide as their sum, either pairing, mixed signs of positions."""
    A = int(g.integers(1, 9))
    dims = [int(2 * g.integers(0, 40)) for _ in range(A)]
    if sum(dims) == 0:
        dims[0] = 2
    span = sum(dims)
    D = span + int(g.choice([0, 0, 2, 8, 16]))
    if D > 1024:
        return None
    T, Hq, Hk = int(g.integers(1, 40)), int(g.integers(1, 6)), int(g.integers(0, 4))
    return T, Hq, Hk, D, tuple(dims), int(g.integers(0, 2)), float(g.choice([1.0, 0.75])), int(g.integers(2, 1 << 16))


@pytest.mark.parametrize("seed", range(24))
def test_rope_multi_random_geometry(et, orc, seed):
    """Seeded random axis geometries in every storage type: oracle parity
    (per-axis PAIR tolerance, tail bits kept) and the scalar path's bits
    equal to the vector path's."""
    g = np.random.default_rng([4747, seed])
    case = None
    while case is None:
        case = _random_case(g)
    T, Hq, Hk, D, dims, layout, mu, pos_hi = case
    for dt in DTS:
        q, k, pos, inv = _inputs(case, dt, 1000 + seed)
        qt, kt = dev(q), (dev(k) if k is not None else None)
        et.rope_multi(qt, kt, dev(pos), dims, dev(inv), attn_scaling=mu, layout=layout)
        for name, src, t in (("q", q, qt), ("k", k, kt)):
            if src is None:
                continue
            ref, y64 = orc.rope_multi(src, pos, dims, inv, mu, layout)
            assert_multi(host(t), y64, ref, dims, layout, f"random {seed} {dt} {case} {name}")
        qm = _misaligned(dev(q))
        et.rope_multi(qm, None, dev(pos), dims, dev(inv), attn_scaling=mu, layout=layout)
        assert_bits(host(qm), host(qt), f"random {seed} {dt} {case} misaligned")
