"""Batch invariance and fused = unfused on the GPU.

Batch invariance ("Elementwise kernels in C ..." 2.1: a row's bits never
depend on its batch): every row op gives identical bits for a row computed
alone (batch 1) and inside batches of 64 and of a full prefill.

Fused = unfused ("Operations" 10 Fused ops): fused add+RMSNorm and fused
RMSNorm+RoPE agree with the unfused GPU chain within 1e-4 (f32) / 1e-2 (bf16)
relative, the page's tolerance for fused ops.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import assert_bits, dev, host, pair_norms, widen

pytestmark = pytest.mark.gpu

DTS = ["f32", "bf16", "f16"]


@pytest.fixture(scope="module")
def et():
    import elementwise_transformer_amd as m
    assert torch.cuda.is_available()
    return m


def _x(shape, dt, seed):
    g = np.random.default_rng([99, seed, *shape])
    return wl.store(g.standard_normal(shape).astype(np.float32) * 2, dt)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("d", [64, 1000, 4096, 8192, 40000])
def test_rmsnorm_rows_batch_invariant(et, dt, d):
    x = dev(_x((64, d), dt, 1))
    w = dev(wl.store(np.linspace(0.5, 1.5, d, dtype=np.float32), dt))
    full = host(et.rmsnorm(x, w, 1e-5))
    for r in (0, 1, 31, 63):
        one = host(et.rmsnorm(x[r:r + 1].contiguous(), w, 1e-5))
        assert_bits(one[0], full[r], f"rmsnorm row {r} d={d}")
    y2, h2 = et.add_rmsnorm(x, x.flip(0).contiguous(), w, 1e-5)
    y2, h2 = host(y2), host(h2)
    xf = x.flip(0).contiguous()
    for r in (0, 5, 63):
        y1, h1 = et.add_rmsnorm(x[r:r + 1].contiguous(), xf[r:r + 1].contiguous(), w, 1e-5)
        assert_bits(host(h1)[0], h2[r], f"h row {r}")
        assert_bits(host(y1)[0], y2[r], f"add_rmsnorm row {r}")


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("D,r,layout", [(128, 128, 0), (128, 64, 1), (96, 96, 0), (10, 6, 1)])
def test_qknorm_tokens_batch_invariant(et, dt, D, r, layout):
    T, Hq, Hk = 64, 8, 2
    q, k = _x((T, Hq, D), dt, 2), _x((T, Hk, D), dt, 3)
    gq = dev(wl.store(np.linspace(0.5, 1.5, D, dtype=np.float32), dt))
    gk = dev(wl.store(np.linspace(1.5, 0.5, D, dtype=np.float32), dt))
    pos = dev(np.random.default_rng(4).integers(0, 1 << 20, T).astype(np.int32))
    inv = dev(wl.inv_freq(1e4, r))
    qt, kt = dev(q), dev(k)
    et.rmsnorm_rope_qk(qt, gq, kt, gk, 1e-6, pos, inv, d_rot=r, layout=layout)
    for t in (0, 17, 63):
        q1, k1 = dev(q[t:t + 1]), dev(k[t:t + 1])
        et.rmsnorm_rope_qk(q1, gq, k1, gk, 1e-6, pos[t:t + 1].contiguous(), inv, d_rot=r,
                           layout=layout)
        assert_bits(host(q1)[0], host(qt)[t], f"q token {t}")
        assert_bits(host(k1)[0], host(kt)[t], f"k token {t}")


def test_prefill_slice_equals_full(et):
    """Rows of the 4096-token bf16 prefill computed as a 64-row slice equal
    the same rows of the full call."""
    w = wl.WORKLOADS[2]
    x, r, gain, eps = wl.gen_add_rmsnorm(w)
    xt, rt, gt = dev(x), dev(r), dev(gain)
    y, h = et.add_rmsnorm(xt, rt, gt, eps)
    y, h = host(y), host(h)
    for s in (0, 1000, 4032):
        ys, hs = et.add_rmsnorm(xt[s:s + 64].contiguous(), rt[s:s + 64].contiguous(), gt, eps)
        assert_bits(host(ys), y[s:s + 64], f"y slice {s}")
        assert_bits(host(hs), h[s:s + 64], f"h slice {s}")
    q, k, gq, gk, pos, inv = wl.gen_qknorm(w)
    s = w.rope
    qt, kt = dev(q), dev(k)
    et.rmsnorm_rope_qk(qt, dev(gq), kt, dev(gk), s.eps, dev(pos), dev(inv), d_rot=s.r,
                       layout=s.layout)
    qs, ks = dev(q[100:164]), dev(k[100:164])
    et.rmsnorm_rope_qk(qs, dev(gq), ks, dev(gk), s.eps, dev(pos[100:164]), dev(inv), d_rot=s.r,
                       layout=s.layout)
    assert_bits(host(qs), host(qt)[100:164], "q slice")
    assert_bits(host(ks), host(kt)[100:164], "k slice")


def _rel_close(a, b, rel, what):
    a, b = widen(a), widen(b)
    err = np.abs(a - b)
    lim = rel * np.maximum(np.abs(a), np.abs(b)) + 1e-30
    assert np.all(err <= lim), f"{what}: max rel {np.max(err / (np.abs(b) + 1e-30)):.3g}"


@pytest.mark.parametrize("dt", DTS)
def test_fused_add_rmsnorm_equals_unfused(et, dt):
    rel = 1e-4 if dt == "f32" else 1e-2
    x, res = dev(_x((33, 4096), dt, 5)), dev(_x((33, 4096), dt, 6))
    w = dev(wl.store(np.linspace(0.5, 1.5, 4096, dtype=np.float32), dt))
    y, h = et.add_rmsnorm(x, res, w, 1e-5)
    h2 = et.add(x, res)
    y2 = et.rmsnorm(h2, w, 1e-5)
    assert_bits(host(h), host(h2), "h")
    _rel_close(host(y), host(y2), rel, f"fused add+rmsnorm {dt}")


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("D,r,layout", [(128, 128, 0), (128, 64, 1)])
def test_fused_rmsnorm_rope_equals_unfused(et, dt, D, r, layout):
    rel = 1e-4 if dt == "f32" else 1e-2
    T, Hq, Hk = 16, 4, 2
    q, k = _x((T, Hq, D), dt, 7), _x((T, Hk, D), dt, 8)
    gq = dev(wl.store(np.linspace(0.5, 1.5, D, dtype=np.float32), dt))
    gk = dev(wl.store(np.linspace(1.5, 0.5, D, dtype=np.float32), dt))
    pos = dev(np.arange(T, dtype=np.int32) * 300)
    inv = dev(wl.inv_freq(1e4, r))
    qf, kf = dev(q), dev(k)
    et.rmsnorm_rope_qk(qf, gq, kf, gk, 1e-6, pos, inv, d_rot=r, attn_scaling=1.25, layout=layout)
    qu = et.rmsnorm(dev(q).view(T * Hq, D), gq, 1e-6).view(T, Hq, D)
    ku = et.rmsnorm(dev(k).view(T * Hk, D), gk, 1e-6).view(T, Hk, D)
    et.rope_qk(qu, ku, pos, inv, d_rot=r, attn_scaling=1.25, layout=layout)
    for name, a, b in (("q", qf, qu), ("k", kf, ku)):
        an, bn = widen(host(a)), widen(host(b))
        # rotated entries: relative to the pair's length (a cos - b sin cancels
        # per element); normalised-only tail: relative to the entry
        scale = np.abs(bn)
        scale[..., :r] = pair_norms(bn, r, layout)[..., :r]
        assert np.all(np.abs(an - bn) <= rel * scale + 1e-30), f"fused qknorm {name} {dt}"


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("d", [64, 4096, 8192, 40000])
def test_rmsnorm_scalar_path_same_bits(et, dt, d):
    """A misaligned buffer takes the scalar path, which keeps the vector
    path's element ownership and summation tree: identical bits."""
    x = dev(_x((8, d), dt, 11))
    r = dev(_x((8, d), dt, 12))
    w = dev(wl.store(np.linspace(0.5, 1.5, d, dtype=np.float32), dt))
    flat = torch.empty(x.numel() + 8, dtype=x.dtype, device="cuda")
    xm = flat[1:1 + x.numel()].view(x.shape)
    xm.copy_(x)
    assert xm.data_ptr() % 16 != 0
    assert_bits(host(et.rmsnorm(xm, w, 1e-5)), host(et.rmsnorm(x, w, 1e-5)), f"rmsnorm d={d}")
    ya, ha = et.add_rmsnorm(x, r, w, 1e-5)
    yb, hb = et.add_rmsnorm(xm, r, w, 1e-5)
    assert_bits(host(hb), host(ha), f"h d={d}")
    assert_bits(host(yb), host(ya), f"add_rmsnorm d={d}")
