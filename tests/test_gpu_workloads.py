"""Full-size workloads on the GPU, in the launch configuration the benchmark
times, checked against the oracle on sampled rows (the oracle is row-wise, so
a sampled row is checked exactly as in a full comparison).

Workloads (shapes of Llama-style prefill and decode):
  2  Llama-3-8B prefill, bf16, T = 4096 (the benchmark step)
  3  decode, f32, 256 sequences of one token
  4  partial (r = 64 of 128) interleaved RoPE, f32, T = 16384, mu = 1.1
  5  large hidden, bf16, T = 8192, hidden 8192, in-place fused add + RMSNorm
  2 in f16: the prefill step with f16 storage (the benchmark's f16 step)
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import assert_bits, assert_close, assert_pair, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def et():
    import elementwise_transformer_amd as m
    assert torch.cuda.is_available()
    return m


def _sample(n, k, seed):
    g = np.random.default_rng([77, seed, n])
    pick = set(g.choice(n, size=min(k, n), replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(pick))


def _check_norm(et, orc, w, in_place=None):
    rows, d, eps = w.rmsnorm
    x, gain, eps = wl.gen_rmsnorm(w)
    y = host(et.rmsnorm(dev(x), dev(gain), eps))
    rs = _sample(rows, 24, w.number)
    yr, y64 = orc.rmsnorm(x[rs], gain, eps)
    assert_close(y[rs], y64, yr, f"rmsnorm workload {w.number}")


def _check_add_rmsnorm(et, orc, w):
    rows, d, eps, in_place = w.add_rmsnorm
    x, r, gain, eps = wl.gen_add_rmsnorm(w)
    xt, rt = dev(x), dev(r)
    if in_place:
        et.add_rmsnorm(xt, rt, dev(gain), eps, out=xt, h=rt)
        y, h = host(xt), host(rt)
    else:
        yt, ht = et.add_rmsnorm(xt, rt, dev(gain), eps)
        y, h = host(yt), host(ht)
    rs = _sample(rows, 24, w.number)
    yr, hr, y64 = orc.add_rmsnorm(x[rs], r[rs], gain, eps)
    assert_bits(h[rs], hr, f"h workload {w.number}")
    assert_close(y[rs], y64, yr, f"y workload {w.number}")


def _check_rope(et, orc, w):
    s = w.rope
    q, k, pos, inv = wl.gen_rope(w)
    qt, kt = dev(q), (dev(k) if k is not None else None)
    et.rope_qk(qt, kt, dev(pos), dev(inv), d_rot=s.r, attn_scaling=s.mu, layout=s.layout)
    ts = _sample(s.T, 32, w.number)
    for name, src, t in (("q", q, qt), ("k", k, kt)):
        if src is None:
            continue
        got = host(t)[ts]
        ref, y64 = orc.rope(src[ts], pos[ts], s.r, inv, s.mu, s.layout)
        assert_pair(got, y64, ref, s.r, s.layout, f"rope {name} workload {w.number}")
        assert_bits(got[..., s.r:], src[ts][..., s.r:], "pass-through")


def _check_qknorm(et, orc, w):
    s = w.rope
    q, k, gq, gk, pos, inv = wl.gen_qknorm(w)
    qt, kt = dev(q), (dev(k) if k is not None else None)
    et.rmsnorm_rope_qk(qt, dev(gq), kt, dev(gk) if k is not None else None, s.eps, dev(pos),
                       dev(inv), d_rot=s.r, attn_scaling=s.mu, layout=s.layout)
    ts = _sample(s.T, 32, w.number + 10)
    for name, src, gain, t in (("q", q, gq, qt), ("k", k, gk, kt)):
        if src is None:
            continue
        got = host(t)[ts]
        ref, y64 = orc.rmsnorm_rope(src[ts], gain, s.eps, pos[ts], s.r, inv, s.mu, s.layout)
        assert_pair(got, y64, ref, s.r, s.layout, f"qknorm {name} workload {w.number}")
        assert_close(got[..., s.r:], y64[..., s.r:], ref[..., s.r:], "qknorm tail")


def _check_silu(et, orc, w):
    rows, cols, _ = w.silu
    gate, up = wl.gen_silu(w)
    y = host(et.silu_mul(dev(gate), dev(up)))
    rs = _sample(rows, 12, w.number)
    yr, y64 = orc.silu_mul(gate[rs], up[rs])
    assert_close(y[rs], y64, yr, f"silu_mul workload {w.number}")


def _check_add(et, orc, w):
    rows, d = w.add
    a, b = wl.gen_add(w)
    y = host(et.add(dev(a), dev(b)))
    rs = _sample(rows, 24, w.number)
    assert_bits(y[rs], orc.add(a[rs], b[rs]), f"add workload {w.number}")


def _check_embedding(et, orc, w):
    table, ids = wl.gen_embedding(w)
    tt = dev(table)
    out = host(et.embedding(tt, dev(ids)))
    rs = _sample(ids.size, 32, w.number)
    assert_bits(out[rs], orc.embedding(table, ids[rs]), f"embedding workload {w.number}")


def _check_argmax(et, orc, w):
    x, plan = wl.gen_argmax(w)
    got = host(et.argmax(dev(x)))
    assert_bits(got, orc.argmax(x), f"argmax workload {w.number}")
    for r in plan["nans"]:
        assert got[r] >= 0
    got1 = host(et.argmax(dev(x), split=False))
    assert_bits(got1, got, "argmax without a workspace")


CHECKS = {
    2: ["embedding", "add", "rmsnorm", "add_rmsnorm", "rope", "qknorm", "silu", "argmax"],
    3: ["embedding", "rmsnorm", "rope", "qknorm", "argmax"],
    4: ["rope", "qknorm"],
    5: ["add_rmsnorm", "rope", "qknorm", "silu"],
}
FN = {"embedding": _check_embedding, "add": _check_add, "rmsnorm": _check_norm,
      "add_rmsnorm": _check_add_rmsnorm, "rope": _check_rope, "qknorm": _check_qknorm,
      "silu": _check_silu, "argmax": _check_argmax}


@pytest.mark.parametrize("number,op", [(n, op) for n, ops in CHECKS.items() for op in ops])
def test_workload(et, orc, number, op):
    print(f"workload {number} {op}", flush=True)
    FN[op](et, orc, wl.WORKLOADS[number])
    torch.cuda.synchronize()


@pytest.mark.parametrize("op", CHECKS[2])
def test_prefill_f16(et, orc, op):
    """The prefill step's ops at full size with f16 storage, as the benchmark
    times them: sampled rows against the oracle (1 f16 ulp; bits where the
    op is exact)."""
    print(f"prefill f16 {op}", flush=True)
    FN[op](et, orc, dataclasses.replace(wl.WORKLOADS[2], dtype="f16"))
    torch.cuda.synchronize()


@pytest.mark.parametrize("layout,r", [(0, 128), (1, 64)])
def test_rope_and_qknorm_past_128_mib_with_mixed_heads(et, orc, layout, r):
    """RoPE and the fused RMSNorm+RoPE on bf16 q [70000, 5, 128] and k [70000,
    3, 128]: 143 MB rotated, so the stores are non-temporal, and every store
    instruction of a wave covers query and key heads of one token, so each one
    takes the path for waves that straddle the two (the large-hidden shape,
    64 + 8 heads, never does).  Sampled tokens against the oracle."""
    T, Hq, Hk, D, eps, mu = 70000, 5, 3, 128, 1e-5, 1.0
    g = np.random.default_rng([31, layout, r])
    q = wl.store(g.standard_normal((T, Hq, D)).astype(np.float32), "bf16")
    k = wl.store(g.standard_normal((T, Hk, D)).astype(np.float32), "bf16")
    gq = wl.store(g.uniform(0.5, 1.5, D).astype(np.float32), "bf16")
    gk = wl.store(g.uniform(0.5, 1.5, D).astype(np.float32), "bf16")
    pos = g.integers(0, 1 << 17, T).astype(np.int32)
    inv = wl.inv_freq(5e5, r)
    assert T * (Hq + Hk) * D * 2 > 128 << 20
    ts = _sample(T, 40, 900 + layout)
    qt, kt = dev(q), dev(k)
    et.rope_qk(qt, kt, dev(pos), dev(inv), d_rot=r, attn_scaling=mu, layout=layout)
    for name, src, t in (("q", q, qt), ("k", k, kt)):
        got = host(t)[ts]
        ref, y64 = orc.rope(src[ts], pos[ts], r, inv, mu, layout)
        assert_pair(got, y64, ref, r, layout, f"rope {name}")
        assert_bits(got[..., r:], src[ts][..., r:], "pass-through")
    qt, kt = dev(q), dev(k)
    et.rmsnorm_rope_qk(qt, dev(gq), kt, dev(gk), eps, dev(pos), dev(inv), d_rot=r, attn_scaling=mu,
                       layout=layout)
    for name, src, gain, t in (("q", q, gq, qt), ("k", k, gk, kt)):
        got = host(t)[ts]
        ref, y64 = orc.rmsnorm_rope(src[ts], gain, eps, pos[ts], r, inv, mu, layout)
        assert_pair(got, y64, ref, r, layout, f"qknorm {name}")
        assert_close(got[..., r:], y64[..., r:], ref[..., r:], "qknorm tail")
