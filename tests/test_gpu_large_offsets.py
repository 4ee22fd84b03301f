"""Tensors past 2^31 elements, through the C ABI: every element offset, row
offset and store resource must hold 64-bit positions (bf16 storage, 4.3 GB
and more per tensor).  Inputs are drawn on the device; the oracle runs on
sampled rows, tokens or elements (rows, tokens and elements are
independent), including the first and the last, with each op's tolerance.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import assert_bits, assert_close, assert_pair, check_layernorm, check_softmax, host

pytestmark = pytest.mark.gpu

BIG = (1 << 31) + 1000


@pytest.fixture(scope="module")
def et():
    import elementwise_transformer_amd as m
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return m


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _randn(shape, seed, scale=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda") * scale).to(torch.bfloat16)


def test_embedding_rows_past_2_31(et, orc):
    V, d = 270000, 8192                              # 2.2e9 elements; row V-1 starts at 2.2e9
    table = _randn((V, d), 1)
    ids = np.array([V - 1, 0, 262144, V - 2, 131072, -1, V, 262145], np.int32)
    out = host(et.embedding(table, torch.from_numpy(ids).cuda()))
    ok = (ids >= 0) & (ids < V)
    rows = host(table[torch.from_numpy(ids[ok]).long().cuda()])
    remap = np.where(ok, np.cumsum(ok) - 1, ids).astype(np.int32)   # the gathered rows as the table
    remap[~ok] = len(rows)                                           # out of range there too
    assert_bits(out, orc.embedding(rows, remap), "embedding past 2^31")


def test_norms_rows_past_2_31(et, orc):
    rows, d = (1 << 19) + 3, 4096                    # 2.15e9 elements per tensor
    x = _randn((rows, d), 2, 2.0)
    res = _randn((rows, d), 3)
    w = _randn((d,), 4, 0.2) + 1.0
    b = _randn((d,), 5)
    pick = [0, 1, (1 << 18) + 7, rows - 2, rows - 1]
    xs, rs, ws, bs = host(x[pick]), host(res[pick]), host(w), host(b)
    y = et.rmsnorm(x, w, 1e-5)
    yr, y64 = orc.rmsnorm(xs, ws, 1e-5)
    assert_close(host(y[pick]), y64, yr, "rmsnorm past 2^31")
    y = et.layernorm(x, w, b, 1e-5, out=y)
    ly, ly64 = orc.layernorm(xs, ws, bs, 1e-5)
    check_layernorm(host(y[pick]), xs, ws, bs, 1e-5, ly, ly64, "layernorm past 2^31")
    y, h = et.add_rmsnorm(x, res, w, 1e-5, out=y)
    oy, oh, oy64 = orc.add_rmsnorm(xs, rs, ws, 1e-5)
    assert_bits(host(h[pick]), oh, "add_rmsnorm h past 2^31")
    assert_close(host(y[pick]), oy64, oy, "add_rmsnorm y past 2^31")


def test_flat_ops_past_2_31(et, orc):
    a = _randn((BIG,), 6, 3.0)
    b = _randn((BIG,), 7)
    g = np.random.default_rng(8)
    pick = np.concatenate([[0, 1, (1 << 31) - 1, 1 << 31], g.integers(0, BIG, 2000), BIG - 1 - np.arange(40)])
    pt = torch.from_numpy(pick).cuda()
    a_s, b_s = host(a[pt]), host(b[pt])
    y = et.add(a, b)
    assert_bits(host(y[pt]), orc.add(a_s, b_s), "add past 2^31")
    y = et.silu_mul(a, b, out=y)
    yr, y64 = orc.silu_mul(a_s, b_s)
    assert_close(host(y[pt]), y64, yr, "silu_mul past 2^31")


@pytest.mark.parametrize("layout", [0, 1])
def test_rope_tokens_past_2_31(et, orc, layout):
    T, H, D, r = (1 << 16) + 1, 32, 1024, 256       # 2.15e9 elements of q
    q = _randn((T, H, D), 9)
    pos = np.random.default_rng(10).integers(0, 1 << 20, T).astype(np.int32)
    inv = wl.inv_freq(1e4, r)
    toks = [0, 1, 1 << 15, T - 2, T - 1]
    q_s = host(q[toks])
    et.rope_qk(q, None, torch.from_numpy(pos).cuda(), torch.from_numpy(inv).cuda(), d_rot=r,
               layout=layout)
    ref, y64 = orc.rope(q_s, pos[toks], r, inv, 1.0, layout)
    got = host(q[toks])
    assert_pair(got, y64, ref, r, layout, f"rope past 2^31 layout={layout}")
    assert_bits(got[..., r:], q_s[..., r:], "rope pass-through past 2^31")


def test_softmax_argmax_rows_past_2_31(et, orc):
    rows, n = 16385, 131072                          # 2.15e9 elements
    x = _randn((rows, n), 11, 3.0)
    pick = [0, 1, 8192, rows - 2, rows - 1]
    xs = host(x[pick])
    am = host(et.argmax(x))
    assert_bits(am[pick], orc.argmax(xs), "argmax past 2^31")
    y = et.softmax(x, 0.7)
    sy, sy64 = orc.softmax(xs, 0.7)
    check_softmax(host(y[pick]), xs, 0.7, sy, sy64, "softmax past 2^31")
