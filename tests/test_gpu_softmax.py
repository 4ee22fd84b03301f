"""GPU parity of the softmax-with-temperature entry point against the CPU
oracle, through the C ABI.

Tolerances, derived from the f32 arithmetic of the kernels (u = 2^-24):
  f32   |got - y| <= u (2|z| + 3|M| + 3|z - M| + 128) y + 2^-140, with z = x/t
        and M the row max.  z = x * (1/t) carries two roundings (2 u |z|);
        z - m_c one more plus the chunk max's own; the output is
        exp(z - m_c) * (exp(m_c - M) / S), where |m_c - M| <= |z - M| and
        |m_c| <= |M| + |z - M|; the exponentials (the hardware exp2 of
        d log2 e: about |d| u from the product, plus one ulp), the division
        and the final product a few ulp each; the sum of a row's exponentials
        at most 32 sequential additions per thread, a 6-level butterfly, 16
        wave partials and the chunk combine -- well under 128 u in all.
        Results below 2^-126 may come out as 0 (the hardware exp2 returns no
        subnormals).
  bf16, f16  at most 1 ulp from the oracle's correctly rounded value (the
        f32 result above is far inside half an ulp of either); results below
        2^-126 may also come out as 0.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import assert_bits, check_softmax, dev, host, widen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def et():
    import elementwise_transformer_amd as m
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return m


def _rng(*key):
    return np.random.default_rng([4343, *key])


def _logits(shape, dt, key, scale=3.0):
    x = (_rng(*key).standard_normal(shape) * scale).astype(np.float32)
    return wl.store(x, dt)


SHAPES = [(1, 1), (3, 5), (4, 64), (7, 100), (5, 1000), (3, 4096), (2, 8191), (2, 32768),
          (2, 32769), (3, 40000), (2, 128256)]


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", SHAPES)
def test_softmax_matches_oracle(et, orc, dt, shape):
    for t in (1.0, 0.7):
        xs = _logits(shape, dt, (shape[1], 1 if dt == "f32" else 2))
        y, y64 = orc.softmax(xs, t)
        got = host(et.softmax(dev(xs), t))
        check_softmax(got, xs, t, y, y64, f"{dt} {shape} t={t}")
        assert np.all(np.abs(y64.sum(axis=1) - 1.0) < 1e-12)


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n", [40000, 128256])
def test_softmax_workspace_and_single_block_agree(et, dt, n):
    """Long rows: the single-launch split (workspace) and one workgroup per
    row (no workspace) give identical bits."""
    xs = dev(_logits((5, n), dt, (n, 3)))
    a = host(et.softmax(xs, 0.9, split=True))
    b = host(et.softmax(xs, 0.9, split=False))
    assert_bits(a, b, f"{dt} n={n}")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n", [40000, 128256])
def test_softmax_bounded_wait_fallback_same_bits(et, dt, n):
    """Forced from the host: with a wait limit of 0 no workgroup waits for the
    row's other partials, every one computes the row statistics itself --
    same bits; the workspace is left zero-filled after each call."""
    xs = dev(_logits((7, n), dt, (n, 7)))
    ws = torch.zeros(et.softmax_workspace_bytes(7, n), dtype=torch.uint8, device="cuda")
    a = host(et.softmax(xs, 1.1, workspace=ws))
    cnt = ws[:7 * 8].cpu().numpy()
    assert not cnt.any()
    b = host(et.softmax(xs, 1.1, workspace=ws, wait_limit=0))
    assert not ws[:7 * 8].cpu().numpy().any()
    c = host(et.softmax(xs, 1.1, workspace=ws, wait_limit=1))
    d = host(et.softmax(xs, 1.1, workspace=ws))
    assert int(torch.count_nonzero(ws)) == 0
    assert_bits(b, a, f"{dt} n={n} fallback")
    assert_bits(c, a, f"{dt} n={n} wait 1")
    assert_bits(d, a, f"{dt} n={n} reuse")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n", [40000, 128256])
@pytest.mark.parametrize("limit", [0, 1, None])
def test_softmax_in_place_with_workspace(et, orc, dt, n, limit):
    """y == x with a workspace, with the bounded wait forced to give up (0),
    nearly so (1) or not at all: the same bits as out of place, against the
    oracle, and the workspace left zero-filled.  (In place, no workgroup may
    read a chunk another one is already writing.)"""
    x = _logits((6, n), dt, (n, 17))
    xs = dev(x)
    ref = host(et.softmax(xs, 0.9))
    ws = torch.zeros(et.softmax_workspace_bytes(6, n), dtype=torch.uint8, device="cuda")
    for rep in range(2):
        xi = xs.clone()
        et.softmax(xi, 0.9, out=xi, workspace=ws, wait_limit=limit)
        assert_bits(host(xi), ref, f"{dt} n={n} in place limit {limit} call {rep}")
        assert int(torch.count_nonzero(ws)) == 0, "workspace not left zero-filled"
    y, y64 = orc.softmax(x, 0.9)
    check_softmax(ref, x, 0.9, y, y64, f"{dt} n={n}")


def test_softmax_wait_limit_rejects_bad_values(et):
    x = torch.zeros((1, 40000), device="cuda")
    for bad in (-1, 65537):
        with pytest.raises(et.ETError):
            et.softmax(x, 1.0, wait_limit=bad)


def _masked(n, dt, key, spans):
    """N(0, 3) logits with the given [a, b) spans set to -inf."""
    x = (_rng(*key).standard_normal((len(spans), n)) * 3).astype(np.float32)
    for r, sp in enumerate(spans):
        for a, b in sp:
            x[r, a:b] = -np.inf
    return wl.store(x, dt)


def _mask_spans(n, rng):
    """Rows of masked logits: a whole first chunk, the last chunk (partial
    when n is not a multiple of 8192), every chunk but one, a top-k style
    mask keeping 50 random entries, two whole chunks in the middle, and
    masks that start and end inside chunks."""
    C = 8192
    chunks = -(-n // C)
    keep = np.sort(rng.choice(n, 50, replace=False))
    topk = []
    prev = 0
    for k in keep:
        if k > prev:
            topk.append((prev, int(k)))
        prev = int(k) + 1
    topk.append((prev, n))
    mid = chunks // 2
    return [
        [(0, C)],
        [((chunks - 1) * C, n)],
        [(0, mid * C), ((mid + 1) * C, n)],
        topk,
        [(C, 3 * C)],
        [(C // 2, C + C // 2), (n - C - 100, n - 7)],
    ]


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n", [40000, 128256])
def test_softmax_masked_chunks(et, orc, dt, n):
    """Whole chunks of -inf (masked logits, a top-k mask, a short last
    chunk): finite probabilities, 0 on the masked entries, against the
    oracle; the one-launch exchange, the forced fallback, the two-launch
    in-place path and one workgroup per row all give the same bits."""
    spans = _mask_spans(n, _rng(n, 23))
    xs = _masked(n, dt, (n, 24), spans)
    y, y64 = orc.softmax(xs, 0.8)
    assert np.all(np.isfinite(y64))
    xd = dev(xs)
    ws = torch.zeros(et.softmax_workspace_bytes(len(spans), n), dtype=torch.uint8, device="cuda")
    a = host(et.softmax(xd, 0.8, workspace=ws))
    check_softmax(a, xs, 0.8, y, y64, f"{dt} n={n} masked")
    wa = widen(a)
    assert np.all(np.isfinite(wa))
    assert np.all(wa[np.isneginf(widen(xs))] == 0.0)
    assert_bits(host(et.softmax(xd, 0.8, workspace=ws, wait_limit=0)), a, f"{dt} n={n} fallback")
    assert_bits(host(et.softmax(xd, 0.8, split=False)), a, f"{dt} n={n} one workgroup per row")
    xi = xd.clone()
    et.softmax(xi, 0.8, out=xi, workspace=ws)
    assert_bits(host(xi), a, f"{dt} n={n} in place")
    assert int(torch.count_nonzero(ws)) == 0


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("rows,n", [(3, 1024 * 8192), (1, 1024 * 8192 + 3), (2, (1 << 24) + 5)])
def test_softmax_very_long_rows(et, orc, dt, rows, n):
    """Rows past 1024 chunks of 8192 take two launches (chunk statistics,
    then combine and write): one launch would need all of a row's chunk
    workgroups resident together.  At exactly 1024 chunks, the one-launch
    exchange.  Against the oracle, the same bits as one workgroup per row
    (no workspace), the same again on a reused workspace, which every call
    leaves zero-filled."""
    x = _logits((rows, n), dt, (n, 11))
    xs = dev(x)
    ws = torch.zeros(et.softmax_workspace_bytes(rows, n), dtype=torch.uint8, device="cuda")
    a = host(et.softmax(xs, 0.8, workspace=ws))
    assert int(torch.count_nonzero(ws)) == 0, "workspace not left zero-filled"
    assert_bits(host(et.softmax(xs, 0.8, workspace=ws)), a, f"{dt} {rows}x{n} reused workspace")
    assert_bits(host(et.softmax(xs, 0.8, split=False)), a, f"{dt} {rows}x{n} one workgroup per row")
    y, y64 = orc.softmax(x, 0.8)
    check_softmax(a, x, 0.8, y, y64, f"{dt} {rows}x{n}")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n", [100, 4096, 32768, 40000, 128256])
def test_softmax_batch_invariance_and_in_place(et, dt, n):
    """A row's bits do not depend on the rows beside it; y == x works."""
    rows = 64 if n <= 4096 else 9
    xs = _logits((rows, n), dt, (n, 4))
    xd = dev(xs)
    full = host(et.softmax(xd, 1.3))
    for r in (0, rows // 2, rows - 1):
        one = host(et.softmax(dev(np.ascontiguousarray(xs[r:r + 1])), 1.3))
        assert_bits(one[0], full[r], f"{dt} n={n} row {r}")
    inplace = xd.clone()
    et.softmax(inplace, 1.3, out=inplace)
    assert_bits(host(inplace), full, f"{dt} n={n} in place")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n", [7, 1001, 40003])
def test_softmax_scalar_path(et, orc, dt, n):
    """Misaligned buffers and lengths that are not whole vectors take the
    scalar loads with the same ownership; results match the oracle."""
    xs = _logits((3, n), dt, (n, 5))
    y, y64 = orc.softmax(xs, 0.8)
    t = dev(xs)
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    mis = flat[1:1 + t.numel()].view(t.shape)
    mis.copy_(t)
    assert mis.data_ptr() % 16 != 0
    got = host(et.softmax(mis, 0.8))
    check_softmax(got, xs, 0.8, y, y64, f"{dt} n={n} misaligned")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n", [16, 5000, 40000])
def test_softmax_special_values(et, orc, dt, n):
    """NaN anywhere, all -inf, a +inf entry: NaN rows; a single -inf entry
    gets 0; logits of 1e4 stay finite (the max is subtracted)."""
    x = (_rng(n, 6).standard_normal((6, n)) * 2).astype(np.float32)
    x[0, n // 3] = np.nan
    x[1, :] = -np.inf
    x[2, n // 2] = np.inf
    x[3, n - 1] = -np.inf
    x[4, :] += 1.0e4
    x[5, :] -= 1.0e4
    xs = wl.store(x, dt)
    y, y64 = orc.softmax(xs, 1.0)
    got = host(et.softmax(dev(xs), 1.0))
    assert np.all(np.isnan(widen(got[:3])))
    assert widen(got[3:4])[0, n - 1] == 0.0
    assert np.all(np.isfinite(widen(got[3:])))
    check_softmax(got[3:], xs[3:], 1.0, y[3:], y64[3:], f"{dt} n={n} special")


def test_softmax_empty_and_degenerate(et):
    x = torch.empty((0, 10), device="cuda")
    assert et.softmax(x).shape == (0, 10)
    x = torch.empty((4, 0), device="cuda")
    assert et.softmax(x).shape == (4, 0)
    one = et.softmax(torch.tensor([[3.0]], device="cuda"))
    assert float(one[0, 0]) == 1.0
    with pytest.raises(Exception):
        et.softmax(torch.ones((2, 3), device="cuda"), 0.0)


def test_softmax_decode_logits_full_size(et, orc):
    """The decode logits at full size, [256, 128256] f32 N(0, 3) with planted
    ties and NaN rows, temperature 0.7, in the launch configuration the
    benchmark times (split over workgroups): sampled rows against the oracle,
    every row summing to 1 where it holds no NaN."""
    w = wl.WORKLOADS[3]
    lg, _ = wl.gen_argmax(w)
    xd = dev(lg)
    got_d = et.softmax(xd, 0.7)
    sums = got_d.double().sum(dim=1).cpu().numpy()
    nan_rows = np.any(np.isnan(lg), axis=1)
    assert np.all(np.abs(sums[~nan_rows] - 1.0) < 1e-4)
    got = host(got_d)
    rows = sorted(set([0, 1, 127, 255] + list(np.flatnonzero(nan_rows)[:2])))
    sub = np.ascontiguousarray(lg[rows])
    y, y64 = orc.softmax(sub, 0.7)
    check_softmax(got[rows], sub, 0.7, y, y64, "decode logits")
