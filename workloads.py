"""Seeded synthetic inputs for the memory-bound transformer ops.

This module only draws random inputs and describes workload shapes; it holds
none of the ops' arithmetic.  Both the HIP path (through the tests and the
benchmark) and the CPU oracle are fed from it, and it imports neither.

Storage: f32 tensors are ``numpy.float32``; f16 tensors ``numpy.float16``; bf16 tensors are ``numpy.uint16``
arrays of bfloat16 bits, drawn in f32 and converted by torch's CPU cast
(round to nearest even).

Seeding: every (workload, tensor group) pair gets its own PCG64 stream,
``numpy.random.default_rng([1000 + workload number, group id])``, so one op's
inputs can be drawn without drawing every tensor listed before it.

"N(0, s)" means a normal with standard deviation s; "U(a, b)" is uniform.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np

# Group ids (the second seed word).
G_EMBED, G_ADD, G_RMSNORM, G_ADD_RMSNORM, G_ROPE, G_QKNORM, G_SILU, G_ARGMAX, G_ROPE_MULTI = range(9)


def rng(workload: int, group: int) -> np.random.Generator:
    return np.random.default_rng([1000 + workload, group])


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """f32 values -> bfloat16 bits (torch's CPU cast, round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bfloat16 bits -> the same values as float32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def store(a: np.ndarray, dtype: str) -> np.ndarray:
    """f32 values -> storage form: float32, bf16 bits (uint16) or float16
    (numpy's cast, round to nearest even; past 65504 infinite)."""
    a = np.asarray(a, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(a)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return np.ascontiguousarray(a.astype(np.float16))
    return np.ascontiguousarray(a)


def normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    out = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def uniform(g: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    return g.uniform(lo, hi, size=shape).astype(np.float32)


def inv_freq(theta: float, r: int) -> np.ndarray:
    """RoPE frequency table w_i = theta^(-2i/r), i < r/2: an input of the op,
    built once per (theta, r) in f64 and rounded to f32."""
    i = np.arange(r // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / r).astype(np.float32)


# --------------------------------------------------------------------------
# Workload descriptions (shapes from the Llama-style prefill/decode settings).

@dataclass(frozen=True)
class RopeShape:
    T: int
    Hq: int
    Hk: int            # 0: Q only
    D: int
    r: int
    layout: int        # 0 half, 1 interleaved
    theta: float
    mu: float
    pos: str           # "arange" or "uniform:<hi>"
    eps: float         # for the fused RMSNorm+RoPE on the same shapes


@dataclass(frozen=True)
class MultiRopeShape:
    """Multi-axis RoPE over a latent video grid: one token per (frame, row,
    column), frame-major; the position vector of a token is its grid index."""
    frames: int
    height: int
    width: int
    Hq: int
    Hk: int
    D: int
    dims: Tuple[int, ...]      # per-axis widths (frame, row, column)
    thetas: Tuple[float, ...]  # per-axis bases
    layout: int
    mu: float

    @property
    def T(self) -> int:
        return self.frames * self.height * self.width


@dataclass(frozen=True)
class Workload:
    number: int
    name: str
    dtype: str                                      # "f32" or "bf16"
    embed: Optional[Tuple[int, int, int, float]] = None   # (V, d, n, std)
    add: Optional[Tuple[int, int]] = None                 # [rows, d]
    rmsnorm: Optional[Tuple[int, int, float]] = None      # (rows, d, eps)
    add_rmsnorm: Optional[Tuple[int, int, float, bool]] = None  # (rows, d, eps, in_place)
    rope: Optional[RopeShape] = None
    silu: Optional[Tuple[int, int, float]] = None          # (rows, cols, std)
    argmax: Optional[Tuple[int, int]] = None               # [rows, n]
    argmax_dtype: str = "f32"
    rope_multi: Optional[MultiRopeShape] = None
    extra: Dict[str, object] = field(default_factory=dict)


WORKLOADS: Dict[int, Workload] = {
    # Tiny f32 decoder-layer chain (correctness only).
    1: Workload(1, "tiny-f32-chain", "f32",
                embed=(256, 64, 8, 1.0), add=(8, 64), rmsnorm=(8, 64, 1e-5),
                add_rmsnorm=(8, 64, 1e-5, False),
                rope=RopeShape(8, 4, 0, 16, 16, 0, 1e4, 1.0, "arange", 1e-5),
                silu=(8, 128, 1.0), argmax=(8, 256)),
    # Llama-3-8B-shaped prefill, bf16 storage, T = 4096 (one sequence).
    2: Workload(2, "llama3-8b-prefill-bf16-T4096", "bf16",
                embed=(128256, 4096, 4096, 1.0), add=(4096, 4096),
                rmsnorm=(4096, 4096, 1e-5), add_rmsnorm=(4096, 4096, 1e-5, False),
                rope=RopeShape(4096, 32, 8, 128, 128, 0, 5e5, 1.0, "arange", 1e-5),
                silu=(4096, 14336, 1.0), argmax=(1, 128256)),
    # Decode step, f32, 256 sequences of one token each.
    3: Workload(3, "decode-f32-B256", "f32",
                embed=(128256, 4096, 256, 0.02), rmsnorm=(256, 4096, 1e-6),
                rope=RopeShape(256, 32, 8, 128, 128, 0, 5e5, 1.0, "uniform:8192", 1e-6),
                argmax=(256, 128256)),
    # Partial / interleaved RoPE stress, f32.
    4: Workload(4, "partial-interleaved-rope-f32-T16384", "f32",
                rope=RopeShape(16384, 16, 0, 128, 64, 1, 1e4, 1.1, "uniform:1048576", 1e-6)),
    # Large-hidden chain, bf16, T = 8192, hidden 8192, in-place fused add+norm.
    5: Workload(5, "large-hidden-bf16-T8192-H8192", "bf16",
                add_rmsnorm=(8192, 8192, 1e-5, True),
                rope=RopeShape(8192, 64, 8, 128, 128, 0, 1e6, 1.0, "arange", 1e-5),
                silu=(8192, 28672, 2.0)),
    # Multi-axis (3D) RoPE of a video diffusion transformer, bf16: a latent
    # grid of 16 frames x 30 x 40 (19,200 tokens), 24 query and 24 key heads
    # of 128, axis widths 16 / 56 / 56, base 256 on every axis.
    6: Workload(6, "video-dit-3d-rope-bf16-T19200", "bf16",
                rope_multi=MultiRopeShape(16, 30, 40, 24, 24, 128, (16, 56, 56), (256.0, 256.0, 256.0),
                                          0, 1.0)),
}


# --------------------------------------------------------------------------
# Generators.  Each returns numpy arrays in storage form (see module doc).

def gen_embedding(w: Workload, n: Optional[int] = None):
    V, d, n_full, std = w.embed
    g = rng(w.number, G_EMBED)
    table = normal(g, (V, d), std)
    ids = g.integers(0, V, size=n_full, dtype=np.int64).astype(np.int32)
    if n is not None:
        ids = ids[:n].copy()
    return store(table, w.dtype), ids


def gen_embedding_ids(w: Workload, j: int) -> np.ndarray:
    """Set j >= 1 of extra token ids for the embedding gather (same
    distribution as gen_embedding's, U[0, V), its own stream
    default_rng([1000 + workload, G_EMBED, j])): a benchmark that repeats
    the gather rotates through such sets so it never re-reads rows the
    previous call left in the caches."""
    V, _, n, _ = w.embed
    g = np.random.default_rng([1000 + w.number, G_EMBED, j])
    return g.integers(0, V, size=n, dtype=np.int64).astype(np.int32)


def gen_add(w: Workload):
    rows, d = w.add
    g = rng(w.number, G_ADD)
    a = normal(g, (rows, d))
    b = normal(g, (rows, d))
    return store(a, w.dtype), store(b, w.dtype)


def gen_rmsnorm(w: Workload):
    rows, d, eps = w.rmsnorm
    g = rng(w.number, G_RMSNORM)
    x = normal(g, (rows, d))
    gain = uniform(g, (d,), 0.5, 1.5)
    if w.number == 1:
        x[3, :] = 0.0               # one all-zero row
    return store(x, w.dtype), store(gain, w.dtype), eps


def gen_add_rmsnorm(w: Workload):
    rows, d, eps, _ = w.add_rmsnorm
    g = rng(w.number, G_ADD_RMSNORM)
    x = normal(g, (rows, d))
    res = normal(g, (rows, d))
    gain = uniform(g, (d,), 0.5, 1.5)
    if w.number == 1:
        x[3, :] = 0.0
        res[3, :] = 0.0             # the sum row is all zero too
    return store(x, w.dtype), store(res, w.dtype), store(gain, w.dtype), eps


def positions(spec: str, T: int, g: np.random.Generator) -> np.ndarray:
    if spec == "arange":
        return np.arange(T, dtype=np.int32)
    kind, hi = spec.split(":")
    assert kind == "uniform"
    return g.integers(0, int(hi), size=T, dtype=np.int64).astype(np.int32)


def gen_rope(w: Workload):
    """Q, K (K is None when Hk == 0), positions, inv_freq."""
    s = w.rope
    g = rng(w.number, G_ROPE)
    q = normal(g, (s.T, s.Hq, s.D))
    k = normal(g, (s.T, s.Hk, s.D)) if s.Hk else None
    pos = positions(s.pos, s.T, g)
    return (store(q, w.dtype), None if k is None else store(k, w.dtype), pos,
            inv_freq(s.theta, s.r))


def grid_positions(frames: int, height: int, width: int) -> np.ndarray:
    """int32 [frames * height * width, 3]: (frame, row, column) of each token,
    frame-major."""
    f, h, c = np.meshgrid(np.arange(frames), np.arange(height), np.arange(width), indexing="ij")
    return np.stack([f.ravel(), h.ravel(), c.ravel()], axis=1).astype(np.int32)


def multi_inv_freq(dims, thetas) -> np.ndarray:
    """Per-axis frequency tables w = theta_a^(-2j/d_a), j < d_a/2, concatenated."""
    return np.concatenate([inv_freq(t, d) for d, t in zip(dims, thetas)]).astype(np.float32)


def gen_rope_multi(w: Workload):
    """Q, K, positions [T, 3], concatenated inv_freq for the multi-axis RoPE."""
    s = w.rope_multi
    g = rng(w.number, G_ROPE_MULTI)
    q = normal(g, (s.T, s.Hq, s.D))
    k = normal(g, (s.T, s.Hk, s.D)) if s.Hk else None
    pos = grid_positions(s.frames, s.height, s.width)
    return (store(q, w.dtype), None if k is None else store(k, w.dtype), pos,
            multi_inv_freq(s.dims, s.thetas))


def gen_qknorm(w: Workload):
    """Q, K, gains g_q, g_k, positions, inv_freq for the fused RMSNorm+RoPE."""
    s = w.rope
    g = rng(w.number, G_QKNORM)
    q = normal(g, (s.T, s.Hq, s.D))
    k = normal(g, (s.T, s.Hk, s.D)) if s.Hk else None
    gq = uniform(g, (s.D,), 0.5, 1.5)
    gk = uniform(g, (s.D,), 0.5, 1.5)
    pos = positions(s.pos, s.T, g)
    return (store(q, w.dtype), None if k is None else store(k, w.dtype),
            store(gq, w.dtype), store(gk, w.dtype), pos, inv_freq(s.theta, s.r))


def gen_silu(w: Workload):
    rows, cols, std = w.silu
    g = rng(w.number, G_SILU)
    gate = normal(g, (rows, cols), std)
    up = normal(g, (rows, cols), std)
    if w.number == 1:
        gate[0, 0], gate[0, 1], gate[0, 2] = 1e4, -1e4, 0.0
    return store(gate, w.dtype), store(up, w.dtype)


def gen_argmax(w: Workload):
    """Logits with planted ties and NaNs; returns (logits f32/bf16, plan)."""
    rows, n = w.argmax
    g = rng(w.number, G_ARGMAX)
    std = 3.0 if w.number == 3 else 1.0
    x = normal(g, (rows, n), std)
    plan = {"ties": [], "nans": []}
    if w.number == 1:
        top = np.float32(x[1].max() + 1.0)
        x[1, [10, 100, 200]] = top          # one maximum at three indices
        x[2, 0] = np.nan
        x[3, :] = np.nan
        x[4, :] = -np.inf
        x[5, :] = -1.0
        x[5, 5] = -0.0
        x[5, 9] = 0.0
        x[6, 17] = np.inf
        x[6, 200] = np.inf
        x[7, int(np.argmax(x[7]))] = np.nan
        plan = {"ties": [1, 5, 6], "nans": [2, 3, 7]}
    elif rows >= 100:
        k = max(1, rows // 100)
        chosen = g.choice(rows, size=2 * k, replace=False)
        ties, nans = sorted(chosen[:k].tolist()), sorted(chosen[k:].tolist())
        for r in ties:
            m = int(np.argmax(x[r]))
            a = int(g.integers(0, max(1, m))) if m > 0 else 0
            b = int(g.integers(m + 1, n)) if m < n - 1 else n - 1
            x[r, a] = x[r, m]
            x[r, b] = x[r, m]
        for r in nans:
            m = int(np.argmax(x[r]))
            x[r, 0] = np.nan
            x[r, m] = np.nan
            idx = g.choice(n, size=max(1, n // 100), replace=False)
            x[r, idx] = np.nan
        plan = {"ties": ties, "nans": nans}
    return store(x, w.argmax_dtype), plan
