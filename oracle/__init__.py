"""CPU oracle for the memory-bound transformer ops (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and the two share no code: this module wraps
``oracle.c`` (plain C, f64 math) through ctypes and converts numpy arrays.

Storage types: ``numpy.float32`` arrays are f32; ``numpy.uint16`` arrays hold
bfloat16 bits.  Every function returns the rounded output(s) in the input's
storage type and, where a tolerance needs it, the unrounded f64 result.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F32, BF16, F16 = 0, 1, 2

CFLAGS = ["-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra: Optional[list] = None) -> str:
    """Compile ``src`` (default: oracle.c) into the shared library ``out``."""
    cmd = ["gcc", *CFLAGS, *(extra or []), "-I", HERE, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float16:
        return F16
    raise TypeError(f"oracle storage must be float32, uint16 (bf16 bits) or float16, got {a.dtype}")


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


_i64, _f32, _int, _vp = ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_void_p


class Oracle:
    """ctypes view of one build of ``oracle.c``."""

    def __init__(self, path: str = LIB):
        self.path = path
        lib = ctypes.CDLL(path)
        self.lib = lib
        lib.orc_set_threads.argtypes = [_int]
        lib.orc_get_threads.restype = _int
        lib.orc_bf16_from_f64.argtypes = [ctypes.c_double]
        lib.orc_bf16_from_f64.restype = ctypes.c_uint16
        lib.orc_f16_from_f64.argtypes = [ctypes.c_double]
        lib.orc_f16_from_f64.restype = ctypes.c_uint16
        lib.orc_round_to.argtypes = [_int, _vp, _i64, _vp]
        lib.orc_rope_angle.argtypes = [ctypes.c_int32, _f32]
        lib.orc_rope_angle.restype = _f32
        lib.orc_rmsnorm.argtypes = [_int, _vp, _vp, _i64, _i64, _f32, _vp, _vp]
        lib.orc_softmax.argtypes = [_int, _vp, _i64, _i64, _f32, _vp, _vp]
        lib.orc_layernorm.argtypes = [_int, _vp, _vp, _vp, _i64, _i64, _f32, _vp, _vp]
        lib.orc_geglu.argtypes = [_int, _vp, _vp, _i64, _int, _vp, _vp]
        lib.orc_rope_cache.argtypes = [_vp, _i64, _i64, _vp, _vp]
        lib.orc_rope_multi.argtypes = [_int, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _f32, _int,
                                       _vp]
        lib.orc_rope_cached.argtypes = [_int, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _i64, _f32,
                                        _int, _vp]
        lib.orc_add_rmsnorm.argtypes = [_int, _vp, _vp, _vp, _i64, _i64, _f32, _vp, _vp, _vp]
        lib.orc_rope.argtypes = [_int, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _f32, _int, _vp]
        lib.orc_rmsnorm_rope.argtypes = [_int, _vp, _vp, _f32, _vp, _i64, _i64, _i64, _i64,
                                         _vp, _f32, _int, _vp]
        lib.orc_silu_mul.argtypes = [_int, _vp, _vp, _i64, _vp, _vp]
        lib.orc_add.argtypes = [_int, _vp, _vp, _i64, _vp]
        lib.orc_embedding.argtypes = [_int, _vp, _i64, _vp, _i64, _i64, _vp]
        lib.orc_argmax.argtypes = [_int, _vp, _i64, _i64, _vp]
        for f in ("orc_set_threads", "orc_rmsnorm", "orc_add_rmsnorm", "orc_rope",
                  "orc_rmsnorm_rope", "orc_silu_mul", "orc_add", "orc_embedding",
                  "orc_argmax"):
            getattr(lib, f).restype = None

    # -- helpers -----------------------------------------------------------
    def set_threads(self, n: int) -> None:
        self.lib.orc_set_threads(int(n))

    def threads(self) -> int:
        return int(self.lib.orc_get_threads())

    def bf16_from_f64(self, v: float) -> int:
        return int(self.lib.orc_bf16_from_f64(float(v)))

    def f16_from_f64(self, v: float) -> int:
        return int(self.lib.orc_f16_from_f64(float(v)))

    def round_to(self, v: np.ndarray, dtype: str) -> np.ndarray:
        """The storage rounding every op applies: f64 values -> "f32" (float32),
        "bf16" (uint16 bits) or "f16" (float16)."""
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty(v.shape, {"f32": np.float32, "bf16": np.uint16, "f16": np.float16}[dtype])
        self.lib.orc_round_to({"f32": F32, "bf16": BF16, "f16": F16}[dtype], _p(v), v.size, _p(out))
        return out

    def rope_angle(self, p: int, w: float) -> np.float32:
        return np.float32(self.lib.orc_rope_angle(int(p), float(w)))

    # -- ops -----------------------------------------------------------------
    def rmsnorm(self, x: np.ndarray, w: np.ndarray, eps: float):
        """[rows, d] -> (y in storage type, y64)."""
        x = np.ascontiguousarray(x)
        dt = _dt(x)
        rows, d = x.shape
        assert w.dtype == x.dtype and w.shape == (d,)
        y = np.empty_like(x)
        y64 = np.empty(x.shape, np.float64)
        self.lib.orc_rmsnorm(dt, _p(x), _p(np.ascontiguousarray(w)), rows, d, eps, _p(y64), _p(y))
        return y, y64

    def add_rmsnorm(self, x: np.ndarray, res: np.ndarray, w: np.ndarray, eps: float):
        """[rows, d] x, residual -> (y, h, y64) with h = x + residual."""
        x = np.ascontiguousarray(x)
        res = np.ascontiguousarray(res)
        dt = _dt(x)
        rows, d = x.shape
        assert res.shape == x.shape and res.dtype == x.dtype and w.shape == (d,)
        y = np.empty_like(x)
        h = np.empty_like(x)
        y64 = np.empty(x.shape, np.float64)
        self.lib.orc_add_rmsnorm(dt, _p(x), _p(res), _p(np.ascontiguousarray(w)), rows, d, eps,
                                 _p(y64), _p(y), _p(h))
        return y, h, y64

    def rope(self, x: np.ndarray, pos: np.ndarray, r: int, inv_freq: np.ndarray,
             mu: float, layout: int):
        """x [T, H, D] (not modified) -> (rotated copy, y64)."""
        out = np.array(x, copy=True, order="C")
        dt = _dt(out)
        T, H, D = out.shape
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        inv_freq = np.ascontiguousarray(inv_freq, dtype=np.float32)
        assert pos.shape == (T,)
        y64 = np.empty(out.shape, np.float64)
        self.lib.orc_rope(dt, _p(out), _p(pos), T, H, D, r, _p(inv_freq), mu, layout, _p(y64))
        return out, y64

    def rmsnorm_rope(self, x: np.ndarray, g: np.ndarray, eps: float, pos: np.ndarray, r: int,
                     inv_freq: np.ndarray, mu: float, layout: int):
        """x [T, H, D] (not modified), per-head gain g [D] -> (result, y64)."""
        out = np.array(x, copy=True, order="C")
        dt = _dt(out)
        T, H, D = out.shape
        assert g.shape == (D,) and g.dtype == out.dtype
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        inv_freq = np.ascontiguousarray(inv_freq, dtype=np.float32)
        y64 = np.empty(out.shape, np.float64)
        self.lib.orc_rmsnorm_rope(dt, _p(out), _p(np.ascontiguousarray(g)), eps, _p(pos), T, H, D,
                                  r, _p(inv_freq), mu, layout, _p(y64))
        return out, y64

    def silu_mul(self, gate: np.ndarray, up: np.ndarray):
        gate = np.ascontiguousarray(gate)
        up = np.ascontiguousarray(up)
        dt = _dt(gate)
        assert up.shape == gate.shape and up.dtype == gate.dtype
        y = np.empty_like(gate)
        y64 = np.empty(gate.shape, np.float64)
        self.lib.orc_silu_mul(dt, _p(gate), _p(up), gate.size, _p(y64), _p(y))
        return y, y64

    def add(self, a: np.ndarray, b: np.ndarray):
        a = np.ascontiguousarray(a)
        b = np.ascontiguousarray(b)
        dt = _dt(a)
        assert b.shape == a.shape and b.dtype == a.dtype
        y = np.empty_like(a)
        self.lib.orc_add(dt, _p(a), _p(b), a.size, _p(y))
        return y

    def embedding(self, table: np.ndarray, ids: np.ndarray):
        table = np.ascontiguousarray(table)
        dt = _dt(table)
        V, d = table.shape
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        out = np.empty((ids.size, d), table.dtype)
        self.lib.orc_embedding(dt, _p(table), V, _p(ids), ids.size, d, _p(out))
        return out

    def argmax(self, x: np.ndarray):
        """[rows, n] -> int32 [rows]."""
        x = np.ascontiguousarray(x)
        dt = _dt(x)
        rows, n = x.shape
        out = np.empty(rows, np.int32)
        self.lib.orc_argmax(dt, _p(x), rows, n, _p(out))
        return out

    def softmax(self, x: np.ndarray, t: float = 1.0):
        """[rows, n] -> (y in storage type, y64): softmax of x / t per row."""
        x = np.ascontiguousarray(x)
        dt = _dt(x)
        rows, n = x.shape
        y = np.empty_like(x)
        y64 = np.empty(x.shape, np.float64)
        self.lib.orc_softmax(dt, _p(x), rows, n, t, _p(y64), _p(y))
        return y, y64

    def layernorm(self, x: np.ndarray, g: np.ndarray, b: Optional[np.ndarray], eps: float):
        """[rows, d] -> (y, y64); b may be None (no bias)."""
        x = np.ascontiguousarray(x)
        dt = _dt(x)
        rows, d = x.shape
        assert g.dtype == x.dtype and g.shape == (d,)
        if b is not None:
            assert b.dtype == x.dtype and b.shape == (d,)
            b = np.ascontiguousarray(b)
        y = np.empty_like(x)
        y64 = np.empty(x.shape, np.float64)
        self.lib.orc_layernorm(dt, _p(x), _p(np.ascontiguousarray(g)), _p(b) if b is not None else None,
                               rows, d, eps, _p(y64), _p(y))
        return y, y64

    def geglu(self, gate: np.ndarray, up: np.ndarray, form: int = 0):
        """GELU(gate) * up; form 0 = erf (exact), 1 = tanh approximation."""
        gate = np.ascontiguousarray(gate)
        up = np.ascontiguousarray(up)
        dt = _dt(gate)
        assert up.shape == gate.shape and up.dtype == gate.dtype
        y = np.empty_like(gate)
        y64 = np.empty(gate.shape, np.float64)
        self.lib.orc_geglu(dt, _p(gate), _p(up), gate.size, form, _p(y64), _p(y))
        return y, y64

    def rope_cache(self, inv_freq: np.ndarray, max_pos: int, r: int):
        """(cos, sin) f32 [max_pos, r/2] of the RoPE angles."""
        inv = np.ascontiguousarray(inv_freq, dtype=np.float32)
        c = np.empty((max_pos, r // 2), np.float32)
        s = np.empty((max_pos, r // 2), np.float32)
        self.lib.orc_rope_cache(_p(inv), max_pos, r, _p(c), _p(s))
        return c, s

    def rope_cached(self, x: np.ndarray, pos: np.ndarray, r: int, cos_c: np.ndarray, sin_c: np.ndarray,
                    mu: float, layout: int):
        """x [T, H, D] (not modified) -> (rotated copy, y64), rotation from the cache."""
        out = np.array(x, copy=True, order="C")
        T, H, D = out.shape
        y64 = np.empty(out.shape, np.float64)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        cos_c = np.ascontiguousarray(cos_c, dtype=np.float32)
        sin_c = np.ascontiguousarray(sin_c, dtype=np.float32)
        self.lib.orc_rope_cached(_dt(out), _p(out), _p(pos), T, H, D, r, _p(cos_c), _p(sin_c),
                                 cos_c.shape[0], mu, layout, _p(y64))
        return out, y64


    def rope_multi(self, x: np.ndarray, pos: np.ndarray, dims, inv_freq: np.ndarray, mu: float,
                   layout: int):
        """x [T, H, D] (not modified), pos int32 [T, A], dims [A] (even), inv_freq f32
        [sum(dims)/2] (axis a's frequencies at offset sum(dims[:a])/2) -> (rotated copy, y64)."""
        out = np.array(x, copy=True, order="C")
        T, H, D = out.shape
        pos = np.ascontiguousarray(pos, dtype=np.int32).reshape(T, -1)
        dims = np.ascontiguousarray(dims, dtype=np.int64)
        assert pos.shape[1] == dims.size and int(dims.sum()) <= D and not np.any(dims % 2)
        inv = np.ascontiguousarray(inv_freq, dtype=np.float32)
        assert inv.size >= int(dims.sum()) // 2
        y64 = np.empty(out.shape, np.float64)
        self.lib.orc_rope_multi(_dt(out), _p(out), _p(pos), T, H, D, dims.size, _p(dims), _p(inv),
                                mu, layout, _p(y64))
        return out, y64


_default: Optional[Oracle] = None


def load(rebuild: bool = False) -> Oracle:
    """The oracle built from ``oracle.c`` (compiled here if missing or stale)."""
    global _default
    if _default is None or rebuild:
        stale = (not os.path.exists(LIB)
                 or os.path.getmtime(LIB) < max(os.path.getmtime(SRC),
                                                os.path.getmtime(os.path.join(HERE, "oracle.h"))))
        if rebuild or stale:
            build()
        _default = Oracle(LIB)
    return _default
