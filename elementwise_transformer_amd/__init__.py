"""Memory-bound transformer ops on AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libet.so`` (C ABI in ``include/et.h``).  Every
function here only checks tensor placement, derives sizes and pointers, and
calls the matching ``et_*_f32`` / ``et_*_bf16`` / ``et_*_f16`` entry point on
the current torch stream; all arithmetic runs in the library's HIP kernels.  There is no
other implementation: if the library is missing, importing this package
raises.

Tensors must be CUDA (ROCm) tensors, contiguous, float32, bfloat16 or float16.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch  # loaded first so libet.so binds to the HIP runtime torch uses

__all__ = ["rmsnorm", "add_rmsnorm", "layernorm", "rope", "rope_qk", "rmsnorm_rope_qk", "rope_cache",
           "rope_qk_cached", "rope_multi", "silu_mul", "geglu", "add", "embedding", "argmax",
           "argmax_workspace_bytes", "softmax", "softmax_workspace_bytes", "ETError", "lib", "LIB_PATH",
           "ROPE_HALF", "ROPE_INTERLEAVED", "GELU_ERF", "GELU_TANH", "abi_version"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libet.so")
ROPE_HALF, ROPE_INTERLEAVED = 0, 1

STATUS = {0: "ET_OK", 1: "ET_ERR_NULL_POINTER", 2: "ET_ERR_BAD_SIZE", 3: "ET_ERR_BAD_ARG",
          4: "ET_ERR_OVERLAP", 5: "ET_ERR_WORKSPACE", 6: "ET_ERR_HIP"}


class ETError(RuntimeError):
    """A non-OK et_status from the library."""

    def __init__(self, fn: str, code: int):
        self.code = code
        self.status = STATUS.get(code, f"status {code}")
        super().__init__(f"{fn}: {self.status} ({_status_string(code)})")


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing; build it with "
                      "`python elementwise_transformer_amd/_build.py` (needs hipcc for gfx950)")

lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _f32, _int, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                             ctypes.c_size_t)
_SIGS = {
    "rmsnorm": [_vp, _vp, _vp, _i64, _i64, _f32, _vp],
    "add_rmsnorm": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp],
    "rope": [_vp, _vp, _i64, _i64, _i64, _i64, _vp, _f32, _int, _vp],
    "rope_qk": [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _f32, _int, _vp],
    "rmsnorm_rope_qk": [_vp, _vp, _i64, _vp, _vp, _i64, _f32, _vp, _i64, _i64, _i64, _vp, _f32,
                        _int, _vp],
    "silu_mul": [_vp, _vp, _vp, _i64, _vp],
    "add": [_vp, _vp, _vp, _i64, _vp],
    "embedding": [_vp, _i64, _vp, _vp, _i64, _i64, _vp],
    "argmax": [_vp, _i64, _i64, _vp, _vp, _sz, _vp],
    "softmax": [_vp, _vp, _i64, _i64, _f32, _vp, _sz, _vp],
    "layernorm": [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp],
    "geglu": [_vp, _vp, _vp, _i64, _int, _vp],
    "rope_qk_cached": [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _vp, _i64, _f32, _int,
                       _vp],
    "rope_multi": [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _vp, _f32, _int, _vp],
}
for _op, _args in _SIGS.items():
    for _sfx in ("f32", "bf16", "f16"):
        _f = getattr(lib, f"et_{_op}_{_sfx}")
        _f.argtypes = _args
        _f.restype = ctypes.c_int
lib.et_argmax_workspace_bytes.argtypes = [_i64, _i64]
lib.et_argmax_workspace_bytes.restype = _sz
lib.et_softmax_workspace_bytes.argtypes = [_i64, _i64]
lib.et_softmax_workspace_bytes.restype = _sz
lib.et_argmax_noalloc.argtypes = [_int, _vp, _i64, _i64, _vp, _vp]
lib.et_argmax_noalloc.restype = ctypes.c_int
lib.et_softmax_wait_limit.argtypes = [_int, _vp, _vp, _i64, _i64, _f32, _vp, _sz, _int, _vp]
lib.et_softmax_wait_limit.restype = ctypes.c_int
lib.et_rope_cache_f32.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp]
lib.et_rope_cache_f32.restype = ctypes.c_int
lib.et_status_string.argtypes = [ctypes.c_int]
lib.et_status_string.restype = ctypes.c_char_p
lib.et_abi_version.argtypes = []
lib.et_abi_version.restype = ctypes.c_int


def _status_string(code: int) -> str:
    return lib.et_status_string(code).decode()


def abi_version() -> int:
    return int(lib.et_abi_version())


def _sfx(t: torch.Tensor) -> str:
    if t.dtype == torch.float32:
        return "f32"
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float16:
        return "f16"
    raise TypeError(f"expected float32, bfloat16 or float16, got {t.dtype}")


def _dev(*ts: Optional[torch.Tensor]) -> None:
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on a ROCm (cuda) device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous (dense row-major)")


def _same(ref: torch.Tensor, *ts: Optional[torch.Tensor]) -> None:
    for t in ts:
        if t is not None and t.dtype != ref.dtype:
            raise TypeError(f"dtype mismatch: {t.dtype} vs {ref.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _call(name: str, *args) -> None:
    code = getattr(lib, name)(*args)
    if code != 0:
        raise ETError(name, code)


# ---------------------------------------------------------------- RMSNorm

def rmsnorm(x: torch.Tensor, w: torch.Tensor, eps: float,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x / sqrt(mean(x^2, -1) + eps) * w over the last axis (et_rmsnorm_*).
    ``out`` may be ``x`` (in place)."""
    d = x.shape[-1]
    out = torch.empty_like(x) if out is None else out
    _dev(x, w, out)
    _same(x, w, out)
    rows = math.prod(x.shape[:-1])
    _call(f"et_rmsnorm_{_sfx(x)}", _ptr(x), _ptr(w), _ptr(out), rows, d, float(eps), _stream(x))
    return out


def layernorm(x: torch.Tensor, gamma: torch.Tensor, beta: Optional[torch.Tensor], eps: float,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = (x - mean) / sqrt(var + eps) * gamma + beta over the last axis
    (et_layernorm_*); beta may be None.  ``out`` may be ``x`` (in place)."""
    d = x.shape[-1]
    out = torch.empty_like(x) if out is None else out
    _dev(x, gamma, beta, out)
    _same(x, gamma, beta, out)
    rows = math.prod(x.shape[:-1])
    _call(f"et_layernorm_{_sfx(x)}", _ptr(x), _ptr(gamma), _ptr(beta), _ptr(out), rows, d, float(eps),
          _stream(x))
    return out


def add_rmsnorm(x: torch.Tensor, residual: torch.Tensor, w: torch.Tensor, eps: float,
                out: Optional[torch.Tensor] = None,
                h: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """h = x + residual; y = rmsnorm(h) (et_add_rmsnorm_*).  Returns (y, h).
    ``out`` may be ``x`` and ``h`` may be ``residual`` (in place)."""
    d = x.shape[-1]
    out = torch.empty_like(x) if out is None else out
    h = torch.empty_like(x) if h is None else h
    _dev(x, residual, w, out, h)
    _same(x, residual, w, out, h)
    if residual.shape != x.shape:
        raise ValueError("residual must have the shape of x")
    rows = math.prod(x.shape[:-1])
    _call(f"et_add_rmsnorm_{_sfx(x)}", _ptr(x), _ptr(residual), _ptr(w), _ptr(out), _ptr(h), rows,
          d, float(eps), _stream(x))
    return out, h


# ------------------------------------------------------------------- RoPE

def _rope_common(pos: torch.Tensor, inv_freq: torch.Tensor) -> None:
    _dev(pos, inv_freq)
    if pos.dtype != torch.int32:
        raise TypeError("pos must be int32")
    if inv_freq.dtype != torch.float32:
        raise TypeError("inv_freq must be float32")


def rope(x: torch.Tensor, pos: torch.Tensor, inv_freq: torch.Tensor, d_rot: Optional[int] = None,
         attn_scaling: float = 1.0, layout: int = ROPE_HALF) -> torch.Tensor:
    """In-place rotary embedding of x [T, H, D] (et_rope_*); returns x."""
    T, H, D = x.shape
    d_rot = D if d_rot is None else int(d_rot)
    _dev(x)
    _rope_common(pos, inv_freq)
    _call(f"et_rope_{_sfx(x)}", _ptr(x), _ptr(pos), T, H, D, d_rot, _ptr(inv_freq),
          float(attn_scaling), int(layout), _stream(x))
    return x


def rope_qk(q: torch.Tensor, k: Optional[torch.Tensor], pos: torch.Tensor, inv_freq: torch.Tensor,
            d_rot: Optional[int] = None, attn_scaling: float = 1.0,
            layout: int = ROPE_HALF) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """In-place rotary embedding of q [T, Hq, D] and k [T, Hk, D] in one
    launch (et_rope_qk_*); returns (q, k)."""
    T, Hq, D = q.shape
    Hk = 0 if k is None else k.shape[1]
    if k is not None and (k.shape[0] != T or k.shape[2] != D):
        raise ValueError("k must be [T, Hk, D] with q's T and D")
    d_rot = D if d_rot is None else int(d_rot)
    _dev(q, k)
    _same(q, k)
    _rope_common(pos, inv_freq)
    _call(f"et_rope_qk_{_sfx(q)}", _ptr(q), Hq, _ptr(k), Hk, _ptr(pos), T, D, d_rot, _ptr(inv_freq),
          float(attn_scaling), int(layout), _stream(q))
    return q, k


def rope_cache(inv_freq: torch.Tensor, max_pos: int, d_rot: Optional[int] = None,
               out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None
               ) -> Tuple[torch.Tensor, torch.Tensor]:
    """(cos, sin) f32 [max_pos, d_rot/2] of the angles et_rope_* uses
    (et_rope_cache_f32); d_rot defaults to 2 * len(inv_freq)."""
    _dev(inv_freq)
    if inv_freq.dtype != torch.float32:
        raise TypeError("inv_freq must be float32")
    d_rot = 2 * inv_freq.numel() if d_rot is None else int(d_rot)
    if inv_freq.numel() < d_rot // 2:
        raise ValueError("inv_freq needs d_rot/2 entries")
    shape = (int(max_pos), d_rot // 2)
    if out is None:
        out = (torch.empty(shape, dtype=torch.float32, device=inv_freq.device),
               torch.empty(shape, dtype=torch.float32, device=inv_freq.device))
    cos_c, sin_c = out
    _dev(cos_c, sin_c)
    for c in (cos_c, sin_c):
        if c.dtype != torch.float32 or tuple(c.shape) != shape:
            raise ValueError(f"cache buffers must be float32 {shape}")
    _call("et_rope_cache_f32", _ptr(inv_freq), shape[0], d_rot, _ptr(cos_c), _ptr(sin_c),
          _stream(inv_freq))
    return cos_c, sin_c


def rope_qk_cached(q: torch.Tensor, k: Optional[torch.Tensor], pos: torch.Tensor,
                   cos_cache: torch.Tensor, sin_cache: torch.Tensor, d_rot: Optional[int] = None,
                   attn_scaling: float = 1.0,
                   layout: int = ROPE_HALF) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """In-place rotary embedding of q [T, Hq, D] and k [T, Hk, D] with the
    rotation read from cos_cache / sin_cache f32 [max_pos, d_rot/2]
    (et_rope_qk_cached_*); returns (q, k)."""
    T, Hq, D = q.shape
    Hk = 0 if k is None else k.shape[1]
    if k is not None and (k.shape[0] != T or k.shape[2] != D):
        raise ValueError("k must be [T, Hk, D] with q's T and D")
    d_rot = D if d_rot is None else int(d_rot)
    _dev(q, k, cos_cache, sin_cache)
    _same(q, k)
    _rope_common(pos, cos_cache)
    if sin_cache.dtype != torch.float32 or sin_cache.shape != cos_cache.shape:
        raise ValueError("sin_cache must match cos_cache (float32)")
    if cos_cache.dim() != 2 or cos_cache.shape[1] != d_rot // 2:
        raise ValueError("caches must be [max_pos, d_rot/2]")
    _call(f"et_rope_qk_cached_{_sfx(q)}", _ptr(q), Hq, _ptr(k), Hk, _ptr(pos), T, D, d_rot,
          _ptr(cos_cache), _ptr(sin_cache), cos_cache.shape[0], float(attn_scaling), int(layout),
          _stream(q))
    return q, k


def rope_multi(q: torch.Tensor, k: Optional[torch.Tensor], pos: torch.Tensor, dims,
               inv_freq: torch.Tensor, attn_scaling: float = 1.0,
               layout: int = ROPE_HALF) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """In-place multi-axis RoPE of q [T, Hq, D] and k [T, Hk, D]: pos int32
    [T, len(dims)], dims the per-axis widths (even), inv_freq f32
    [sum(dims)/2] (axis a's frequencies from sum(dims[:a])/2)
    (et_rope_multi_*); returns (q, k)."""
    T, Hq, D = q.shape
    Hk = 0 if k is None else k.shape[1]
    if k is not None and (k.shape[0] != T or k.shape[2] != D):
        raise ValueError("k must be [T, Hk, D] with q's T and D")
    dims_arr = (ctypes.c_int64 * len(dims))(*[int(d) for d in dims])
    _dev(q, k)
    _same(q, k)
    _rope_common(pos, inv_freq)
    if pos.dim() != 2 or pos.shape[0] != T or pos.shape[1] != len(dims):
        raise ValueError("pos must be [T, len(dims)]")
    if inv_freq.numel() < sum(int(d) for d in dims) // 2:
        raise ValueError("inv_freq needs sum(dims)/2 entries")
    _call(f"et_rope_multi_{_sfx(q)}", _ptr(q), Hq, _ptr(k), Hk, _ptr(pos), T, D, len(dims),
          ctypes.cast(dims_arr, ctypes.c_void_p), _ptr(inv_freq), float(attn_scaling), int(layout),
          _stream(q))
    return q, k


def rmsnorm_rope_qk(q: torch.Tensor, gq: torch.Tensor, k: Optional[torch.Tensor],
                    gk: Optional[torch.Tensor], eps: float, pos: torch.Tensor,
                    inv_freq: torch.Tensor, d_rot: Optional[int] = None,
                    attn_scaling: float = 1.0,
                    layout: int = ROPE_HALF) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """In place: per-head RMSNorm over D with gains gq / gk, then RoPE
    (et_rmsnorm_rope_qk_*); returns (q, k)."""
    T, Hq, D = q.shape
    Hk = 0 if k is None else k.shape[1]
    if k is not None and (k.shape[0] != T or k.shape[2] != D):
        raise ValueError("k must be [T, Hk, D] with q's T and D")
    d_rot = D if d_rot is None else int(d_rot)
    _dev(q, gq, k, gk)
    _same(q, gq, k, gk)
    _rope_common(pos, inv_freq)
    _call(f"et_rmsnorm_rope_qk_{_sfx(q)}", _ptr(q), _ptr(gq), Hq, _ptr(k), _ptr(gk), Hk, float(eps),
          _ptr(pos), T, D, d_rot, _ptr(inv_freq), float(attn_scaling), int(layout), _stream(q))
    return q, k


# ------------------------------------------------------- flat ops, gather

GELU_ERF = 0
GELU_TANH = 1


def geglu(gate: torch.Tensor, up: torch.Tensor, approximate: int = GELU_ERF,
          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = gelu(gate) * up elementwise (et_geglu_*); approximate GELU_ERF
    (exact) or GELU_TANH.  ``out`` may be gate or up."""
    out = torch.empty_like(gate) if out is None else out
    _dev(gate, up, out)
    _same(gate, up, out)
    _call(f"et_geglu_{_sfx(gate)}", _ptr(gate), _ptr(up), _ptr(out), gate.numel(), int(approximate),
          _stream(gate))
    return out


def silu_mul(gate: torch.Tensor, up: torch.Tensor,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = silu(gate) * up elementwise (et_silu_mul_*)."""
    out = torch.empty_like(gate) if out is None else out
    _dev(gate, up, out)
    _same(gate, up, out)
    if up.numel() != gate.numel() or out.numel() != gate.numel():
        raise ValueError("gate, up and out must have the same number of elements")
    _call(f"et_silu_mul_{_sfx(gate)}", _ptr(gate), _ptr(up), _ptr(out), gate.numel(), _stream(gate))
    return out


def add(a: torch.Tensor, b: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = a + b elementwise (et_add_*); ``out`` may be ``a`` or ``b``."""
    out = torch.empty_like(a) if out is None else out
    _dev(a, b, out)
    _same(a, b, out)
    if b.numel() != a.numel() or out.numel() != a.numel():
        raise ValueError("a, b and out must have the same number of elements")
    _call(f"et_add_{_sfx(a)}", _ptr(a), _ptr(b), _ptr(out), a.numel(), _stream(a))
    return out


def embedding(table: torch.Tensor, ids: torch.Tensor,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[t] = table[ids[t]] (et_embedding_*); a bad id gives a NaN row."""
    V, d = table.shape
    n = ids.numel()
    out = torch.empty((n, d), dtype=table.dtype, device=table.device) if out is None else out
    _dev(table, ids, out)
    _same(table, out)
    if ids.dtype != torch.int32:
        raise TypeError("ids must be int32")
    _call(f"et_embedding_{_sfx(table)}", _ptr(table), V, _ptr(ids), _ptr(out), n, d,
          _stream(table))
    return out


def argmax_workspace_bytes(rows: int, n: int) -> int:
    return int(lib.et_argmax_workspace_bytes(int(rows), int(n)))


def argmax(x: torch.Tensor, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, split: bool = True) -> torch.Tensor:
    """Greedy argmax over the last axis (et_argmax_*): int32 per row, -1 for a
    row with no number.  ``split`` lets long rows spread over several
    workgroups through a workspace: zero-filled here unless given; a given
    one must be zero-filled before its first use (each call leaves it so)."""
    n = x.shape[-1]
    rows = math.prod(x.shape[:-1])
    out = torch.empty(rows, dtype=torch.int32, device=x.device) if out is None else out
    _dev(x, out)
    if out.dtype != torch.int32:
        raise TypeError("out must be int32")
    ws_ptr, ws_bytes = None, 0
    if split:
        need = argmax_workspace_bytes(rows, n)
        if need > 0:
            if workspace is None:
                workspace = torch.zeros(need, dtype=torch.uint8, device=x.device)
            _dev(workspace)
            ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    _call(f"et_argmax_{_sfx(x)}", _ptr(x), rows, n, _ptr(out), ws_ptr, ws_bytes, _stream(x))
    return out


def softmax_workspace_bytes(rows: int, n: int) -> int:
    return int(lib.et_softmax_workspace_bytes(int(rows), int(n)))


_STORAGE = {"f32": 0, "bf16": 1, "f16": 2}


def softmax(x: torch.Tensor, temperature: float = 1.0, out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, split: bool = True,
            wait_limit: Optional[int] = None) -> torch.Tensor:
    """Softmax of x / temperature over the last axis (et_softmax_*); out may be
    x.  ``split`` lets rows longer than 32768 elements spread over several
    workgroups through a workspace: zero-filled here unless given; a given
    one must be zero-filled before its first use (each call leaves it so).
    ``wait_limit`` (tests of the bounded wait) calls et_softmax_wait_limit
    with that many polls per thread instead."""
    n = x.shape[-1]
    rows = math.prod(x.shape[:-1])
    out = torch.empty_like(x) if out is None else out
    _dev(x, out)
    _same(x, out)
    ws_ptr, ws_bytes = None, 0
    if split:
        need = softmax_workspace_bytes(rows, n)
        if need > 0:
            if workspace is None:
                workspace = torch.zeros(need, dtype=torch.uint8, device=x.device)
            _dev(workspace)
            ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    if wait_limit is None:
        _call(f"et_softmax_{_sfx(x)}", _ptr(x), _ptr(out), rows, n, float(temperature), ws_ptr,
              ws_bytes, _stream(x))
    else:
        _call("et_softmax_wait_limit", _STORAGE[_sfx(x)], _ptr(x), _ptr(out), rows, n,
              float(temperature), ws_ptr, ws_bytes, int(wait_limit), _stream(x))
    return out
