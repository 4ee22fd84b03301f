"""Benchmark of the memory-bound transformer ops on one MI355X.

Default workload: the large-hidden chain, bf16 storage with f32 math, T =
8192 tokens, hidden 8192 -- in-place fused residual-add + RMSNorm [8192,
8192], RoPE on Q [8192, 64, 128] and K [8192, 8, 128], fused RMSNorm + RoPE
on the same shapes, SiLU-mul [8192, 28672].  It is the largest of the
configurations.

Timed region: K steps (one step = one pass of every op of the workload)
launched back to back on one stream; ``value`` = a step's algorithmic bytes
x K / wall time.  Algorithmic bytes: each input read once and each output
written once (in-place RoPE counts only the rotated entries).  Every op
rotates through buffer sets whose footprint is at least 768 MB, three times
the 256 MB Infinity Cache, so no launch is served from lines an earlier
launch left there.  The dominant op (SiLU-mul) is bracketed by HIP events in
every step: that is the ``roofline`` record.

After the timed region, every op is timed alone: ``--op-launches`` launches
(at least 20) over its rotated sets, one pair of HIP events per launch,
whatever ``--steps`` is (``ops``); the same for the other configurations --
Llama-3-8B prefill (T = 4096), decode (256 sequences), partial/interleaved
RoPE (T = 16384) -- under ``configs``; the ops beyond the step under
``next_ops``; plain-stream yardsticks under ``stream_ceiling``; and the CPU
oracle on a bounded sample of the same workload (``cpu_baseline``).

``--dispatch-log FILE`` writes the label of every library call in launch
order; ``--summarize DIR`` turns a rocprofv3 kernel trace or counter run of
such a bench run into a per-op table (one row per op and launch shape).

    python bench.py [--steps K] [--warmup W] [--workload 2|3|4|5]
    python bench.py --summarize DIR --dispatch-log FILE [--title T] [--command C]
"""
from __future__ import annotations

import argparse
import csv
import gc
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0          # MI355X HBM3E peak, vendor figure (8 TB/s)
MIN_FOOTPRINT = 768_000_000  # bytes per rotation: three times the 256 MB Infinity Cache
MIN_OP_LAUNCHES = 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", type=int, default=5)
    p.add_argument("--configs", default="2,3,4",
                   help="other workloads whose ops are timed one by one after the timed region "
                        "(comma-separated numbers; empty for none)")
    p.add_argument("--op-launches", type=int, default=100,
                   help=f"launches per op in the per-op passes (at least {MIN_OP_LAUNCHES})")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after the timed region, stream 256 MiB in and out with the plain-stream "
                        "probe (a copy of known size, to scale HBM traffic counters)")
    p.add_argument("--no-next-ops", action="store_true",
                   help="skip timing the ops beyond the step (softmax, LayerNorm, GeGLU, ...)")
    p.add_argument("--no-stream-ceiling", action="store_true",
                   help="skip timing the plain-stream probe (probe/libet_probe.so)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="least CPU time spent timing the oracle")
    p.add_argument("--dispatch-log", default=None,
                   help="write (run) or read (--summarize) the label of every library call")
    p.add_argument("--summarize", default=None,
                   help="summarise the rocprofv3 output under this directory and exit")
    p.add_argument("--title", default="", help="--summarize: heading of the summary")
    p.add_argument("--command", default="", help="--summarize: the command that made the profile")
    p.add_argument("--labels", default="",
                   help="--summarize: comma-separated label prefixes to report (default: all)")
    return p.parse_args()


# ------------------------------------------------------------------ timing

class TimingEvents:
    """A pair of HIP timing events recorded on a given stream.

    They are created with hipEventDisableSystemFence: a timing marker needs no
    system-scope release, and that release adds about 2 us to the interval it
    brackets.  The HIP runtime is the one torch has already loaded."""

    _hip = None
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            hip = ctypes.CDLL("libamdhip64.so.7")
            vp = ctypes.c_void_p
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [vp, vp]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            hip.hipEventDestroy.argtypes = [vp]
            hip.hipMemcpyAsync.argtypes = [vp, vp, ctypes.c_size_t, ctypes.c_int, vp]
            cls._hip = hip
        return cls._hip

    def __init__(self, stream):
        import ctypes
        hip = self._lib()
        self._stream = ctypes.c_void_p(stream.cuda_stream)
        self._ev = []
        for _ in range(2):
            e = ctypes.c_void_p()
            rc = hip.hipEventCreateWithFlags(ctypes.byref(e), self.FLAGS)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self._ev.append(e)

    def start(self):
        self._check(self._hip.hipEventRecord(self._ev[0], self._stream))

    def stop(self):
        self._check(self._hip.hipEventRecord(self._ev[1], self._stream))

    def elapsed_ms(self):
        import ctypes
        f = ctypes.c_float()
        self._check(self._hip.hipEventElapsedTime(ctypes.byref(f), self._ev[0], self._ev[1]))
        return f.value

    def close(self):
        for e in self._ev:
            self._hip.hipEventDestroy(e)
        self._ev = []

    @staticmethod
    def _check(rc):
        if rc != 0:
            raise RuntimeError(f"HIP event call failed ({rc})")


class DispatchLog:
    """The label of every library call, in launch order, as runs of
    (label, calls).  Every entry point the benchmark calls enqueues exactly
    one kernel at these sizes, so the n-th library kernel of a profile of
    this run belongs to the n-th logged call (--summarize checks that each
    label maps to one kernel and launch shape)."""

    def __init__(self):
        self.runs = []
        self.info = {}

    def add(self, label, calls, **info):
        if calls <= 0:
            return
        if self.runs and self.runs[-1][0] == label:
            self.runs[-1][1] += calls
        else:
            self.runs.append([label, calls])
        if info:
            self.info.setdefault(label, {}).update(info)

    def write(self, path):
        with open(path, "w") as fh:
            json.dump({"runs": self.runs, "info": self.info}, fh)


LOG = DispatchLog()


_HOLD = None


def _hold(stream, launches):
    """Keep `stream` busy while the host enqueues `launches` timed launches
    (probe_hold_kernel, about 60 us of host time per launch, at most 100 ms),
    so that kernels shorter than the host's enqueue time still run back to
    back and their events time the GPU.  A no-op if the probe library cannot
    be loaded."""
    global _HOLD
    if _HOLD is None:
        import ctypes
        try:
            lib = ctypes.CDLL(os.path.join(ROOT, "probe", "libet_probe.so"))
            f = lib.et_probe_hold
            f.argtypes = [ctypes.c_int64, ctypes.c_void_p]
            f.restype = ctypes.c_int
            _HOLD = f
        except (OSError, AttributeError):
            _HOLD = False
    if _HOLD:
        import ctypes
        us = min(100000, 60 * launches)
        if _HOLD(us, ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("probe hold kernel failed to launch")


def _time_launches(stream, fn, sets, launches, label, warm=5):
    """Per-launch HIP-event times (ms) of fn(i), i over rotating buffer sets.
    The events are created before the loop and Python's collector is paused
    inside it, so no host pause lands between an event and its launch; a
    hold kernel ahead of the loop lets the host enqueue the whole batch
    before the first timed launch runs."""
    import torch
    for i in range(warm):
        fn(i)
    evs = [TimingEvents(stream) for _ in range(launches)]
    torch.cuda.synchronize()
    _hold(stream, launches)
    gc.disable()
    try:
        for j, ev in enumerate(evs):
            ev.start()
            fn(warm + j)
            ev.stop()
    finally:
        gc.enable()
    torch.cuda.synchronize()
    LOG.add(label, warm + launches)
    t = [ev.elapsed_ms() for ev in evs]
    for ev in evs:
        ev.close()
    return t


def _stats(t_ms, nbytes, rows=None):
    t = np.asarray(t_ms, dtype=np.float64)
    if t.size == 0 or not np.all(np.isfinite(t)) or np.any(t <= 0):
        raise RuntimeError("no valid timing samples")
    avg = float(np.mean(t))
    gbps = nbytes / (avg * 1e-3) / 1e9
    rec = {"bytes": int(nbytes), "avg_us": round(avg * 1e3, 2),
           "median_us": round(float(np.median(t)) * 1e3, 2),
           "p10_us": round(float(np.percentile(t, 10)) * 1e3, 2),
           "p90_us": round(float(np.percentile(t, 90)) * 1e3, 2),
           "samples": int(t.size), "GBps": round(gbps, 1), "frac_peak": round(gbps / PEAK_GBPS, 4)}
    if t.size >= 40:
        # Launches back to back can slow as the GPU's clock drops under
        # sustained load: the first 20 launches' mean and the slowest mean of
        # 20 consecutive launches show it.
        blocks = [float(np.mean(t[j:j + 20])) for j in range(0, t.size - 19, 20)]
        rec["first20_us"] = round(blocks[0] * 1e3, 2)
        rec["slowest20_us"] = round(max(blocks) * 1e3, 2)
    if rows:
        rec["rows_per_s"] = float(f"{rows / (avg * 1e-3):.4g}")
    return rec


# --------------------------------------------------------------------- ops

# The kernel sources each op is built from (relative to csrc/): a profile
# or counter record of an op stays valid while these files are unchanged.
OP_SOURCES = {
    "silu_mul": ["eltwise.hip", "et_common.hpp"], "add": ["eltwise.hip", "et_common.hpp"],
    "rmsnorm": ["norm.hip", "norm_common.hpp", "et_common.hpp"],
    "add_rmsnorm": ["norm.hip", "norm_common.hpp", "et_common.hpp"],
    "rope": ["rope.hip", "et_common.hpp"], "rmsnorm_rope": ["rope.hip", "et_common.hpp"],
    "embedding": ["gather.hip", "et_common.hpp"], "argmax": ["argmax.hip", "et_common.hpp"],
    "softmax": ["softmax.hip", "et_common.hpp"],
    "layernorm": ["layernorm.hip", "norm_common.hpp", "et_common.hpp"],
    "geglu_erf": ["eltwise.hip", "et_common.hpp"], "geglu_tanh": ["eltwise.hip", "et_common.hpp"],
    "rope_cached": ["rope.hip", "et_common.hpp"], "rope_multi": ["rope.hip", "et_common.hpp"],
}


def op_sources_sha256(op):
    src = os.path.join(ROOT, "elementwise_transformer_amd", "csrc")
    h = hashlib.sha256()
    for f in OP_SOURCES[op]:
        with open(os.path.join(src, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


class Op:
    """One op of a workload: fn(i) launches it on buffer set i % sets.
    rw = (algorithmic bytes read, bytes written) per launch."""

    def __init__(self, cfg, name, rw, kernel, fn, sets, footprint, rows=None):
        self.cfg, self.name, self.kernel = cfg, name, kernel
        self.read_bytes, self.write_bytes = rw
        self.nbytes = self.read_bytes + self.write_bytes
        self.fn, self.sets, self.footprint, self.rows = fn, sets, footprint, rows
        self.label = f"{cfg}/{name}"


def n_sets(footprint):
    """Buffer sets whose total footprint is at least MIN_FOOTPRINT."""
    return max(1, -(-MIN_FOOTPRINT // int(footprint)))


def to_dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:      # bf16 bits
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def build_ops(w, et, torch, rotate=True):
    """Device buffers (rotating sets) and one launcher per op, with its
    algorithmic bytes; the first set holds the workload's inputs, the others
    are copies (for the gather: further id sets of the same distribution)."""
    import workloads as wl
    cfg = f"w{w.number}"
    ops = []

    def k_of(foot):
        return n_sets(foot) if rotate else 1

    def copies(t, k):
        return [t] + [t.clone() for _ in range(k - 1)]

    if w.embed:
        V, d, n, _ = w.embed
        table, ids = wl.gen_embedding(w)
        tt = to_dev(torch, table)
        es = tt.element_size()
        k = k_of(2 * n * d * es)
        idl = [to_dev(torch, ids)] + [to_dev(torch, wl.gen_embedding_ids(w, j)) for j in range(1, k)]
        outs = [torch.empty((n, d), dtype=tt.dtype, device="cuda") for _ in range(k)]
        ops.append(Op(cfg, "embedding", (n * d * es + 4 * n, n * d * es), "embedding_kernel",
                      lambda i, k=k, tt=tt, idl=idl, outs=outs: et.embedding(tt, idl[i % k], out=outs[i % k]),
                      k, 2 * n * d * es))
        del table
    if w.add:
        rows, d = w.add
        a, b = wl.gen_add(w)
        at = to_dev(torch, a)
        es = at.element_size()
        k = k_of(3 * rows * d * es)
        A, B = copies(at, k), copies(to_dev(torch, b), k)
        Y = [torch.empty_like(at) for _ in range(k)]
        ops.append(Op(cfg, "add", (2 * rows * d * es, rows * d * es), "eltwise_vec",
                      lambda i, k=k, A=A, B=B, Y=Y: et.add(A[i % k], B[i % k], out=Y[i % k]), k,
                      3 * rows * d * es))
    if w.rmsnorm:
        rows, d, _ = w.rmsnorm
        x, g, eps = wl.gen_rmsnorm(w)
        xt, gt = to_dev(torch, x), to_dev(torch, g)
        es = xt.element_size()
        k = k_of(2 * rows * d * es)
        X, Y = copies(xt, k), [torch.empty_like(xt) for _ in range(k)]
        ops.append(Op(cfg, "rmsnorm", (rows * d * es + d * es, rows * d * es), "rmsnorm_rows",
                      lambda i, k=k, X=X, Y=Y, gt=gt, eps=eps: et.rmsnorm(X[i % k], gt, eps, out=Y[i % k]),
                      k, 2 * rows * d * es))
    if w.add_rmsnorm:
        rows, d, _, in_place = w.add_rmsnorm
        x, r, g, eps = wl.gen_add_rmsnorm(w)
        xt, rt, gt = to_dev(torch, x), to_dev(torch, r), to_dev(torch, g)
        es = xt.element_size()
        foot = (2 if in_place else 4) * rows * d * es
        k = k_of(foot)
        X, R = copies(xt, k), copies(rt, k)
        if in_place:
            fn = lambda i, k=k, X=X, R=R, gt=gt, eps=eps: et.add_rmsnorm(X[i % k], R[i % k], gt, eps,
                                                                          out=X[i % k], h=R[i % k])
        else:
            Y = [torch.empty_like(xt) for _ in range(k)]
            H = [torch.empty_like(xt) for _ in range(k)]
            fn = lambda i, k=k, X=X, R=R, Y=Y, H=H, gt=gt, eps=eps: et.add_rmsnorm(
                X[i % k], R[i % k], gt, eps, out=Y[i % k], h=H[i % k])
        ops.append(Op(cfg, "add_rmsnorm", (2 * rows * d * es + d * es, 2 * rows * d * es), "rmsnorm_rows",
                      fn, k, foot))
    if w.rope:
        s = w.rope
        heads = s.Hq + s.Hk
        q, kk, pos, inv = wl.gen_rope(w)
        qt = to_dev(torch, q)
        es = qt.element_size()
        foot = s.T * heads * s.D * es
        k = k_of(foot)
        Q = copies(qt, k)
        K = copies(to_dev(torch, kk), k) if kk is not None else [None] * k
        pt, ft = to_dev(torch, pos), to_dev(torch, inv)
        ops.append(Op(cfg, "rope", (s.T * heads * s.r * es + 4 * s.T + 4 * (s.r // 2),
                                    s.T * heads * s.r * es), "rope_qk_kernel",
                      lambda i, k=k, Q=Q, K=K, pt=pt, ft=ft, s=s: et.rope_qk(
                          Q[i % k], K[i % k], pt, ft, d_rot=s.r, attn_scaling=s.mu, layout=s.layout),
                      k, foot))
        del q, kk
        q2, k2, gq, gk, pos2, inv2 = wl.gen_qknorm(w)
        Q2 = copies(to_dev(torch, q2), k)
        K2 = copies(to_dev(torch, k2), k) if k2 is not None else [None] * k
        gqt = to_dev(torch, gq)
        gkt = to_dev(torch, gk) if k2 is not None else None
        p2t, f2t = to_dev(torch, pos2), to_dev(torch, inv2)
        ops.append(Op(cfg, "rmsnorm_rope", (s.T * heads * s.D * es + 2 * s.D * es + 4 * s.T + 4 * (s.r // 2),
                                            s.T * heads * s.D * es), "rmsnorm_rope_kernel",
                      lambda i, k=k, Q2=Q2, K2=K2, gqt=gqt, gkt=gkt, p2t=p2t, f2t=f2t, s=s:
                      et.rmsnorm_rope_qk(Q2[i % k], gqt, K2[i % k], gkt, s.eps, p2t, f2t, d_rot=s.r,
                                         attn_scaling=s.mu, layout=s.layout),
                      k, foot, rows=s.T * heads))
        del q2, k2
    if w.silu:
        rows, cols, _ = w.silu
        gate, up = wl.gen_silu(w)
        gt_ = to_dev(torch, gate)
        del gate
        ut = to_dev(torch, up)
        del up
        es = gt_.element_size()
        k = k_of(3 * rows * cols * es)
        G, U = copies(gt_, k), copies(ut, k)
        Y = [torch.empty_like(gt_) for _ in range(k)]
        ops.append(Op(cfg, "silu_mul", (2 * rows * cols * es, rows * cols * es), "eltwise_vec",
                      lambda i, k=k, G=G, U=U, Y=Y: et.silu_mul(G[i % k], U[i % k], out=Y[i % k]), k,
                      3 * rows * cols * es))
    if w.argmax:
        rows, n = w.argmax
        lg, _ = wl.gen_argmax(w)
        lt = to_dev(torch, lg)
        k = k_of(lt.numel() * lt.element_size())
        L = copies(lt, k)
        ao = torch.empty(rows, dtype=torch.int32, device="cuda")
        ws = torch.zeros(max(16, et.argmax_workspace_bytes(rows, n)), dtype=torch.uint8, device="cuda")
        ops.append(Op(cfg, "argmax", (rows * n * lt.element_size(), 4 * rows), "argmax_rows",
                      lambda i, k=k, L=L, ao=ao, ws=ws: et.argmax(L[i % k], out=ao, workspace=ws), k,
                      rows * n * lt.element_size()))
    torch.cuda.synchronize()
    return ops


def time_ops(ops, stream, launches, ceiling=None, cases=None):
    """Each op alone: `launches` event-timed launches over its rotated sets."""
    out = {}
    for op in ops:
        t = _time_launches(stream, op.fn, op.sets, launches, op.label)
        LOG.info.setdefault(op.label, {}).update(
            {"bytes": op.nbytes, "bytes_read": op.read_bytes, "bytes_written": op.write_bytes,
             "rows": op.rows, "op": op.name, "kernel": op.kernel,
             "sources_sha256": op_sources_sha256(op.name)})
        rec = _stats(t, op.nbytes, op.rows)
        rec["kernel"] = op.kernel
        rec["sets"] = op.sets
        rec["footprint_MB"] = round(op.sets * op.footprint / 1e6, 1)
        case = (cases or {}).get(op.name)
        if ceiling and case in ceiling:
            rec["stream_ceiling"] = case
            rec["frac_of_ceiling"] = round(rec["GBps"] / ceiling[case]["GBps"], 4)
        out[op.name] = rec
    return out


# ---------------------------------------------------------- stream ceiling

# Plain streams the kernels are measured against: (name, operand bytes,
# reads, writes, device-scope stores, persistent-grid workgroups (0: one
# per tile), in place).  Each op is compared with the stream of its own
# shape, with non-temporal stores as the kernels use.
#   large hidden (T = 8192): fused add+RMSNorm reads and writes back x and
#     the residual, 128 MiB each; RoPE q and k, 144 MiB, in place; SiLU-mul
#     operands 448 MiB.
#   prefill (T = 4096): [4096, 4096] bf16 operands of 32 MiB; q and k of the
#     RoPE 40 MiB in place; SiLU-mul operands 112 MiB.
#   decode: the logits [256, 128256] f32 (125 MiB) argmax reads.
#   partial RoPE: q [16384, 16, 128] f32 (128 MiB) the fused RMSNorm+RoPE
#     rewrites in place.
#   next rows: softmax of the decode logits (1 read, 1 write), LayerNorm
#     [4096, 4096] bf16, GeGLU [4096, 14336] bf16, the video RoPE's q and k
#     (225 MiB in place).
#   yardsticks at 32 and 64 MiB, one read and one write: the kernels' grid
#     (one workgroup per tile), persistent grids of 1024 and 2048
#     workgroups, and the runtime's device-to-device copy.
MIB = 1 << 20
CEILING_CASES = [
    ("inplace_2R2W_128MiB", 128 * MIB, 2, 2, 0, 0, True),
    ("inplace_144MiB", 8192 * 72 * 128 * 2, 1, 1, 0, 0, True),
    ("2R1W_448MiB", 8192 * 28672 * 2, 2, 1, 0, 0, False),
    ("1R1W_32MiB", 32 * MIB, 1, 1, 0, 0, False),
    ("2R1W_32MiB", 32 * MIB, 2, 1, 0, 0, False),
    ("2R2W_32MiB", 32 * MIB, 2, 2, 0, 0, False),
    ("inplace_40MiB", 4096 * 40 * 128 * 2, 1, 1, 0, 0, True),
    ("2R1W_112MiB", 4096 * 14336 * 2, 2, 1, 0, 0, False),
    ("read_125MiB", 256 * 128256 * 4, 1, 0, 0, 0, False),
    ("inplace_128MiB", 128 * MIB, 1, 1, 0, 0, True),
    ("1R1W_125MiB", 256 * 128256 * 4, 1, 1, 0, 0, False),
    ("inplace_225MiB", 19200 * 48 * 128 * 2, 1, 1, 0, 0, True),
    ("1R1W_32MiB_persist1024", 32 * MIB, 1, 1, 0, 1024, False),
    ("1R1W_32MiB_persist2048", 32 * MIB, 1, 1, 0, 2048, False),
    ("1R1W_64MiB", 64 * MIB, 1, 1, 0, 0, False),
    ("1R1W_64MiB_persist1024", 64 * MIB, 1, 1, 0, 1024, False),
    ("1R1W_64MiB_persist2048", 64 * MIB, 1, 1, 0, 2048, False),
]
MEMCPY_CASES = [("memcpy_32MiB", 32 * MIB), ("memcpy_64MiB", 64 * MIB)]

OP_CEILING = {
    "w5": {"add_rmsnorm": "inplace_2R2W_128MiB", "rope": "inplace_144MiB",
           "rmsnorm_rope": "inplace_144MiB", "silu_mul": "2R1W_448MiB"},
    "w2": {"rmsnorm": "1R1W_32MiB", "embedding": "1R1W_32MiB", "add": "2R1W_32MiB",
           "add_rmsnorm": "2R2W_32MiB", "rope": "inplace_40MiB",
           "rmsnorm_rope": "inplace_40MiB", "silu_mul": "2R1W_112MiB"},
    "w3": {"argmax": "read_125MiB"},
    "w4": {"rmsnorm_rope": "inplace_128MiB"},
    "next": {"softmax": "1R1W_125MiB", "layernorm": "1R1W_32MiB", "geglu_erf": "2R1W_112MiB",
             "geglu_tanh": "2R1W_112MiB", "rope_cached": "inplace_40MiB",
             "rope_multi": "inplace_225MiB"},
}


def _probe():
    import ctypes
    path = os.path.join(ROOT, "probe", "libet_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing; build it with `python probe/build.py`")
    lib = ctypes.CDLL(path)
    f = lib.et_probe_stream
    vp = ctypes.c_void_p
    f.argtypes = [vp, vp, vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, vp]
    f.restype = ctypes.c_int
    return f


def stream_ceiling(torch, stream, launches=40):
    """Per-launch HIP-event times of plain HBM streams (probe/libet_probe.so:
    16-byte non-temporal loads, stores by the given policy, nothing computed
    between) and of the runtime's device-to-device copy, each over rotating
    buffer sets of at least 1 GiB, so every launch streams from HBM.
    Algorithmic bytes = (reads + writes) x operand bytes; the best of 4 and
    8 vectors per lane is kept."""
    f = _probe()
    out = {}
    for name, nb, nr, nw, dev, persist, inplace in CEILING_CASES:
        sets = max(4, -(-(1 << 30) // (4 * nb)))
        bufs = [[torch.randint(0, 256, (nb,), dtype=torch.uint8, device="cuda") for _ in range(4)]
                for _ in range(sets)]
        best = None
        for u in (4, 8):
            def fn(i, u=u):
                a, b, y, h = bufs[i % sets]
                if inplace:
                    y, h = a, b
                rc = f(a.data_ptr(), b.data_ptr(), y.data_ptr(), h.data_ptr(), nb, nr, nw, u, dev,
                       persist, stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"et_probe_stream failed ({rc}) on {name}")
            t = _time_launches(stream, fn, sets, launches, f"probe/{name}/u{u}")
            avg = float(np.mean(t))
            if best is None or avg < best[0]:
                best = (avg, t, u)
        rec = _stats(best[1], (nr + nw) * nb)
        rec["vectors_per_lane"] = best[2]
        rec["workgroups"] = persist if persist else "one per tile"
        out[name] = rec
        del bufs
    hip = TimingEvents._lib()
    for name, nb in MEMCPY_CASES:
        sets = max(4, -(-(1 << 30) // (2 * nb)))
        bufs = [[torch.randint(0, 256, (nb,), dtype=torch.uint8, device="cuda") for _ in range(2)]
                for _ in range(sets)]

        def cp(i):
            a, y = bufs[i % sets]
            rc = hip.hipMemcpyAsync(y.data_ptr(), a.data_ptr(), nb, 3, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"hipMemcpyAsync failed ({rc})")
        t = _time_launches_plain(stream, cp, launches)
        rec = _stats(t, 2 * nb)
        rec["what"] = "hipMemcpyAsync device to device"
        out[name] = rec
        del bufs
    return out


def _time_launches_plain(stream, fn, launches, warm=5):
    """_time_launches for work that is not a library call (not logged)."""
    import torch
    for i in range(warm):
        fn(i)
    evs = [TimingEvents(stream) for _ in range(launches)]
    torch.cuda.synchronize()
    _hold(stream, launches)
    gc.disable()
    try:
        for j, ev in enumerate(evs):
            ev.start()
            fn(warm + j)
            ev.stop()
    finally:
        gc.enable()
    torch.cuda.synchronize()
    t = [ev.elapsed_ms() for ev in evs]
    for ev in evs:
        ev.close()
    return t


def copy_calibration(torch, stream):
    """A plain copy of known size for scaling the HBM traffic counters: the
    probe's one-read, one-write stream over 256 MiB, three launches (logged
    as calibration/copy_256MiB)."""
    f = _probe()
    nb = 256 * MIB
    a = torch.randint(0, 256, (nb,), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(a)
    for _ in range(3):
        if f(a.data_ptr(), a.data_ptr(), y.data_ptr(), y.data_ptr(), nb, 1, 1, 4, 0, 0,
             stream.cuda_stream) != 0:
            raise RuntimeError("et_probe_stream failed (calibration)")
    torch.cuda.synchronize()
    LOG.add("calibration/copy_256MiB", 3, bytes_read=nb, bytes_written=nb)


# ---------------------------------------------------------------- next ops

def time_next_ops(et, torch, wl, stream, launches):
    """Per-launch HIP-event times of the ops beyond the step, each on the
    inputs its workload names, over rotated sets (footprint >= 768 MB):
      softmax   temperature 0.7 over the decode logits [256, 128256] f32
      layernorm [4096, 4096] bf16 with gain and bias (the prefill hidden size)
      geglu     [4096, 14336] bf16, erf and tanh forms (the prefill FFN size)
      rope_cached  the prefill RoPE (q [4096,32,128], k [4096,8,128] bf16,
                positions 0..4095) with the rotation read from a cos/sin
                cache [4096, 64] f32 built by the library
      rope_multi  3D RoPE of a video DiT: q and k [19200, 24, 128] bf16 over a
                16 x 30 x 40 latent grid, axis widths 16 / 56 / 56
      f16_step  the whole prefill step (every op of it, same shapes and
                inputs) with f16 storage, one event pair per step
    Algorithmic bytes: each input read once, each output written once."""
    out = {}

    def record(name, workload, nbytes, t, kernels, sets, foot, written=None):
        """written: algorithmic bytes written per launch (default: half)."""
        rec = _stats(t, nbytes)
        rec.update({"workload": workload, "kernels": kernels, "sets": sets,
                    "footprint_MB": round(sets * foot / 1e6, 1)})
        out[name] = rec
        if name in OP_SOURCES:
            wb = nbytes // 2 if written is None else written
            LOG.info.setdefault(f"next/{name}", {}).update(
                {"bytes": nbytes, "bytes_read": nbytes - wb, "bytes_written": wb, "op": name,
                 "kernel": kernels, "sources_sha256": op_sources_sha256(name)})

    lg, _ = wl.gen_argmax(wl.WORKLOADS[3])
    rows, n = lg.shape
    foot = 2 * lg.nbytes
    k = n_sets(foot)
    xs = [torch.from_numpy(lg).cuda() for _ in range(k)]
    ys = [torch.empty_like(x) for x in xs]
    ws = torch.zeros(max(et.softmax_workspace_bytes(rows, n), 16), dtype=torch.uint8, device="cuda")
    t = _time_launches(stream, lambda i: et.softmax(xs[i % k], 0.7, out=ys[i % k], workspace=ws), k,
                       launches, "next/softmax")
    record("softmax", "decode logits [256,128256] f32, temperature 0.7", 2 * rows * n * 4, t,
           "softmax_chunks (one launch)", k, foot)
    del xs, ys, ws

    g = np.random.default_rng([1002, 40])
    d = 4096
    x0 = torch.from_numpy(g.standard_normal((4096, d)).astype(np.float32)).to("cuda", torch.bfloat16)
    foot = 2 * x0.numel() * 2
    k = n_sets(foot)
    xs = [x0] + [x0.clone() for _ in range(k - 1)]
    ys = [torch.empty_like(x0) for _ in range(k)]
    gam = torch.from_numpy(g.uniform(0.5, 1.5, d).astype(np.float32)).to("cuda", torch.bfloat16)
    bet = torch.from_numpy(g.standard_normal(d).astype(np.float32)).to("cuda", torch.bfloat16)
    t = _time_launches(stream, lambda i: et.layernorm(xs[i % k], gam, bet, 1e-5, out=ys[i % k]), k,
                       launches, "next/layernorm")
    record("layernorm", "[4096,4096] bf16 with gain and bias, eps 1e-5", 2 * 4096 * d * 2 + 2 * d * 2, t,
           "layernorm_rows", k, foot, written=4096 * d * 2)
    del xs, ys

    g = np.random.default_rng([1002, 41])
    shape = (4096, 14336)
    g0 = torch.from_numpy(g.standard_normal(shape).astype(np.float32)).to("cuda", torch.bfloat16)
    u0 = torch.from_numpy(g.standard_normal(shape).astype(np.float32)).to("cuda", torch.bfloat16)
    foot = 3 * g0.numel() * 2
    k = n_sets(foot)
    gs = [g0] + [g0.clone() for _ in range(k - 1)]
    us = [u0] + [u0.clone() for _ in range(k - 1)]
    ys = [torch.empty_like(g0) for _ in range(k)]
    for form, name in ((et.GELU_ERF, "geglu_erf"), (et.GELU_TANH, "geglu_tanh")):
        t = _time_launches(stream, lambda i, form=form: et.geglu(gs[i % k], us[i % k], form,
                                                                 out=ys[i % k]), k,
                           launches, f"next/{name}")
        record(name, f"[4096,14336] bf16, {'erf' if form == 0 else 'tanh'} form", 3 * 4096 * 14336 * 2,
               t, "eltwise_vec", k, foot, written=4096 * 14336 * 2)
    del gs, us, ys

    w = wl.WORKLOADS[2]
    s = w.rope
    q, kk, pos, inv = wl.gen_rope(w)
    q0, k0 = to_dev(torch, q), to_dev(torch, kk)
    foot = (q0.numel() + k0.numel()) * 2
    k = n_sets(foot)
    qs = [q0] + [q0.clone() for _ in range(k - 1)]
    ks = [k0] + [k0.clone() for _ in range(k - 1)]
    pt = torch.from_numpy(pos).cuda()
    cc, sc = et.rope_cache(torch.from_numpy(inv).cuda(), s.T, s.r)
    LOG.add("next/rope_cache_build", 1)
    t = _time_launches(stream, lambda i: et.rope_qk_cached(qs[i % k], ks[i % k], pt, cc, sc,
                                                           d_rot=s.r, attn_scaling=s.mu,
                                                           layout=s.layout), k, launches,
                       "next/rope_cached")
    heads = s.Hq + s.Hk
    record("rope_cached", "prefill RoPE q [4096,32,128] k [4096,8,128] bf16, cache [4096,64] f32",
           2 * s.T * heads * s.r * 2 + 4 * s.T + 2 * s.T * (s.r // 2) * 4, t, "rope_qk_kernel (cached)",
           k, foot, written=s.T * heads * s.r * 2)
    del qs, ks

    w = wl.WORKLOADS[6]
    m = w.rope_multi
    q, kk, pos, inv = wl.gen_rope_multi(w)
    q0, k0 = to_dev(torch, q), to_dev(torch, kk)
    foot = (q0.numel() + k0.numel()) * 2
    k = n_sets(foot)
    qs = [q0] + [q0.clone() for _ in range(k - 1)]
    ks = [k0] + [k0.clone() for _ in range(k - 1)]
    pt = torch.from_numpy(pos).cuda()
    ft = torch.from_numpy(inv).cuda()
    t = _time_launches(stream, lambda i: et.rope_multi(qs[i % k], ks[i % k], pt, m.dims, ft,
                                                       attn_scaling=m.mu, layout=m.layout), k,
                       launches, "next/rope_multi")
    span = sum(m.dims)
    record("rope_multi", "video DiT 3D RoPE q,k [19200,24,128] bf16, grid 16x30x40, widths 16/56/56",
           2 * m.T * (m.Hq + m.Hk) * span * 2 + 4 * 3 * m.T + 4 * (span // 2), t, "rope_multi_kernel",
           k, foot, written=m.T * (m.Hq + m.Hk) * span * 2)
    del qs, ks

    import dataclasses
    wf = dataclasses.replace(wl.WORKLOADS[2], dtype="f16")
    ops = build_ops(wf, et, torch)
    for op in ops:
        op.label = f"f16/{op.name}"

    def step(i):
        for op in ops:
            op.fn(i)
    t = _time_launches_plain(stream, step, 40, warm=5)
    for _ in range(45):
        for op in ops:
            LOG.add(op.label, 1)
    record("f16_step", "the prefill step of llama3-8b-prefill-T4096 with f16 storage",
           sum(op.nbytes for op in ops), t, "the step's eight kernels, f16 instances", 1,
           sum(op.sets * op.footprint for op in ops))
    del ops
    return out


# ------------------------------------------------------------ CPU baseline

def cpu_baseline(w, min_seconds, frac=8):
    """The CPU oracle as it stands, timed on a bounded sample of the same
    workload: every op of the step on the first 1/frac of its rows (tokens),
    repeated until at least min_seconds of work; GB/s of the sample's
    algorithmic bytes."""
    import oracle
    import workloads as wl
    orc = oracle.load()
    calls = []            # (bytes, closure)
    es = 4 if w.dtype == "f32" else 2

    def head(a, n):
        return None if a is None else np.ascontiguousarray(a[:n])

    if w.embed:
        V, d, n, _ = w.embed
        table, ids = wl.gen_embedding(w)
        m = max(1, n // frac)
        ids = ids[:m].copy()
        calls.append((2 * m * d * es + 4 * m, lambda: orc.embedding(table, ids)))
    if w.add:
        rows, d = w.add
        a, b = wl.gen_add(w)
        m = max(1, rows // frac)
        a, b = head(a, m), head(b, m)
        calls.append((3 * m * d * es, lambda: orc.add(a, b)))
    if w.rmsnorm:
        rows, d, _ = w.rmsnorm
        x, g, eps1 = wl.gen_rmsnorm(w)
        m = max(1, rows // frac)
        x = head(x, m)
        calls.append((2 * m * d * es, lambda: orc.rmsnorm(x, g, eps1)))
    if w.add_rmsnorm:
        rows, d, _, _ = w.add_rmsnorm
        xa, ra, ga, eps2 = wl.gen_add_rmsnorm(w)
        m = max(1, rows // frac)
        xa, ra = head(xa, m), head(ra, m)
        calls.append((4 * m * d * es, lambda: orc.add_rmsnorm(xa, ra, ga, eps2)))
    if w.rope:
        s = w.rope
        m = max(1, s.T // frac)
        q, k, pos, inv = wl.gen_rope(w)
        q, k, pos = head(q, m), head(k, m), pos[:m].copy()

        def rope_both():
            orc.rope(q, pos, s.r, inv, s.mu, s.layout)
            if k is not None:
                orc.rope(k, pos, s.r, inv, s.mu, s.layout)
        calls.append((2 * m * (s.Hq + s.Hk) * s.r * es, rope_both))
        q2, k2, gq, gk, pos2, inv2 = wl.gen_qknorm(w)
        q2, k2, pos2 = head(q2, m), head(k2, m), pos2[:m].copy()

        def qk_both():
            orc.rmsnorm_rope(q2, gq, s.eps, pos2, s.r, inv2, s.mu, s.layout)
            if k2 is not None:
                orc.rmsnorm_rope(k2, gk, s.eps, pos2, s.r, inv2, s.mu, s.layout)
        calls.append((2 * m * (s.Hq + s.Hk) * s.D * es, qk_both))
    if w.silu:
        rows, cols, _ = w.silu
        gate, up = wl.gen_silu(w)
        m = max(1, rows // frac)
        gate, up = head(gate, m), head(up, m)
        calls.append((3 * m * cols * es, lambda: orc.silu_mul(gate, up)))
    if w.argmax:
        rows, n = w.argmax
        lg, _ = wl.gen_argmax(w)
        m = max(1, rows // frac)
        lg = head(lg, m)
        calls.append((m * n * lg.itemsize, lambda: orc.argmax(lg)))
    step_bytes = sum(b for b, _ in calls)
    reps, t_total = 0, 0.0
    while t_total < min_seconds or reps == 0:
        t0 = time.perf_counter()
        for _, fn in calls:
            fn()
        t_total += time.perf_counter() - t0
        reps += 1
    cpu = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(reps * step_bytes / t_total / 1e9, 3), "unit": "GB/s",
            "cores": orc.threads(), "cpu": cpu, "kind": "oracle", "seconds": round(t_total, 2),
            "sample": f"{reps} passes of every op of {w.name} on its first 1/{frac} of rows "
                      f"(tokens): {step_bytes} algorithmic bytes per pass"}


def cpu_next_ops(next_ops, min_seconds):
    """The CPU oracle as it stands on a bounded sample of each next op's
    workload (same generators, shapes and distributions, fewer rows or
    tokens), timed like cpu_baseline: GB/s of algorithmic bytes, added to
    that op's record as cpu_GBps with the sample named."""
    import dataclasses
    import oracle
    import workloads as wl
    orc = oracle.load()

    def put(name, fn, nbytes, sample):
        if name not in next_ops:
            return
        reps, t = 0, 0.0
        while t < min_seconds or reps == 0:
            t0 = time.perf_counter()
            fn()
            t += time.perf_counter() - t0
            reps += 1
        next_ops[name]["cpu_GBps"] = round(reps * nbytes / t / 1e9, 3)
        next_ops[name]["cpu_sample"] = sample

    lg, _ = wl.gen_argmax(wl.WORKLOADS[3])
    lg = np.ascontiguousarray(lg[:32])
    put("softmax", lambda: orc.softmax(lg, 0.7), 2 * lg.size * 4, "32 of the 256 rows")
    g = np.random.default_rng([1002, 40])
    x = wl.store(g.standard_normal((512, 4096)).astype(np.float32), "bf16")
    gm = wl.store(g.uniform(0.5, 1.5, 4096).astype(np.float32), "bf16")
    bt = wl.store(g.standard_normal(4096).astype(np.float32), "bf16")
    put("layernorm", lambda: orc.layernorm(x, gm, bt, 1e-5), 2 * x.size * 2 + 2 * 4096 * 2,
        "512 of the 4096 rows")
    g = np.random.default_rng([1002, 41])
    ga = wl.store(g.standard_normal((512, 14336)).astype(np.float32), "bf16")
    ua = wl.store(g.standard_normal((512, 14336)).astype(np.float32), "bf16")
    for form, name in ((0, "geglu_erf"), (1, "geglu_tanh")):
        put(name, lambda: orc.geglu(ga, ua, form), 3 * ga.size * 2, "512 of the 4096 rows")
    w2 = wl.WORKLOADS[2]
    s = w2.rope
    q, k, pos, inv = wl.gen_rope(w2)
    q, k, pos = np.ascontiguousarray(q[:512]), np.ascontiguousarray(k[:512]), pos[:512].copy()
    oc, osn = orc.rope_cache(inv, s.T, s.r)

    def cached():
        orc.rope_cached(q, pos, s.r, oc, osn, s.mu, s.layout)
        orc.rope_cached(k, pos, s.r, oc, osn, s.mu, s.layout)
    put("rope_cached", cached, 2 * 512 * (s.Hq + s.Hk) * s.r * 2 + 4 * 512 + 2 * 512 * (s.r // 2) * 4,
        "512 of the 4096 tokens")
    w6 = wl.WORKLOADS[6]
    m = w6.rope_multi
    q, k, pos, inv = wl.gen_rope_multi(w6)
    q, k, pos = np.ascontiguousarray(q[:2400]), np.ascontiguousarray(k[:2400]), pos[:2400].copy()

    def multi():
        orc.rope_multi(q, pos, m.dims, inv, m.mu, m.layout)
        orc.rope_multi(k, pos, m.dims, inv, m.mu, m.layout)
    put("rope_multi", multi, 2 * 2400 * (m.Hq + m.Hk) * sum(m.dims) * 2 + 12 * 2400,
        "2400 of the 19200 tokens (two frames)")
    if "f16_step" in next_ops:
        c = cpu_baseline(dataclasses.replace(w2, dtype="f16"), min_seconds)
        next_ops["f16_step"]["cpu_GBps"] = c["value"]
        next_ops["f16_step"]["cpu_sample"] = c["sample"]


# -------------------------------------------------------- profile summary

_LIB_KERNEL = re.compile(r"(?<![A-Za-z0-9_])(et|etprobe)::")


def _is_library_kernel(name):
    """Kernels of libet.so (namespace et) and of the stream probe
    (namespace etprobe); everything else in a trace is torch's or the
    runtime's."""
    return _LIB_KERNEL.search(name) is not None


def _short(name):
    """The demangled name without its return type, anonymous namespaces
    and parameter list."""
    name = name.replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    return name.split("(")[0]


def _read_csv(path):
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _find(d, pattern):
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    return hits[0] if hits else None


def _dispatch_labels(log, n_kernels):
    seq = []
    for label, calls in log["runs"]:
        seq.extend([label] * calls)
    if len(seq) != n_kernels:
        raise SystemExit(f"the profile holds {n_kernels} library kernels but the dispatch log "
                         f"{len(seq)} calls: they do not belong to the same run")
    return seq


def summarize(d, log_path, title, command, prefixes=()):
    """Markdown summary of a rocprofv3 run of this benchmark: a kernel trace
    (kernel_trace.csv) gives one row per (op, kernel, launch shape) with
    average / median / p10 / p90 durations and GB/s of algorithmic bytes; a
    counter run (counter_collection.csv with FETCH_SIZE or WRITE_SIZE) gives
    HBM bytes per launch, scaled by the counter's reading for the 256 MiB
    calibration copy.  Rows are labelled from the dispatch log, so a kernel
    that serves two ops or two shapes gets two rows; a row above peak
    bandwidth is marked invalid."""
    log = json.load(open(log_path))
    info = log.get("info", {})
    keep = (lambda lab: any(lab.startswith(p) for p in prefixes)) if prefixes else (lambda lab: True)
    lines = [f"# {title or 'rocprofv3 summary'}", ""]
    if command:
        lines += ["Command:", "", "```", command, "```", ""]
    trace = _find(d, "*kernel_trace.csv")
    stats = _find(d, "*kernel_stats.csv")
    counters = _find(d, "*counter_collection.csv")
    if trace:
        rows = [r for r in _read_csv(trace) if _is_library_kernel(r["Kernel_Name"])]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        labels = _dispatch_labels(log, len(rows))
        groups = {}
        for lab, r in zip(labels, rows):
            grid = f'{r["Grid_Size_X"]}x{r.get("Grid_Size_Y", "1")}x{r.get("Grid_Size_Z", "1")}'
            blk = f'{r["Workgroup_Size_X"]}x{r.get("Workgroup_Size_Y", "1")}x{r.get("Workgroup_Size_Z", "1")}'
            key = (lab, _short(r["Kernel_Name"]), grid, blk, r.get("LDS_Block_Size", ""),
                   r.get("VGPR_Count", r.get("Arch_VGPR_Count", "")))
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3   # us
            groups.setdefault(key, []).append(dur)
        per_label = {}
        for key in groups:
            per_label.setdefault(key[0], []).append(key)
        for lab, keys in per_label.items():
            if len(keys) != 1 and not lab.startswith("probe/") and not lab.startswith("f16/"):
                raise SystemExit(f"label {lab} maps to {len(keys)} kernels or launch shapes: {keys}")
        lines += ["Kernel trace: one row per op (label) and launch shape; durations in us from "
                  "the trace's start and end timestamps; GB/s = algorithmic bytes / average "
                  "duration; % of the 8 TB/s HBM peak.", "",
                  "| label | kernel | grid | workgroup | VGPRs | calls | avg us | median | p10 | p90 | "
                  "algorithmic MB | GB/s | % peak | sources sha256 (16) |",
                  "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
        for key, durs in groups.items():
            lab, kern, grid, blk, lds, vgpr = key
            if not keep(lab):
                continue
            t = np.asarray(durs)
            nb = info.get(lab, {}).get("bytes")
            if nb:
                gbps = nb / (t.mean() * 1e-6) / 1e9
                frac = gbps / PEAK_GBPS
                g_s = f"{gbps:.1f}"
                f_s = f"{100 * frac:.1f}" + (" INVALID: above peak" if frac > 1.0 else "")
                mb = f"{nb / 1e6:.2f}"
            else:
                g_s = f_s = mb = "-"
            sha = info.get(lab, {}).get("sources_sha256", "")[:16] or "-"
            lines.append(f"| {lab} | `{kern[:90]}` | {grid} | {blk} | {vgpr} | {t.size} | {t.mean():.2f} | "
                         f"{np.median(t):.2f} | {np.percentile(t, 10):.2f} | {np.percentile(t, 90):.2f} | "
                         f"{mb} | {g_s} | {f_s} | {sha} |")
        lines.append("")
        if stats:
            # rocprofv3's own --stats rows (per kernel name, every launch of it
            # in the run) for the kernels of the rows above.
            names = {r["Kernel_Name"] for lab, r in zip(labels, rows) if keep(lab)}
            lines += ["rocprofv3 --stats rows of these kernels (all their launches in the run):", "",
                      "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
            for r in _read_csv(stats):
                if r["Name"] in names:
                    lines.append(f"| `{_short(r['Name'])[:90]}` | {r['Calls']} | "
                                 f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                                 f"{float(r['MaxNs']) / 1e3:.2f} |")
            lines.append("")
    if counters:
        rows = [r for r in _read_csv(counters) if _is_library_kernel(r["Kernel_Name"])]
        by_disp = {}
        for r in rows:
            by_disp.setdefault(int(r["Dispatch_Id"]), []).append(r)
        disp = sorted(by_disp)
        labels = _dispatch_labels(log, len(disp))
        vals = {}
        names = set()
        for lab, did in zip(labels, disp):
            for r in by_disp[did]:
                names.add(r["Counter_Name"])
                vals.setdefault((lab, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
        cal = "calibration/copy_256MiB"
        lines += ["HBM traffic counters (KiB per dispatch in rocprofv3; here bytes per launch, "
                  "scaled by factor = true bytes / counter bytes of the calibration copy).", ""]
        for cname in sorted(names):
            key = "bytes_read" if cname.startswith("FETCH") else "bytes_written"
            c = vals.get((cal, cname))
            truth = info.get(cal, {}).get(key)
            factor = truth / (np.mean(c) * 1024) if c and truth else None
            lines += [f"Counter {cname}: the calibration copy counts {np.mean(c) * 1024:.0f} B for the "
                      f"{truth} B it {'reads' if key == 'bytes_read' else 'writes'}, factor {factor:.4f}."
                      if factor else f"Counter {cname}: no calibration.",
                      "", f"| label | launches | counter bytes per launch | scaled bytes | algorithmic "
                          f"{'read' if key == 'bytes_read' else 'written'} bytes | sources sha256 |",
                      "|---|---|---|---|---|---|"]
            for (lab, cn), v in vals.items():
                if cn != cname or lab == cal or not keep(lab):
                    continue
                raw = float(np.mean(v)) * 1024
                sc = raw * factor if factor else float("nan")
                nb = info.get(lab, {}).get(key, "-")
                sha = info.get(lab, {}).get("sources_sha256", "-")
                lines.append(f"| {lab} | {len(v)} | {raw:.0f} | {sc:.0f} | {nb} | {sha} |")
            lines.append("")
    print("\n".join(lines))


def traffic_record(label):
    """HBM bytes per launch of the op with this dispatch label, from the
    committed counter summaries (profiles/*_hbm_counters.md: FETCH_SIZE and
    WRITE_SIZE rows, scaled by a plain copy of known size), when both were
    taken on the current sources of the op's kernel; else None."""
    op = label.split("/")[-1]
    want = op_sources_sha256(op) if op in OP_SOURCES else None
    total, seen = 0.0, set()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_counters.md"))):
        cname = None
        for line in open(path):
            m = re.match(r"Counter (\w+):", line)
            if m:
                cname = m.group(1)
                continue
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if cname and len(cells) == 6 and cells[0] == label and cells[5] == want:
                try:
                    total += float(cells[3])
                    seen.add(cname)
                except ValueError:
                    pass
    return round(total) if {"FETCH_SIZE", "WRITE_SIZE"} <= seen else None


# -------------------------------------------------------------------- main

def main():
    args = parse()
    if args.summarize:
        if not args.dispatch_log:
            raise SystemExit("--summarize needs --dispatch-log")
        summarize(args.summarize, args.dispatch_log, args.title, args.command,
                  tuple(x for x in args.labels.split(",") if x))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the ops shard by rows with "
                          "no communication, so per-GPU throughput is the one-GPU figure",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    launches = max(MIN_OP_LAUNCHES, args.op_launches)
    import torch
    import elementwise_transformer_amd as et
    import workloads as wl

    w = wl.WORKLOADS[args.workload]
    ops = build_ops(w, et, torch)
    stream = torch.cuda.current_stream()
    for s in range(args.warmup):
        for op in ops:
            op.fn(s)
            LOG.add(op.label, 1)
    torch.cuda.synchronize()

    # Timed region: K steps back to back on one stream (the host issues a
    # step in far less time than the GPU runs it, so the queue stays ahead);
    # step s uses buffer set s of every op.  A pair of HIP events on the
    # launch stream (torch's current stream, which the binding passes to every
    # entry point) brackets the dominant op in every step.
    dom = max(range(len(ops)), key=lambda i: ops[i].nbytes)
    evs = [TimingEvents(stream) for _ in range(args.steps)]
    torch.cuda.synchronize()
    gc.disable()                      # no collector pause inside the timed region
    t0 = time.perf_counter()
    for s in range(args.steps):
        for i, op in enumerate(ops):
            if i == dom:
                evs[s].start()
            op.fn(args.warmup + s)
            if i == dom:
                evs[s].stop()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    for s in range(args.steps):
        for op in ops:
            LOG.add(op.label, 1)
    dom_ms = [ev.elapsed_ms() for ev in evs]
    for ev in evs:
        ev.close()
    step_bytes = sum(op.nbytes for op in ops)
    ms_step = wall * 1e3 / args.steps

    # After the timed region: plain-stream yardsticks, then every op alone.
    ceiling = None if args.no_stream_ceiling else stream_ceiling(torch, stream)
    cfg = f"w{args.workload}"
    per_op = time_ops(ops, stream, launches, ceiling, OP_CEILING.get(cfg))
    if args.copy_calibration:
        copy_calibration(torch, stream)
    dom_op = ops[dom]
    del ops
    gc.collect()
    torch.cuda.empty_cache()

    configs = {}
    for c in [int(x) for x in args.configs.split(",") if x.strip()]:
        if c == args.workload:
            continue
        wc = wl.WORKLOADS[c]
        cops = build_ops(wc, et, torch)
        configs[wc.name] = {"workload": c, "storage": wc.dtype,
                            "ops": time_ops(cops, stream, launches, ceiling, OP_CEILING.get(f"w{c}"))}
        del cops
        gc.collect()
        torch.cuda.empty_cache()

    next_ops = None if args.no_next_ops else time_next_ops(et, torch, wl, stream, launches)
    if ceiling and next_ops:
        for name, rec in next_ops.items():
            case = OP_CEILING["next"].get(name)
            if case:
                rec["stream_ceiling"] = case
                rec["frac_of_ceiling"] = round(rec["GBps"] / ceiling[case]["GBps"], 4)

    # Roofline of the dominant kernel from its in-step launches.
    dstat = _stats(dom_ms, dom_op.nbytes)
    achieved = dstat["GBps"]
    roofline = {"bound": "hbm", "kernel": dom_op.kernel, "op": dom_op.name, "achieved": achieved,
                "peak": PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4),
                "traffic": traffic_record(dom_op.label), "bytes_per_launch": dom_op.nbytes,
                "avg_launch_us": dstat["avg_us"], "median_launch_us": dstat["median_us"],
                "samples": dstat["samples"],
                "timing": "HIP events around the op in every step of the timed region"}
    case = OP_CEILING.get(cfg, {}).get(dom_op.name)
    if ceiling and case:
        roofline["stream_ceiling"] = {"case": case, "GBps": ceiling[case]["GBps"],
                                      "frac_of_ceiling": round(achieved / ceiling[case]["GBps"], 4)}
    for name, rec in per_op.items():
        tr = traffic_record(f"{cfg}/{name}")
        if tr is not None:
            rec["traffic_bytes"] = tr

    # The step as plain streams: each op's bytes at the rate of the stream
    # of its shape and store policy, against the measured step.
    step_ceiling = None
    cases = OP_CEILING.get(cfg, {})
    if ceiling and cases and all(n in cases for n in per_op):
        eq_s = sum(per_op[n]["bytes"] / (ceiling[cases[n]]["GBps"] * 1e9) for n in per_op)
        step_ceiling = {"stream_step_us": round(eq_s * 1e6, 2), "step_us": round(ms_step * 1e3, 2),
                        "frac": round(eq_s * 1e3 / ms_step, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)
        if next_ops:
            cpu_next_ops(next_ops, 1.0)
    if args.dispatch_log:
        LOG.write(args.dispatch_log)

    s = w.rope
    value = step_bytes / (ms_step * 1e-3) / 1e9
    line = {
        "metric": "achieved HBM GB/s (% of MI355X peak) per op; rows/s for fused RMSNorm+RoPE",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "frac_peak": round(value / PEAK_GBPS, 4),
        "rmsnorm_rope_rows_per_s": per_op.get("rmsnorm_rope", {}).get("rows_per_s"),
        "config": {"workload": w.name, "storage": w.dtype, "step_bytes": step_bytes,
                   "ops": list(per_op),
                   "T": s.T if s else None, "heads_q": s.Hq if s else None,
                   "heads_kv": s.Hk if s else None, "head_dim": s.D if s else None,
                   "hidden": (w.add_rmsnorm or w.rmsnorm or (None, None))[1],
                   "intermediate": w.silu[1] if w.silu else None,
                   "vocab": w.embed[0] if w.embed else None,
                   "rotation": f"buffer sets of >= {MIN_FOOTPRINT // 10**6} MB per op"},
        "ops": per_op,
        "roofline": roofline,
        "configs": configs,
        "stream_ceiling": ceiling,
        "step_vs_stream_ceiling": step_ceiling,
        "next_ops": next_ops,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
