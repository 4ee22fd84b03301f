"""Benchmark of the memory-bound transformer ops on one MI355X.

One step = one pass of every op on the workload's synthetic inputs:
embedding gather, residual add, RMSNorm, fused add+RMSNorm, RoPE on Q and K,
fused RMSNorm+RoPE on Q and K, SiLU-mul and greedy argmax (the ops a workload
names; workload 2, the default, names them all).  Each op has its own
buffers, so no op reads what the previous op just wrote (the 256 MB
Infinity Cache cannot serve an op from its predecessor's output), and one
step moves far more than 256 MB, so every op starts cold.

Prints ONE JSON line: whole-step throughput in GB/s of algorithmic HBM
traffic (each input read once, each output written once; in-place RoPE counts
only rotated entries), per-op GB/s and fraction of the 8 TB/s peak from HIP
events on the launch stream, rows/s for the fused RMSNorm+RoPE, the roofline
record of the dominant kernel and the CPU oracle timed on a sample.  After the
timed region it also times plain HBM streams (libet_probe.so: loads and stores
only, at the step's operand sizes and store policies) and reports each op's
fraction of the stream of its own shape.

    python bench.py [--steps K] [--warmup W] [--workload 2|3|4|5]
"""
from __future__ import annotations

import argparse
import gc
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after the timed region, run three 256 MiB device-to-device copies (a "
                        "plain copy kernel of known size, to scale HBM traffic counters)")
    p.add_argument("--no-next-ops", action="store_true",
                   help="skip timing the ops beyond the step (softmax, LayerNorm, GeGLU)")
    p.add_argument("--no-stream-ceiling", action="store_true",
                   help="skip timing the plain-stream probe (libet_probe.so)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="least CPU time spent timing the oracle on whole steps")
    return p.parse_args()


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


class Op:
    def __init__(self, name, nbytes, fn, kernel, rows=None):
        self.name, self.nbytes, self.fn, self.kernel, self.rows = name, nbytes, fn, kernel, rows
        self.ms = []


def build_ops(w, et, torch):
    """Device buffers and one closure per op, with algorithmic bytes."""
    import workloads as wl
    from_np = lambda a: (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
                         if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a))).cuda()
    es = 4 if w.dtype == "f32" else 2
    ops = []
    if w.embed:
        V, d, n, _ = w.embed
        table, ids = wl.gen_embedding(w)
        tt, it = from_np(table), from_np(ids)
        out = torch.empty((n, d), dtype=tt.dtype, device="cuda")
        ops.append(Op("embedding", 2 * n * d * es + 4 * n, lambda: et.embedding(tt, it, out=out),
                      "embedding_kernel"))
    if w.add:
        rows, d = w.add
        a, b = wl.gen_add(w)
        at, bt = from_np(a), from_np(b)
        yt = torch.empty_like(at)
        ops.append(Op("add", 3 * rows * d * es, lambda: et.add(at, bt, out=yt), "eltwise_vec"))
    if w.rmsnorm:
        rows, d, eps = w.rmsnorm
        x, g, eps = wl.gen_rmsnorm(w)
        xt, gt = from_np(x), from_np(g)
        yn = torch.empty_like(xt)
        ops.append(Op("rmsnorm", 2 * rows * d * es + d * es,
                      lambda: et.rmsnorm(xt, gt, eps, out=yn), "rmsnorm_rows"))
    if w.add_rmsnorm:
        rows, d, eps, in_place = w.add_rmsnorm
        x, r, g, eps = wl.gen_add_rmsnorm(w)
        xa, ra, ga = from_np(x), from_np(r), from_np(g)
        if in_place:
            fn = lambda: et.add_rmsnorm(xa, ra, ga, eps, out=xa, h=ra)
        else:
            ya, ha = torch.empty_like(xa), torch.empty_like(xa)
            fn = lambda: et.add_rmsnorm(xa, ra, ga, eps, out=ya, h=ha)
        ops.append(Op("add_rmsnorm", 4 * rows * d * es + d * es, fn, "rmsnorm_rows"))
    if w.rope:
        s = w.rope
        q, k, pos, inv = wl.gen_rope(w)
        qt, kt, pt, ft = from_np(q), (from_np(k) if k is not None else None), from_np(pos), from_np(inv)
        heads = s.Hq + s.Hk
        ops.append(Op("rope", 2 * s.T * heads * s.r * es + 4 * s.T + 4 * (s.r // 2),
                      lambda: et.rope_qk(qt, kt, pt, ft, d_rot=s.r, attn_scaling=s.mu,
                                         layout=s.layout), "rope_qk_kernel"))
        q2, k2, gq, gk, pos2, inv2 = wl.gen_qknorm(w)
        q2t, k2t = from_np(q2), (from_np(k2) if k2 is not None else None)
        gqt, gkt = from_np(gq), (from_np(gk) if k2 is not None else None)
        p2t, f2t = from_np(pos2), from_np(inv2)
        ops.append(Op("rmsnorm_rope", 2 * s.T * heads * s.D * es + 2 * s.D * es + 4 * s.T
                      + 4 * (s.r // 2),
                      lambda: et.rmsnorm_rope_qk(q2t, gqt, k2t, gkt, s.eps, p2t, f2t, d_rot=s.r,
                                                 attn_scaling=s.mu, layout=s.layout),
                      "rmsnorm_rope_kernel", rows=s.T * heads))
    if w.silu:
        rows, cols, _ = w.silu
        gate, up = wl.gen_silu(w)
        gt_, ut = from_np(gate), from_np(up)
        ys = torch.empty_like(gt_)
        ops.append(Op("silu_mul", 3 * rows * cols * es, lambda: et.silu_mul(gt_, ut, out=ys),
                      "eltwise_vec"))
    if w.argmax:
        rows, n = w.argmax
        lg, _ = wl.gen_argmax(w)
        lt = from_np(lg)
        ao = torch.empty(rows, dtype=torch.int32, device="cuda")
        ws = torch.zeros(max(1, et.argmax_workspace_bytes(rows, n)), dtype=torch.uint8, device="cuda")
        ops.append(Op("argmax", rows * n * lt.element_size() + 4 * rows,
                      lambda: et.argmax(lt, out=ao, workspace=ws), "argmax_chunks"))
    return ops


COUNTER_SUMMARY = {2: "prefill_bf16_T4096_hbm_counters.md"}


# The kernel sources each step op is built from (relative to csrc/): a
# counter record stays valid while these files are unchanged.
OP_SOURCES = {
    "silu_mul": ["eltwise.hip", "et_common.hpp"], "add": ["eltwise.hip", "et_common.hpp"],
    "rmsnorm": ["norm.hip", "norm_common.hpp", "et_common.hpp"],
    "add_rmsnorm": ["norm.hip", "norm_common.hpp", "et_common.hpp"],
    "rope": ["rope.hip", "et_common.hpp"], "rmsnorm_rope": ["rope.hip", "et_common.hpp"],
    "embedding": ["gather.hip", "et_common.hpp"], "argmax": ["argmax.hip", "et_common.hpp"],
}


def op_sources_sha256(op):
    src = os.path.join(ROOT, "elementwise_transformer_amd", "csrc")
    h = hashlib.sha256()
    for f in OP_SOURCES[op]:
        with open(os.path.join(src, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_record(workload, op):
    """HBM bytes per launch of `op` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy of known size),
    if that summary covers this workload and was taken on the current sources
    of that op's kernel; else None."""
    name = COUNTER_SUMMARY.get(workload)
    path = os.path.join(ROOT, "profiles", name) if name else ""
    if not name or not os.path.exists(path) or op not in OP_SOURCES:
        return None
    text = open(path).read()
    m = re.search(r"traffic bytes per launch:\s*" + re.escape(op) + r"\s+([0-9.eE+]+)\s+sources sha256\s+"
                  r"([0-9a-f]{64})", text)
    if not m:
        return None
    return float(m.group(1)) if op_sources_sha256(op) == m.group(2) else None


def _time_launches(stream, fn, sets, launches):
    """Per-launch HIP-event times (ms) of fn(i), i over rotating buffer sets.
    The events are created before the loop and Python's collector is paused
    inside it, so no host pause lands between an event and its launch."""
    import gc
    import torch
    for i in range(sets * 2):
        fn(i)
    evs = [TimingEvents(stream) for _ in range(launches)]
    torch.cuda.synchronize()
    gc.disable()
    try:
        for i, ev in enumerate(evs):
            ev.start()
            fn(i)
            ev.stop()
    finally:
        gc.enable()
    torch.cuda.synchronize()
    t = [ev.elapsed_ms() for ev in evs]
    for ev in evs:
        ev.close()
    return t


# Plain streams the kernels are measured against: (name, operand bytes,
# reads, writes, device-scope stores).  32 MiB is one [4096, 4096] bf16
# operand of the prefill row ops (RMSNorm and the gather read one and write
# one, add reads two and writes one, fused add+RMSNorm reads two and writes
# two); 112 MiB one [4096, 14336] bf16 operand of the prefill SiLU-mul (two
# reads, one write) and GeGLU; 125 MiB the decode logits [256, 128256] f32
# softmax reads and writes; 225 MiB the q and k [19200, 24, 128] bf16 the
# multi-axis RoPE rotates in place; "inplace" cases write back over what they read
# (the output buffer is the input), as RoPE does to q and k [4096, 32 + 8,
# 128] bf16 (40 MiB).  Non-temporal and device-scope stores are the two
# policies the kernels choose between by output size.
CEILING_CASES = [
    ("read_32MiB", 32 << 20, 1, 0, 0),
    ("write_32MiB", 32 << 20, 0, 1, 0),
    ("1R1W_32MiB", 32 << 20, 1, 1, 0),
    ("1R1W_32MiB_dev", 32 << 20, 1, 1, 1),
    ("2R1W_32MiB", 32 << 20, 2, 1, 0),
    ("2R1W_32MiB_dev", 32 << 20, 2, 1, 1),
    ("2R2W_32MiB", 32 << 20, 2, 2, 0),
    ("2R1W_112MiB", 4096 * 14336 * 2, 2, 1, 0),
    ("2R1W_112MiB_dev", 4096 * 14336 * 2, 2, 1, 1),
    ("1R1W_125MiB", 256 * 128256 * 4, 1, 1, 0),
    ("inplace_225MiB", 19200 * 48 * 128 * 2, 1, 1, 0),
    ("inplace_40MiB_dev", 4096 * 40 * 128 * 2, 1, 1, 1),
]
# Cases only the large-hidden chain (workload 5: T = 8192, hidden 8192, FFN
# 28672, bf16) needs, measured when that workload runs: its in-place fused
# add+RMSNorm (x and residual, 128 MiB each, written back), its RoPE's q and
# k (144 MiB in place) and its SiLU-mul operands (448 MiB).
WORKLOAD_CASES = {5: [
    ("inplace_2R2W_128MiB", 8192 * 8192 * 2, 2, 2, 0),
    ("inplace_144MiB", 8192 * 72 * 128 * 2, 1, 1, 0),
    ("2R1W_448MiB", 8192 * 28672 * 2, 2, 1, 0),
]}


# The plain stream of each prefill-step op's shape and store policy (the
# policy its kernel picks at that output size); RoPE rotates q (32 MiB) and k
# (8 MiB) in place, so its stream writes back over what it reads.
OP_CEILING = {2: {"rmsnorm": "1R1W_32MiB", "embedding": "1R1W_32MiB", "add": "2R1W_32MiB_dev",
                  "add_rmsnorm": "2R2W_32MiB", "rope": "inplace_40MiB_dev",
                  "rmsnorm_rope": "inplace_40MiB_dev", "silu_mul": "2R1W_112MiB_dev"},
              5: {"add_rmsnorm": "inplace_2R2W_128MiB", "rope": "inplace_144MiB",
                  "rmsnorm_rope": "inplace_144MiB", "silu_mul": "2R1W_448MiB"}}


# The same for the ops timed beyond the step (their kernels' store policies:
# non-temporal for softmax, LayerNorm and the multi-axis RoPE, device scope
# for GeGLU and the cached RoPE at these sizes).
NEXT_CEILING = {"softmax": "1R1W_125MiB", "layernorm": "1R1W_32MiB", "geglu_erf": "2R1W_112MiB_dev",
                "geglu_tanh": "2R1W_112MiB_dev", "rope_cached": "inplace_40MiB_dev",
                "rope_multi": "inplace_225MiB"}


def stream_ceiling(torch, stream, workload, launches=40):
    """Per-launch HIP-event times of plain HBM streams (libet_probe.so: 16-byte
    non-temporal loads, stores by the given policy, nothing computed between),
    each case over rotating buffer sets whose footprint is several times the
    256 MB Infinity Cache, so every launch streams from HBM.  Algorithmic
    bytes = (reads + writes) x operand bytes; the best of 4 and 8 vectors
    per lane is kept."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "elementwise_transformer_amd", "libet_probe.so"))
    f = lib.et_probe_stream
    vp = ctypes.c_void_p
    f.argtypes = [vp, vp, vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, vp]
    f.restype = ctypes.c_int
    out = {}
    for name, nb, nr, nw, dev in CEILING_CASES + WORKLOAD_CASES.get(workload, []):
        sets = max(4, -(-(1 << 30) // (4 * nb)))
        bufs = [[torch.randint(0, 256, (nb,), dtype=torch.uint8, device="cuda") for _ in range(4)]
                for _ in range(sets)]
        best = None
        for u in (4, 8):
            def fn(i, u=u):
                a, b, y, h = bufs[i % sets]
                if name.startswith("inplace"):
                    y, h = a, b
                rc = f(a.data_ptr(), b.data_ptr(), y.data_ptr(), h.data_ptr(), nb, nr, nw, u, dev,
                       stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"et_probe_stream failed ({rc}) on {name}")
            t = _time_launches(stream, fn, sets, launches)
            avg = float(np.mean(t))
            if best is None or avg < best[0]:
                best = (avg, float(np.median(t)), u)
        gbps = (nr + nw) * nb / (best[0] * 1e-3) / 1e9
        out[name] = {"bytes": (nr + nw) * nb, "avg_us": round(best[0] * 1e3, 2),
                     "median_us": round(best[1] * 1e3, 2), "vectors_per_lane": best[2],
                     "GBps": round(gbps, 1), "frac_peak": round(gbps / PEAK_GBPS, 4)}
        del bufs
    return out


def time_next_ops(et, torch, wl, stream, sets=3, launches=60):
    """Per-launch HIP-event times of the ops beyond the step, each on the
    inputs its workload names:
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

    def record(name, workload, nbytes, t, kernels):
        avg = float(np.mean(t))
        gbps = nbytes / (avg * 1e-3) / 1e9
        out[name] = {"workload": workload, "bytes": nbytes, "avg_us": round(avg * 1e3, 2),
                     "median_us": round(float(np.median(t)) * 1e3, 2), "samples": len(t),
                     "GBps": round(gbps, 1), "frac_peak": round(gbps / PEAK_GBPS, 4),
                     "kernels": kernels}

    lg, _ = wl.gen_argmax(wl.WORKLOADS[3])
    rows, n = lg.shape
    xs = [torch.from_numpy(lg).cuda() for _ in range(sets)]
    ys = [torch.empty_like(x) for x in xs]
    ws = torch.zeros(max(et.softmax_workspace_bytes(rows, n), 16), dtype=torch.uint8, device="cuda")
    t = _time_launches(stream, lambda i: et.softmax(xs[i % sets], 0.7, out=ys[i % sets], workspace=ws),
                       sets, launches)
    record("softmax", "decode logits [256,128256] f32, temperature 0.7", 2 * rows * n * 4, t,
           "softmax_chunks (one launch)")
    del xs, ys, ws

    g = np.random.default_rng([1002, 40])
    d = 4096
    xs = [torch.from_numpy(g.standard_normal((4096, d)).astype(np.float32)).to("cuda", torch.bfloat16)
          for _ in range(sets)]
    ys = [torch.empty_like(x) for x in xs]
    gam = torch.from_numpy(g.uniform(0.5, 1.5, d).astype(np.float32)).to("cuda", torch.bfloat16)
    bet = torch.from_numpy(g.standard_normal(d).astype(np.float32)).to("cuda", torch.bfloat16)
    t = _time_launches(stream, lambda i: et.layernorm(xs[i % sets], gam, bet, 1e-5, out=ys[i % sets]),
                       sets, launches)
    record("layernorm", "[4096,4096] bf16 with gain and bias, eps 1e-5", 2 * 4096 * d * 2 + 2 * d * 2, t,
           "layernorm_rows")
    del xs, ys

    g = np.random.default_rng([1002, 41])
    shape = (4096, 14336)
    gs = [torch.from_numpy(g.standard_normal(shape).astype(np.float32)).to("cuda", torch.bfloat16)
          for _ in range(sets)]
    us = [torch.from_numpy(g.standard_normal(shape).astype(np.float32)).to("cuda", torch.bfloat16)
          for _ in range(sets)]
    ys = [torch.empty_like(x) for x in gs]
    for form, name in ((et.GELU_ERF, "geglu_erf"), (et.GELU_TANH, "geglu_tanh")):
        t = _time_launches(stream, lambda i: et.geglu(gs[i % sets], us[i % sets], form, out=ys[i % sets]),
                           sets, launches)
        record(name, f"[4096,14336] bf16, {'erf' if form == 0 else 'tanh'} form", 3 * 4096 * 14336 * 2, t,
               "eltwise_vec")
    del gs, us, ys

    w = wl.WORKLOADS[2]
    s = w.rope
    q, k, pos, inv = wl.gen_rope(w)
    qs = [torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda() for _ in range(sets)]
    ks = [torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).cuda() for _ in range(sets)]
    pt = torch.from_numpy(pos).cuda()
    cc, sc = et.rope_cache(torch.from_numpy(inv).cuda(), s.T, s.r)
    t = _time_launches(stream, lambda i: et.rope_qk_cached(qs[i % sets], ks[i % sets], pt, cc, sc,
                                                           d_rot=s.r, attn_scaling=s.mu,
                                                           layout=s.layout), sets, launches)
    heads = s.Hq + s.Hk
    record("rope_cached", "prefill RoPE q [4096,32,128] k [4096,8,128] bf16, cache [4096,64] f32",
           2 * s.T * heads * s.r * 2 + 4 * s.T + 2 * s.T * (s.r // 2) * 4, t, "rope_qk_kernel (cached)")
    del qs, ks

    w = wl.WORKLOADS[6]
    m = w.rope_multi
    q, k, pos, inv = wl.gen_rope_multi(w)
    qs = [torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda() for _ in range(sets)]
    ks = [torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).cuda() for _ in range(sets)]
    pt = torch.from_numpy(pos).cuda()
    ft = torch.from_numpy(inv).cuda()
    t = _time_launches(stream, lambda i: et.rope_multi(qs[i % sets], ks[i % sets], pt, m.dims, ft,
                                                       attn_scaling=m.mu, layout=m.layout), sets, launches)
    span = sum(m.dims)
    record("rope_multi", "video DiT 3D RoPE q,k [19200,24,128] bf16, grid 16x30x40, widths 16/56/56",
           2 * m.T * (m.Hq + m.Hk) * span * 2 + 4 * 3 * m.T + 4 * (span // 2), t, "rope_multi_kernel")
    del qs, ks

    import dataclasses
    wf = dataclasses.replace(wl.WORKLOADS[2], dtype="f16")
    ops = build_ops(wf, et, torch)
    t = _time_launches(stream, lambda i: [op.fn() for op in ops], 1, 40)
    record("f16_step", "the prefill step of llama3-8b-prefill-T4096 with f16 storage",
           sum(op.nbytes for op in ops), t, "the step's eight kernels, f16 instances")
    return out


def cpu_baseline(w, min_seconds):
    """The CPU oracle as it stands, timed on whole steps of the same workload
    (every op at full size), repeated until at least min_seconds of work."""
    import oracle
    import workloads as wl
    orc = oracle.load()
    calls = []            # (bytes, closure)
    es = 4 if w.dtype == "f32" else 2
    if w.embed:
        V, d, n, _ = w.embed
        table, ids = wl.gen_embedding(w)
        calls.append((2 * n * d * es + 4 * n, lambda: orc.embedding(table, ids)))
    if w.add:
        rows, d = w.add
        a, b = wl.gen_add(w)
        calls.append((3 * rows * d * es, lambda: orc.add(a, b)))
    if w.rmsnorm:
        rows, d, eps = w.rmsnorm
        x, g, eps1 = wl.gen_rmsnorm(w)
        calls.append((2 * rows * d * es, lambda: orc.rmsnorm(x, g, eps1)))
    if w.add_rmsnorm:
        rows, d, eps, _ = w.add_rmsnorm
        xa, ra, ga, eps2 = wl.gen_add_rmsnorm(w)
        calls.append((4 * rows * d * es, lambda: orc.add_rmsnorm(xa, ra, ga, eps2)))
    if w.rope:
        s = w.rope
        q, k, pos, inv = wl.gen_rope(w)
        def rope_both():
            orc.rope(q, pos, s.r, inv, s.mu, s.layout)
            if k is not None:
                orc.rope(k, pos, s.r, inv, s.mu, s.layout)
        calls.append((2 * s.T * (s.Hq + s.Hk) * s.r * es, rope_both))
        q2, k2, gq, gk, pos2, inv2 = wl.gen_qknorm(w)
        def qk_both():
            orc.rmsnorm_rope(q2, gq, s.eps, pos2, s.r, inv2, s.mu, s.layout)
            if k2 is not None:
                orc.rmsnorm_rope(k2, gk, s.eps, pos2, s.r, inv2, s.mu, s.layout)
        calls.append((2 * s.T * (s.Hq + s.Hk) * s.D * es, qk_both))
    if w.silu:
        rows, cols, _ = w.silu
        gate, up = wl.gen_silu(w)
        calls.append((3 * rows * cols * es, lambda: orc.silu_mul(gate, up)))
    if w.argmax:
        rows, n = w.argmax
        lg, _ = wl.gen_argmax(w)
        calls.append((rows * n * lg.itemsize, lambda: orc.argmax(lg)))
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
            "sample": f"{reps} whole steps of the same workload ({step_bytes} algorithmic bytes "
                      f"each), all ops at full size"}


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


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the ops shard by rows with "
                          "no communication, so per-GPU throughput is the one-GPU figure",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import elementwise_transformer_amd as et
    import workloads as wl

    w = wl.WORKLOADS[args.workload]
    ops = build_ops(w, et, torch)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for op in ops:
            op.fn()
    torch.cuda.synchronize()

    # Timed region: K eager steps, launched back to back on one stream (the
    # host issues a step in far less time than the GPU runs it, so the queue
    # stays ahead).  Inside it, HIP events on the launch stream (torch's
    # current stream, which the binding passes to every entry point) bracket the
    # dominant op in every fourth step and, two steps later, one other op in
    # turn: every op gets live per-launch durations, while each event record
    # (a marker packet that costs the queue a few microseconds) touches only
    # a quarter of the steps.
    dom = max(range(len(ops)), key=lambda i: ops[i].nbytes)
    others = [i for i in range(len(ops)) if i != dom]
    plan = []
    for s in range(args.steps):
        pair = {}
        if s % 4 == 0:
            pair[dom] = TimingEvents(stream)
        elif s % 4 == 2 and others:
            j = others[(s // 4) % len(others)]
            pair[j] = TimingEvents(stream)
        plan.append(pair)
    torch.cuda.synchronize()
    gc.disable()                      # no collector pause inside the timed region
    t0 = time.perf_counter()
    for s in range(args.steps):
        pair = plan[s]
        for i, op in enumerate(ops):
            ev = pair.get(i)
            if ev:
                ev.start()
            op.fn()
            if ev:
                ev.stop()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    for s in range(args.steps):
        for i, ev in plan[s].items():
            ops[i].ms.append(ev.elapsed_ms())
            ev.close()

    # Ops beyond the step (the next rows built to the same bar), each timed on
    # its own workload after the timed region, as back-to-back launches over
    # rotating buffer sets with one pair of events per launch.
    next_ops = None if args.no_next_ops else time_next_ops(et, torch, wl, stream)
    ceiling = None if args.no_stream_ceiling else stream_ceiling(torch, stream, args.workload)

    # Attainable-bandwidth context: a plain device-to-device copy as large as
    # the dominant op's largest operand (read once, written once), timed the
    # same way after the timed region.
    copy_ctx = None
    if not args.copy_calibration:
        nb = max(op.nbytes for op in ops) // 3
        src = torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        ms = []
        for _ in range(10):
            ev = TimingEvents(stream)
            ev.start()
            dst.copy_(src)
            ev.stop()
            torch.cuda.synchronize()
            ms.append(ev.elapsed_ms())
            ev.close()
        med = float(np.median(ms))
        copy_ctx = {"bytes": 2 * nb, "median_us": round(med * 1e3, 2),
                    "GBps": round(2 * nb / (med * 1e-3) / 1e9, 1),
                    "what": "device-to-device copy of one operand-sized buffer (torch copy_)"}
        del src, dst

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    step_bytes = sum(op.nbytes for op in ops)
    ms_step = wall * 1e3 / args.steps
    per_op = {}
    for op in ops:
        avg = float(np.mean(op.ms))
        med = float(np.median(op.ms))
        # (argmax's per-launch time covers its two kernels)
        gbps = op.nbytes / (avg * 1e-3) / 1e9
        rec = {"bytes": op.nbytes, "avg_us": round(avg * 1e3, 2), "median_us": round(med * 1e3, 2),
               "samples": len(op.ms),
               "GBps": round(gbps, 1), "frac_peak": round(gbps / PEAK_GBPS, 4)}
        if op.rows:
            rec["rows_per_s"] = float(f"{op.rows / (avg * 1e-3):.4g}")
        case = OP_CEILING.get(args.workload, {}).get(op.name)
        if ceiling and case:
            rec["stream_ceiling"] = case
            rec["frac_of_ceiling"] = round(gbps / ceiling[case]["GBps"], 4)
        per_op[op.name] = rec
    dom = ops[dom]
    dom_avg_s = float(np.mean(dom.ms)) * 1e-3
    achieved = dom.nbytes / dom_avg_s / 1e9
    roofline = {"bound": "hbm", "kernel": dom.kernel, "op": dom.name, "achieved": round(achieved, 1),
                "peak": PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4),
                "traffic": traffic_record(args.workload, dom.name), "bytes_per_launch": dom.nbytes,
                "avg_launch_us": round(dom_avg_s * 1e6, 2),
                "note": "SiLU-mul and RoPE kernels whose output fits the 256 MB Infinity Cache use "
                        "device-scope stores; the cache writes part of their output back to HBM "
                        "after the kernel ends, so their per-kernel figures exclude that part, "
                        "while the whole-step value includes it"}
    case = OP_CEILING.get(args.workload, {}).get(dom.name)
    if ceiling and case:
        roofline["stream_ceiling"] = {"case": case, "GBps": ceiling[case]["GBps"],
                                      "frac_of_ceiling": round(achieved / ceiling[case]["GBps"], 4)}

    # The step as plain streams: each op's bytes at the measured rate of the
    # stream of its shape and store policy (an op with no such stream, the
    # latency-bound argmax, at its own time), against the measured step.
    step_ceiling = None
    cases = OP_CEILING.get(args.workload, {})
    if ceiling and cases:
        eq_s = sum(op.nbytes / (ceiling[cases[op.name]]["GBps"] * 1e9) if op.name in cases
                   else float(np.mean(op.ms)) * 1e-3 for op in ops)
        step_ceiling = {"stream_step_us": round(eq_s * 1e6, 2), "step_us": round(ms_step * 1e3, 2),
                        "frac": round(eq_s * 1e3 / ms_step, 4)}
    if ceiling and next_ops:
        for name, rec in next_ops.items():
            case = NEXT_CEILING.get(name)
            if case:
                rec["stream_ceiling"] = case
                rec["frac_of_ceiling"] = round(rec["GBps"] / ceiling[case]["GBps"], 4)
            elif name == "f16_step" and step_ceiling and args.workload == 2:
                # the f16 step moves the bf16 step's bytes in the same shapes
                rec["stream_step_us"] = step_ceiling["stream_step_us"]
                rec["frac_of_ceiling"] = round(step_ceiling["stream_step_us"] / rec["avg_us"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)
        if next_ops:
            cpu_next_ops(next_ops, 1.0)

    s = w.rope
    line = {
        "metric": "achieved HBM GB/s (% of MI355X peak) per op; rows/s for fused RMSNorm+RoPE",
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "frac_peak": round(step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_GBPS, 4),
        "config": {"workload": w.name, "storage": w.dtype, "step_bytes": step_bytes,
                   "ops": [op.name for op in ops],
                   "T": s.T if s else None, "heads_q": s.Hq if s else None,
                   "heads_kv": s.Hk if s else None, "head_dim": s.D if s else None,
                   "hidden": (w.add_rmsnorm or w.rmsnorm or (None, None))[1],
                   "intermediate": w.silu[1] if w.silu else None,
                   "vocab": w.embed[0] if w.embed else None},
        "ops": per_op,
        "roofline": roofline,
        "copy_context": copy_ctx,
        "stream_ceiling": ceiling,
        "step_vs_stream_ceiling": step_ceiling,
        "next_ops": next_ops,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
