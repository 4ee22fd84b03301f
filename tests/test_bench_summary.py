"""The benchmark's profile summary on the CPU (bench.py --summarize and the
traffic lookup the roofline record uses), on synthetic rocprofv3 output:
library kernels are matched to the logged calls in launch order, torch's own
kernels are skipped, each (label, kernel, launch shape) gets its own row, a
row faster than the HBM peak is marked invalid, a log that does not belong to
the run is refused, and counter rows are scaled by the calibration copy."""
import contextlib
import csv
import io
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id",
              "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size",
              "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X",
              "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]

SILU = "void et::(anonymous namespace)::eltwise_vec<et::Bf16, 1, 2>(et::Bf16 const*, long)"
ARG = "void et::(anonymous namespace)::argmax_rows<float, 256, true>(float const*, long, int*)"
TORCH = "void at::native::(anonymous namespace)::offset::elementwise_kernel<128, 4>(int)"
PROBE = "void etprobe::(anonymous namespace)::stream_kernel<1, 1, 4, 2, false>(void const*, long)"


def _trace(path, kernels):
    """kernels: (name, duration ns, grid) in dispatch order."""
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, TRACE_COLS)
        w.writeheader()
        t = 1000
        for i, (name, dur, grid) in enumerate(kernels, 1):
            row = {c: 0 for c in TRACE_COLS}
            row.update({"Kind": "KERNEL_DISPATCH", "Dispatch_Id": i, "Kernel_Name": name,
                        "Start_Timestamp": t, "End_Timestamp": t + dur, "Workgroup_Size_X": 256,
                        "Workgroup_Size_Y": 1, "Workgroup_Size_Z": 1, "Grid_Size_X": grid,
                        "Grid_Size_Y": 1, "Grid_Size_Z": 1, "VGPR_Count": 32})
            w.writerow(row)
            t += dur + 500


def _log(path, runs, info):
    with open(path, "w") as fh:
        json.dump({"runs": runs, "info": info}, fh)


def _summary(*args, **kw):
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        bench.summarize(*args, **kw)
    return out.getvalue()


def test_trace_rows_by_label_and_shape(tmp_path):
    d = tmp_path / "trace"
    d.mkdir()
    # torch kernels in between are skipped; the silu label is one row; the
    # argmax label runs at two shapes under two labels
    _trace(d / "run_kernel_trace.csv",
           [(TORCH, 5000, 64), (SILU, 200_000, 1024), (SILU, 220_000, 1024), (TORCH, 7000, 64),
            (ARG, 20_000, 262144), (ARG, 5_000, 256), (ARG, 5_000, 256), (PROBE, 1000, 512)])
    info = {"w5/silu_mul": {"bytes": 1_409_286_144, "sources_sha256": "ab" * 32},
            "w3/argmax": {"bytes": 131_334_144},
            "w2/argmax": {"bytes": 513_024}}
    _log(d / "dispatch.json", [["w5/silu_mul", 2], ["w3/argmax", 1], ["w2/argmax", 2], ["probe/x/u4", 1]],
         info)
    text = _summary(str(d), str(d / "dispatch.json"), "t", "cmd")
    rows = [ln for ln in text.splitlines() if ln.startswith("| w") or ln.startswith("| probe")]
    assert len(rows) == 4
    silu = next(r for r in rows if r.startswith("| w5/silu_mul"))
    cells = [c.strip() for c in silu.strip("|").split("|")]
    assert cells[5] == "2" and cells[6] == "210.00"                 # calls, average us
    assert abs(float(cells[11]) - 1_409_286_144 / 210e-6 / 1e9) < 0.1  # GB/s
    assert cells[13] == "abababababababab"
    assert "INVALID" not in silu
    w3 = next(r for r in rows if r.startswith("| w3/argmax"))
    assert "262144x1x1" in w3 and "INVALID" not in w3
    # 131 MB in 20 us would be 6.6 TB/s: valid; the same bytes in 5 us would not be
    assert "cmd" in text


def test_trace_row_above_peak_is_marked(tmp_path):
    d = tmp_path / "t"
    d.mkdir()
    _trace(d / "k_kernel_trace.csv", [(ARG, 5_000, 262144)])
    _log(d / "l.json", [["w3/argmax", 1]], {"w3/argmax": {"bytes": 131_334_144}})
    text = _summary(str(d), str(d / "l.json"), "t", "")
    assert "INVALID: above peak" in text


def test_trace_refuses_a_foreign_log(tmp_path):
    d = tmp_path / "t"
    d.mkdir()
    _trace(d / "k_kernel_trace.csv", [(SILU, 1000, 64), (SILU, 1000, 64)])
    _log(d / "l.json", [["w5/silu_mul", 3]], {})
    with pytest.raises(SystemExit):
        _summary(str(d), str(d / "l.json"), "t", "")


def test_trace_refuses_one_label_at_two_shapes(tmp_path):
    d = tmp_path / "t"
    d.mkdir()
    _trace(d / "k_kernel_trace.csv", [(ARG, 1000, 256), (ARG, 1000, 512)])
    _log(d / "l.json", [["w3/argmax", 2]], {})
    with pytest.raises(SystemExit):
        _summary(str(d), str(d / "l.json"), "t", "")


def test_label_prefix_filter(tmp_path):
    d = tmp_path / "t"
    d.mkdir()
    _trace(d / "k_kernel_trace.csv", [(SILU, 1000, 64), (ARG, 1000, 256)])
    _log(d / "l.json", [["w5/silu_mul", 1], ["w3/argmax", 1]], {})
    text = _summary(str(d), str(d / "l.json"), "t", "", prefixes=("w3/",))
    assert "| w3/argmax" in text and "| w5/silu_mul" not in text


def _counters(path, rows):
    """rows: (dispatch id, kernel, counter, value in KiB)."""
    cols = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
            "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size",
            "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value",
            "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, cols)
        w.writeheader()
        for did, name, cname, val in rows:
            r = {c: 0 for c in cols}
            r.update({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": cname, "Counter_Value": val})
            w.writerow(r)


def test_counters_scaled_and_traffic_lookup(tmp_path, monkeypatch):
    # a fake tree: the op's sources, whose hash the counter rows must carry
    root = tmp_path / "root"
    src = root / "elementwise_transformer_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "eltwise.hip").write_text("kernel v1\n")
    (src / "et_common.hpp").write_text("common\n")
    (root / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(root))
    sha = bench.op_sources_sha256("silu_mul")
    info = {"w5/silu_mul": {"bytes": 3000, "bytes_read": 2000, "bytes_written": 1000, "sources_sha256": sha},
            "calibration/copy_256MiB": {"bytes_read": 1 << 28, "bytes_written": 1 << 28}}
    runs = [["w5/silu_mul", 2], ["calibration/copy_256MiB", 1]]
    for cname, cal_kib, silu_kib in (("FETCH_SIZE", (1 << 27) / 1024, 1000 / 1024),
                                     ("WRITE_SIZE", (1 << 28) / 1024, 1000 / 1024)):
        d = tmp_path / cname
        d.mkdir()
        _counters(d / "pmc_counter_collection.csv",
                  [(3, SILU, cname, silu_kib), (5, TORCH, cname, 99.0), (7, SILU, cname, silu_kib),
                   (9, PROBE, cname, cal_kib)])
        _log(d / "l.json", runs, info)
        text = _summary(str(d), str(d / "l.json"), "c", "")
        factor = 2.0 if cname == "FETCH_SIZE" else 1.0
        assert f"factor {factor:.4f}" in text
        line = next(ln for ln in text.splitlines() if ln.startswith("| w5/silu_mul"))
        cells = [c.strip() for c in line.strip("|").split("|")]
        assert cells[1] == "2" and float(cells[2]) == 1000.0
        assert abs(float(cells[3]) - 1000.0 * factor) < 1.0
        assert cells[4] == ("2000" if cname == "FETCH_SIZE" else "1000") and cells[5] == sha
        (root / "profiles" / f"{cname}_hbm_counters.md").write_text(text)
    assert bench.traffic_record("w5/silu_mul") == 3000
    # once the kernel's source changes, the committed counters no longer apply
    (src / "eltwise.hip").write_text("kernel v2\n")
    assert bench.traffic_record("w5/silu_mul") is None


def test_more_than_one_gpu_is_refused():
    """bench.py --gpus N > 1 exits with a message (one GPU only) before
    touching a device."""
    import json
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
