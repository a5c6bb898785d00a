"""Host-side logic of bench.py, on small synthetic profiler outputs (no GPU):
the per-linear kernel-time summary of a kernel trace, the HBM bytes per
launch from two counter runs, and the cost-curve tables of a --shapes run.
Each fixture is written here, with the column names rocprofv3 uses, so that
the expected figures follow from the fixture by hand."""
import csv
import json
import os

import pytest

import bench


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def _dispatch(i, name, start, dur):
    return {"Dispatch_Id": str(i), "Kernel_Name": name, "Start_Timestamp": str(start),
            "End_Timestamp": str(start + dur)}


GEMV = "void w4::w4a16_gemv_kernel<4>(w4::LinearArgs)"
LDS = "void w4::w4a16_mfma_lds_kernel<4, 8>(w4::LinearArgs)"
RED = "void w4::splitk_reduce_kernel<2>(float const*, float*, unsigned short*, float, int, int, int, int)"
PASS0 = "void w4::(anonymous namespace)::w4_pass_kernel<0, 8, 4>(w4::PassLinear const*, w4::(anonymous namespace)::PassArgs)"
OTHER = "void at::native::vectorized_elementwise_kernel<4>(int)"


def test_trace_summary_adds_each_reduction_to_the_linear_before_it(tmp_path):
    # M = 1: two linears, the second with a reduction; M = 64: one linear with
    # a reduction; a foreign kernel in between belongs to no linear, and a
    # reduction after it is not counted; a persistent pass dispatch at M = 1
    # would be a whole pass (not mixed in here: its own run)
    rows = [_dispatch(1, GEMV, 1000, 10000), _dispatch(2, GEMV, 12000, 20000), _dispatch(3, RED, 33000, 4000),
            _dispatch(4, OTHER, 40000, 1000), _dispatch(5, RED, 42000, 9000),
            _dispatch(6, LDS, 50000, 40000), _dispatch(7, RED, 91000, 6000)]
    _write_csv(str(tmp_path / "t" / "run_kernel_trace.csv"), rows)
    s = bench.trace_summary(str(tmp_path / "t"))
    assert s["1"]["dispatches"] == 2 and s["64"]["dispatches"] == 1
    assert s["1"]["mean_us"] == pytest.approx((10 + 20 + 4) / 2)
    assert s["1"]["kernel_mean_us"] == pytest.approx(15.0)
    assert s["64"]["mean_us"] == pytest.approx(46.0) and s["64"]["kernel_mean_us"] == pytest.approx(40.0)
    assert s["1"]["kernels"] == ["w4::w4a16_gemv_kernel<4>"]
    assert "5" not in s


def test_trace_summary_names_the_persistent_pass_kernel(tmp_path):
    _write_csv(str(tmp_path / "p" / "run_kernel_trace.csv"), [_dispatch(1, PASS0, 0, 7000000)])
    s = bench.trace_summary(str(tmp_path / "p"))
    assert s["1"] == {"kernels": ["w4::w4_pass_kernel<0, 8, 4>"], "dispatches": 1, "mean_us": 7000.0,
                      "kernel_mean_us": 7000.0}


def _counter_rows(values):
    return [{"Dispatch_Id": str(i), "Kernel_Name": n, "Counter_Name": c, "Counter_Value": str(v)}
            for i, (n, c, v) in enumerate(values)]


def test_traffic_scales_by_the_copy_and_counts_reductions_with_their_linear(tmp_path):
    copy = "void w4::bench_copy_kernel(unsigned int __vector(4)*, unsigned int __vector(4) const*, unsigned long)"
    mib = 4
    # the copy of 4 MiB reads back as 2 MiB fetched (factor 2) and 4 MiB written (factor 1)
    fetch = _counter_rows([(copy, "FETCH_SIZE", mib * 1024 / 2), (GEMV, "FETCH_SIZE", 100.0),
                           (GEMV, "FETCH_SIZE", 300.0), (RED, "FETCH_SIZE", 50.0), (LDS, "FETCH_SIZE", 1000.0),
                           (RED, "FETCH_SIZE", 200.0)])
    write = _counter_rows([(copy, "WRITE_SIZE", mib * 1024), (GEMV, "WRITE_SIZE", 1.0), (GEMV, "WRITE_SIZE", 3.0),
                           (RED, "WRITE_SIZE", 2.0), (LDS, "WRITE_SIZE", 10.0), (RED, "WRITE_SIZE", 4.0)])
    _write_csv(str(tmp_path / "f" / "run_counter_collection.csv"), fetch)
    _write_csv(str(tmp_path / "w" / "run_counter_collection.csv"), write)
    out = bench.traffic_from_pmc(str(tmp_path / "f"), str(tmp_path / "w"), mib, str(tmp_path / "traffic.json"))
    assert out["FETCH_SIZE_factor"] == pytest.approx(2.0) and out["WRITE_SIZE_factor"] == pytest.approx(1.0)
    assert out["launch"] == {"1": "linear", "64": "linear"}
    p1, p64 = out["passes"]["1"], out["passes"]["64"]
    assert p1["launches_counted"] == 2 and p64["launches_counted"] == 1
    # KiB counts x factor x 1024 bytes, averaged over the linears
    assert p1["fetch_size_bytes_per_launch"] == int((100 + 300 + 50) * 2 * 1024 / 2)
    assert p1["write_size_bytes_per_launch"] == int((1 + 3 + 2) * 1024 / 2)
    assert p64["hbm_bytes_per_launch"] == int((1000 + 200) * 2 * 1024) + int((10 + 4) * 1024)
    assert json.load(open(tmp_path / "traffic.json")) == out
    assert out["source_digest"] == bench.source_digest()


def test_curve_tables_ratios_and_layer_sums(tmp_path):
    lines = []
    for name, t1 in (("q", 10.0), ("k", 5.0), ("v", 5.0), ("o", 10.0), ("gate", 20.0), ("up", 20.0), ("down", 20.0)):
        for M, f in ((1, 1.0), (5, 1.2)):
            us = t1 * f * (2.0 if name == "k" and M == 5 else 1.0)
            lines.append(json.dumps({"linear": name, "M": M, "us": us, "us_min": us * 0.99, "us_max": us * 1.01,
                                     "tbps": 1.0, "roofline_frac": 0.5}))
    p = tmp_path / "shapes.jsonl"
    p.write_text("\n".join(["[bench] progress line"] + lines) + "\n")
    text = bench.curve_tables(str(p))
    rows = {ln.split("|")[1].strip(): ln for ln in text.splitlines() if ln.startswith("| ")}
    assert "| q | 10.0 | 12.0 |" in text
    # t(5)/t(1): q 1.2, k 2.4; one layer (7 launches): (90 * 1.2 + 6) / 90
    assert "| k | 1.00 | 2.40 |" in text
    assert rows["one layer, 7 launches"].split("|")[3].strip() == "%.2f" % ((90 * 1.2 + 6) / 90)
    assert "one layer, fused (4 launches)" not in text  # no fused shapes in this run
    assert "| q | 0.020 | 0.020 |" in text  # spread (max - min) / median


def test_more_than_one_gpu_is_refused_with_a_message():
    # the bench measures one GPU's throughput; --gpus N > 1 exits before any
    # device work, saying so
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, cwd=root)
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU" in r.stderr and r.stdout == ""
