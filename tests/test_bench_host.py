"""Host logic of bench.py that needs no GPU: the one-GPU refusal, the
rocprofv3 counter parsing behind `roofline.traffic`, the copy-calibrated
scaling of a traffic record and its invalidation when the kernels change."""
import csv
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_counters(path, rows):
    """rows: (dispatch, kernel, counter, value); one row per XCD instance is
    how rocprofv3 reports a counter, so a dispatch may appear several times."""
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (d, k, c, v) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c,
                        "Counter_Value": v})


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_counter_means_sums_instances_and_averages_dispatches(tmp_path):
    p = tmp_path / "c.csv"
    write_counters(p, [
        (1, "void st::conv_rows<...>", "FETCH_SIZE", 10.0),
        (1, "void st::conv_rows<...>", "FETCH_SIZE", 5.0),       # second instance of dispatch 1
        (2, "torch fill", "FETCH_SIZE", 999.0),                  # not a matching kernel
        (3, "void st::conv_rows<...>", "FETCH_SIZE", 25.0),
    ])
    mean, n = bench._counter_means(str(p), ("conv_rows",))["FETCH_SIZE"]
    assert n == 2 and mean == pytest.approx(20.0)
    mx, n = bench._counter_means(str(p), ("conv_rows",), pick_max=True)["FETCH_SIZE"]
    assert n == 2 and mx == pytest.approx(25.0)
    with pytest.raises(SystemExit):
        bench._counter_means(str(p), ("no_such_kernel",))


@pytest.mark.parametrize("stage,kernel", [("conv", "conv_rows"), ("strided", "conv_sx_mfma<16, 4, 2, false>"),
                                          ("transposed", "conv_sx_mfma<16, 4, 2, true>")])
def test_traffic_record_scaling_and_staleness(tmp_path, monkeypatch, stage, kernel):
    kib = 1024.0
    copy_kib = bench.COPY_BYTES / kib
    # the copy's read counter reads half its bytes, its write counter all of them
    write_counters(tmp_path / "cf.csv", [(1, "elementwise_kernel fill", "FETCH_SIZE", 1.0),
                                         (2, "vectorized_elementwise_kernel mul", "FETCH_SIZE", copy_kib / 2)])
    write_counters(tmp_path / "cw.csv", [(1, "elementwise_kernel fill", "WRITE_SIZE", copy_kib),
                                         (2, "vectorized_elementwise_kernel mul", "WRITE_SIZE", copy_kib)])
    write_counters(tmp_path / "f.csv", [(5, kernel, "FETCH_SIZE", 300.0), (6, kernel, "FETCH_SIZE", 100.0)])
    write_counters(tmp_path / "w.csv", [(5, kernel, "WRITE_SIZE", 50.0), (6, kernel, "WRITE_SIZE", 50.0)])
    out = tmp_path / "rec.json"
    args = types.SimpleNamespace(record_traffic=[str(tmp_path / n) for n in ("f.csv", "w.csv", "cf.csv", "cw.csv")],
                                 workload=None, record_stage=stage, record_out=str(out))
    bench.record_traffic(args)
    rec = json.loads(out.read_text())
    assert rec["stage"] == stage
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["traffic_bytes"] == pytest.approx((200.0 * 2.0 + 50.0) * kib)

    import synth
    wl = synth.workload(synth.BENCH_WORKLOAD)
    monkeypatch.setattr(bench, "traffic_path", lambda w, s: str(out))
    assert bench.load_traffic(wl, stage) == pytest.approx(rec["traffic_bytes"])
    # a record of another stage, or of kernels whose sources changed since, is not reported
    other = "pool" if stage != "pool" else "conv"
    assert bench.load_traffic(wl, other) is None
    rec["source_digest"] = "0" * 64
    out.write_text(json.dumps(rec))
    assert bench.load_traffic(wl, stage) is None


def test_traffic_paths_are_distinct_per_stage():
    import synth
    wl = synth.workload(synth.BENCH_WORKLOAD)
    paths = {bench.traffic_path(wl, s) for s in ("conv", "strided", "transposed", "pool")}
    assert len(paths) == 4
    assert bench.traffic_path(wl, "conv").endswith(f"traffic_{wl.name}.json")
