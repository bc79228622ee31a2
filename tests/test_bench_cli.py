"""bench.py's command line without a GPU: more than one GPU is refused with a
message and exit status 2, before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _counter_csv(d, rows):
    """A rocprofv3 counter_collection.csv with (kernel, counter, value) rows."""
    import csv
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, c, v) in enumerate(rows):
            w.writerow([i + 1, k, c, v])


def test_summarize_counters_scales_by_the_calibration_copy(tmp_path):
    """FETCH_SIZE / WRITE_SIZE are scaled so that the 1 GiB calibration copy reads
    1 GiB (median of its dispatches), then averaged over the GEMM's dispatches."""
    sys.path.insert(0, ROOT)
    import bench
    gemm = "void nel::(anonymous namespace)::heads_loss_kernel<3>(nel::ExitSet, int)"
    copy = "void at::native::vectorized_elementwise_kernel<4, AUnaryFunctor<float> >"
    gib_kib = float(1 << 20)
    # fetch reads half the bytes (scale 2), write reads them exactly (scale 1)
    _counter_csv(str(tmp_path / "pf"), [(copy, "FETCH_SIZE", gib_kib / 2)] * 3 +
                 [(gemm, "FETCH_SIZE", 1000.0), (gemm, "FETCH_SIZE", 3000.0)])
    _counter_csv(str(tmp_path / "pw"), [(copy, "WRITE_SIZE", gib_kib), (copy, "WRITE_SIZE", gib_kib),
                                        (copy, "WRITE_SIZE", 5 * gib_kib),
                                        (gemm, "WRITE_SIZE", 500.0)])
    out = str(tmp_path / "traffic.json")
    res = bench.summarize_counters(str(tmp_path / "pf"), str(tmp_path / "pw"), out=out)
    assert res["fetch_scale"] == 2.0 and res["write_scale"] == 1.0
    assert res["heads_loss_fetch_bytes"] == 2000.0 * 1024 * 2.0
    assert res["heads_loss_write_bytes"] == 500.0 * 1024
    assert res["heads_loss_bytes_per_launch"] == 2000.0 * 2048 + 500.0 * 1024
    assert res["source_hash"] == bench.kernel_source_hash()
    # the record is used only while the GEMM sources are unchanged
    assert bench.measured_traffic(out) == res["heads_loss_bytes_per_launch"]
    import json
    with open(out) as f:
        d = json.load(f)
    d["source_hash"] = "0" * 16
    with open(out, "w") as f:
        json.dump(d, f)
    assert bench.measured_traffic(out) is None
    assert bench.measured_traffic(str(tmp_path / "missing.json")) is None
