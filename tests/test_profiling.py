"""The measurement helper (moe_decode_02_amd/profiling.py) on synthetic
rocprofv3 CSV files: copy-calibrated HBM bytes, the source-hash gate that
keeps a stale traffic figure out of bench.py, kernel-trace statistics, and
per-counter means."""
import csv
import os

import pytest

from moe_decode_02_amd import profiling

DECODE = "void (anonymous namespace)::moe_kernel<1, 0, 1, 1, true, false>(Params)"
COPY = "(anonymous namespace)::copy_kernel(HIP_vector_type<unsigned int, 4u> const*, ...)"


def write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_is_calibrated_by_the_copy_kernel(tmp_path):
    # the copy reads and writes 1 GiB; FETCH_SIZE reports half of it, WRITE_SIZE all of it
    kib = profiling.COPY_BYTES / 1024
    write_counters(tmp_path / "f", [(COPY, "FETCH_SIZE", kib / 2), (DECODE, "FETCH_SIZE", 400000.0),
                                    (DECODE, "FETCH_SIZE", 400002.0), ("other", "FETCH_SIZE", 9.0)])
    write_counters(tmp_path / "w", [(COPY, "WRITE_SIZE", kib), (DECODE, "WRITE_SIZE", 683.0),
                                    (DECODE, "WRITE_SIZE", 683.0)])
    out = tmp_path / "traffic.txt"
    profiling.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(out), "cmd")
    tr = profiling.read_traffic(str(out))
    assert tr["read"] == pytest.approx(400001.0 * 1024 * 2, rel=1e-9)
    assert tr["write"] == pytest.approx(683.0 * 1024, rel=1e-9)


def test_traffic_of_another_kernel_source_is_not_reported(tmp_path):
    out = tmp_path / "traffic.txt"
    out.write_text("kernel_source_sha256 = 00\nhbm_read_bytes_per_launch = 1\nhbm_write_bytes_per_launch = 2\n")
    assert profiling.read_traffic(str(out)) is None
    assert profiling.read_traffic(str(tmp_path / "missing.txt")) is None
    out.write_text(f"kernel_source_sha256 = {profiling.kernel_source_sha()}\n"
                   "hbm_read_bytes_per_launch = 1\nhbm_write_bytes_per_launch = 2\n")
    assert profiling.read_traffic(str(out)) == {"read": 1.0, "write": 2.0}


def test_kernel_trace_statistics(tmp_path):
    d = tmp_path / "t"
    os.makedirs(d)
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for i, us in enumerate([130.0, 136.0, 142.0]):
            w.writerow({"Kernel_Name": DECODE, "Start_Timestamp": 10**9 * i, "End_Timestamp": 10**9 * i + int(us * 1000)})
    durs = profiling.kernel_durations(str(d))
    assert durs[DECODE] == [130.0, 136.0, 142.0]
    out = tmp_path / "stats.txt"
    profiling.write_stats(str(d), str(out), "cmd")
    line = [ln for ln in out.read_text().splitlines() if ln.startswith("void")][0].split()
    assert line[-5:] == ["3", "136.00", "136.00", "130.00", "142.00"]


def test_counter_means_of_the_decode_kernel(tmp_path):
    write_counters(tmp_path / "c", [(DECODE, "TCC_HIT_sum", 10.0), (DECODE, "TCC_HIT_sum", 30.0),
                                    (DECODE, "TCC_MISS_sum", 5.0), (COPY, "TCC_HIT_sum", 1e9)])
    out = tmp_path / "counters.txt"
    profiling.write_counters(str(tmp_path / "c"), str(out), "cmd")
    text = out.read_text()
    assert "TCC_HIT_sum = 20   (dispatches 2)" in text
    assert "TCC_MISS_sum = 5   (dispatches 1)" in text


def test_unfused_traffic_per_layer(tmp_path):
    """The multi-launch path's summary sums every uf_ kernel's calibrated bytes
    and divides by the layers (dispatches of its combine kernel)."""
    kib = profiling.COPY_BYTES / 1024
    gemv = "void (anonymous namespace)::uf_gemv<1, 1, 1>((anonymous namespace)::UfGemv)"
    comb = "void (anonymous namespace)::uf_combine<1>(void const*, float const*, ...)"
    pref = "(anonymous namespace)::uf_prefetch((anonymous namespace)::UfPrefetch)"
    write_counters(tmp_path / "f", [(COPY, "FETCH_SIZE", kib / 2), (gemv, "FETCH_SIZE", 100.0),
                                    (gemv, "FETCH_SIZE", 300.0), (comb, "FETCH_SIZE", 10.0),
                                    (comb, "FETCH_SIZE", 10.0), (pref, "FETCH_SIZE", 50.0),
                                    (DECODE, "FETCH_SIZE", 1e9)])
    write_counters(tmp_path / "w", [(COPY, "WRITE_SIZE", kib), (gemv, "WRITE_SIZE", 4.0),
                                    (gemv, "WRITE_SIZE", 4.0), (comb, "WRITE_SIZE", 2.0), (comb, "WRITE_SIZE", 2.0)])
    out = tmp_path / "u.txt"
    profiling.write_unfused_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(out), "cmd")
    kv = dict(ln.split(" = ") for ln in out.read_text().splitlines() if " = " in ln and not ln.startswith("#"))
    assert int(kv["layers"]) == 2
    # reads: (100 + 300 + 10 + 10 + 50) KiB x 2 (FETCH_SIZE counts half) over 2 layers; the decode kernel is not counted
    assert float(kv["hbm_read_bytes_per_layer"]) == pytest.approx(470 * 1024 * 2 / 2, rel=1e-6)
    assert float(kv["hbm_write_bytes_per_layer"]) == pytest.approx(12 * 1024 / 2, rel=1e-6)
