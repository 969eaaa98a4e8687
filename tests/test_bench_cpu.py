"""Host logic of bench.py on the CPU: the one-GPU guard, the calibrated
traffic record (per-dispatch counter CSVs -> bytes per call), the traffic
lookup that bench.py reports, and the result-traffic cut."""
import argparse
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("extra", [[], ["--workload", "mlp_down"]])
def test_more_than_one_gpu_exits_with_a_message(extra):
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"] + extra, cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _counters(path, dispatches):
    """rocprofv3 counter-collection rows: one per (dispatch, counter instance)."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for disp, (name, instances) in enumerate(dispatches, start=1):
            for v in instances:
                w.writerow(dict(Dispatch_Id=disp, Kernel_Name=name, Counter_Name="C",
                                Counter_Value=v))
    return str(path)


COPY = "__amd_rocclr_copyBuffer"


def _record(tmp_path, monkeypatch, workload, fetch, write, B=None, mib=1):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    args = argparse.Namespace(
        workload=workload, B=B, surface="tokens", op="sum", copy_calibration_mib=mib,
        record_traffic=[_counters(tmp_path / "f.csv", fetch), _counters(tmp_path / "w.csv", write)])
    bench.record_traffic(args)
    with open(tmp_path / "traffic.json") as f:
        return json.load(f)


def test_traffic_is_scaled_by_the_calibration_copy(tmp_path, monkeypatch):
    # A 1 MiB copy that FETCH_SIZE reads as 512 KiB (factor 2) and WRITE_SIZE
    # as 1024 KiB (factor 1); a small input upload that is also a copy; two
    # calls of a head dispatch (instances summing to 100 and 102 KiB) and its
    # combine dispatch (2 KiB).
    head = "void sbk::head_gemm_kernel<1, 0, 2, false>(sbk::HeadArgs)"
    comb = "sbk::combine_kernel(HIP_vector_type<int, 2u> const*, ...)"
    fetch = [(COPY, [3.0]), (COPY, [256.0, 256.0]), (head, [60.0, 40.0]), (comb, [1.0, 1.0]),
             (head, [50.0, 52.0]), (comb, [2.0])]
    write = [(COPY, [1.0]), (COPY, [512.0, 512.0]), (head, [4.0, 1.0]), (comb, [0.5]),
             (head, [3.0, 2.0]), (comb, [0.5])]
    rec = _record(tmp_path, monkeypatch, "dense_decode", fetch, write)
    assert rec["kernel_source_sha256"] == bench.kernel_source_hash()
    e = rec["workloads"]["dense_decode/tokens/B16"]
    assert e["fetch_factor"] == 2.0 and e["write_factor"] == 1.0
    assert "head_gemm" in e["kernel"] and "combine_kernel" in e["kernel"]
    assert e["fetch_bytes"] == 103 * 1024 * 2
    assert e["write_bytes"] == int(5.5 * 1024)
    assert e["dispatches"] == 2
    assert bench.recorded_traffic("dense_decode", "tokens", 16) == 103 * 2048 + int(5.5 * 1024)
    assert bench.recorded_traffic("dense_decode", "tokens", 8) is None


def test_traffic_of_33_to_64_rows_adds_the_hidden_row_pack(tmp_path, monkeypatch):
    pack = "void sbk::pack_hidden_kernel<4>(unsigned short const*, long, int, int, unsigned short*)"
    head = "void sbk::head_gemm_kernel<4, 0, 2, true>(sbk::HeadArgs)"
    comb = "sbk::combine_kernel(HIP_vector_type<int, 2u> const*, ...)"
    fetch = [(COPY, [512.0]), (pack, [1.0]), (head, [200.0]), (comb, [1.0]),
             (pack, [1.0]), (head, [200.0]), (comb, [1.0])]
    write = [(COPY, [1024.0]), (pack, [0.5]), (head, [2.0]), (comb, [0.25]),
             (pack, [0.5]), (head, [2.0]), (comb, [0.25])]
    rec = _record(tmp_path, monkeypatch, "moe_decode", fetch, write)
    e = rec["workloads"]["moe_decode/tokens/B64"]
    assert "pack_hidden" in e["kernel"] and "head_gemm" in e["kernel"]
    assert e["fetch_bytes"] == 202 * 1024 * 2
    assert e["write_bytes"] == int(2.75 * 1024)


def test_traffic_without_the_head_kernel_is_refused(tmp_path, monkeypatch):
    fetch = [(COPY, [512.0]), ("some_other_kernel", [1.0])]
    with pytest.raises(SystemExit):
        _record(tmp_path, monkeypatch, "dense_decode", fetch, fetch)


def test_recorded_traffic_is_dropped_after_a_kernel_source_change(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps({"kernel_source_sha256": "0" * 64, "workloads": {
        "dense_decode/tokens/B16": {"fetch_bytes": 1, "write_bytes": 2}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.recorded_traffic("dense_decode", "tokens", 16) is None


def test_result_traffic_cut():
    # int32 IDs against V fp32 logits per row
    assert bench.result_cut_percent(4 * 16, 4 * 16 * 151936) == pytest.approx(
        100.0 * (1.0 - 1.0 / 151936), rel=1e-12)
    assert bench.result_cut_percent(1, 1) == 0.0
