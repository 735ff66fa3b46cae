"""Host logic of the benchmark's counter-traffic summary (no GPU): two
rocprofv3 --pmc counter files (FETCH_SIZE, WRITE_SIZE in KiB per dispatch) are
scaled by the readings of a 1 GiB copy, and the summary is honoured only while
the kernel's sources are unchanged."""

import argparse
import csv
import os

import bench


def _csv(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "p_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, val) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": val})


def test_traffic_summary_roundtrip(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    k = "void hm::(anonymous namespace)::decode_step_fixed<16, 1, 2, 1, true>(hm::DecodeArgs)"
    copy = "void at::native::elementwise_kernel<direct_copy_kernel_cuda>"
    # FETCH_SIZE reads half of the copy's bytes, WRITE_SIZE all of them
    _csv(tmp_path / "f", "FETCH_SIZE", [(copy, 12.0), (k, 2100.0), (k, 2200.0), (copy, 524288.0)])
    _csv(tmp_path / "w", "WRITE_SIZE", [(copy, 4.0), (k, 4300.0), (k, 4300.0), (copy, 1048576.0)])
    args = argparse.Namespace(config=2, traffic_kernel="decode_step_fixed",
                              traffic_from=(str(tmp_path / "f"), str(tmp_path / "w")), traffic_cmd="a ;; b")
    bench.write_traffic(args)
    got = bench.read_traffic("decode_step_fixed", "width2048-bf16")
    assert got == round((2150.0 * 2 + 4300.0) * 1024)
    # a changed kernel source voids the measurement
    monkeypatch.setattr(bench, "kernel_fingerprint", lambda kernel: "0" * 16)
    assert bench.read_traffic("decode_step_fixed", "width2048-bf16") is None
    assert bench.read_traffic("chunk_mfma_kernel", "width2048-bf16") is None
