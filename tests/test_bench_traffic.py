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


def test_stack_token_traffic_sums_every_layer(tmp_path, monkeypatch):
    """The stack's generated token is one launch of 24 gates and 24 out_projs:
    its traffic is 24 x (mean gate + mean out_proj) per counter, scaled by the
    copy, and other kernels in the run (the start-of-generation prepare) do not
    count."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    gate = "void hm::(anonymous namespace)::gemm_stream_lds_kernel<3, 1, true, 32, -1, 16>(hm::GemmArgs)"
    outp = "void hm::(anonymous namespace)::gemm_stream_dl_kernel<6>(hm::GemmArgs)"
    prep = "void hm::(anonymous namespace)::prepare_kernel<16>(hm::PrepArgs)"
    copy = "void at::native::elementwise_kernel<direct_copy_kernel_cuda>"
    _csv(tmp_path / "f", "FETCH_SIZE", [(copy, 524288.0), (prep, 9999.0), (gate, 100.0), (outp, 10.0), (gate, 300.0),
                                        (outp, 30.0)])
    _csv(tmp_path / "w", "WRITE_SIZE", [(copy, 1048576.0), (prep, 9999.0), (gate, 50.0), (outp, 5.0)])
    args = argparse.Namespace(config=5, traffic_kernel="stack_token",
                              traffic_from=(str(tmp_path / "f"), str(tmp_path / "w")), traffic_cmd="a ;; b")
    bench.write_traffic(args)
    got = bench.read_traffic("stack_token", "stack24-bf16")
    assert got == round(24 * ((200.0 + 20.0) * 2 + (50.0 + 5.0)) * 1024)
    text = (tmp_path / "profiles" / "stack_token.stack24-bf16.traffic.txt").read_text()
    assert "algorithmic_bytes_per_launch: 1635778560" in text


def test_stack_prompt_gemm_traffic_is_per_layer(tmp_path, monkeypatch):
    """A layer's prompt GEMMs are two gemm_dl8_kernel dispatches (in_proj and
    out_proj): the summary is 2 x the mean dispatch per counter, scaled by the
    copy, against the two GEMMs' algorithmic bytes; the row pass and the
    operator's kernels in the same run do not count."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    dl8 = "void hm::(anonymous namespace)::gemm_dl8_kernel<64>(hm::GemmArgs)"
    rms = "hm::(anonymous namespace)::row_rms_kernel(hm::RmsArgs)"
    op = "void hm::(anonymous namespace)::chunk_mfma_kernel<16, 128, 1, false, false>(hm::OpArgs)"
    copy = "void at::native::elementwise_kernel<direct_copy_kernel_cuda>"
    _csv(tmp_path / "f", "FETCH_SIZE", [(copy, 524288.0), (rms, 777.0), (dl8, 3000.0), (op, 555.0), (dl8, 1000.0)])
    _csv(tmp_path / "w", "WRITE_SIZE", [(copy, 1048576.0), (rms, 1.0), (dl8, 600.0), (op, 5.0), (dl8, 200.0)])
    args = argparse.Namespace(config=5, traffic_kernel="stack_prompt_gemm",
                              traffic_from=(str(tmp_path / "f"), str(tmp_path / "w")), traffic_cmd="a ;; b")
    bench.write_traffic(args)
    got = bench.read_traffic("stack_prompt_gemm", "stack24-bf16")
    assert got == round(2 * (2000.0 * 2 + 400.0) * 1024)
    M, D = 64 * 2048, 2048
    alg = 2 * (M * D + 3 * D * D + 3 * M * D) + 2 * (M * D + D * D + M * D)
    assert bench.stack_prompt_gemm_bytes(__import__("workloads").get_config(5)) == alg == 3254779904
    text = (tmp_path / "profiles" / "stack_prompt_gemm.stack24-bf16.traffic.txt").read_text()
    assert f"algorithmic_bytes_per_launch: {alg}" in text


def test_trace_summary_from_kernel_stats(tmp_path):
    """rocprofv3 --stats rows of two processes are merged per kernel, sorted by
    total time, with calls, mean/min/max per dispatch and the command."""
    d = tmp_path / "trace" / "host"
    d.mkdir(parents=True)
    fields = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"]
    for pid, rows in (("1", [("kA", 4, 4000, 500, 1500), ("kB", 1, 9000, 9000, 9000)]),
                      ("2", [("kA", 2, 2000, 800, 1200)])):
        with open(d / f"{pid}_kernel_stats.csv", "w", newline="") as fh:
            w = csv.DictWriter(fh, fieldnames=fields)
            w.writeheader()
            for name, calls, tot, lo, hi in rows:
                w.writerow({"Name": name, "Calls": calls, "TotalDurationNs": tot, "AverageNs": tot / calls,
                            "Percentage": 0, "MinNs": lo, "MaxNs": hi, "StdDev": 0})
    out = tmp_path / "sum.txt"
    args = argparse.Namespace(summarize_trace=(str(tmp_path / "trace"), str(out)), summary_title="t",
                              traffic_cmd="rocprofv3 ... -- python3 bench.py")
    bench.write_trace_summary(args)
    lines = [l for l in out.read_text().splitlines() if l.startswith(("kA", "kB"))]
    assert lines[0].split()[:2] == ["kB", "1"] and lines[1].split()[:2] == ["kA", "6"]
    assert lines[1].split()[2:5] == ["1.00", "0.50", "1.50"]   # 6000 ns / 6 calls, min 500, max 1500
    assert "python3 bench.py" in out.read_text()


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "4"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_stack_token_bytes_per_layer():
    """Weights (W_in 3D x D, W_out D x D in bf16), the state read and written
    (2 x 8 d bytes per row and channel) and four bf16 activation rows."""
    from workloads import get_config
    cfg = get_config(5)
    D, B = 2048, 64
    per_layer = 4 * D * D * 2 + B * D * 16 * 16 + 4 * B * D * 2
    assert bench.stack_token_bytes(cfg) == 24 * per_layer == 1635778560
