"""Host logic of the benchmark script, on the CPU: the one-GPU guard, the
reduction of the two HBM byte-counter runs, and the source-hash gate that
withdraws a traffic figure once the measured kernel's source changes."""

import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

COPY = "void at::native::vectorized_elementwise_kernel<neg_kernel_cuda>"  # any name holding the copy fragment
QUANT = "void qw::(anonymous namespace)::quant_subgroup_batched_kernel<4, 8>(qw::QuantBatch)"
GEMV = "void qw::(anonymous namespace)::gemv8_kernel<4, 1, 16, 256>(qw::GemvBatch<256>)"


def _counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size",
                                          "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, grid, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Grid_Size": grid,
                        "Counter_Name": counter, "Counter_Value": value})


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def _summary(tmp_path):
    # the copy reads 1 GiB and writes 1 GiB: FETCH_SIZE counts half of it,
    # WRITE_SIZE all of it, so fetch counts scale by 2 and write counts by 1
    _counters(tmp_path / "f", "FETCH_SIZE", [
        (COPY, 1 << 20, 524288.0),
        (QUANT, 4096, 900.0), (QUANT, 4096, 1100.0),   # mean 1000 KiB
        (GEMV, 5439488, 100.0),
        (GEMV, 64, 99999.0),                           # another grid: not the measured launch
    ])
    _counters(tmp_path / "w", "WRITE_SIZE", [
        (COPY, 1 << 20, 1048576.0),
        (QUANT, 4096, 300.0),
        (GEMV, 5439488, 50.0),
    ])
    return bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"), copy_mib=1024)


def test_pmc_summary_scales_by_the_copy(tmp_path):
    s = _summary(tmp_path)
    assert s["fetch_factor"] == 2.0 and s["write_factor"] == 1.0
    k = s["kernels"]
    assert k["quantize_pack_batched"]["traffic_bytes"] == (1000 * 2 + 300) * 1024
    assert k["quantize_pack_batched"]["dispatches"] == [2, 1]
    assert k["gemv_batched_m1"]["traffic_bytes"] == (100 * 2 + 50) * 1024
    assert k["gemv_batched_m1"]["dispatches"] == [1, 1]
    # kernels without counts in both runs are left out
    assert "gemm" not in k and "gptq_hessian_k1368" not in k
    assert set(s["source_sha256"]) >= {"quantize.hip", "gemv.hip", "qw_internal.h"}


def test_traffic_is_withdrawn_when_the_source_changes(tmp_path, monkeypatch):
    s = _summary(tmp_path)
    f = tmp_path / "traffic.md"
    f.write_text("# summary\n\n```json\n" + json.dumps(s) + "\n```\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("quantize_pack_batched") == (1000 * 2 + 300) * 1024
    assert bench.measured_traffic("gemv_batched_m1") == (100 * 2 + 50) * 1024
    assert bench.measured_traffic("gemm") is None            # not measured
    assert bench.measured_traffic("no_such_label") is None
    # another hash for the GEMV source withdraws the GEMV figure only
    s["source_sha256"]["gemv.hip"] = "0" * 16
    f.write_text("```json\n" + json.dumps(s) + "\n```\n")
    assert bench.measured_traffic("gemv_batched_m1") is None
    assert bench.measured_traffic("quantize_pack_batched") == (1000 * 2 + 300) * 1024
    # a change of the shared header withdraws every figure
    s["source_sha256"]["qw_internal.h"] = "0" * 16
    f.write_text("```json\n" + json.dumps(s) + "\n```\n")
    assert bench.measured_traffic("quantize_pack_batched") is None
    # a missing or unreadable summary gives null, not an error
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.md"))
    assert bench.measured_traffic("quantize_pack_batched") is None


def test_clock_sampler_reports_nothing_without_a_gpu():
    # switched off, or with no device to read, the sampler yields no figure
    # and does not raise; the timed region runs the same either way
    with bench.ClockSampler(enabled=False) as off:
        pass
    assert off.summary() is None
    with bench.ClockSampler() as c:
        pass
    if not c.enabled:
        assert c.summary() is None


def test_clock_summary_medians():
    # samples of the first skip_s seconds (the ramp, and figures the device
    # has not refreshed yet) are left out
    c = bench.ClockSampler(enabled=False, skip_s=0.4)
    c.samples = [(0.1, 700.0, 300), (0.39, 2400.0, 300),
                 (0.5, 1800.0, 1300), (0.6, 2000.0, 1400), (0.7, None, None), (0.8, 1900.0, None)]
    s = c.summary()
    assert s["gfx_mhz_median"] == 1900 and s["gfx_mhz_min"] == 1800 and s["gfx_mhz_max"] == 2000
    assert s["socket_w_median"] == 1350 and s["samples"] == 3
    c.samples = c.samples[:2]
    assert c.summary() is None
