"""Host logic of the rocprofv3 harness: CSV parsing, calibration, the
achieved-rate and utilisation arithmetic and the traffic record, on small
hand-made files (no GPU, no profiler)."""

import csv
import json

import pytest

from transformer_attention_tiled_amd import rocprof_harness as h

P = "void attn::(anonymous namespace)::prefill_pp_kernel<128, true>(attn::PrefillArgs, float, int)"
PP = "void attn::(anonymous namespace)::prefill_pp_paged_kernel<128, true>(attn::PagedArgs, float, int)"
D = "void attn::(anonymous namespace)::decode_kernel<128>(attn::PagedArgs, float)"
M = "void attn::(anonymous namespace)::decode_merge_kernel<128>(attn::PagedArgs, int)"


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_durations_in_dispatch_order(tmp_path):
    p = tmp_path / "r_kernel_trace.csv"
    hdr = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    _write(p, hdr, [
        ["KERNEL_DISPATCH", 3, P, 5000, 8000],       # 3.0 us
        ["KERNEL_DISPATCH", 1, P, 1000, 3000],       # 2.0 us
        ["KERNEL_DISPATCH", 2, PP, 0, 99000],        # other kernel, not matched
        ["KERNEL_DISPATCH", 4, D, 0, 1500],
        ["KERNEL_DISPATCH", 5, M, 0, 500],
    ])
    assert h.kernel_durations(str(p), h.KERNELS["prefill"]) == [2.0, 3.0]
    # the decode name must not match the merge kernel
    assert h.kernel_durations(str(p), h.KERNELS["decode"]) == [1.5]
    assert h.kernel_durations(str(p), h.KERNELS["merge"]) == [0.5]
    st = h.timed_stats([9.0, 2.0, 3.0, 4.0], 3)
    assert st == {"launches": 4, "timed": 3, "mean_us": 3.0, "min_us": 2.0, "max_us": 4.0}


def test_counter_values_sum_instances_per_dispatch(tmp_path):
    p = tmp_path / "r_counter_collection.csv"
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    _write(p, hdr, [
        [1, P, "FETCH_SIZE", 10.0],
        [1, P, "FETCH_SIZE", 5.0],   # a second instance of the same dispatch
        [2, P, "FETCH_SIZE", 20.0],
        [2, P, "WRITE_SIZE", 7.0],
        [3, D, "FETCH_SIZE", 1.0],
    ])
    assert h.counter_values(str(p), h.KERNELS["prefill"], "FETCH_SIZE") == [15.0, 20.0]
    assert h.counter_values(str(p), h.KERNELS["prefill"], "WRITE_SIZE") == [7.0]
    assert h.counter_values(str(p), h.KERNELS["decode"], "FETCH_SIZE") == [1.0]


def test_calibration_and_traffic():
    # a copy of 1 GiB whose read counter shows half the bytes and whose write
    # counter shows all of them (what MI355X reports)
    cal = h.calibration(copy_fetch_kib=524288.0, copy_write_kib=1048576.0)
    assert cal["fetch_scale"] == pytest.approx(2.0)
    assert cal["write_scale"] == pytest.approx(1.0)
    assert h.traffic_bytes(100.0, 50.0, cal) == pytest.approx(100 * 1024 * 2 + 50 * 1024)


def test_mfma_utilisation():
    # every SIMD busy for half of the CU busy cycles
    assert h.mfma_utilisation(mfma_busy_cycles=1024 * 500, busy_cu_cycles=256 * 1000) == 0.5


def _raw():
    return {
        "prefill_flops": 2.0e12,
        "prefill_trace": {"launches": 20, "timed": 16, "mean_us": 1600.0, "min_us": 1590.0,
                          "max_us": 1610.0},
        "decode_bytes": 160_000_000,
        "decode_trace": {"launches": 24, "timed": 16, "mean_us": 30.0, "min_us": 29.0,
                         "max_us": 31.0},
        "merge_trace": {"launches": 24, "timed": 16, "mean_us": 10.0, "min_us": 9.0,
                        "max_us": 11.0},
        "copy_fetch_kib": 524288.0, "copy_write_kib": 1048576.0,
        "prefill_fetch_kib": 1000.0, "prefill_write_kib": 2000.0,
        "decode_fetch_kib": 300.0, "decode_write_kib": 4.0,
        "merge_fetch_kib": 8.0, "merge_write_kib": 1.0,
        "prefill_sq": {c: 1.0 for c in h.SQ_COUNTERS} | {"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 7.0,
                                                       "SQ_BUSY_CU_CYCLES": 256 * 10.0},
    }


def test_summary_rates_and_fractions():
    rep = h.summarise(_raw())
    p, d = rep["prefill"], rep["decode"]
    assert p["tflops"] == pytest.approx(2.0e12 / 1600e-6 / 1e12)          # 1250
    assert p["frac_bf16_peak"] == pytest.approx(1250.0 / h.PEAK_BF16_TFLOPS)
    assert p["hbm_bytes"] == pytest.approx(1000 * 1024 * 2 + 2000 * 1024)
    assert p["mfma_util"] == pytest.approx(0.7)
    assert d["gbs_split"] == pytest.approx(160e6 / 30e-6 / 1e9)             # 5333
    assert d["gbs_split_plus_merge"] == pytest.approx(4000.0)
    assert d["frac_hbm_split_plus_merge"] == pytest.approx(0.5)
    md = h.markdown(rep, "cmd")
    assert "1250.0 TFLOP/s" in md and "4000 GB/s" in md and "70.0%" in md


def test_update_traffic_record(tmp_path):
    rep = h.summarise(_raw())
    path = tmp_path / "hbm_traffic.json"
    path.write_text(json.dumps({"_about": "kept", "other": {"x": 1}}))
    h.update_traffic(rep, str(path))
    rec = json.loads(path.read_text())
    assert rec["_about"] == "kept" and rec["other"] == {"x": 1}
    e = rec[h.TRAFFIC_KEYS["prefill"]]
    assert e["source"] == "prefill_bf16.hip" and len(e["source_sha256_16"]) == 16
    assert e["fetch_bytes"] == pytest.approx(1000 * 1024 * 2.0)
    assert e["write_bytes"] == pytest.approx(2000 * 1024 * 1.0)
    dec = rec[h.TRAFFIC_KEYS["decode"]]
    assert dec["merge_kernel_fetch_kib"] == 8.0
    assert rec["calibration"]["fetch_scale"] == pytest.approx(2.0)


def test_harness_imports_no_torch():
    # the harness process must not touch the GPU: it imports no torch
    lines = [l.strip() for l in open(h.__file__)]
    assert not any(l.startswith(("import torch", "from torch")) for l in lines)
