"""Host logic of the counter summaries that feed bench.py's roofline.traffic."""
import csv
import json
import os

from kv_cache_attention_step_amd import profiling as P


def _write_counters(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for disp, name, vals in rows:
            for v in vals:   # one row per counter instance; summed per dispatch
                w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter,
                            "Counter_Value": v})


def test_traffic_summary_calibrates_and_checks_sources(tmp_path):
    qkv = "(anonymous namespace)::qkv_rope_cache_bf16_d128(unsigned short const*, int)"
    fetch_dir, write_dir = str(tmp_path / "f"), str(tmp_path / "w")
    # the copy reads 256 MiB but the counter shows half; two projection dispatches
    pre = "(anonymous namespace)::qkv_prepass_kernel(int const*, int)"
    _write_counters(fetch_dir, "FETCH_SIZE", [
        (1, "__amd_rocclr_copyBuffer", [65536.0, 65536.0]),
        (2, pre, [1.0]), (3, qkv, [100.0, 200.0]),
        (4, pre, [1.0]), (5, qkv, [150.0, 150.0]),
    ])
    _write_counters(write_dir, "WRITE_SIZE", [
        (1, "void at::native::vectorized_elementwise_kernel<16, FillFunctor>", [524288.0]),
        (2, pre, [1.0]), (3, qkv, [10.0]),
        (4, pre, [1.0]), (5, qkv, [30.0]),
    ])
    rec = P.summarize(fetch_dir, write_dir)
    assert rec["calibration"]["fetch_factor"] == 2.0
    assert rec["calibration"]["write_factor"] == 1.0
    k = rec["kernels"]["qkv_rope_cache_write"]
    assert k["fetch_kib"] == 300.0 and k["write_kib"] == 20.0
    assert k["traffic_bytes"] == (300.0 * 2.0 + 20.0) * 1024
    path = tmp_path / "t.json"
    path.write_text(json.dumps(rec))
    assert P.load_traffic(str(path), "qkv_rope_cache_write") == k["traffic_bytes"]
    assert P.load_traffic(str(path), "varlen_bidir_attention") is None
    rec["sources_sha256"] = "0" * 64            # taken on other kernel sources
    path.write_text(json.dumps(rec))
    assert P.load_traffic(str(path), "qkv_rope_cache_write") is None
    assert P.load_traffic(str(tmp_path / "missing.json"), "qkv_rope_cache_write") is None


def test_stats_markdown(tmp_path):
    f = tmp_path / "s.csv"
    with open(f, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                           "Percentage", "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow({"Name": "void (anonymous namespace)::attn_bf16_d128<true, true>(X)",
                    "Calls": 3, "TotalDurationNs": 600000, "AverageNs": 200000,
                    "Percentage": 60.0, "MinNs": 190000, "MaxNs": 210000})
        w.writerow({"Name": "(anonymous namespace)::topk_kernel(float const*)", "Calls": 3,
                    "TotalDurationNs": 60000, "AverageNs": 20000, "Percentage": 6.0,
                    "MinNs": 19000, "MaxNs": 21000})
    md = P.stats_markdown(str(f)).splitlines()
    assert md[2].startswith("| `attn_bf16_d128<true, true>` | 3 | 200.0 |")
    assert md[3].startswith("| `topk_kernel` | 3 | 20.0 |")


def test_mfma_summary_busy_fraction(tmp_path):
    d = tmp_path / "m"
    os.makedirs(d)
    qkv = "void (anonymous namespace)::qkv_rope_cache_bf16_d128<Gemm8<256>, true>(int)"
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        # 2 XCDs, 8 SIMDs: GRBM_GUI_ACTIVE is summed over the XCDs (2 x 100 clocks
        # in 50 ns: 2 GHz), SQ counters over the SIMDs
        for disp, busy in ((1, 600.0), (2, 200.0)):
            row = {"Dispatch_Id": disp, "Kernel_Name": qkv, "Start_Timestamp": 1000,
                   "End_Timestamp": 1050}
            w.writerow({**row, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES", "Counter_Value": busy})
            w.writerow({**row, "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 200.0})
            w.writerow({**row, "Counter_Name": "SQ_INSTS_VALU_MFMA_MOPS_BF16", "Counter_Value": 2.0})
            w.writerow({**row, "Kernel_Name": "qkv_prepass_kernel(int)", "Dispatch_Id": disp + 10,
                        "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 2.0})
    rec = P.mfma_summary(str(d), n_simd=8, n_xcd=2)
    k = rec["qkv_rope_cache_write"]
    assert k["dispatches"] == 2
    assert abs(k["mfma_busy"] - (600 / 800 + 200 / 800) / 2) < 1e-12
    assert k["bf16_mfma_flops"] == 1024.0
    assert k["clock_ghz"] == 2.0 and k["us"] == 0.05


def test_summaries_add_the_kernels_of_one_call(tmp_path):
    """An entry point that launches two matching kernels per call (256-row tiles,
    then 128-row tiles): figures per call are sums over both dispatches, counted
    by the once-per-call pre-pass; the busy fraction is weighted by clocks."""
    main = "void (anonymous namespace)::qkv_rope_cache_bf16_d128<Gemm8<256>, true>(int)"
    tail = "void (anonymous namespace)::qkv_rope_cache_bf16_d128<Gemm8<128>, false>(int)"
    pre = "(anonymous namespace)::qkv_prepass_kernel(int const*, int)"
    fetch_dir, write_dir = str(tmp_path / "f"), str(tmp_path / "w")
    _write_counters(fetch_dir, "FETCH_SIZE", [
        (1, "__amd_rocclr_copyBuffer", [131072.0]),
        (2, pre, [1.0]), (3, main, [250.0]), (4, tail, [50.0])])
    _write_counters(write_dir, "WRITE_SIZE", [
        (1, "void at::native::vectorized_elementwise_kernel<16, FillFunctor>", [524288.0]),
        (2, pre, [1.0]), (3, main, [15.0]), (4, tail, [5.0])])
    k = P.summarize(fetch_dir, write_dir)["kernels"]["qkv_rope_cache_write"]
    assert k["fetch_kib"] == 300.0 and k["write_kib"] == 20.0
    d = tmp_path / "m"
    os.makedirs(d)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        # main: 300 clocks per XCD in 150 ns, 75 % busy; tail: 100 clocks in 50 ns, 25 % busy
        for disp, name, grbm, busy, ns in ((3, main, 600.0, 1800.0, 150), (4, tail, 200.0, 200.0, 50)):
            row = {"Dispatch_Id": disp, "Kernel_Name": name, "Start_Timestamp": 1000,
                   "End_Timestamp": 1000 + ns}
            w.writerow({**row, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES", "Counter_Value": busy})
            w.writerow({**row, "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": grbm})
            w.writerow({**row, "Counter_Name": "SQ_INSTS_VALU_MFMA_MOPS_BF16", "Counter_Value": 1.0})
        w.writerow({"Dispatch_Id": 2, "Kernel_Name": pre, "Start_Timestamp": 0, "End_Timestamp": 10,
                    "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 2.0})
    m = P.mfma_summary(str(d), n_simd=8, n_xcd=2)["qkv_rope_cache_write"]
    assert m["dispatches"] == 2
    assert abs(m["mfma_busy"] - 2000.0 / (400.0 * 8)) < 1e-12
    assert m["bf16_mfma_flops"] == 1024.0 and m["us"] == 0.2 and m["clock_ghz"] == 2.0
