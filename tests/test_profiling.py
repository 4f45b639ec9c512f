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
    _write_counters(fetch_dir, "FETCH_SIZE", [
        (1, "__amd_rocclr_copyBuffer", [65536.0, 65536.0]),
        (2, qkv, [100.0, 200.0]),
        (3, qkv, [150.0, 150.0]),
    ])
    _write_counters(write_dir, "WRITE_SIZE", [
        (1, "void at::native::vectorized_elementwise_kernel<16, FillFunctor>", [524288.0]),
        (2, qkv, [10.0]),
        (3, qkv, [30.0]),
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
