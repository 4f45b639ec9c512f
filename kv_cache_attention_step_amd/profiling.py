"""HBM traffic of the step's kernels from rocprofv3 counter runs.

Two counter passes over the same bench command, one with FETCH_SIZE and one
with WRITE_SIZE (KiB per dispatch, summed over the counter's instances), give
the bytes a kernel moves between the L2 and memory. Each counter is scaled by
what it reads for a kernel of known size run in the same process: the bench
with --calib copies a 256 MiB buffer once (read 256 MiB, write 256 MiB), and
the Infinity-Cache flush between steps fills a 512 MiB buffer (write 512 MiB).

    python -m kv_cache_attention_step_amd.profiling traffic FETCH_DIR WRITE_DIR OUT_JSON
    python -m kv_cache_attention_step_amd.profiling traffic-multi OUT_JSON LABEL=FETCH_DIR,WRITE_DIR ...
    python -m kv_cache_attention_step_amd.profiling stats KERNEL_STATS_CSV
    python -m kv_cache_attention_step_amd.profiling mfma COUNTER_DIR N_SIMD N_XCD

FETCH_DIR / WRITE_DIR hold the rocprofv3 csv output (*counter_collection.csv).
OUT_JSON records the per-dispatch averages, the calibration factors and a
SHA-256 of the kernel sources the counters were taken on; bench.py reports the
traffic only while those sources are unchanged. traffic-multi does the same for
several labelled runs (one bench component each, every run calibrated by its
own copy and fill); kernels of the run labelled "step" keep their plain names,
the others are stored as LABEL:name. `stats` prints the kernel table of a
`rocprofv3 --kernel-trace --stats` run as markdown. `mfma` prints, per kernel,
the matrix-unit busy fraction, the bf16 MFMA work, the LDS instructions and the
clock (one XCD's busy clocks over the dispatch's duration) per dispatch.
"""
import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# kernel of each step component, as rocprofv3 names it (substring match). A
# (kernels, once) pair covers an entry point that may launch several matching
# kernels per call (the projection: 256-row tiles, then 128-row tiles for the
# rows past the last whole round): figures are per call, summed over the
# matching dispatches and divided by the dispatches of `once`, a kernel the
# entry point launches exactly once per call.
KERNELS = {
    "qkv_rope_cache_write": ("qkv_rope_cache_bf16_d128", "qkv_prepass_kernel"),
    "varlen_bidir_attention": "attn_bf16_d128<true",
    "attention_one_pass": "attn_bf16_d128<false",
    "importance_topk": "topk_kernel",
    "verify_rows": "verify_rows",
    "lmhead_partials": "lmhead_partials",
    "fork_view_pages": "fork_kernel",
    "commit_accepted": "commit_kernel",
    "linear_residual": "linear_residual_dma",
}
CALIB_COPY_KIB = 256 * 1024   # the --calib copy: reads and writes this much
CALIB_FILL_KIB = 512 * 1024   # the flush fill: writes this much


def sources_digest(csrc: str = CSRC) -> str:
    """SHA-256 over the device sources (file names and contents, sorted)."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(csrc, "*"))):
        if os.path.splitext(path)[1] in (".hip", ".hpp", ".cpp", ".h"):
            h.update(os.path.basename(path).encode())
            h.update(open(path, "rb").read())
    return h.hexdigest()


def per_dispatch(csv_dir: str, counter: str):
    """{dispatch id: (kernel name, counter value summed over instances)}"""
    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {csv_dir}")
    out = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = (f, r["Dispatch_Id"])
            name, val = out.get(key, (r["Kernel_Name"], 0.0))
            out[key] = (name, val + float(r["Counter_Value"]))
    return out


def _names(spec):
    """(substring of the component's kernels, substring of its once-per-call kernel)"""
    return spec if isinstance(spec, tuple) else (spec, spec)


def _mean_for(disp, spec):
    """Mean per call of the counter over the component's dispatches, and the calls."""
    sub, once = _names(spec)
    vals = [v for (n, v) in disp.values() if sub in n]
    calls = sum(1 for (n, _) in disp.values() if once in n)
    return (sum(vals) / calls, calls) if vals and calls else (None, 0)


def summarize(fetch_dir: str, write_dir: str):
    fetch = per_dispatch(fetch_dir, "FETCH_SIZE")
    write = per_dispatch(write_dir, "WRITE_SIZE")
    # calibration: the largest copy dispatch (FETCH) and the largest fill (WRITE)
    # the --calib device copy (a blit kernel; other copy kernels convert dtypes)
    copies = [v for (n, v) in fetch.values() if "copybuffer" in n.lower()]
    fills = [v for (n, v) in write.values() if "fill" in n.lower()]
    if not copies or not fills:
        raise RuntimeError("calibration dispatches not found (run the bench with --calib)")
    f_fetch = CALIB_COPY_KIB / max(copies)
    f_write = CALIB_FILL_KIB / max(fills)
    kernels = {}
    for key, spec in KERNELS.items():
        fk, nf = _mean_for(fetch, spec)
        wk, nw = _mean_for(write, spec)
        if fk is None or wk is None:
            continue
        kernels[key] = {
            "fetch_kib": round(fk, 1), "write_kib": round(wk, 1), "dispatches": [nf, nw],
            "traffic_bytes": round((fk * f_fetch + wk * f_write) * 1024.0),
        }
    return {"calibration": {"copy_fetch_kib": round(max(copies), 1),
                            "fill_write_kib": round(max(fills), 1),
                            "fetch_factor": round(f_fetch, 5), "write_factor": round(f_write, 5)},
            "kernels": kernels, "sources_sha256": sources_digest()}


def summarize_multi(pairs):
    """pairs: [(label, fetch_dir, write_dir)]; one record with every labelled
    run's kernels (label "step" unprefixed) and its calibration."""
    out = {"calibration": {}, "kernels": {}, "sources_sha256": sources_digest()}
    for label, fd, wd in pairs:
        rec = summarize(fd, wd)
        out["calibration"][label] = rec["calibration"]
        for k, v in rec["kernels"].items():
            out["kernels"][k if label == "step" else f"{label}:{k}"] = v
    return out


def mfma_summary(csv_dir: str, n_simd: int, n_xcd: int):
    """{kernel: dict(dispatches, mfma_busy, bf16_mfma_flops, lds_insts, clock_ghz, us)}
    averaged over dispatches. rocprofv3 reports each counter summed over its
    hardware instances: SQ counters over every SIMD's sequencer, GRBM_GUI_ACTIVE
    over the XCDs (each counts its own busy clocks), so one XCD's busy clocks
    are GRBM_GUI_ACTIVE / n_xcd and the matrix-unit busy fraction is
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / n_xcd x n_simd)."""
    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {csv_dir}")
    disp = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            key = (f, r["Dispatch_Id"])
            d = disp.setdefault(key, {"name": r["Kernel_Name"],
                                      "ns": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])})
            c = r["Counter_Name"]
            d[c] = d.get(c, 0.0) + float(r["Counter_Value"])
    out = {}
    for key, spec in KERNELS.items():
        sub, once = _names(spec)
        ds = [d for d in disp.values() if sub in d["name"] and d.get("GRBM_GUI_ACTIVE")]
        calls = sum(1 for d in disp.values() if once in d["name"])
        if not ds or not calls:
            continue
        # per call: work and time summed over the call's dispatches; the busy
        # fraction and the clock weighted by each dispatch's busy clocks
        per_call = lambda f: sum(f(d) for d in ds) / calls
        xcd_clocks = lambda d: d["GRBM_GUI_ACTIVE"] / n_xcd
        clocks = sum(xcd_clocks(d) for d in ds)
        ns = sum(d["ns"] for d in ds)
        out[key] = {
            "dispatches": len(ds),
            "mfma_busy": round(sum(d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for d in ds) /
                               (clocks * n_simd), 4),
            "bf16_mfma_flops": per_call(lambda d: d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512),
            "lds_insts": per_call(lambda d: d.get("SQ_INSTS_LDS", 0.0)),
            "lds_bank_conflict_cycles": per_call(lambda d: d.get("SQ_LDS_BANK_CONFLICT", 0.0)),
            "clock_ghz": round(clocks / ns if ns > 0 else 0.0, 3),
            "us": round(ns * 1e-3 / calls, 2)}
    return out


def load_traffic(path: str, kernel: str):
    """Bytes per launch of `kernel` recorded in `path`, or None when the file is
    missing or was taken on other kernel sources."""
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else float(k["traffic_bytes"])


def stats_markdown(stats_csv: str, top: int = 14) -> str:
    """Markdown table of a rocprofv3 *kernel_stats.csv (time per kernel)."""
    rows = list(csv.DictReader(open(stats_csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["| kernel | calls | avg us | min us | max us | % of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in rows[:top]:
        name = r["Name"]
        short = name.replace("(anonymous namespace)::", "")
        if short.startswith("void "):
            short = short[5:]
        short = short.split("(")[0]
        if len(short) > 70:
            short = short[:67] + "..."
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.2f} |")
    return "\n".join(lines)


if __name__ == "__main__":
    if len(sys.argv) == 5 and sys.argv[1] == "traffic":
        rec = summarize(sys.argv[2], sys.argv[3])
        with open(sys.argv[4], "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec, indent=1))
    elif len(sys.argv) >= 4 and sys.argv[1] == "traffic-multi":
        pairs = []
        for arg in sys.argv[3:]:
            label, dirs = arg.split("=", 1)
            fd, wd = dirs.split(",")
            pairs.append((label, fd, wd))
        rec = summarize_multi(pairs)
        with open(sys.argv[2], "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec, indent=1))
    elif len(sys.argv) == 3 and sys.argv[1] == "stats":
        print(stats_markdown(sys.argv[2]))
    elif len(sys.argv) == 5 and sys.argv[1] == "mfma":
        for k, v in mfma_summary(sys.argv[2], int(sys.argv[3]), int(sys.argv[4])).items():
            print(k, json.dumps(v))
    else:
        sys.exit(__doc__)
