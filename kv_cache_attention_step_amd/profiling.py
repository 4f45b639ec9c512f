"""HBM traffic of the step's kernels from rocprofv3 counter runs.

Two counter passes over the same bench command, one with FETCH_SIZE and one
with WRITE_SIZE (KiB per dispatch, summed over the counter's instances), give
the bytes a kernel moves between the L2 and memory. Each counter is scaled by
what it reads for a kernel of known size run in the same process: the bench
with --calib copies a 256 MiB buffer once (read 256 MiB, write 256 MiB), and
the Infinity-Cache flush between steps fills a 512 MiB buffer (write 512 MiB).

    python -m kv_cache_attention_step_amd.profiling traffic FETCH_DIR WRITE_DIR OUT_JSON
    python -m kv_cache_attention_step_amd.profiling stats KERNEL_STATS_CSV

FETCH_DIR / WRITE_DIR hold the rocprofv3 csv output (*counter_collection.csv).
OUT_JSON records the per-dispatch averages, the calibration factors and a
SHA-256 of the kernel sources the counters were taken on; bench.py reports the
traffic only while those sources are unchanged. `stats` prints the kernel
table of a `rocprofv3 --kernel-trace --stats` run as markdown.
"""
import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# kernel of each step component, as rocprofv3 names it (substring match)
KERNELS = {
    "qkv_rope_cache_write": "qkv_rope_cache_bf16_d128",
    "varlen_bidir_attention": "attn_bf16_d128",
    "importance_topk": "topk_kernel",
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


def _mean_for(disp, substr):
    vals = [v for (n, v) in disp.values() if substr in n]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def summarize(fetch_dir: str, write_dir: str):
    fetch = per_dispatch(fetch_dir, "FETCH_SIZE")
    write = per_dispatch(write_dir, "WRITE_SIZE")
    # calibration: the largest copy dispatch (FETCH) and the largest fill (WRITE)
    copies = [v for (n, v) in fetch.values() if "copy" in n.lower()]
    fills = [v for (n, v) in write.values() if "fill" in n.lower()]
    if not copies or not fills:
        raise RuntimeError("calibration dispatches not found (run the bench with --calib)")
    f_fetch = CALIB_COPY_KIB / max(copies)
    f_write = CALIB_FILL_KIB / max(fills)
    kernels = {}
    for key, sub in KERNELS.items():
        fk, nf = _mean_for(fetch, sub)
        wk, nw = _mean_for(write, sub)
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
    elif len(sys.argv) == 3 and sys.argv[1] == "stats":
        print(stats_markdown(sys.argv[2]))
    else:
        sys.exit(__doc__)
