"""Summaries of rocprofv3 output for the committed profiles.

    python -m gqa_attention_flashattention_amd.profile_summary trace <results.db> --title T --cmd C
        per-kernel dispatch count and duration statistics from a
        `rocprofv3 --kernel-trace` database (markdown table on stdout), one
        row per (kernel, grid size): one kernel serves several workloads
    python -m gqa_attention_flashattention_amd.profile_summary traffic \
            --fetch <dir> --write <dir> --cmd-fetch C1 --cmd-write C2 --copy-mib N
        FETCH_SIZE / WRITE_SIZE per dispatch from two `rocprofv3 --pmc` runs,
        each scaled by what the same counter reads for the plain device copy of
        N MiB that `bench.py --copy-calibration N` runs first; writes a
        markdown table on stdout and updates profiles/traffic.json (keyed
        "kernel@grid threads"), which bench.py reports as `roofline.traffic`
        while the kernel source it was measured on is unchanged (sha256
        recorded per kernel).
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import sqlite3
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")

# kernel short name -> source file whose hash guards its traffic record
KERNEL_SOURCES = {
    "decode_split_kernel": "csrc/decode.hip",
    "decode_combine_kernel": "csrc/decode.hip",
    "prefill_bf16_kernel": "csrc/prefill_bf16.hip",
    "prefill_f32_kernel": "csrc/prefill_f32.hip",
}


def short_name(name: str) -> str:
    m = re.search(r"(\w+_kernel<[^>]*>)", name)
    if m:
        return m.group(1).replace(" ", "")
    m = re.search(r"(\w+_kernel)", name)
    return m.group(1) if m else name.split("(")[0][:60]


def source_sha(kernel_short: str) -> str | None:
    for prefix, rel in KERNEL_SOURCES.items():
        if kernel_short.startswith(prefix):
            with open(os.path.join(PKG, rel), "rb") as f:
                return hashlib.sha256(f.read()).hexdigest()
    return None


def trace_table(db_path: str) -> list[tuple]:
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, grid_x * grid_y * grid_z, duration from kernels").fetchall()
    agg = collections.defaultdict(list)
    for name, grid, dur in rows:
        agg[(short_name(name), int(grid))].append(dur / 1e3)
    out = []
    for (k, g), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        out.append((k, g, len(v), statistics.mean(v), statistics.median(v), min(v), max(v)))
    return out


def counters(run_dir: str) -> dict:
    """{"kernel short name@grid threads": {counter: [value per dispatch]}}"""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            key = (r["Dispatch_Id"], r["Counter_Name"])
            per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = f'{short_name(r["Kernel_Name"])}@{int(r["Grid_Size"])}'
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for d, cs in per.items():
        for c, v in cs.items():
            out[names[d]][c].append(v)
    return out


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--title", default="kernel trace")
    t.add_argument("--cmd", default="")
    tr = sub.add_parser("traffic")
    tr.add_argument("--fetch", required=True)
    tr.add_argument("--write", required=True)
    tr.add_argument("--cmd-fetch", default="")
    tr.add_argument("--cmd-write", default="")
    tr.add_argument("--copy-mib", type=float, required=True)
    tr.add_argument("--title", default="HBM traffic per dispatch")
    args = ap.parse_args()

    if args.mode == "trace":
        print(f"# {args.title}\n")
        if args.cmd:
            print(f"Command:\n\n    {args.cmd}\n")
        print("| kernel | grid threads | dispatches | avg us | median us | min us | max us |")
        print("|---|---|---|---|---|---|---|")
        for k, g, n, a, m, lo, hi in trace_table(args.db):
            if len(k) > 90:
                k = k[:87] + "..."
            print(f"| `{k}` | {g} | {n} | {a:.2f} | {m:.2f} | {lo:.2f} | {hi:.2f} |")
        return

    fetch = counters(args.fetch)
    write = counters(args.write)
    copy_kib = args.copy_mib * 1024.0

    def copy_value(table, counter):
        for k, cs in table.items():
            if "copy" in k.lower() or "elementwise" in k.lower():
                vals = sorted(cs.get(counter, []))
                big = [v for v in vals if v > 0.5 * copy_kib]
                if big:
                    return statistics.median(big)
        raise RuntimeError(f"no calibration copy kernel with {counter} near {copy_kib} KiB")

    f_scale = copy_kib / copy_value(fetch, "FETCH_SIZE")
    w_scale = copy_kib / copy_value(write, "WRITE_SIZE")
    print(f"# {args.title}\n")
    print("Commands:\n")
    print(f"    {args.cmd_fetch}\n    {args.cmd_write}\n")
    print(f"Calibration: a device copy of {args.copy_mib:g} MiB reads FETCH_SIZE x{1 / f_scale:.4f} "
          f"and WRITE_SIZE x{1 / w_scale:.4f} of its size; the figures below are scaled by "
          f"{f_scale:.4f} and {w_scale:.4f}.\n")
    print("| kernel | dispatches | FETCH KiB (median) | WRITE KiB (median) | scaled bytes per dispatch |")
    print("|---|---|---|---|---|")
    record = {}
    if os.path.exists(TRAFFIC_JSON):
        record = json.load(open(TRAFFIC_JSON))
    for k in sorted(set(fetch) | set(write)):
        fv = fetch.get(k, {}).get("FETCH_SIZE", [])
        wv = write.get(k, {}).get("WRITE_SIZE", [])
        if not fv or not wv:
            continue
        fm, wm = statistics.median(fv), statistics.median(wv)
        scaled = (fm * f_scale + wm * w_scale) * 1024.0
        shown = k if len(k) <= 90 else k[:87] + "..."
        print(f"| `{shown}` | {len(fv)} | {fm:.0f} | {wm:.0f} | {scaled:.4g} |")
        sha = source_sha(k)
        if sha:
            record[k] = {"fetch_kib": fm, "write_kib": wm, "fetch_scale": f_scale,
                         "write_scale": w_scale, "bytes_per_dispatch": scaled,
                         "source_sha256": sha}
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(record, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main()
