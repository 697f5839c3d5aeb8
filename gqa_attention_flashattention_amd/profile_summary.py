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
    python -m gqa_attention_flashattention_amd.profile_summary gqa --run G=<dir> [...] \
            --kernel K --kv-bytes N --copy-mib M --cmd C
        FETCH_SIZE per dispatch of kernel K in one `rocprofv3 --pmc FETCH_SIZE`
        run per G (query heads per KV head), scaled by that run's copy
        calibration, against the N bytes of K and V the launch must read:
        the GQA reuse check (the fetched bytes must not grow with G).
    python -m gqa_attention_flashattention_amd.profile_summary mfma <dir> [<dir> ...] --cmd C ...
        MFMA utilisation per dispatch from `rocprofv3 --pmc` runs that hold
        GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES and, where collected,
        SQ_VALU_MFMA_COEXEC_CYCLES, SQ_INSTS_VALU, SQ_INSTS_MFMA and
        SQ_INSTS_VALU_MFMA_MOPS_BF16; writes a markdown table on stdout and
        updates profiles/mfma.json (same keys and source guard as
        traffic.json), which bench.py reports beside the prefill roofline.
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
MFMA_JSON = os.path.join(ROOT, "profiles", "mfma.json")

# MI355X: 8 XCDs (GRBM_GUI_ACTIVE is summed over one counter per XCD), 256
# compute units of 4 SIMDs; one SIMD retires 1024 dense bf16 MFMA flops per
# cycle (a 32x32x16 MFMA, 32768 flops, every 32 cycles); one unit of
# SQ_INSTS_VALU_MFMA_MOPS_BF16 is 512 flops.
XCDS = 8
SIMDS = 256 * 4
BF16_FLOPS_PER_SIMD_CYCLE = 1024
FLOPS_PER_MOP = 512

# kernel short name -> source file whose hash guards its traffic record
KERNEL_SOURCES = {
    "decode_split_kernel": "csrc/decode.hip",
    "decode_stream_kernel": "csrc/decode.hip",
    "decode_wide_kernel": "csrc/decode.hip",
    "decode_combine_kernel": "csrc/decode.hip",
    "decode_combine_rows_kernel": "csrc/decode.hip",
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


def mfma_table(run_dirs: list[str]) -> dict:
    """{"kernel@grid": {figure: median over dispatches}} for kernels that
    issued MFMAs; counters of one kernel may come from several runs."""
    merged = collections.defaultdict(dict)
    for d in run_dirs:
        for k, cs in counters(d).items():
            merged[k].update({c: statistics.median(v) for c, v in cs.items()})
            merged[k]["dispatches"] = max(merged[k].get("dispatches", 0),
                                          max(len(v) for v in cs.values()))
    out = {}
    for k, c in merged.items():
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        grbm = c.get("GRBM_GUI_ACTIVE", 0.0)
        if busy <= 0 or grbm <= 0:
            continue
        cycles = grbm / XCDS
        rec = {"dispatches": int(c["dispatches"]), "cycles": cycles,
               "mfma_busy": busy / (SIMDS * cycles)}
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in c:
            rec["mfma_valu_coexec"] = c["SQ_VALU_MFMA_COEXEC_CYCLES"] / (SIMDS * cycles)
        if c.get("SQ_INSTS_MFMA", 0) > 0 and "SQ_INSTS_VALU" in c:
            rec["valu_insts_per_mfma"] = c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"]
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:
            flops = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * FLOPS_PER_MOP
            rec["counted_mfma_flops"] = flops
            rec["mfma_rate_frac"] = flops / (BF16_FLOPS_PER_SIMD_CYCLE * SIMDS * cycles)
        out[k] = rec
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
    gq_ = sub.add_parser("gqa")
    gq_.add_argument("--run", action="append", required=True, help="G=<rocprofv3 output dir>")
    gq_.add_argument("--kernel", required=True, help="kernel short-name prefix")
    gq_.add_argument("--kv-bytes", type=float, required=True)
    gq_.add_argument("--copy-mib", type=float, required=True)
    gq_.add_argument("--cmd", default="")
    gq_.add_argument("--title", default="GQA reuse: HBM fetch of the decode split kernel against G")
    mf = sub.add_parser("mfma")
    mf.add_argument("dirs", nargs="+")
    mf.add_argument("--cmd", action="append", default=[])
    mf.add_argument("--title", default="MFMA utilisation per dispatch")
    args = ap.parse_args()

    if args.mode == "gqa":
        copy_kib = args.copy_mib * 1024.0
        print(f"# {args.title}\n")
        if args.cmd:
            print(f"Command (one run per G):\n\n    {args.cmd}\n")
        print(f"FETCH_SIZE of each run is scaled by what it reads for a plain device copy of "
              f"{args.copy_mib:g} MiB run first in the same process. K/V bytes per launch: "
              f"{args.kv_bytes:.6g}.\n")
        print("| G (query heads per KV head) | kernel@grid | dispatches | FETCH KiB (median) "
              "| calibration | fetched bytes | fetched / K+V bytes |")
        print("|---|---|---|---|---|---|---|")
        for spec in args.run:
            g, d = spec.split("=", 1)
            table = counters(d)
            cal = None
            for k, cs in table.items():
                if "copy" in k.lower() or "elementwise" in k.lower():
                    big = [v for v in cs.get("FETCH_SIZE", []) if v > 0.5 * copy_kib]
                    if big:
                        cal = copy_kib / statistics.median(big)
            if cal is None:
                raise RuntimeError(f"{d}: no calibration copy")
            for k, cs in sorted(table.items()):
                if not k.startswith(args.kernel):
                    continue
                fm = statistics.median(cs["FETCH_SIZE"])
                b = fm * cal * 1024.0
                print(f"| {g} | `{k}` | {len(cs['FETCH_SIZE'])} | {fm:.0f} | x{cal:.4f} | {b:.6g} "
                      f"| {b / args.kv_bytes:.4f} |")
        return

    if args.mode == "mfma":
        table = mfma_table(args.dirs)
        print(f"# {args.title}\n")
        print("Commands:\n")
        for c in args.cmd:
            print(f"    {c}")
        print("\nCycles = GRBM_GUI_ACTIVE / 8 (one counter per XCD, summed); MFMA busy = "
              "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles); co-exec likewise with "
              "SQ_VALU_MFMA_COEXEC_CYCLES; MFMA rate = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flops / "
              "(1024 flops per SIMD cycle x 1024 SIMDs x cycles), the fraction of the "
              "bf16 MFMA peak at the clock the kernel ran at.\n")
        print("| kernel | dispatches | cycles | MFMA busy | MFMA+VALU co-exec | VALU insts / MFMA "
              "| counted MFMA flops | MFMA rate |")
        print("|---|---|---|---|---|---|---|---|")
        record = json.load(open(MFMA_JSON)) if os.path.exists(MFMA_JSON) else {}

        def f(rec, key, fmt):
            return format(rec[key], fmt) if key in rec else "-"

        for k in sorted(table):
            r = table[k]
            shown = k if len(k) <= 90 else k[:87] + "..."
            print(f"| `{shown}` | {r['dispatches']} | {r['cycles']:.4g} | {f(r, 'mfma_busy', '.1%')} "
                  f"| {f(r, 'mfma_valu_coexec', '.1%')} | {f(r, 'valu_insts_per_mfma', '.2f')} "
                  f"| {f(r, 'counted_mfma_flops', '.4g')} | {f(r, 'mfma_rate_frac', '.1%')} |")
            sha = source_sha(k)
            if sha:
                record[k] = dict(r, source_sha256=sha)
        os.makedirs(os.path.dirname(MFMA_JSON), exist_ok=True)
        with open(MFMA_JSON, "w") as fh:
            json.dump(record, fh, indent=1, sort_keys=True)
        return

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
