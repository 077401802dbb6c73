"""Summaries of rocprofv3 output for profiles/ (text only).

kernel-stats: rocprofv3 --kernel-trace --stats --output-format csv run
    -> a markdown table of per-kernel calls and durations.
traffic: two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of a bench
    command with --calibrate-copy MIB -> HBM bytes per split launch, each
    counter scaled by what it reads for the calibration kernel (neg over
    MIB MiB of fp32: MIB MiB read, MIB MiB written).

Usage:
  python -m block_sparse_paged_split_amd.profile_summary kernel-stats STATS_CSV OUT_MD --command CMD
  python -m block_sparse_paged_split_amd.profile_summary traffic FETCH_CSV WRITE_CSV OUT_MD \
      --workload W --calibrate-mib MIB --algorithmic-bytes B --command CMD --command CMD
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import re
import os

PKG = os.path.dirname(os.path.abspath(__file__))


# sources that decide the split kernel's code and launch shape
DIGEST_SOURCES = ("wise_split.hip", "wise_select.h", "wise_internal.h", "wise_api.hip")


def split_source_digest() -> str:
    """sha256 of the split kernel's sources with comments and whitespace
    removed, so that counters stay attributed across comment-only edits."""
    h = hashlib.sha256()
    for name in DIGEST_SOURCES:
        text = open(os.path.join(PKG, "csrc", name)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(name.encode() + b"\0" + "".join(text.split()).encode() + b"\0")
    return h.hexdigest()


def k_only_kernel(name: str) -> bool:
    """A K-only (LSE route) instantiation: split_static_kernel<bf16, D, K-only>
    or split_fused_kernel<bf16, D, waves, K-only, max blocks>."""
    m = re.search(r"split_(static|fused)_kernel<([^>]*)>", name)
    if not m:
        return False
    args = [a.strip() for a in m.group(2).split(",")]
    pos = 2 if m.group(1) == "static" else 3
    return len(args) > pos and args[pos] == "true"


def short(name: str) -> str:
    for key in ("split_fused_kernel", "split_static_kernel", "split_listed_kernel", "plan_kernel", "finish_kernel",
                "compact_pages_kernel", "snapshot_kernel", "restore_kernel", "read_probe_kernel"):
        if key in name:
            tmpl = name[name.find("<"): name.find(">") + 1] if "<" in name else ""
            return key + tmpl
    return name if len(name) < 70 else name[:67] + "..."


def duration_groups(trace_csv: str, min_share: float = 0.02):
    """Per kernel, its dispatch durations split into groups wherever the
    sorted durations jump by more than 15% (one kernel serves calls of very
    different sizes: a sparse call and a dense one of the same launch
    shape): [(kernel, [(dispatches, mean us, min us, max us), ...])] for the
    kernels holding at least min_share of the traced time."""
    durs = {}
    for r in csv.DictReader(open(trace_csv)):
        if r.get("Kind", "KERNEL_DISPATCH") != "KERNEL_DISPATCH":
            continue
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        durs.setdefault(r["Kernel_Name"], []).append(d)
    total = sum(sum(v) for v in durs.values()) or 1.0
    out = []
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        if sum(v) / total < min_share:
            continue
        v = sorted(v)
        groups, cur = [], [v[0]]
        for x in v[1:]:
            if x > cur[-1] * 1.15:
                groups.append(cur)
                cur = [x]
            else:
                cur.append(x)
        groups.append(cur)
        out.append((name, [(len(g), sum(g) / len(g), g[0], g[-1]) for g in groups]))
    return out


def kernel_stats(stats_csv: str, out_md: str, command: str) -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = ["# Kernel durations: rocprofv3 --kernel-trace --stats", "",
             "Command (run from /tmp with TMPDIR=/tmp; R = the repository root):", "",
             "```", command, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}% |")
    trace_csv = stats_csv.replace("_kernel_stats.csv", "_kernel_trace.csv")
    if os.path.exists(trace_csv):
        lines += ["", "Dispatch durations of the main kernels, grouped where the sorted durations jump by",
                  "more than 15% (calls of different sizes on the same kernel):", "",
                  "| kernel | dispatches | mean (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
        for name, groups in duration_groups(trace_csv):
            for n, mean, lo, hi in groups:
                lines.append(f"| {short(name)} | {n} | {mean:.2f} | {lo:.2f} | {hi:.2f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def _per_kernel(counter_csv: str, counter: str):
    vals = {}
    for r in csv.DictReader(open(counter_csv)):
        if r.get("Counter_Name") != counter:
            continue
        vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def traffic(fetch_csv: str, write_csv: str, out_md: str, workload: str, mib: int, algo: float,
            commands) -> None:
    f = _per_kernel(fetch_csv, "FETCH_SIZE")
    w = _per_kernel(write_csv, "WRITE_SIZE")
    known = mib * 1024.0  # KiB read by the calibration kernel, and KiB written
    cal_f = [v for k, v in f.items() if "neg" in k.lower()]
    cal_w = [v for k, v in w.items() if "neg" in k.lower()]
    if not cal_f or not cal_w:
        raise SystemExit("calibration kernel not found in the counter output")
    scale_f = known / max(cal_f[0])
    scale_w = known / max(cal_w[0])
    # the decode split kernel (the K-only instantiations of the LSE route are not counted)
    split = [k for k in f if "split_" in k and "kernel" in k and not k_only_kernel(k)]
    fk = [x for k in split for x in f[k]]
    wk = [x for k in split for x in w.get(k, [])]
    fetch_kib = sum(fk) / len(fk)
    write_kib = sum(wk) / len(wk) if wk else 0.0
    traffic_bytes = (fetch_kib * scale_f + write_kib * scale_w) * 1024.0
    rec = {"workload": workload, "kernel_source_sha256": split_source_digest(),
           "split_launches": len(fk), "fetch_kib_per_launch": round(fetch_kib, 1),
           "write_kib_per_launch": round(write_kib, 1),
           "calibration_mib": mib, "fetch_scale": round(scale_f, 4), "write_scale": round(scale_w, 4),
           "traffic_bytes_per_launch": round(traffic_bytes),
           "algorithmic_bytes_per_launch": round(algo),
           "traffic_over_algorithmic": round(traffic_bytes / algo, 4) if algo else None}
    lines = [f"# HBM traffic of the split-KV kernel: {workload}", "",
             "Two counter runs of the same bench command (FETCH_SIZE, then WRITE_SIZE, KiB per",
             "dispatch summed over the L2 channels), each scaled by what the counter reads for the",
             f"calibration kernel (neg over {mib} MiB of fp32: {mib} MiB read, {mib} MiB written).",
             "bench.py reports traffic_bytes_per_launch as roofline.traffic while the split",
             "kernel's sources (" + ", ".join(DIGEST_SOURCES) + "),",
             "comments and whitespace removed, still hash to kernel_source_sha256.", "",
             "Commands:", "", "```"]
    lines += list(commands) + ["```", "", "```json", json.dumps(rec, indent=1), "```", ""]
    open(out_md, "w").write("\n".join(lines))


def parity_classes(record_json, out_md, command):
    """profiles/ summary of the selection ambiguity classes that one GPU test
    session recorded (tests/conftest.py writes the JSON when
    WISE_PARITY_RECORD is set), grouped by workload."""
    rec = json.load(open(record_json))
    tot, groups = rec["totals"], {}
    for r in rec["calls"]:
        key = r["what"].split(" ")[0]
        if r["kind"] == "lse":
            key = "LSE route: " + key
        g = groups.setdefault(key, {"calls": 0, "units": 0, "near_eta": 0, "near_tie": 0, "mismatch": 0,
                                    "max_abs": 0.0})
        g["calls"] += 1
        for k in ("units", "near_eta", "near_tie", "mismatch"):
            g[k] += r[k]
        if r.get("max_abs") is not None:
            g["max_abs"] = max(g["max_abs"], r["max_abs"])
    lines = ["# Selection ambiguity classes: GPU vs the fp64 oracle", "",
             "Every GPU-vs-oracle comparison of one run of the GPU test suite (MI355X),",
             "grouped by workload.  A unit is one (row, head) of a call; `units` counts",
             "every unit compared (all modes).  Class A: a discovery unit whose oracle",
             "running sum lies within 1e-6 of eta at the cut.  Class B: a discovery unit",
             "(not in class A) whose K-th and (K+1)-th masses tie within 1e-6 relative",
             "(the exact-tie tests put every unit here on purpose).  A support mismatch",
             "would be excused only when it is exactly the moved cut (A) or the swapped",
             "tied pair (B); any other difference fails the test.  The LSE route's rows",
             "compare supports, tags and counters only (it writes no output).", "",
             "Command (from the repository root), then this summary:", "", "```", command,
             "python -m block_sparse_paged_split_amd.profile_summary parity-classes "
             "$OUT/parity_classes.json profiles/parity_classes.md --command '...'", "```", "",
             f"Totals: {len(rec['calls'])} calls, {tot['units']} units; class A {tot['near_eta']}, "
             f"class B {tot['near_tie']};",
             f"support mismatches {tot['mismatch']} (moved cut {tot['excused_a']}, tied swap {tot['excused_b']}).",
             "", "| workload | calls | units | class A | class B | mismatches | max abs error |",
             "|---|---|---|---|---|---|---|"]
    for key, g in groups.items():
        lines.append(f"| {key} | {g['calls']} | {g['units']} | {g['near_eta']} | {g['near_tie']} | "
                     f"{g['mismatch']} | {g['max_abs']:.2e} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("kernel-stats")
    a.add_argument("stats_csv")
    a.add_argument("out_md")
    a.add_argument("--command", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("out_md")
    b.add_argument("--workload", required=True)
    b.add_argument("--calibrate-mib", type=int, required=True)
    b.add_argument("--algorithmic-bytes", type=float, required=True)
    b.add_argument("--command", action="append", default=[])
    c = sub.add_parser("parity-classes")
    c.add_argument("record_json")
    c.add_argument("out_md")
    c.add_argument("--command", required=True)
    args = ap.parse_args()
    if args.what == "parity-classes":
        parity_classes(args.record_json, args.out_md, args.command)
    elif args.what == "kernel-stats":
        kernel_stats(args.stats_csv, args.out_md, args.command)
    else:
        traffic(args.fetch_csv, args.write_csv, args.out_md, args.workload, args.calibrate_mib,
                args.algorithmic_bytes, args.command)


if __name__ == "__main__":
    main()
