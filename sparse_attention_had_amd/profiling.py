"""Turn rocprofv3 CSV output into the short summaries kept under profiles/.

    python -m sparse_attention_had_amd.profiling stats  <kernel_stats.csv> <out.md> --cmd "..."
    python -m sparse_attention_had_amd.profiling traffic --fetch <fetch csv> --write <write csv> \
        --workload NAME --out profiles/traffic_had_attention_NAME.json --cmd "..."
    python -m sparse_attention_had_amd.profiling counters --csv <pass 1 csv> --cmd "..." \
        [--csv <pass 2 csv> --cmd "..."] --kernel had_attn_kernel --workload NAME --out <out.md>

The traffic run profiles `bench.py --traffic-probe`, which launches the
attention kernel a few times and then one plain device-to-device copy of
COPY_BYTES bytes (read COPY_BYTES, write COPY_BYTES).  FETCH_SIZE and
WRITE_SIZE of the attention kernel are scaled by what the same counters read
for that copy, so the result is in bytes of HBM traffic per launch.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys

COPY_BYTES = 64 << 20
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# The sources the attention kernel is compiled from: a counter record taken on
# them stays valid while they are unchanged.
ATTENTION_SOURCES = ("had_attention.hip", "had_internal.h")


def source_hash(files=ATTENTION_SOURCES) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_attention_had_amd", "csrc")
    for f in sorted(files):
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def _counter_rows(path, counter):
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Dispatch_Id"], r["Kernel_Name"])
        out[key] = out.get(key, 0.0) + float(r["Counter_Value"])
    return out


def _split(rows):
    attn = [v for (d, name), v in rows.items() if "had_attn_kernel" in name]
    copy = [v for (d, name), v in rows.items()
            if "had_" not in name and ("copy" in name.lower() or "elementwise" in name.lower())]
    return attn, copy


def traffic(fetch_csv, write_csv, workload, out, cmd):
    fa, fc = _split(_counter_rows(fetch_csv, "FETCH_SIZE"))
    wa, wc = _split(_counter_rows(write_csv, "WRITE_SIZE"))
    if not fa or not wa or not fc or not wc:
        raise SystemExit("missing attention or copy dispatches in the counter files")
    copy_fetch_kib = max(fc)   # the 64 MiB copy is the largest elementwise dispatch
    copy_write_kib = max(wc)
    f_scale = (COPY_BYTES / 1024.0) / copy_fetch_kib
    w_scale = (COPY_BYTES / 1024.0) / copy_write_kib
    fetch_b = statistics.median(fa) * 1024.0 * f_scale
    write_b = statistics.median(wa) * 1024.0 * w_scale
    rec = {
        "kernel": "had_attn_kernel",
        "workload": workload,
        "source_hash": source_hash(),
        "fetch_bytes_per_launch": fetch_b,
        "write_bytes_per_launch": write_b,
        "bytes_per_launch": fetch_b + write_b,
        "raw_fetch_kib": statistics.median(fa),
        "raw_write_kib": statistics.median(wa),
        "copy_probe_bytes": COPY_BYTES,
        "copy_fetch_kib": copy_fetch_kib,
        "copy_write_kib": copy_write_kib,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "command": cmd,
    }
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def stats(stats_csv, out_md, cmd, title):
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# {title}", "", "Command:", "", "```", cmd, "```", "",
             "| kernel | calls | total ns | average ns | min ns | max ns | % |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "").replace("void ", "")
        short = name.split("(")[0]
        lines.append(f"| `{short}` | {r['Calls']} | {r['TotalDurationNs']} | "
                     f"{float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} | "
                     f"{float(r['Percentage']):.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counters(csvs, cmds, kernel, workload, out_md, sources=ATTENTION_SOURCES):
    """SQ counters of one kernel, one rocprofv3 --pmc pass per CSV: the mean
    over its dispatches of each counter (summed over the counter's instances
    within a dispatch), and that mean divided by SQ_WAVES (waves per dispatch).
    `sources` are the files the kernel is compiled from (their hash heads the
    summary)."""
    means, ndisp = {}, {}
    for path in csvs:
        per = {}
        for r in csv.DictReader(open(path)):
            if kernel not in r["Kernel_Name"]:
                continue
            d = per.setdefault(r["Dispatch_Id"], {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        for name in sorted({c for d in per.values() for c in d}):
            vals = [d[name] for d in per.values() if name in d]
            means[name] = statistics.fmean(vals)
            ndisp[name] = len(vals)
    waves = means.get("SQ_WAVES")
    lines = [f"# SQ counters, `{kernel}`, {workload}", "",
             f"Kernel sources: sha256 prefix `{source_hash(sources)}` of "
             f"{', '.join('`' + f + '`' for f in sources)}.", "",
             "Commands (one counter pass each):", "", "```"] + list(cmds) + ["```", "",
             "| counter | mean per dispatch | per wave | dispatches |", "|---|---|---|---|"]
    for name, v in means.items():
        pw = f"{v / waves:.4g}" if waves else "—"
        lines.append(f"| `{name}` | {v:.6g} | {pw} | {ndisp[name]} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", default="rocprofv3 kernel statistics")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--cmd", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--csv", action="append", required=True)
    c.add_argument("--sources", action="append", default=None,
                   help="source files of the kernel (default: the attention kernel's)")
    c.add_argument("--cmd", action="append", required=True)
    c.add_argument("--kernel", default="had_attn_kernel")
    c.add_argument("--workload", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd_name == "stats":
        stats(a.csv, a.out, a.cmd, a.title)
    elif a.cmd_name == "counters":
        counters(a.csv, a.cmd, a.kernel, a.workload, a.out,
                 tuple(a.sources) if a.sources else ATTENTION_SOURCES)
    else:
        traffic(a.fetch, a.write, a.workload, a.out, a.cmd)


if __name__ == "__main__":
    sys.exit(main())
