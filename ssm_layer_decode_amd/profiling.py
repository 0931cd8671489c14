"""Summaries of rocprofv3 output for the decode kernels.

``traffic``: per-launch HBM bytes of a kernel from two counter runs
(``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``, each reported in KiB per
dispatch).  Each counter is scaled by what it reads for the plain copy probe
``probe_copy_kernel`` of known size in the same run (bytes copied / counter
bytes), which corrects for whatever the counter does not see or double counts.

    python -m ssm_layer_decode_amd.profiling traffic \
        --fetch <dir>/run_counter_collection.csv --write <dir2>/run_counter_collection.csv \
        --kernel rssm_decode_kernel --copy-bytes 2147483648 --out profiles/<name>.json

``stats``: a markdown table of a ``--kernel-trace --stats`` kernel_stats.csv.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import sys


def _counter_rows(path, counter):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"{path}: no {counter} rows")
    return rows


def _mean_for(rows, needle):
    vals = [v for n, v in rows if needle in n]
    if not vals:
        raise SystemExit(f"no dispatch of {needle}")
    return sum(vals) / len(vals), len(vals)


def traffic(fetch_csv, write_csv, kernel, copy_bytes, sha=None, algorithmic=None):
    fr = _counter_rows(fetch_csv, "FETCH_SIZE")
    wr = _counter_rows(write_csv, "WRITE_SIZE")
    cf, _ = _mean_for(fr, "probe_copy_kernel")
    cw, _ = _mean_for(wr, "probe_copy_kernel")
    sf = copy_bytes / (cf * 1024.0)
    sw = copy_bytes / (cw * 1024.0)
    kf, nf = _mean_for(fr, kernel)
    kw, nw = _mean_for(wr, kernel)
    fetch = kf * 1024.0 * sf
    write = kw * 1024.0 * sw
    d = {"kernel": kernel, "dispatches": [nf, nw],
         "fetch_KiB_per_dispatch_raw": kf, "write_KiB_per_dispatch_raw": kw,
         "copy_probe_bytes": copy_bytes, "copy_fetch_KiB_raw": cf, "copy_write_KiB_raw": cw,
         "fetch_scale": sf, "write_scale": sw,
         "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
         "hbm_bytes_per_launch": fetch + write}
    if sha:
        d["kernel_src_sha"] = sha
    if algorithmic:
        d["algorithmic_bytes_per_launch"] = algorithmic
        d["traffic_over_algorithmic"] = (fetch + write) / algorithmic
    return d


def stats_table(path, top=8):
    with open(path) as f:
        rows = list(csv.DictReader(f))
    out = ["| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        out.append(f"| {r['Name'][:72]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", default="rssm_decode_kernel")
    t.add_argument("--copy-bytes", type=int, default=2 << 30)
    t.add_argument("--sha", default=None)
    t.add_argument("--algorithmic", type=float, default=None)
    t.add_argument("--out", default=None)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    a = ap.parse_args(argv)
    if a.cmd == "traffic":
        d = traffic(a.fetch, a.write, a.kernel, a.copy_bytes, a.sha, a.algorithmic)
        txt = json.dumps(d, indent=1)
        if a.out:
            open(a.out, "w").write(txt + "\n")
        print(txt)
    else:
        print(stats_table(a.csv))


if __name__ == "__main__":
    sys.exit(main())
