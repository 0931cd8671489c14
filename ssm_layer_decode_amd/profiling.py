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

``suite``: markdown tables of the JSON lines of ``bench.py --suite ...``.

``counters``: mean of each counter of a kernel over its dispatches in one
or more ``--pmc`` runs, split into non-flush and flush steps by the window
position of each dispatch (a layer that starts empty).
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


def counter_summary(paths, kernel, window, first_position=0):
    """Mean of every counter over a kernel's dispatches in rocprofv3
    counter-collection CSVs (one pass per file), split by window position: a
    decode layer that starts empty is at position (first_position + i) mod L
    at its i-th dispatch, and position L - 1 is the flush step.  Returns
    {counter: (non-flush mean, flush mean)} and the dispatch resources
    (VGPR, accumulation VGPR, SGPR, LDS bytes) of the kernel."""
    out, res = {}, {}
    for path in paths:
        per = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if kernel not in r.get("Kernel_Name", ""):
                    continue
                per.setdefault(r["Counter_Name"], []).append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
                for k in ("VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "LDS_Block_Size", "Scratch_Size"):
                    if k in r:
                        res[k] = r[k]
        for name, vals in per.items():
            vals.sort()
            nf = [v for i, (_, v) in enumerate(vals) if (first_position + i) % window != window - 1]
            fl = [v for i, (_, v) in enumerate(vals) if (first_position + i) % window == window - 1]
            mean = lambda x: sum(x) / len(x) if x else float("nan")
            out[name] = (mean(nf), mean(fl))
    if not out:
        raise SystemExit(f"no dispatch of {kernel}")
    return out, res


def counter_table(paths, kernel, window, first_position=0) -> str:
    c, res = counter_summary(paths, kernel, window, first_position)
    lines = [f"Dispatch resources: " + ", ".join(f"{k} {v}" for k, v in res.items()), "",
             "| counter | non-flush dispatches (mean) | flush dispatches (mean) |", "|---|---|---|"]
    lines += [f"| {k} | {a:.6g} | {b:.6g} |" for k, (a, b) in sorted(c.items())]
    return "\n".join(lines)


def stats_table(path, top=8):
    with open(path) as f:
        rows = list(csv.DictReader(f))
    out = ["| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        out.append(f"| {r['Name'][:72]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    return "\n".join(out)


def _f(x, nd=1):
    return f"{x:.{nd}f}" if isinstance(x, float) else str(x)


def suite_markdown(jsonl_path) -> str:
    """Markdown tables of a ``bench.py --suite ...`` run (one JSON line per
    measurement)."""
    rows = [json.loads(l) for l in open(jsonl_path) if l.startswith("{")]
    by = {}
    for r in rows:
        by.setdefault(r["suite"], []).append(r)
    out = []
    if "decode" in by:
        out += ["## Decode at other shapes (ReplaySSM vs conventional fused decode, same inputs)", "",
                "| case | workload | tokens/s | algorithmic GB/s | us/step | conventional tokens/s | conventional GB/s | speedup |",
                "|---|---|---|---|---|---|---|---|"]
        out += [f"| {r['case']} | {r['workload']} | {r['tokens_per_s']:.3e} | {r['GBps']:.0f} | {r['us_per_step']:.1f} | "
                f"{r['conventional_tokens_per_s']:.3e} | {r['conventional_GBps']:.0f} | {r['speedup']:.2f}x |" for r in by["decode"]]
        out.append("")
    if "window" in by:
        out += ["## Window sweep (Mamba-2 serving shape, B = 256; a key per head, or keys shared by groups of heads)", "",
                "| key heads | L | tokens/s | algorithmic GB/s | us/step | algorithmic MB per token |", "|---|---|---|---|---|---|"]
        out += [f"| {r.get('key_heads', 128)} | {r['L']} | {r['tokens_per_s']:.3e} | {r['GBps']:.0f} | {r['us_per_step']:.1f} | "
                + (f"{r['bytes_per_token'] / 1e6:.3f} |" if "bytes_per_token" in r else "-- |") for r in by["window"]]
        out.append("")
    if "batch" in by:
        out += ["## Batch sweep (Mamba-2 shape; independent layers rotated so every checkpoint read is cache-cold)", "",
                "| B | layers rotated | tokens/s (one layer) | GB/s | us per layer-step | conventional us | speedup |",
                "|---|---|---|---|---|---|---|"]
        out += [f"| {r['B']} | {r['layers_rotated']} | {r['tokens_per_s']:.3e} | {r['GBps']:.0f} | {r['us_per_layer_step']:.1f} | "
                f"{r['conventional_us_per_layer_step']:.1f} | {r['speedup']:.2f}x |" for r in by["batch"]]
        out.append("")
    if "spec" in by:
        out += ["## Speculative verify + commit, Mamba-2 shape, B = 512 (accepted length uniform in 0..T)", "",
                "| T | ReplaySSM us/round | snapshot us/round | speedup | ReplaySSM verify-only / conventional decode step | "
                "snapshot round / conventional decode step | ReplaySSM verified tokens/s | snapshot verified tokens/s |",
                "|---|---|---|---|---|---|---|---|"]
        out += [f"| {r['T']} | {r['replay_us_per_round']:.0f} | {r['snapshot_us_per_round']:.0f} | {r['speedup']:.2f}x | "
                f"{r['replay_verify_over_conv_decode_step']:.2f} | {r['snapshot_round_over_conv_decode_step']:.2f} | "
                f"{r['replay_verified_tokens_per_s']:.3e} | {r['snapshot_verified_tokens_per_s']:.3e} |" for r in by["spec"]]
        r0 = by["spec"][0]
        out += ["", f"Conventional decode step at B = 512: {r0['conv_decode_step_us']:.0f} us; ReplaySSM decode step: "
                    f"{r0['replay_decode_step_us']:.0f} us.", ""]
    if "graph" in by:
        out += ["## Small batches: decode launched one by one vs replayed from a captured HIP graph (Mamba-2 shape)", "",
                "| B | layers rotated | eager us per layer-step | graph us per layer-step |", "|---|---|---|---|"]
        out += [f"| {r['B']} | {r['layers']} | {r['eager_us_per_layer_step']:.1f} | {r['graph_us_per_layer_step']:.1f} |"
                for r in by["graph"]]
        out.append("")
    if "ceiling" in by:
        out += ["## Read ceiling against the write share (chunked-read probe, 2 GiB, 32 KiB per workgroup)", "",
                "| bytes written per 32 KiB read | write share of traffic | read GB/s | read + write GB/s |",
                "|---|---|---|---|"]
        out += [f"| {r['write_bytes_per_32KiB']} | {100 * r['write_share']:.1f} % | {r['read_GBps']:.0f} | "
                f"{r['total_GBps']:.0f} |" for r in by["ceiling"]]
        out.append("")
    if "verify_h7" in by:
        out += ["## Verify alone, every sequence at h = 7 (B = 512, Mamba-2 shape, fp32)", "",
                "| T | us per launch | algorithmic GB per launch | algorithmic GB/s |", "|---|---|---|---|"]
        out += [f"| {r['T']} | {r['verify_us']:.1f} | {r['algorithmic_bytes_per_launch']/1e9:.3f} | {r['GBps']:.0f} |"
                for r in by["verify_h7"]]
        out.append("")
    if "spec_copies" in by:
        out += ["## Speculative verify + commit reading a copy or an fp16 checkpoint (B = 512, Mamba-2 shape)", "",
                "| checkpoint | read copy | T | heads per tile | us per round (verify + commit) | verify-only us | verified tokens/s |",
                "|---|---|---|---|---|---|---|"]
        out += [f"| {r['ckpt']} | {r['read_copy']} | {r['T']} | {r['heads_per_tile']} | {r['us_per_round']:.0f} | "
                f"{r['verify_only_us']:.0f} | {r['verified_tokens_per_s']:.3e} |" for r in by["spec_copies"]]
        out.append("")
    if "read_copy" in by:
        out += ["## Read copies and the fp16 checkpoint (window-averaged decode step)", "",
                "| case | checkpoint | read copy | layers rotated | tokens/s | algorithmic GB/s | us per layer-step |",
                "|---|---|---|---|---|---|---|"]
        out += [f"| {r['case']} | {r.get('ckpt', 'f32')} | {r['read_copy']} | {r['layers_rotated']} | {r['tokens_per_s']:.3e} | "
                f"{r['GBps']:.0f} | {r['us_per_layer_step']:.1f} |" for r in by["read_copy"]]
        out.append("")
    if "prefill" in by:
        out += ["## Prefill of a prompt from an empty state vs decoding it token by token", "",
                "| case | T | kernel | prefill ms | prefill tokens/s | decode tokens/s | speedup | algorithmic GB/s | TFLOP/s | peak |",
                "|---|---|---|---|---|---|---|---|---|---|"]
        out += [f"| {r['case']} | {r['T']} | {r.get('kernel', 'rssm_prefill_kernel')} | {r['prefill_ms']:.2f} | "
                f"{r['prefill_tokens_per_s']:.3e} | {r['decode_tokens_per_s']:.3e} | "
                f"{r['speedup_vs_decode']:.2f}x | {r['algorithmic_GBps']:.0f} | {r['TFLOPs']:.1f} | "
                f"{r.get('TFLOPs_peak', r.get('TFLOPs_peak_fp32_valu'))} ({r.get('peak_of', 'fp32 VALU')}) |" for r in by["prefill"]]
        out.append("")
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
    u = sub.add_parser("suite")
    u.add_argument("jsonl")
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--kernel", default="rssm_decode_kernel")
    c.add_argument("--window", type=int, default=16)
    c.add_argument("--first-position", type=int, default=0)
    a = ap.parse_args(argv)
    if a.cmd == "counters":
        print(counter_table(a.csv, a.kernel, a.window, a.first_position))
        return 0
    if a.cmd == "suite":
        print(suite_markdown(a.jsonl))
        return 0
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
