"""Turn rocprofv3 outputs into the committed profile summaries.

Inputs (CSV files that rocprofv3 writes into its -d directory):
  --trace-stats  <..._kernel_stats.csv>       from  --kernel-trace --stats
  --fetch        <..._counter_collection.csv> from  --pmc FETCH_SIZE
  --write        <..._counter_collection.csv> from  --pmc WRITE_SIZE

Counters are calibrated against the plain device-to-device copy that bench.py
runs (``__amd_rocclr_copyBuffer`` of the whole history, a known number of
bytes read and written): each counter is scaled by known_bytes / counter
reading of that copy.  The HBM traffic of the kernel is then reported per
launch, next to its algorithmic bytes.

Outputs: profiles/<name>.md (human summary, with the commands) and
profiles/<name>_traffic.json (the record bench.py reads; it carries a hash of
the kernel sources so bench.py drops it once the kernel changes).
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def main():
    import bench

    ap = argparse.ArgumentParser()
    ap.add_argument("--trace-stats", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--stats-only", metavar="TITLE",
                    help="write profiles/<name>.md with the kernel-trace table only")
    ap.add_argument("--kernel-summary", metavar="TITLE",
                    help="write profiles/<name>.md for the kernels matching --kernel of a "
                         "bench.py --profile run: trace, HBM counters per dispatch, SQ counters")
    ap.add_argument("--copy-bytes", type=float, help="bytes read (= written) by the calibration copy")
    ap.add_argument("--alg-bytes", type=float, help="algorithmic bytes of one run of the workload")
    ap.add_argument("--alg-flops", type=float, help="algorithmic FLOPs of one run (matrix-core kernels)")
    ap.add_argument("--flops-peak", type=float, default=2500.0, help="dense peak in TFLOP/s for --alg-flops")
    ap.add_argument("--sq", nargs="*", default=[], help="counter CSVs of SQ passes")
    ap.add_argument("--name", default="full_fwd_stream_L32_d896")
    ap.add_argument("--kernel", default="full_fwd_stream_kernel")
    ap.add_argument("--commands", default="", help="text of the commands that made the CSVs")
    args = ap.parse_args()
    if args.stats_only:
        return stats_only(args)
    if args.kernel_summary:
        return kernel_summary(args)
    if not (args.fetch and args.write):
        raise SystemExit("--fetch and --write are required (or use --stats-only)")

    from depth_wise_attention_attnres_amd.workloads import WORKLOADS
    wl = WORKLOADS[bench.WORKLOAD]
    n, T, d = wl.n_hist, wl.T, wl.d
    copy_bytes = n * T * d * 2  # the history copy bench.py runs: bytes read == bytes written

    def counter(path):
        rs = rows(path)
        cp = [float(r["Counter_Value"]) * 1024 for r in rs if "copyBuffer" in r["Kernel_Name"]]
        k = [float(r["Counter_Value"]) * 1024 for r in rs if args.kernel in r["Kernel_Name"]]
        if not cp or len(k) < n:
            raise SystemExit(f"{path}: missing copy or kernel dispatches")
        factor = copy_bytes / (sum(cp) / len(cp))
        return factor, [v * factor for v in k[-n:]]  # the last full sweep, read l = 0..n-1

    f_fac, fetch = counter(args.fetch)
    w_fac, write = counter(args.write)
    alg_r = [((l + 1) * 2 * d + 4 * l) * T for l in range(n)]
    alg_w = [(2 * d + 4 + 4) * T for l in range(n)]
    per_launch = [a + b for a, b in zip(fetch, write)]
    mean_traffic = sum(per_launch) / n
    mean_alg = sum(bench.read_bytes_per_token(l, d) * T for l in range(n)) / n

    stats = [r for r in rows(args.trace_stats) if args.kernel in r["Name"]]
    if not stats:
        raise SystemExit("kernel not in trace stats")
    st = stats[0]

    rec = {
        "kernel": st["Name"],
        "workload": bench.WORKLOAD,
        "kernel_source_hash": bench.kernel_source_hash(),
        "bytes_per_launch": mean_traffic,
        "algorithmic_bytes_per_launch": mean_alg,
        "fetch_scale": f_fac,
        "write_scale": w_fac,
        "fetch_over_algorithmic": sum(fetch) / sum(alg_r),
        "write_over_algorithmic": sum(write) / sum(alg_w),
        "trace_calls": int(st["Calls"]),
        "trace_average_ns": float(st["AverageNs"]),
    }
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"{args.name}_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)

    gbs = mean_alg / (float(st["AverageNs"]) * 1e-9) / 1e9
    lines = [
        f"# {args.name}: Full AttnRes forward, read by read, L=32 / d=896 / 16384 tokens, bf16",
        "",
        "Commands (run from /tmp with TMPDIR=/tmp on the machine that holds the GPU; $R = the repo root):",
        "",
        "```",
        args.commands.strip() or "(commands not given)",
        "```",
        "",
        "## rocprofv3 --kernel-trace --stats",
        "",
        "| kernel | calls | average ns | min ns | max ns | share |",
        "|---|---|---|---|---|---|",
    ]
    for r in rows(args.trace_stats)[:4]:
        name = r["Name"] if len(r["Name"]) < 90 else r["Name"][:87] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                     f"{r['MaxNs']} | {r['Percentage']}% |")
    lines += [
        "",
        f"Mean algorithmic bytes per launch (65 reads, l = 0..64): {mean_alg / 1e6:.1f} MB; "
        f"over the trace average duration: **{gbs:.0f} GB/s = {gbs / 8000 * 100:.1f}% of 8 TB/s**.",
        "",
        "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)",
        "",
        f"Calibration on the plain copy of the history ({copy_bytes / 1e9:.3f} GB read and written, "
        f"`__amd_rocclr_copyBuffer`): FETCH_SIZE x {f_fac:.3f}, WRITE_SIZE x {w_fac:.3f}.",
        "",
        "| read l | fetched MB | algorithmic read MB | written MB | algorithmic write MB |",
        "|---|---|---|---|---|",
    ]
    for l in [0, 1, 8, 16, 32, 48, 64]:
        lines.append(f"| {l} | {fetch[l] / 1e6:.1f} | {alg_r[l] / 1e6:.1f} | {write[l] / 1e6:.1f} | "
                     f"{alg_w[l] / 1e6:.1f} |")
    lines += [
        "",
        f"Over the sweep: fetched / algorithmic = {rec['fetch_over_algorithmic']:.4f}, "
        f"written / algorithmic = {rec['write_over_algorithmic']:.4f}; "
        f"mean HBM traffic per launch {mean_traffic / 1e6:.1f} MB vs {mean_alg / 1e6:.1f} MB "
        "algorithmic.",
        "",
        f"Kernel source hash at measurement: `{rec['kernel_source_hash']}`.",
    ]
    with open(os.path.join(ROOT, "profiles", f"{args.name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(rec, indent=1))


def kernel_summary(args):
    """Trace, HBM traffic and SQ counters of the kernels (matching --kernel) of
    one run of a workload; counters are scaled by the calibration copy."""
    def sel(path):
        return [r for r in rows(path) if any(k in r["Kernel_Name"] for k in args.kernel.split(","))]

    def per_dispatch(path):
        rs = rows(path)
        cp = [float(r["Counter_Value"]) * 1024 for r in rs if "copyBuffer" in r["Kernel_Name"]
              or "copy" in r["Kernel_Name"].lower() and "attnres" not in r["Kernel_Name"]]
        if not cp:
            raise SystemExit(f"{path}: no calibration copy dispatch")
        factor = args.copy_bytes / max(cp)
        by = {}
        for r in sel(path):
            by.setdefault(int(r["Dispatch_Id"]), 0.0)
            by[int(r["Dispatch_Id"])] += float(r["Counter_Value"]) * 1024 * factor
        ids = sorted(by)
        half = ids[len(ids) // 2:]  # the second of the two runs
        return factor, sum(by[i] for i in half)

    f_fac, fetched = per_dispatch(args.fetch)
    w_fac, written = per_dispatch(args.write)
    st = [r for r in rows(args.trace_stats) if any(k in r["Name"] for k in args.kernel.split(","))]
    total_ns = sum(float(r["TotalDurationNs"]) for r in st) / 2  # per run (two runs)
    lines = [f"# {args.name}: {args.kernel_summary}", "",
             "Commands (run from /tmp with TMPDIR=/tmp on the machine that holds the GPU; $R = the repo root):", "",
             "```", args.commands.strip(), "```", "",
             "## rocprofv3 --kernel-trace --stats", "",
             "| kernel | calls | average ns | total ns |", "|---|---|---|---|"]
    for r in st:
        lines.append(f"| `{r['Name'][:100]}` | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                     f"{float(r['TotalDurationNs']):.0f} |")
    gbs = args.alg_bytes / (total_ns * 1e-9) / 1e9
    lines += ["", f"One run: {total_ns / 1e6:.2f} ms of kernel time; algorithmic bytes "
              f"{args.alg_bytes / 1e9:.2f} GB -> {gbs:.0f} GB/s = {gbs / 80:.1f}% of 8 TB/s." +
              (f" Algorithmic FLOPs {args.alg_flops / 1e12:.3f} T -> "
               f"{args.alg_flops / (total_ns * 1e-9) / 1e12:.0f} TFLOP/s = "
               f"{100 * args.alg_flops / (total_ns * 1e-9) / 1e12 / args.flops_peak:.1f}% of the "
               f"{args.flops_peak:.0f} TFLOP/s dense peak." if args.alg_flops else ""), "",
              "## HBM traffic of one run (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)", "",
              f"Calibration on the history copy ({args.copy_bytes / 1e9:.2f} GB read and written): "
              f"FETCH_SIZE x {f_fac:.3f}, WRITE_SIZE x {w_fac:.3f}.", "",
              f"Fetched {fetched / 1e9:.2f} GB, written {written / 1e9:.2f} GB, together "
              f"{(fetched + written) / args.alg_bytes:.3f} x the algorithmic bytes."]
    if args.sq:
        agg = {}
        waves = 0.0
        for path in args.sq:
            for r in sel(path):
                agg[r["Counter_Name"]] = agg.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        waves = agg.get("SQ_WAVES", 0.0)
        lines += ["", "## SQ counters (both runs; per wave where it applies)", "",
                  "| counter | total | per wave |", "|---|---|---|"]
        for k in sorted(agg):
            lines.append(f"| {k} | {agg[k]:.4g} | {agg[k] / waves if waves else 0:.1f} |")
    with open(os.path.join(ROOT, "profiles", f"{args.name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stats_only(args):
    """Kernel-trace summary of every kernel in a run (no counters)."""
    lines = [
        f"# {args.name}: {args.stats_only}",
        "",
        "Commands (run from /tmp with TMPDIR=/tmp on the machine that holds the GPU; $R = the repo root):",
        "",
        "```",
        args.commands.strip(),
        "```",
        "",
        "## rocprofv3 --kernel-trace --stats",
        "",
        "| kernel | calls | average ns | min ns | max ns | share |",
        "|---|---|---|---|---|---|",
    ]
    for r in rows(args.trace_stats):
        name = r["Name"] if len(r["Name"]) < 110 else r["Name"][:107] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                     f"{r['MaxNs']} | {r['Percentage']}% |")
    with open(os.path.join(ROOT, "profiles", f"{args.name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
