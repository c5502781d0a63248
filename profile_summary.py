"""Turns rocprofv3 output of bench.py runs into the short summaries kept in profiles/.

    # kernel-trace statistics -> profiles/<name>.txt
    python3 profile_summary.py trace --dir <rocprofv3 -d dir> --out profiles/<name>.txt \\
        --workload <workload> --command "<the rocprofv3 command line>" [--bench-json <bench output>]

    # two counter runs (FETCH_SIZE, then WRITE_SIZE) -> profiles/traffic.json entry + text
    python3 profile_summary.py traffic --fetch-dir <dir> --write-dir <dir> --workload <workload> \\
        --kernel <substring of the kernel's name> --out profiles/<name>.txt --command "<command lines>" \\
        [--kernels-per-call K]      # a call that launches K kernels matching the substring (the backward: 5)

The counters are scaled by what they read for the calibration copy bench.py runs
(ssm_calib_copy: 1 GiB read and 1 GiB written per dispatch), so HBM bytes per launch
= counter per dispatch x (known bytes / counter per calibration dispatch).  The
traffic entry records the hash of the kernel's sources (bench.src_hash); bench.py
reports it only while the sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CALIB_KERNEL = "calib_copy_kernel"
CALIB_BYTES = 1 << 30


def _csvs(d, suffix):
    found = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not found:
        raise SystemExit(f"no *{suffix} under {d}")
    return found


def _short(name):
    return name.replace("(anonymous namespace)::", "").replace("ssm::", "ssm::")


def trace(args):
    rows = []
    for path in _csvs(args.dir, "kernel_stats.csv"):
        with open(path) as f:
            rows += list(csv.DictReader(f))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"# rocprofv3 kernel trace: {args.workload}", "", "Command (MI355X, one GPU):", f"    {args.command}", ""]
    if args.bench_json:
        with open(args.bench_json) as f:
            b = json.loads([ln for ln in f if ln.startswith("{")][-1])
        lines += [f"Workload: {json.dumps(b['config'])}", "",
                  f"bench.py, same run: {b['roofline']['avg_launch_us']:.2f} us per call (HIP events around "
                  f"{b['steps']} graph-replayed calls), HBM {b['hbm']['achieved']:.0f} GB/s = "
                  f"{b['hbm']['frac']:.4f} of 8 TB/s; median {b['timing']['us_median']:.2f} us "
                  f"(p10 {b['timing']['us_p10']:.2f}, p90 {b['timing']['us_p90']:.2f}) over "
                  f"{b['timing']['iterations']} replays.", ""]
    lines += ["| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{100 * float(r['TotalDurationNs']) / total:.1f} |")
    lines.append("")
    lines.append("(calib_copy_kernel / calib_alu_kernel: bench.py's calibration probes; __amd_rocclr_*: uploads "
                 "and fills outside the timed region.)")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_rows(d):
    rows = []
    for path in _csvs(d, "counter_collection.csv"):
        with open(path) as f:
            rows += list(csv.DictReader(f))
    return rows


def _short_name(name):
    for key in ("bwd_summary_tokseq_kernel", "bwd_summary_kernel", "bwd_combine_kernel", "bwd_main_kernel",
                "bwd_param_sums_kernel", "bwd_bc_out_kernel"):
        if key in name:
            return key
    return _short(name.split("(")[0])


def _per_dispatch(rows, counter, match):
    """Per-dispatch totals of `counter` for kernels whose name contains `match`."""
    tot = {}
    for r in rows:
        if r.get("Counter_Name") != counter or match not in r.get("Kernel_Name", ""):
            continue
        key = (r.get("Dispatch_Id"), r.get("Kernel_Name"))
        tot[key] = tot.get(key, 0.0) + float(r["Counter_Value"])
    return tot


def traffic(args):
    sys.path.insert(0, ROOT)
    import bench
    out = {}
    for counter, d in (("FETCH_SIZE", args.fetch_dir), ("WRITE_SIZE", args.write_dir)):
        rows = _counter_rows(d)
        cal = _per_dispatch(rows, counter, CALIB_KERNEL)
        ker = _per_dispatch(rows, counter, args.kernel)
        if not cal or not ker:
            raise SystemExit(f"{counter}: no dispatches of {CALIB_KERNEL} or {args.kernel}")
        cal_kib = sorted(cal.values())[len(cal) // 2]                # median calibration dispatch
        scale = CALIB_BYTES / (cal_kib * 1024.0)
        vals = list(ker.values())
        calls = len(vals) / args.kernels_per_call
        per_kernel = {}
        for (_, name), v in ker.items():
            per_kernel.setdefault(_short_name(name), []).append(v)
        out[counter] = {"kib_per_dispatch": sum(vals) / calls, "dispatches": len(vals),
                        "calib_kib_per_dispatch": cal_kib, "scale": scale,
                        "kernels": sorted({k[1] for k in ker}),
                        "per_kernel_kib": {k: sum(v) / len(v) for k, v in per_kernel.items()}}
    fetch_b = out["FETCH_SIZE"]["kib_per_dispatch"] * 1024 * out["FETCH_SIZE"]["scale"]
    write_b = out["WRITE_SIZE"]["kib_per_dispatch"] * 1024 * out["WRITE_SIZE"]["scale"]
    import synth
    cfg = synth.CONFIGS[args.workload]
    alg = cfg.algorithmic_bytes() if hasattr(cfg, "algorithmic_bytes") else cfg.algorithmic_bytes_per_step()
    kernel = bench.kernel_of(cfg, bench.kind_of(args.workload)) if args.hash_kernel is None else args.hash_kernel
    entry = {"source_hash": bench.src_hash(kernel), "hbm_bytes_per_launch": fetch_b + write_b,
             "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
             "fetch_scale": out["FETCH_SIZE"]["scale"], "write_scale": out["WRITE_SIZE"]["scale"],
             "algorithmic_bytes": alg, "kernels": out["FETCH_SIZE"]["kernels"]}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data[args.workload] = entry
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    lines = [f"# rocprofv3 HBM counters: {args.workload}", "", "Commands (MI355X, one GPU):"]
    lines += [f"    {c}" for c in args.command.split(" ;; ")]
    lines += ["", "| counter | KiB per call | dispatches | calibration copy KiB per dispatch (1 GiB moved) | "
              "scale | bytes per call |", "|---|---|---|---|---|---|"]
    for counter, b in (("FETCH_SIZE", fetch_b), ("WRITE_SIZE", write_b)):
        o = out[counter]
        lines.append(f"| {counter} | {o['kib_per_dispatch']:.0f} | {o['dispatches']} | {o['calib_kib_per_dispatch']:.0f} | "
                     f"{o['scale']:.4f} | {b / 1e6:.2f} MB |")
    if args.kernels_per_call > 1:
        lines += ["", "| kernel | read MB (scaled) | written MB (scaled) |", "|---|---|---|"]
        for k in out["FETCH_SIZE"]["per_kernel_kib"]:
            rd = out["FETCH_SIZE"]["per_kernel_kib"][k] * 1024 * out["FETCH_SIZE"]["scale"] / 1e6
            wr = out["WRITE_SIZE"]["per_kernel_kib"].get(k, 0.0) * 1024 * out["WRITE_SIZE"]["scale"] / 1e6
            lines.append(f"| {k} | {rd:.2f} | {wr:.2f} |")
    lines += ["", f"HBM traffic per call: {(fetch_b + write_b) / 1e6:.2f} MB against {alg / 1e6:.2f} MB "
                  f"algorithmic ({(fetch_b + write_b) / alg:.3f}x).", f"Kernels: {', '.join(entry['kernels'])}"]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--dir", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--bench-json")
    c = sub.add_parser("traffic")
    c.add_argument("--fetch-dir", required=True)
    c.add_argument("--write-dir", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--kernel", required=True, help="substring of the kernel's name in the counter CSV")
    c.add_argument("--hash-kernel", default=None, help="bench.KERNEL_SRC key for the source hash (default: the "
                                                        "kernel bench.py reports for the workload)")
    c.add_argument("--out", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--kernels-per-call", type=int, default=1)
    a = ap.parse_args()
    trace(a) if a.cmd == "trace" else traffic(a)


if __name__ == "__main__":
    main()
