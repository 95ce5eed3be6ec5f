"""Turns rocprofv3 output of a bench.py run into the short text summaries kept
under profiles/.

  python -m verified_sparse_attention_amd.profile_summary stats \
      --trace DIR --workload NAME --cmd "rocprofv3 ... -- python3 bench.py" --out FILE.txt
      kernel-trace statistics (rocprofv3 --kernel-trace --stats --output-format csv):
      calls, mean / min / max duration per kernel.

  python -m verified_sparse_attention_amd.profile_summary traffic \
      --fetch CSV --write CSV --workload NAME --cmd-fetch "..." --cmd-write "..." --out FILE.json
      HBM bytes per dispatch from two counter runs (FETCH_SIZE, then WRITE_SIZE,
      both in KiB per dispatch).  Each counter is scaled by what it reads for the
      plain device copy that `bench.py --profile` makes just before its decode
      steps (a copy of a known size reads and writes that many bytes), so the
      result is in bytes regardless of how the counter aggregates its channels.

The traffic file carries the digest of the kernel sources it was taken with;
bench.py reports `traffic` only while that digest matches the current sources.
"""
import argparse
import collections
import csv
import glob
import json
import os
import subprocess
import sys

from . import build as _build

# must match the calibration copy in bench.py --profile
CALIBRATION_BYTES = 256 << 20
STAGE_KERNELS = ("k_predict", "k_premerge", "k_select", "k_base", "k_budget", "k_numstat", "k_order", "k_gather", "k_combine", "k_emit",
                 "k_project")


def _demangle(name):
    try:
        out = subprocess.run(["c++filt", name], capture_output=True, text=True, check=True).stdout
        return out.strip()
    except (OSError, subprocess.CalledProcessError):
        return name


def _short(name):
    dm = _demangle(name)
    for k in STAGE_KERNELS:
        if "vattn::%s" % k in dm or "vattn::%s<" % k in dm:
            tmpl = dm.split("vattn::%s" % k, 1)[1]
            tmpl = tmpl.split("(", 1)[0]
            return k + tmpl
    return dm[:60]


def _stage(name):
    dm = _demangle(name)
    for k in STAGE_KERNELS:
        if "vattn::%s" % k in dm:
            return k
    return None


def _find(pattern):
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit("no file matches %s" % pattern)
    return hits[0]


def _grid_rows(trace_dir):
    """Per (decode-step kernel, step kind) statistics from the kernel trace.
    Dispatches are taken in order and cut into decode steps at each k_predict;
    a step's kind is its k_predict's instance and grid, plus "+numerator" when
    the step runs the output-level mode's kernels.  One kind is one workload
    launch, so the headline workload's select, budget and combine are told from
    another workload's with the same number of heads."""
    path = _find(os.path.join(trace_dir, "**", "*kernel_trace.csv"))
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    steps, cur = [], None
    for r in rows:
        st = _stage(r["Kernel_Name"])
        if st is None or st == "k_project":
            continue
        grid = tuple(int(r["Grid_Size_%s" % a]) // max(int(r["Workgroup_Size_%s" % a]), 1) for a in "XYZ")
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if st == "k_predict" or cur is None:
            cur = []
            steps.append(cur)
        cur.append((_short(r["Kernel_Name"]), grid, dur))
    acc = collections.OrderedDict()
    for step in steps:
        head = step[0]
        tag = "%s %s" % (head[0], head[1]) if head[0].startswith("k_predict") else "(no predict)"
        if any(n.startswith("k_numstat") for n, _, _ in step):
            tag += " +numerator"
        for name, grid, dur in step:
            acc.setdefault((name, grid, tag), []).append(dur)
    return acc


def stats(args):
    path = _find(os.path.join(args.trace, "**", "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(path)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = ["# rocprofv3 kernel-trace statistics, workload %s" % args.workload,
             "# command: %s" % args.cmd,
             "# kernel sources digest: %s" % _build.source_hash(),
             "# durations in microseconds; every dispatch of the run is counted "
             "(warm-up, timed, per-stage-timed and rate-check steps of every workload)",
             "%-40s %7s %10s %10s %10s %7s" % ("kernel", "calls", "mean_us", "min_us", "max_us", "share")]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append("%-40s %7d %10.2f %10.2f %10.2f %6.1f%%" % (
            _short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            100.0 * float(r["TotalDurationNs"]) / total))
    try:
        grid = _grid_rows(args.trace)
    except SystemExit:
        grid = {}
    if grid:
        lines += ["", "# decode-step kernels by step kind: grid in workgroups; step = the k_predict instance and grid "
                      "that opened the dispatch's decode step (+numerator: output-level mode); the headline "
                      "workload's steps are marked *",
                  "%-34s %-16s %-52s %7s %9s %9s %9s" % ("kernel", "grid", "step", "calls", "mean_us",
                                                        "median_us", "max_us")]
        for (name, g, tag), d in sorted(grid.items(), key=lambda kv: (str(kv[0][2]), kv[0][0])):
            d = sorted(d)
            star = "*" if args.headline_step and tag == args.headline_step else " "
            lines.append("%-34s %-16s %-52s %7d %9.2f %9.2f %9.2f %s" % (
                name, str(g), str(tag), len(d), sum(d) / len(d), d[len(d) // 2], d[-1], star))
    text = "\n".join(lines) + "\n"
    with open(args.out, "w") as f:
        f.write(text)
    sys.stdout.write(text)


def _per_dispatch(path, counter):
    """{dispatch id: (kernel name, summed counter value)} in dispatch order."""
    acc = collections.OrderedDict()
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        name, v = acc.get(d, (r["Kernel_Name"], 0.0))
        acc[d] = (name, v + float(r["Counter_Value"]))
    return acc


def _calibration(disp):
    """The copy just before the first decode-step kernel of the run."""
    first = min((d for d, (n, _) in disp.items() if _stage(n) == "k_predict"), default=None)
    if first is None:
        raise SystemExit("no k_predict dispatch in the counter file")
    cands = [d for d, (n, _) in disp.items() if "copyBuffer" in n and d < first]
    if not cands:
        raise SystemExit("no calibration copy before the first decode step")
    return disp[max(cands)][1]


def traffic(args):
    fetch = _per_dispatch(args.fetch, "FETCH_SIZE")
    write = _per_dispatch(args.write, "WRITE_SIZE")
    cal_f, cal_w = _calibration(fetch), _calibration(write)
    kib = CALIBRATION_BYTES / 1024.0
    f_scale, w_scale = kib / cal_f, kib / cal_w
    out = {"workload": args.workload, "source_hash": _build.source_hash(),
           "commands": {"fetch": args.cmd_fetch, "write": args.cmd_write},
           "calibration": {"copy_bytes": CALIBRATION_BYTES, "fetch_kib": round(cal_f, 2),
                           "write_kib": round(cal_w, 2), "fetch_scale": round(f_scale, 4),
                           "write_scale": round(w_scale, 4)},
           "kernels": {}}
    for stage in STAGE_KERNELS:
        fs = [v for n, v in fetch.values() if _stage(n) == stage]
        ws = [v for n, v in write.values() if _stage(n) == stage]
        if not fs or not ws:
            continue
        fk, wk = sum(fs) / len(fs), sum(ws) / len(ws)
        out["kernels"][stage] = {
            "dispatches": [len(fs), len(ws)],
            "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
            "hbm_bytes_per_launch": round(fk * 1024 * f_scale + wk * 1024 * w_scale)}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    a = sub.add_parser("stats")
    a.add_argument("--trace", required=True)
    a.add_argument("--workload", required=True)
    a.add_argument("--cmd", required=True)
    a.add_argument("--out", required=True)
    a.add_argument("--headline-step", default=None,
                   help="the headline workload's step kind, e.g. 'k_predict<32, unsigned short, 4> (4, 64, 1)'")
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--workload", required=True)
    b.add_argument("--cmd-fetch", required=True)
    b.add_argument("--cmd-write", required=True)
    b.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    (stats if args.mode == "stats" else traffic)(args)


if __name__ == "__main__":
    main()
