"""Turn rocprofv3 CSV output into the short text summaries kept in profiles/.

Three kinds of summary:

* ``stats``: the per-kernel table of ``rocprofv3 --kernel-trace --stats``
  (calls, average / min / max duration) for the kernels of one run.
* ``traffic``: HBM bytes per launch of one kernel from two ``--pmc`` runs
  (``FETCH_SIZE``, then ``WRITE_SIZE``, both in KiB per dispatch), each scaled
  by the factor that makes the same counter read the known byte count of a
  plain copy kernel (``bench.py --copy-calibration``).  The summary records a
  hash of the library sources, so that a reader (bench.py) can tell whether
  the kernel has changed since the counters were taken.

Usage (paths are the rocprofv3 output directories' CSV files):

  python -m dense_gemm_mxfp8_amd.profiling stats RUN_kernel_stats.csv OUT.md \\
      --cmd "<the rocprofv3 command>" [--match SUBSTRING]
  python -m dense_gemm_mxfp8_amd.profiling traffic --kernel SUBSTRING \\
      --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv \\
      --copy-bytes N --out OUT.md --cmd "<commands>"
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))


# The sources each kernel family is built from: a counter summary stays valid
# while these files are unchanged.
FAMILIES = {
    "gemm": ["csrc/libgemm.hip", "csrc/gemm_mf16.hip", "csrc/gemm_*.h", "../include/libgemm.h"],
    "attention": ["csrc/attention.hip", "../include/attention.h"],
}


def family_of(workload_or_kernel: str) -> str:
    """Kernel family of a workload or kernel name."""
    return "attention" if "attn" in workload_or_kernel else "gemm"


def source_hash(family: str = "gemm") -> str:
    """sha256 over one kernel family's sources, in a fixed order."""
    h = hashlib.sha256()
    files = []
    for pat in FAMILIES[family]:
        files += sorted(glob.glob(os.path.normpath(os.path.join(PKG, pat))))
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def _counter_rows(path: str, counter: str, match: str):
    out = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter and match in r["Kernel_Name"]:
                out.append(float(r["Counter_Value"]))
    return out


def traffic(args) -> None:
    fetch = _counter_rows(args.fetch, "FETCH_SIZE", args.kernel)
    write = _counter_rows(args.write, "WRITE_SIZE", args.kernel)
    cf = _counter_rows(args.copy_fetch, "FETCH_SIZE", args.copy_kernel)
    cw = _counter_rows(args.copy_write, "WRITE_SIZE", args.copy_kernel)
    if not (fetch and write and cf and cw):
        raise SystemExit("missing counter rows (check --kernel / --copy-kernel)")
    # counters read KiB per dispatch; the copy reads and writes copy_bytes
    f_scale = args.copy_bytes / (sum(cf) / len(cf) * 1024.0)
    w_scale = args.copy_bytes / (sum(cw) / len(cw) * 1024.0)
    fetch_b = sum(fetch) / len(fetch) * 1024.0 * f_scale
    write_b = sum(write) / len(write) * 1024.0 * w_scale
    lines = [
        f"# HBM traffic per launch: {args.title or args.kernel}",
        "",
        f"source_sha256: {source_hash(family_of(args.kernel))}",
        f"source_family: {family_of(args.kernel)}",
        f"kernel_match: {args.kernel}",
        f"dispatches: fetch {len(fetch)}, write {len(write)}",
        f"fetch_kib_raw: {sum(fetch) / len(fetch):.1f}",
        f"write_kib_raw: {sum(write) / len(write):.1f}",
        f"copy_bytes: {args.copy_bytes}",
        f"copy_fetch_kib_raw: {sum(cf) / len(cf):.1f}",
        f"copy_write_kib_raw: {sum(cw) / len(cw):.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"fetch_bytes: {fetch_b:.0f}",
        f"write_bytes: {write_b:.0f}",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
        "",
        "Commands:",
        "",
        "```",
        args.cmd.strip(),
        "```",
        "",
    ]
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def stats(args) -> None:
    rows = []
    with open(args.csv) as fh:
        for r in csv.DictReader(fh):
            if args.match and args.match not in r["Name"] and not any(x in r["Name"] for x in args.also):
                continue
            rows.append(r)
    lines = [f"# rocprofv3 kernel statistics{': ' + args.title if args.title else ''}", "",
             f"source_sha256: {source_hash(family_of(args.match))} ({family_of(args.match)} sources)", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    bench = None
    if args.bench_json:
        import json
        with open(args.bench_json) as fh:
            first = fh.readline()
        if first.strip():
            bench = json.loads(first)
    if args.trace:
        # per-dispatch durations of the matching kernel.  With the benchmark's
        # JSON line at hand its timed launches are the `steps` ones before the
        # final single-launch pass (the settle and warm-up launches come
        # first); otherwise the first `skip` launches are dropped.
        durs = []
        with open(args.trace) as fh:
            for r in csv.DictReader(fh):
                if args.match in r["Kernel_Name"]:
                    durs.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        durs.sort()
        if bench is not None and bench.get("steps"):
            tail = int(bench.get("kernel_ms", {}).get("single_launches", 0))
            end = len(durs) - tail
            timed = [d for _, d in durs[end - int(bench["steps"]):end]]
            which = f"the benchmark's {len(timed)} timed steps"
        else:
            timed = [d for _, d in durs[args.skip:]]
            which = f"after the first {args.skip}"
        if timed:
            timed_sorted = sorted(timed)
            lines += ["", f"Timed launches of `{args.match}` ({which}): {len(timed)}, "
                      f"average {sum(timed) / len(timed) / 1e3:.2f} us, "
                      f"median {timed_sorted[len(timed) // 2] / 1e3:.2f} us"]
    if bench is not None:
        if True:
            d = bench
            km = d.get("kernel_ms", {})
            lines += ["", f"The benchmark's own HIP-event timing of the same launches: mean "
                      f"{km.get('mean', float('nan')) * 1e3:.2f} us, median "
                      f"{km.get('median', float('nan')) * 1e3:.2f} us; value {d.get('value')} "
                      f"{d.get('unit')}, roofline.frac {d.get('roofline', {}).get('frac')}."]
    lines += ["", "Command:", "", "```", args.cmd.strip(), "```", ""]
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def counters(args) -> None:
    """Mean of each counter per dispatch of the matching kernel, over one or
    more --pmc runs' counter_collection.csv files, as a markdown table."""
    import collections
    acc = collections.defaultdict(list)
    for path in args.csv:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if args.match in r["Kernel_Name"]:
                    acc[r["Counter_Name"]].append(float(r["Counter_Value"]))
    if not acc:
        raise SystemExit("no counter rows for that kernel")
    lines = [f"# rocprofv3 counters per dispatch: {args.title or args.match}", "",
             f"source_sha256: {source_hash(family_of(args.match))} ({family_of(args.match)} sources)",
             f"kernel_match: {args.match}", "",
             "| counter | dispatches | mean per dispatch |", "|---|---|---|"]
    for k in sorted(acc):
        v = acc[k]
        lines.append(f"| `{k}` | {len(v)} | {sum(v) / len(v):.6g} |")
    if args.note:
        lines += ["", args.note.strip()]
    lines += ["", "Commands:", "", "```", args.cmd.strip(), "```", ""]
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def read_traffic(path: str, family: str = "gemm"):
    """traffic_bytes_per_launch from a traffic summary if its source hash
    matches the current sources of the kernel family, else None."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^source_sha256: (\w+)", text, re.M)
    t = re.search(r"^traffic_bytes_per_launch: (\d+)", text, re.M)
    if not m or not t or m.group(1) != source_hash(family):
        return None
    return int(t.group(1))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--cmd", required=True)
    s.add_argument("--match", default="")
    s.add_argument("--title", default="")
    s.add_argument("--also", action="append", default=[],
                   help="further kernel names to list in the table (e.g. a second kernel of each step)")
    s.add_argument("--trace", default="", help="run_kernel_trace.csv of the same run")
    s.add_argument("--skip", type=int, default=0, help="leading launches to leave out (warm-up)")
    s.add_argument("--bench-json", default="", help="the JSON line bench.py printed in the same run")
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-kernel", default="neg_kernel",
                   help="kernel name of the copy (the calibration run also launches a fill kernel)")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--title", default="")
    c = sub.add_parser("counters")
    c.add_argument("--match", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--title", default="")
    c.add_argument("--note", default="")
    c.add_argument("csv", nargs="+")
    a = ap.parse_args()
    if a.cmd_name == "stats":
        stats(a)
    elif a.cmd_name == "counters":
        counters(a)
    else:
        traffic(a)


if __name__ == "__main__":
    main()
