"""Summaries of rocprofv3 output for the profiles/ folder (host-side tooling).

  python -m randomized_positional_lsh_amd.profsum stats DIR OUT.md --cmd "..."
      Per-kernel rows (calls, mean / min / max duration) of the
      --kernel-trace --stats CSV in DIR for the kernels of this library.

  python -m randomized_positional_lsh_amd.profsum traffic FETCH WRITE CFETCH CWRITE OUT.json \
          --workload mistral --kernel-sha SHA --copy-bytes N --cmd "..."
      HBM bytes per launch of the attention kernel from two --pmc runs
      (FETCH_SIZE, WRITE_SIZE, KiB per dispatch), each scaled by the factor
      that makes the same counter read right on plain device copies of
      known total size (CFETCH / CWRITE runs, N bytes read and N written).
"""

from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics

KERNELS = {"fwd_kernel": "attention (fwd_kernel)", "bins_kernel": "bin boundaries (bins_kernel)"}


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def _short(name: str) -> str | None:
    for k, v in KERNELS.items():
        if k in name:
            return v
    return None


def stats(d: str, out: str, cmd: str) -> None:
    path = _one(os.path.join(d, "**", "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(path)))
    lines = ["# Kernel trace summary", "", f"Command: `{cmd}`", "",
             "| kernel | calls | mean us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        s = _short(r["Name"])
        if s is None:
            continue
        ns = 1e-3
        lines.append(f"| {s} | {r['Calls']} | {float(r['AverageNs']) * ns:.2f} | {float(r['MinNs']) * ns:.2f} | "
                     f"{float(r['MaxNs']) * ns:.2f} | {float(r['Percentage']):.1f}% |")
    lines += ["", f"Source: {os.path.basename(path)} (rocprofv3 --kernel-trace --stats --output-format csv)."]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_kib(d: str, regex_part: str, counter: str) -> list[float]:
    path = _one(os.path.join(d, "**", "*counter_collection.csv"))
    per = {}
    for r in csv.DictReader(open(path)):
        if regex_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise ValueError(f"no {counter} rows for kernels matching {regex_part!r} in {path}")
    return list(per.values())


def traffic(fetch: str, write: str, cfetch: str, cwrite: str, out: str, workload: str, sha: str,
            copy_bytes: int, cmd: str) -> None:
    f = _counter_kib(fetch, "fwd_kernel", "FETCH_SIZE")
    w = _counter_kib(write, "fwd_kernel", "WRITE_SIZE")
    cf = sum(_counter_kib(cfetch, "copyBuffer", "FETCH_SIZE")) * 1024.0
    cw = sum(_counter_kib(cwrite, "copyBuffer", "WRITE_SIZE")) * 1024.0
    sf, sw = copy_bytes / cf, copy_bytes / cw
    fb = statistics.mean(f) * 1024.0 * sf
    wb = statistics.mean(w) * 1024.0 * sw
    res = {"kernel_sha": sha, "workload": workload, "bytes_per_launch": int(round(fb + wb)),
           "fetch_bytes": int(round(fb)), "write_bytes": int(round(wb)),
           "fetch_scale": round(sf, 5), "write_scale": round(sw, 5),
           "dispatches": {"fetch": len(f), "write": len(w)}, "command": cmd}
    with open(out, "w") as fo:
        json.dump(res, fo, indent=1)
        fo.write("\n")
    print(json.dumps(res, indent=1))


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    a.add_argument("out")
    a.add_argument("--cmd", required=True)
    b = sub.add_parser("traffic")
    for x in ("fetch", "write", "cfetch", "cwrite", "out"):
        b.add_argument(x)
    b.add_argument("--workload", required=True)
    b.add_argument("--kernel-sha", required=True)
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--cmd", required=True)
    args = ap.parse_args()
    if args.cmd_name == "stats":
        stats(args.dir, args.out, args.cmd)
    else:
        traffic(args.fetch, args.write, args.cfetch, args.cwrite, args.out, args.workload, args.kernel_sha,
                args.copy_bytes, args.cmd)


if __name__ == "__main__":
    main()
