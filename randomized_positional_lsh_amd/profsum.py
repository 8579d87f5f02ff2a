"""Summaries of rocprofv3 output for the profiles/ folder (host-side tooling).

  python -m randomized_positional_lsh_amd.profsum stats DIR OUT.md --cmd "..."
      Per-kernel rows (calls, mean / min / max duration) of the
      --kernel-trace --stats CSV in DIR for the kernels of this library,
      labelled by kernel and template instance; and, from the per-dispatch
      trace, the count-weighted attention kernel's durations at the
      Mistral shape (--grid: threads per launch, 4096 x 512) split into
      launches that follow a read-only reduction over a large buffer
      (bench.py evicts the caches that way before its cold-cache launches)
      and the others.

  python -m randomized_positional_lsh_amd.profsum util DIR OUT.md --cmd "..." [--kernel K]
      Unit utilisation of one kernel (default the count-weighted attention
      kernel at head_dim 128, bf16, causal, one hash chunk) from one --pmc
      pass of GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES, SQ_ACTIVE_INST_VALU,
      SQ_LDS_IDX_ACTIVE and SQ_LDS_BANK_CONFLICT (means over its dispatches;
      GRBM_GUI_ACTIVE summed over the 8 XCDs, so divided by 8 for cycles).

  python -m randomized_positional_lsh_amd.profsum waves DIR [DIR ...] OUT.md --cmd "..." --kernel K ...
      Per-wave instruction counts and wave states of the named kernels
      (substrings of the demangled name, e.g. "bwd_kernel<128, true, 1,
      false>") from --pmc passes that each hold SQ_WAVES: SQ_INSTS_* over
      SQ_WAVES, and SQ_ACTIVE_INST_ANY, SQ_WAIT_INST_ANY and SQ_WAIT_ANY as
      shares of SQ_WAVE_CYCLES; means over dispatches per (kernel, grid).
      Dispatches that directly follow a bin kernel (the two-launch step's
      attention, which reads its plan records) are left out.

  python -m randomized_positional_lsh_amd.profsum traffic FETCH WRITE CFETCH CWRITE OUT.json \
          --workload mistral --kernel-sha SHA --copy-bytes N --cmd "..."
      HBM bytes per launch of the count-weighted attention kernel at the
      Mistral shape (fwd_kernel<128, bf16, causal, 1 hash chunk, mode 0>),
      over its launches that follow the cache-evicting read, from two --pmc runs
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
import re
import statistics

# Kernel labels.  rocprofv3 reports demangled names; the attention template's
# arguments are <head_dim, bf16, causal, hash chunks, mode> with mode 0
# count-weighted, 1 dense ALiBi, 2 one short attention per hash; the backward
# template's <head_dim, causal, hash chunks, keys side>.
MAIN = "fwd_kernel<128, true, true, 1, 0>"
EVICT = "reduce_kernel"  # torch's reduction kernel: bench.py's read-only cache eviction
_MODES = {"0": "attention, count-weighted", "1": "dense exact ALiBi", "2": "one attention per hash"}
_PLAIN = [
    ("bins_part_kernel", "bin boundaries, parts of 8192 positions"),
    ("bins_kernel", "bin boundaries, one workgroup per hash"),
    ("rowdot_kernel", "backward D = <dO, O>"),
    ("rowmax_kernel", "error row maxima"),
    ("scan_local_kernel", "error product, tile scans"),
    ("scan_carry_kernel", "error product, carries"),
    ("combine_kernel", "error product, combine"),
    ("dots_kernel", "Lanczos dot products"),
    ("sub_proj_kernel", "Lanczos projections"),
    ("scale_kernel", "Lanczos scaling"),
    ("argmax_kernel", "max reduction"),
]


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def _short(name: str) -> str | None:
    m = re.search(r"fwd_kernel<(\d+), (\w+), (\w+), (\d+), (\d)>", name)
    if m:
        return f"{_MODES[m.group(5)]} (fwd_kernel<{', '.join(m.groups())}>)"
    m = re.search(r"bwd_kernel<(\d+), (\w+), (\d+), (\w+)>", name)
    if m:
        side = "dK dV" if m.group(4) == "true" else "dQ"
        return f"backward {side} (bwd_kernel<{', '.join(m.groups())}>)"
    for k, v in _PLAIN:
        if k in name:
            return f"{v} ({k})"
    return None


def stats(d: str, out: str, cmd: str, grid: int = 4096 * 512) -> None:
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
    traces = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if traces:
        seq = sorted(csv.DictReader(open(traces[0])), key=lambda r: int(r["Start_Timestamp"]))
        cold, warm = [], []
        for prev, r in zip([None] + seq[:-1], seq):
            if MAIN not in r["Kernel_Name"] or int(r["Grid_Size_X"]) != grid:
                continue
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
            (cold if prev is not None and EVICT in prev["Kernel_Name"] else warm).append(us)
        if cold or warm:
            lines += ["", f"Count-weighted attention ({MAIN}), launches of {grid // 512} workgroups (the "
                      "Mistral-shaped layer), per dispatch (kernel trace, us):", "",
                      "| launches | calls | median | mean | p10 | p90 |", "|---|---|---|---|---|---|"]
            for name, x in (("after a cache-evicting read (cold)", cold), ("others (warm)", warm)):
                if x:
                    q = statistics.quantiles(x, n=10) if len(x) > 1 else [x[0]] * 9
                    lines.append(f"| {name} | {len(x)} | {statistics.median(x):.2f} | {statistics.mean(x):.2f} | "
                                 f"{q[0]:.2f} | {q[-1]:.2f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def util(d: str, out: str, cmd: str, kernel: str = MAIN, cus: int = 256, simds: int = 1024, xcds: int = 8) -> None:
    path = _one(os.path.join(d, "**", "*counter_collection.csv"))
    per: dict = {}
    for r in csv.DictReader(open(path)):
        if kernel in r["Kernel_Name"]:
            per.setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = float(r["Counter_Value"])
    need = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_LDS_IDX_ACTIVE",
            "SQ_LDS_BANK_CONFLICT")
    rows = [v for v in per.values() if all(k in v for k in need)]
    if not rows:
        raise ValueError(f"no dispatches of {kernel} with counters {need} in {path}")
    m = {k: statistics.mean(v[k] for v in rows) for k in need}
    cyc = m["GRBM_GUI_ACTIVE"] / xcds
    res = [
        ("matrix cores busy (SQ_VALU_MFMA_BUSY_CYCLES / (cycles x SIMDs))", m["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * simds)),
        ("vector ALU instructions active (4 x SQ_ACTIVE_INST_VALU / (cycles x SIMDs))",
         4 * m["SQ_ACTIVE_INST_VALU"] / (cyc * simds)),
        ("LDS busy (SQ_LDS_IDX_ACTIVE / (cycles x CUs))", m["SQ_LDS_IDX_ACTIVE"] / (cyc * cus)),
        ("LDS bank-conflict stalls (SQ_LDS_BANK_CONFLICT / (cycles x CUs))", m["SQ_LDS_BANK_CONFLICT"] / (cyc * cus)),
    ]
    lines = [f"# Unit utilisation of {_short(kernel) or kernel}", "", f"Command: `{cmd}`", "",
             f"Kernel: {kernel}, {len(rows)} dispatches; cycles per dispatch (GRBM_GUI_ACTIVE / {xcds}): {cyc:.0f}.",
             "", "| unit | share of cycles |", "|---|---|"]
    lines += [f"| {name} | {100 * v:.1f}% |" for name, v in res]
    lines += ["", f"Source: {os.path.basename(path)} (rocprofv3 --pmc, counters per dispatch)."]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


_WAVE_ROWS = [
    ("vector instructions (SQ_INSTS_VALU, matrix included)", "SQ_INSTS_VALU"),
    ("matrix instructions (SQ_INSTS_MFMA)", "SQ_INSTS_MFMA"),
    ("transcendental fp32 (SQ_INSTS_VALU_TRANS_F32)", "SQ_INSTS_VALU_TRANS_F32"),
    ("scalar ALU (SQ_INSTS_SALU)", "SQ_INSTS_SALU"),
    ("scalar memory (SQ_INSTS_SMEM)", "SQ_INSTS_SMEM"),
    ("LDS (SQ_INSTS_LDS)", "SQ_INSTS_LDS"),
    ("branches (SQ_INSTS_BRANCH)", "SQ_INSTS_BRANCH"),
]
_STATE_ROWS = [
    ("issuing (SQ_ACTIVE_INST_ANY)", "SQ_ACTIVE_INST_ANY"),
    ("ready, not issued (SQ_WAIT_INST_ANY)", "SQ_WAIT_INST_ANY"),
    ("waiting on dependencies (SQ_WAIT_ANY)", "SQ_WAIT_ANY"),
]


def waves(dirs: list[str], out: str, cmd: str, kernels: list[str]) -> None:
    # (kernel, grid) -> dispatch -> counter -> value, over every pass
    per: dict = {}
    for d in dirs:
        path = _one(os.path.join(d, "**", "*counter_collection.csv"))
        rows = list(csv.DictReader(open(path)))
        names = {int(r["Dispatch_Id"]): r["Kernel_Name"] for r in rows}
        ids = sorted(names)
        after_bins = {b for a, b in zip(ids, ids[1:]) if "bins_" in names[a]}
        for r in rows:
            i = int(r["Dispatch_Id"])
            k = next((k for k in kernels if k in r["Kernel_Name"]), None)
            if k is None or i in after_bins:
                continue
            key = (k, int(r["Grid_Size"]) // int(r["Workgroup_Size"]))
            c = per.setdefault(key, {}).setdefault((d, i), {})
            c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    lines = ["# Instructions and wave states per wave", "", f"Command: `{cmd}`", "",
             "Means over dispatches of each counter divided by SQ_WAVES of the same dispatch; wave states as "
             "shares of SQ_WAVE_CYCLES (quad-cycles per wave).", ""]
    for (k, wgs), disp in sorted(per.items()):
        vals: dict = {}
        for c in disp.values():
            if c.get("SQ_WAVES", 0.0) <= 0.0:
                continue
            for name, v in c.items():
                if name != "SQ_WAVES":
                    vals.setdefault(name, []).append(v / c["SQ_WAVES"])
        if not vals:
            continue
        m = {name: statistics.mean(v) for name, v in vals.items()}
        lines += [f"## {k}, {wgs} workgroups", "", "| per wave | value |", "|---|---|"]
        for label, name in _WAVE_ROWS:
            if name in m:
                lines.append(f"| {label} | {m[name]:.0f} |")
        if "SQ_WAVE_CYCLES" in m:
            wc = m["SQ_WAVE_CYCLES"]
            lines.append(f"| wave life, quad-cycles (SQ_WAVE_CYCLES) | {wc:.0f} |")
            for label, name in _STATE_ROWS:
                if name in m:
                    lines.append(f"| {label} | {100 * m[name] / wc:.0f}% |")
        lines.append("")
    lines.append("Source: counter_collection.csv of each pass (rocprofv3 --pmc, counters per dispatch).")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_kib(d: str, regex_part: str, counter: str, cold_only: bool = False) -> list[float]:
    """Per-dispatch sums of `counter` for kernels matching `regex_part`;
    cold_only: only dispatches that directly follow the cache-evicting read."""
    path = _one(os.path.join(d, "**", "*counter_collection.csv"))
    per, names = {}, {}
    for r in csv.DictReader(open(path)):
        names[int(r["Dispatch_Id"])] = r["Kernel_Name"]
        if regex_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per[int(r["Dispatch_Id"])] = per.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
    if cold_only:
        ids = sorted(names)
        prev = {b: a for a, b in zip(ids, ids[1:])}
        per = {k: v for k, v in per.items() if k in prev and EVICT in names[prev[k]]}
    if not per:
        raise ValueError(f"no {counter} rows for kernels matching {regex_part!r} in {path}")
    return list(per.values())


def traffic(fetch: str, write: str, cfetch: str, cwrite: str, out: str, workload: str, sha: str,
            copy_bytes: int, cmd: str) -> None:
    f = _counter_kib(fetch, MAIN, "FETCH_SIZE", cold_only=True)
    w = _counter_kib(write, MAIN, "WRITE_SIZE", cold_only=True)
    cf = sum(_counter_kib(cfetch, "copyBuffer", "FETCH_SIZE")) * 1024.0
    cw = sum(_counter_kib(cwrite, "copyBuffer", "WRITE_SIZE")) * 1024.0
    sf, sw = copy_bytes / cf, copy_bytes / cw
    fb = statistics.mean(f) * 1024.0 * sf
    wb = statistics.mean(w) * 1024.0 * sw
    res = {"kernel_sha": sha, "workload": workload, "bytes_per_launch": int(round(fb + wb)),
           "fetch_bytes": int(round(fb)), "write_bytes": int(round(wb)),
           "fetch_scale": round(sf, 5), "write_scale": round(sw, 5),
           "dispatches": {"fetch": len(f), "write": len(w)}, "launches": "after a cache-evicting read",
           "command": cmd}
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
    a.add_argument("--grid", type=int, default=4096 * 512)
    c = sub.add_parser("util")
    c.add_argument("dir")
    c.add_argument("out")
    c.add_argument("--cmd", required=True)
    c.add_argument("--kernel", default=MAIN)
    w = sub.add_parser("waves")
    w.add_argument("paths", nargs="+", help="pass directories, then the output file")
    w.add_argument("--cmd", required=True)
    w.add_argument("--kernel", action="append", required=True)
    b = sub.add_parser("traffic")
    for x in ("fetch", "write", "cfetch", "cwrite", "out"):
        b.add_argument(x)
    b.add_argument("--workload", required=True)
    b.add_argument("--kernel-sha", required=True)
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--cmd", required=True)
    args = ap.parse_args()
    if args.cmd_name == "stats":
        stats(args.dir, args.out, args.cmd, args.grid)
    elif args.cmd_name == "waves":
        waves(args.paths[:-1], args.paths[-1], args.cmd, args.kernel)
    elif args.cmd_name == "util":
        util(args.dir, args.out, args.cmd, args.kernel)
    else:
        traffic(args.fetch, args.write, args.cfetch, args.cwrite, args.out, args.workload, args.kernel_sha,
                args.copy_bytes, args.cmd)


if __name__ == "__main__":
    main()
