"""Summaries of rocprofv3 CSV output for the kernels of this library.

    python -m layer_wise_mixed_kvq_amd.profiling stats  <kernel_stats.csv>  --cmd "..." [--out F]
    python -m layer_wise_mixed_kvq_amd.profiling pmc    <counter_collection.csv> --cmd "..." [--out F]
    python -m layer_wise_mixed_kvq_amd.profiling traffic --kernel-regex R --workload W
           --fetch <csv> --write <csv> --copy-fetch <csv> --copy-write <csv> --copy-bytes N
           --alg-bytes-per-launch A --source <file.hip> --out <json>

`traffic` turns the FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch) into HBM bytes per
launch: each counter is scaled by what it reads for a plain copy kernel of known size
(the copy reads N bytes and writes N bytes), so both the KiB unit and any systematic
under- or over-count of the counter on this chip cancel.  The record carries a hash of the
kernel source it was measured on; the benchmark reports the figure only while that hash
still matches.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import re
import statistics
import sys
from collections import OrderedDict, defaultdict


def source_hash(paths) -> str:
    """sha256[:16] over the given source files, in order (the kernel's .hip and headers)."""
    h = hashlib.sha256()
    for path in ([paths] if isinstance(paths, str) else paths):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    name = re.sub(r"\(anonymous namespace\)::", "", name)
    name = re.sub(r"^void ", "", name)
    return name.split("(kvq::")[0] if "(kvq::" in name else name[:90]


def stats_md(path: str, cmd: str, top: int = 12) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["# rocprofv3 kernel statistics", "", f"Command: `{cmd}`", "",
           "| kernel | calls | avg us | min us | max us | total ms | % |", "|---|---|---|---|---|---|---|"]
    for r in rows[:top]:
        out.append("| %s | %s | %.2f | %.2f | %.2f | %.3f | %s |" % (
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e6, r["Percentage"]))
    return "\n".join(out) + "\n"


def _per_dispatch(path: str, kernel_regex: str | None = None):
    """{(dispatch_id): {"name":..., counter: value}} for the matching dispatches."""
    rx = re.compile(kernel_regex) if kernel_regex else None
    d = OrderedDict()
    for r in csv.DictReader(open(path)):
        if rx and not rx.search(r["Kernel_Name"]):
            continue
        e = d.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"]),
                                            "vgpr": int(r["VGPR_Count"]), "lds": int(r["LDS_Block_Size"])})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return d


def pmc_md(path: str, cmd: str, kernel_regex: str | None = None) -> str:
    d = _per_dispatch(path, kernel_regex)
    by_kernel = defaultdict(list)
    for e in d.values():
        by_kernel[_short(e["name"])].append(e)
    counters = sorted({k for e in d.values() for k in e if k.isupper() or "_" in k} - {"name", "grid", "vgpr", "lds"})
    out = ["# rocprofv3 counters (mean per dispatch)", "", f"Command: `{cmd}`", "",
           "| kernel | dispatches | VGPR | LDS B | " + " | ".join(counters) + " |",
           "|---|---|---|---|" + "---|" * len(counters)]
    for k, es in by_kernel.items():
        vals = [statistics.fmean(e.get(c, 0.0) for e in es) for c in counters]
        out.append(f"| {k} | {len(es)} | {es[0]['vgpr']} | {es[0]['lds']} | " +
                   " | ".join(f"{v:.6g}" for v in vals) + " |")
    return "\n".join(out) + "\n"


def _mean_counter(path: str, counter: str, kernel_regex: str | None) -> tuple[float, int]:
    d = _per_dispatch(path, kernel_regex)
    vals = [e[counter] for e in d.values() if counter in e]
    if not vals:
        raise SystemExit(f"{path}: no {counter} values for kernels matching {kernel_regex!r}")
    return statistics.fmean(vals), len(vals)


def traffic(args) -> dict:
    fetch_kib, n_f = _mean_counter(args.fetch, "FETCH_SIZE", args.kernel_regex)
    write_kib, n_w = _mean_counter(args.write, "WRITE_SIZE", args.kernel_regex)
    cf_kib, _ = _mean_counter(args.copy_fetch, "FETCH_SIZE", args.copy_regex)
    cw_kib, _ = _mean_counter(args.copy_write, "WRITE_SIZE", args.copy_regex)
    f_scale = args.copy_bytes / cf_kib      # bytes per counted KiB, reads
    w_scale = args.copy_bytes / cw_kib      # bytes per counted KiB, writes
    rd, wr = fetch_kib * f_scale, write_kib * w_scale
    return {
        "kernel_regex": args.kernel_regex, "workload": args.workload,
        "source": args.source, "source_sha256_16": source_hash(args.source),
        "dispatches": {"fetch": n_f, "write": n_w},
        "fetch_kib_per_launch": fetch_kib, "write_kib_per_launch": write_kib,
        "copy_bytes": args.copy_bytes, "copy_fetch_kib": cf_kib, "copy_write_kib": cw_kib,
        "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
        "traffic_bytes_per_launch": rd + wr,
        "alg_bytes_per_launch": args.alg_bytes_per_launch,
        "traffic_over_alg": (rd + wr) / args.alg_bytes_per_launch if args.alg_bytes_per_launch else None,
        "commands": args.cmd,
    }


def traffic_md(rec: dict) -> str:
    c = rec["commands"] or []
    lines = ["# HBM traffic of %s (%s)" % (rec["kernel_regex"], rec["workload"]), "",
             "Commands:", ""] + [f"    {x}" for x in c] + [
        "",
        "| quantity | value |", "|---|---|",
        f"| FETCH_SIZE per launch (KiB, mean of {rec['dispatches']['fetch']}) | {rec['fetch_kib_per_launch']:.1f} |",
        f"| WRITE_SIZE per launch (KiB, mean of {rec['dispatches']['write']}) | {rec['write_kib_per_launch']:.1f} |",
        f"| copy kernel: bytes read = bytes written | {rec['copy_bytes']} |",
        f"| copy kernel FETCH_SIZE / WRITE_SIZE (KiB) | {rec['copy_fetch_kib']:.1f} / {rec['copy_write_kib']:.1f} |",
        f"| read bytes per launch (scaled) | {rec['read_bytes_per_launch']:.4g} |",
        f"| written bytes per launch (scaled) | {rec['write_bytes_per_launch']:.4g} |",
        f"| HBM traffic per launch | {rec['traffic_bytes_per_launch']:.4g} |",
        f"| algorithmic bytes per launch | {rec['alg_bytes_per_launch']:.4g} |",
        f"| traffic / algorithmic | {rec['traffic_over_alg']:.3f} |",
        f"| kernel sources | {', '.join(rec['source'])} |",
        f"| their sha256[:16] | {rec['source_sha256_16']} |",
    ]
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m layer_wise_mixed_kvq_amd.profiling")
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    s.add_argument("--out")
    p = sub.add_parser("pmc")
    p.add_argument("csv")
    p.add_argument("--cmd", required=True)
    p.add_argument("--kernel-regex")
    p.add_argument("--out")
    t = sub.add_parser("traffic")
    t.add_argument("--kernel-regex", required=True)
    t.add_argument("--copy-regex", default=None)
    t.add_argument("--workload", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--alg-bytes-per-launch", type=float, required=True)
    t.add_argument("--source", action="append", required=True, help="kernel sources (repeat)")
    t.add_argument("--cmd", action="append")
    t.add_argument("--out", required=True, help="JSON record; a .md summary is written beside it")
    t.add_argument("--md")
    a = ap.parse_args(argv)
    if a.what == "stats":
        text = stats_md(a.csv, a.cmd)
    elif a.what == "pmc":
        text = pmc_md(a.csv, a.cmd, a.kernel_regex)
    else:
        rec = traffic(a)
        with open(a.out, "w") as f:
            json.dump(rec, f, indent=1)
        text = traffic_md(rec)
        if a.md:
            with open(a.md, "w") as f:
                f.write(text)
            return
    if getattr(a, "out", None):
        with open(a.out, "w") as f:
            f.write(text)
    else:
        sys.stdout.write(text)


if __name__ == "__main__":
    main()
