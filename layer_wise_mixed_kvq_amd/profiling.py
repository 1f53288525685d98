"""Summaries of rocprofv3 CSV output for the kernels of this library.

    python -m layer_wise_mixed_kvq_amd.profiling stats  <kernel_stats.csv>  --cmd "..." [--out F]
    python -m layer_wise_mixed_kvq_amd.profiling pmc    <counter_collection.csv> --cmd "..." [--out F]
    python -m layer_wise_mixed_kvq_amd.profiling traffic --kernel-regex R --workload W
           --fetch <csv> --write <csv> --copy-fetch <csv> --copy-write <csv> --copy-bytes N
           --alg-bytes-per-launch A --source <file.hip> --out <json>

    python -m layer_wise_mixed_kvq_amd.profiling phases [--config llama] [--layer 3] [--out F]

`phases` (needs the profiling build, `python -m layer_wise_mixed_kvq_amd.build
--phase-timers`) replays a benchmark decode step as a graph in which one layer's launch
records, per wave, the 100 MHz real-time counter at the decode kernel's phase boundaries,
and prints when each phase ends across the launch's waves (relative to its first wave's
entry) and how the work items sat on the XCDs.

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


PHASE_NAMES = {0: "entry", 8: "length known", 9: "first page requested", 10: "q setup done",
               1: "page loop start", 11: "first page done", 2: "page loop end", 12: "residual start",
               13: "residual end", 14: "merge barrier 1", 15: "merge barrier 2", 3: "partials stored",
               4: "split counter known", 5: "exit"}
N_STAMPS = 16


def phase_summary(rec) -> dict:
    """Summary of one launch's phase records: numpy uint64 [n_waves][N_STAMPS] (see kPhaseStamps
    in csrc/kvq_internal.h)."""
    import numpy as np
    live = rec[rec[:, 0] != 0]
    t0 = live[:, 0].min()
    rel = lambda col: (live[:, col].astype(np.int64) - int(t0)) * 10.0 / 1000.0   # us (10 ns ticks)
    out = {"waves": int(len(live)), "phases": {}}
    for k, name in PHASE_NAMES.items():
        sel = live[:, k] != 0
        if not sel.any():
            continue
        v = rel(k)[sel]
        out["phases"][name] = {"waves": int(sel.sum()), "min_us": float(v.min()), "median_us": float(np.median(v)),
                               "p90_us": float(np.percentile(v, 90)), "max_us": float(v.max())}
    # per-wave durations of the page loop, the merge and the combine
    dur = {}
    for a, b, name in ((1, 2, "page loop"), (2, 3, "merge + partial stores"), (3, 4, "store wait + counter"),
                       (4, 5, "after the counter (combine on the last workgroup)"), (0, 1, "prologue")):
        sel = (live[:, a] != 0) & (live[:, b] != 0)
        if sel.any():
            d = (live[sel, b].astype(np.int64) - live[sel, a].astype(np.int64)) * 0.01
            dur[name] = {"median_us": float(np.median(d)), "max_us": float(d.max())}
    out["durations"] = dur
    # page loop end by split index (early- and late-dispatched halves)
    split = (live[:, 7] >> 40).astype(np.int64)
    sel = live[:, 2] != 0
    if sel.any():
        by = {}
        for sp in np.unique(split[sel]):
            v = rel(2)[sel & (split == sp)]
            by[int(sp)] = float(np.median(v))
        out["page_loop_end_median_by_split_us"] = by
    # sharing of compute units: waves of one CU (XCC id and HW_ID bits 8..15: CU, shader
    # array, shader engine), their workgroups in order of entry, and how far apart the page
    # loops of a CU's workgroups end
    cu = ((live[:, 6] >> 32) & 0xF).astype(np.int64) * 256 + ((live[:, 6] >> 8) & 0xFF).astype(np.int64)
    wg = (live[:, 7]).astype(np.int64)
    spread, first_last, wgs_per_cu = [], [], []
    for c in np.unique(cu):
        m = (cu == c) & sel
        if not m.any():
            continue
        ends = {}
        ent = {}
        for w_, e_, t_ in zip(wg[m], rel(2)[m], rel(0)[m]):
            ends[w_] = max(ends.get(w_, 0.0), e_)
            ent[w_] = min(ent.get(w_, 1e9), t_)
        order = sorted(ends, key=lambda k: ent[k])
        wgs_per_cu.append(len(order))
        spread.append(float(rel(2)[m].max() - rel(2)[m].min()))
        if len(order) >= 2:
            first_last.append((ends[order[0]], ends[order[-1]]))
    out["cus"] = {"n": len(spread), "workgroups_per_cu": {int(k): int(v) for k, v in
                                                          zip(*np.unique(wgs_per_cu, return_counts=True))},
                  "loop_end_spread_within_cu_median_us": float(np.median(spread)) if spread else None}
    if first_last:
        fl = np.array(first_last)
        out["cus"]["loop_end_first_vs_last_entered_wg_median_us"] = [float(np.median(fl[:, 0])),
                                                                    float(np.median(fl[:, 1]))]
    # XCD placement: does every (sequence, KV head) keep all its splits on one XCD?
    xcc = ((live[:, 6] >> 32) & 0xF).astype(np.int64)
    item = (live[:, 7] & ((1 << 40) - 1)).astype(np.int64)
    one = all(len(np.unique(xcc[item == it])) == 1 for it in np.unique(item))
    out["xcds"] = {"waves_per_xcd": {int(x): int((xcc == x).sum()) for x in np.unique(xcc)},
                   "every_item_on_one_xcd": bool(one)}
    return out


def phases_md(summ: dict, cmd: str, title: str) -> str:
    lines = [f"# Decode kernel phase timers: {title}", "", f"Command: `{cmd}`", "",
             "Per-wave stamps of the 100 MHz real-time counter (10 ns ticks), relative to the first wave's entry "
             f"into the launch; {summ['waves']} waves.", "",
             "| phase boundary | waves | min us | median us | p90 us | max us |", "|---|---|---|---|---|---|"]
    for name, v in summ["phases"].items():
        lines.append(f"| {name} | {v['waves']} | {v['min_us']:.2f} | {v['median_us']:.2f} | {v['p90_us']:.2f} | "
                     f"{v['max_us']:.2f} |")
    lines += ["", "| per-wave duration | median us | max us |", "|---|---|---|"]
    for name, v in summ["durations"].items():
        lines.append(f"| {name} | {v['median_us']:.2f} | {v['max_us']:.2f} |")
    if "page_loop_end_median_by_split_us" in summ:
        lines += ["", "Page loop end, median by split index (us): " +
                  ", ".join(f"{k}: {v:.2f}" for k, v in summ["page_loop_end_median_by_split_us"].items())]
    if "cus" in summ:
        c = summ["cus"]
        lines += ["", f"Compute units used: {c['n']}; workgroups per CU: {c['workgroups_per_cu']}; page-loop end "
                  f"spread within a CU (median over CUs): {c['loop_end_spread_within_cu_median_us']:.2f} us" +
                  (f"; loop end of the first- and last-entered workgroup of a CU (medians): "
                   f"{c['loop_end_first_vs_last_entered_wg_median_us'][0]:.2f} / "
                   f"{c['loop_end_first_vs_last_entered_wg_median_us'][1]:.2f} us"
                   if "loop_end_first_vs_last_entered_wg_median_us" in c else "")]
    x = summ["xcds"]
    lines += ["", "Waves per XCD: " + ", ".join(f"{k}: {v}" for k, v in x["waves_per_xcd"].items()) +
              f"; every (sequence, KV head) on one XCD: {x['every_item_on_one_xcd']}"]
    return "\n".join(lines) + "\n"


def phases(args) -> str:
    import os
    import numpy as np
    import torch
    from . import _native
    _native.use_phase_timer_build(args.lib)
    from . import _native as nat
    L = nat.lib()
    if not hasattr(L, "kvq_profile_set_phase_buffer"):
        raise SystemExit("libkvq_phases.so lacks the phase timers: build it with "
                         "python -m layer_wise_mixed_kvq_amd.build --phase-timers")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    cfg = bench.CONFIGS[args.config]
    stack = bench.DecodeStack(cfg, "cuda")
    n_rec = stack.H * stack.B * stack.max_pages * 8          # >= workgroups x 8 wave slots
    buf = torch.zeros(n_rec * N_STAMPS, dtype=torch.int64, device="cuda")
    kvq = stack.kvq

    sink = torch.zeros(1, dtype=torch.int64, device="cuda")

    def step():
        for l in range(len(stack.caches)):
            if l == args.layer and args.touch_stride:
                # read one byte per touch_stride bytes of the layer's buffers just before its
                # launch (address translations warm, almost no data cached)
                c = stack.caches[l]
                for t in (c.pages.view(-1), stack.q[l].view(torch.uint8).view(-1), stack.out[l].view(torch.uint8).view(-1)):
                    sink.add_(t[::args.touch_stride].sum())
            if l == args.layer:
                L.kvq_profile_set_phase_buffer(buf.data_ptr(), buf.numel() * 8)
            kvq.kvq_append_decode_attn(stack.model, l, stack.caches[l], stack.k_new[l], stack.v_new[l], stack.pos,
                                       stack.q[l], stack.L, out=stack.out[l], lse=stack.lse[l],
                                       workspace=stack.workspace)
            if l == args.layer:
                L.kvq_profile_set_phase_buffer(None, 0)

    g = bench.capture(step)
    summaries = []
    for r in range(args.reps):
        buf.zero_()
        g.replay()
        torch.cuda.synchronize()
        rec = buf.view(-1, N_STAMPS).cpu().numpy().view(np.uint64)
        summaries.append((phase_summary(rec), rec.copy()))
    # the replay with the median exit time
    summaries.sort(key=lambda s_: s_[0]["phases"]["exit"]["max_us"])
    summ, raw = summaries[len(summaries) // 2]
    if args.raw:
        np.save(args.raw, raw[raw[:, 0] != 0])
    summaries = [s_ for s_, _ in summaries]
    kb, vb = cfg["pairs"][args.layer] if not isinstance(cfg["pairs"][args.layer], str) else (0, 0)
    title = (f"{cfg['workload']}, layer {args.layer} ({cfg['pairs'][args.layer]}); median of {args.reps} graph "
             "replays of the whole step by last exit")
    text = phases_md(summ, args.cmd or " ".join(sys.argv), title)
    summ["exit_max_us_all_replays"] = [s_["phases"]["exit"]["max_us"] for s_ in summaries]
    if args.json:
        with open(args.json, "w") as f:
            json.dump(summ, f, indent=1)
    return text


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
    ph = sub.add_parser("phases")
    ph.add_argument("--config", default="llama")
    ph.add_argument("--layer", type=int, default=3)
    ph.add_argument("--reps", type=int, default=7)
    ph.add_argument("--cmd")
    ph.add_argument("--json")
    ph.add_argument("--lib", help="another phase-timer build of the library to load")
    ph.add_argument("--touch-stride", type=int, default=0,
                    help="before the layer's launch, read one byte per this many bytes of its pool, q and out")
    ph.add_argument("--raw", help="also save that replay's per-wave records (.npy, uint64 [waves][16])")
    ph.add_argument("--out")
    a = ap.parse_args(argv)
    if a.what == "stats":
        text = stats_md(a.csv, a.cmd)
    elif a.what == "pmc":
        text = pmc_md(a.csv, a.cmd, a.kernel_regex)
    elif a.what == "phases":
        text = phases(a)
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
