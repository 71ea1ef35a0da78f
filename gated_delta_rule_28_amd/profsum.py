"""Summaries of rocprofv3 CSV output for the KDA kernels.

    python -m gated_delta_rule_28_amd.profsum stats  KERNEL_STATS_CSV [--trace KERNEL_TRACE_CSV --prefill-calls N] [--top K] --cmd "..." --out FILE.md
    python -m gated_delta_rule_28_amd.profsum traffic FETCH_CSV WRITE_CSV [--prefill-calls N] --cmd "..." --out FILE.md
    python -m gated_delta_rule_28_amd.profsum counters COUNTER_CSV --cmd "..." --out FILE.md

A kda_prefill call on the two-kernel path launches the intra-chunk kernel once
per slab of chunks and the inter-chunk kernel once over all slabs (or once per
slab when the slabs share buffers), partly at the same time; with
--prefill-calls (the number of calls in the profiled run) `stats` adds the
average span of a call (first start to last end of its kernels) and
`traffic` the HBM bytes of a whole call.

`traffic` scales FETCH_SIZE and WRITE_SIZE (KiB per dispatch) by what the same
counters read for the largest `neg` elementwise kernel in the run (bench.py
--calibrate: 1 GiB read + 1 GiB written), and records the HBM bytes per launch
of each KDA kernel, with a hash of the kernel's source, in profiles/traffic.json
(bench.py reports them only while the source is unchanged).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_28_amd", "csrc")

# kernel key -> (substring of the demangled name, source file)
KERNELS = {
    "intra_chunk_kernel": ("intra_chunk_kernel<false>", "kda_prefill_split.hip"),
    "inter_chunk_kernel": ("inter_chunk_kernel<false, true>", "kda_prefill_split.hip"),
    "prefill_kernel": ("prefill_kernel<64, 128, 128, true, false, false>", "kda_prefill.hip"),
    "decode_kernel": ("decode_kernel<128, 128, true, false>", "kda_decode.hip"),
    "decode_multi_kernel": ("decode_multi_kernel<128, 128, true, false, 4, false>", "kda_decode.hip"),
}
CALIB_BYTES = 1 << 30   # bytes read, and bytes written, by the calibration kernel


def source_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def _short(name, n=90):
    name = name.replace("kda::(anonymous namespace)::", "")
    return name if len(name) <= n else name[:n - 3] + "..."


def call_spans(trace, calls):
    """Spans (ns) of the prefill calls: the chunk kernels of the run, in start
    order, split into `calls` equal groups (each call launches the same slabs);
    and the durations (ns) of each call's inter-chunk dispatches in start order
    (the recurrence launch, then the resume launch when there is one)."""
    ks = [r for r in csv.DictReader(open(trace)) if "chunk_kernel" in r["Kernel_Name"]]
    ks.sort(key=lambda r: int(r["Start_Timestamp"]))
    if calls <= 0 or len(ks) % calls:
        raise SystemExit(f"{trace}: {len(ks)} chunk-kernel dispatches do not split into {calls} calls")
    per = len(ks) // calls
    spans, inter = [], []
    for c in range(calls):
        g = ks[c * per:(c + 1) * per]
        spans.append(max(int(r["End_Timestamp"]) for r in g) - min(int(r["Start_Timestamp"]) for r in g))
        inter.append([int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in g
                      if "inter_chunk_kernel" in r["Kernel_Name"]])
    return spans, per, inter


def stats(path, cmd, out, trace=None, calls=0, top=8):
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["# Kernel time (rocprofv3 --kernel-trace --stats)", "", "Command:", "",
             "```", cmd, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in rows[:top]:
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    if trace:
        spans, per, inter = call_spans(trace, calls)
        lines += ["", f"kda_prefill calls: {calls}, {per} chunk-kernel launches each (the intra-chunk kernel per slab and "
                  f"the inter-chunk kernel, overlapping); span of a call (first start to last end): average "
                  f"{sum(spans) / len(spans) / 1e3:.1f} us, min {min(spans) / 1e3:.1f} us, max {max(spans) / 1e3:.1f} us."]
        n_inter = {len(x) for x in inter}
        if n_inter == {2}:
            rec = [x[0] for x in inter]
            res = [x[1] for x in inter]
            lines += ["", "Inter-chunk dispatches of a call: the recurrence launch over all slabs, average "
                      f"{sum(rec) / len(rec) / 1e3:.1f} us (min {min(rec) / 1e3:.1f}, max {max(rec) / 1e3:.1f}), "
                      f"and the resume launch after the slabs, average {sum(res) / len(res) / 1e3:.1f} us (its "
                      "workgroups exit at once when no wait expired); the per-kernel average above mixes the two."]
    open(out, "w").write("\n".join(lines) + "\n")


def _per_kernel(path):
    """kernel name -> counter name -> list of per-dispatch values; plus grid sizes."""
    d = collections.defaultdict(lambda: collections.defaultdict(list))
    grid = {}
    for r in csv.DictReader(open(path)):
        d[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
        grid.setdefault((r["Kernel_Name"], r["Dispatch_Id"]), int(r["Grid_Size"]))
    return d, grid


def _calib(path, counter):
    """Mean counter value of the largest-grid `neg` dispatches (the calibration kernel)."""
    best, vals = -1, []
    for r in csv.DictReader(open(path)):
        if "neg_kernel" not in r["Kernel_Name"] or r["Counter_Name"] != counter:
            continue
        g = int(r["Grid_Size"])
        if g > best:
            best, vals = g, []
        if g == best:
            vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"{path}: no calibration dispatch (run bench.py with --calibrate)")
    return sum(vals) / len(vals)


def _match(d, sub):
    names = [n for n in d if sub in n]
    return names[0] if names else None


def traffic(fetch_csv, write_csv, cmd, out, json_out, calls=0):
    f_d, _ = _per_kernel(fetch_csv)
    w_d, _ = _per_kernel(write_csv)
    f_cal = _calib(fetch_csv, "FETCH_SIZE")
    w_cal = _calib(write_csv, "WRITE_SIZE")
    f_scale = (CALIB_BYTES / 1024) / f_cal
    w_scale = (CALIB_BYTES / 1024) / w_cal
    lines = ["# HBM traffic per launch (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)", "",
             "Commands (one counter per run):", "", "```", cmd, "```", "",
             f"Calibration: a `neg` elementwise kernel reading 1 GiB and writing 1 GiB reads as "
             f"FETCH_SIZE {f_cal:.0f} KiB and WRITE_SIZE {w_cal:.0f} KiB, so the counters are scaled "
             f"by {f_scale:.3f} (fetch) and {w_scale:.3f} (write).", "",
             "| kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM read (GB) | HBM write (GB) | total (GB) |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    res = json.load(open(json_out)) if os.path.exists(json_out) else {}
    for key, (sub, src) in KERNELS.items():
        nf, nw = _match(f_d, sub), _match(w_d, sub)
        if nf is None or nw is None:
            continue
        fv, wv = f_d[nf]["FETCH_SIZE"], w_d[nw]["WRITE_SIZE"]
        fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
        rd, wr = fk * 1024 * f_scale, wk * 1024 * w_scale
        lines.append(f"| `{_short(nf)}` | {len(fv)} | {fk:.0f} | {wk:.0f} | {rd / 1e9:.3f} | "
                     f"{wr / 1e9:.3f} | {(rd + wr) / 1e9:.3f} |")
        res[key] = {"bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr,
                    "source_sha256_16": source_hash(os.path.join(CSRC, src)),
                    "fetch_scale": f_scale, "write_scale": w_scale}
    if calls > 0:
        # a whole kda_prefill call: every dispatch of both chunk kernels, per call
        tot_r = tot_w = 0.0
        for key in ("intra_chunk_kernel", "inter_chunk_kernel"):
            sub = KERNELS[key][0]
            nf, nw = _match(f_d, sub), _match(w_d, sub)
            if nf is None or nw is None:
                raise SystemExit(f"no dispatches of {key} in the counter runs")
            tot_r += sum(f_d[nf]["FETCH_SIZE"]) * 1024 * f_scale
            tot_w += sum(w_d[nw]["WRITE_SIZE"]) * 1024 * w_scale
        rd, wr = tot_r / calls, tot_w / calls
        lines += ["", f"Whole kda_prefill call ({calls} calls in the run, all slabs of both chunk kernels): "
                  f"read {rd / 1e9:.3f} GB, written {wr / 1e9:.3f} GB, total {(rd + wr) / 1e9:.3f} GB per call."]
        n_int = len(f_d[_match(f_d, KERNELS["inter_chunk_kernel"][0])]["FETCH_SIZE"])
        if n_int == 2 * calls:
            lines += ["", "Each call's two inter-chunk dispatches are the recurrence launch over all slabs and the "
                      "resume launch. Counter collection serialises kernels, so the recurrence stops at its first "
                      "slab wait and the resume launch does its work: the per-dispatch figures above are half a "
                      "call's recurrence traffic; the per-call total is unaffected."]
        res["prefill_call"] = {"bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr,
                               "source_sha256_16": source_hash(os.path.join(CSRC, "kda_prefill_split.hip")),
                               "fetch_scale": f_scale, "write_scale": w_scale}
    open(out, "w").write("\n".join(lines) + "\n")
    json.dump(res, open(json_out, "w"), indent=1, sort_keys=True)


def counters(path, cmd, out, simds=1024):
    """Per-kernel means of the counters of one --pmc run (raw or derived, as
    rocprofv3 reports them), over the dispatches that did matrix-core work when
    the run counts SQ_INSTS_VALU_MFMA_MOPS_F16 (counter collection serialises
    kernels, so a one-launch recurrence stops at its first wait and its resume
    launch does the work: the stopped dispatch would only dilute the means)."""
    by = collections.defaultdict(lambda: collections.defaultdict(dict))
    for r in csv.DictReader(open(path)):
        by[r["Kernel_Name"]][r["Dispatch_Id"]][r["Counter_Name"]] = float(r["Counter_Value"])
    lines = ["# Compute counters per dispatch (rocprofv3 --pmc)", "", "Command:", "", "```", cmd, "```", ""]
    for key, (sub, _src) in KERNELS.items():
        n = _match(by, sub)
        if n is None:
            continue
        disp = list(by[n].values())
        mops = "SQ_INSTS_VALU_MFMA_MOPS_F16"
        top = max((x.get(mops, 0.0) for x in disp), default=0.0)
        used = [x for x in disp if top == 0.0 or x.get(mops, 0.0) > 0.01 * top]
        names = sorted({k for x in used for k in x})
        lines.append(f"## `{_short(n)}`")
        lines.append("")
        lines.append(f"- dispatches: {len(used)} of {len(disp)}")
        for k in names:
            v = [x[k] for x in used if k in x]
            lines.append(f"- {k}: {sum(v) / len(v):.6g}")
        lines.append("")
    open(out, "w").write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--trace", default=None)
    a.add_argument("--top", type=int, default=8, help="kernels listed (by total time)")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("--json", default=os.path.join(ROOT, "profiles", "traffic.json"))
    c = sub.add_parser("counters")
    c.add_argument("csv")
    for p in (a, b, c):
        p.add_argument("--cmd", required=True)
        p.add_argument("--out", required=True)
    for p in (a, b):
        p.add_argument("--prefill-calls", type=int, default=0)
    args = ap.parse_args()
    if args.what == "stats":
        stats(args.csv, args.cmd, args.out, args.trace, args.prefill_calls, args.top)
    elif args.what == "traffic":
        traffic(args.fetch_csv, args.write_csv, args.cmd, args.out, args.json, args.prefill_calls)
    else:
        counters(args.csv, args.cmd, args.out)


if __name__ == "__main__":
    main()
