"""Turn rocprofv3 CSV output into the short summaries kept under profiles/.

    python -m gated_delta_rule_08_amd.profiling stats  <kernel_stats.csv>  [--command "..."]
    python -m gated_delta_rule_08_amd.profiling evicted <kernel_trace.csv>
    python -m gated_delta_rule_08_amd.profiling traffic <fetch_counter_collection.csv>
            <write_counter_collection.csv> [--copy-mib 256] [--out profiles/traffic.json]

`stats` prints a table of per-kernel call counts and durations; `evicted` the
same from the kernel trace over the calls that follow a cache-evicting fill only
(the calls bench.py times, without its warm-cache pass).  `traffic`
averages FETCH_SIZE and WRITE_SIZE (KiB per dispatch) per kernel, scales both
by the factor that makes a plain device copy of a known size (an elementwise
multiply by 1 of a 256 MiB tensor) read and write exactly that size, and writes the HBM bytes
per launch of the prefill path (prep, scan and output kernels, and the index kernel where
there is one) and of the decode kernel
(or, for a backward-only run, of the backward's launches), tagged with a digest
of the kernel sources (bench.py reports the figures only while the sources are
unchanged).
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _short(name: str) -> str:
    for key in ("scan_out_kernel", "scan_pair_kernel", "scan_kernel"):
        if key in name:
            return key + (name[name.index("<"):name.index(">") + 1] if "<" in name else "")
    for key in ("prep_kernel", "index_kernel", "decode_kernel", "chunk_small_kernel",
                "zero_kernel", "gather_scatter_kernel", "grad_kernel"):
        if key in name:
            return key
    if "MulFunctor" in name or "mul_kernel" in name:
        return "torch:mul"
    if "FillFunctor" in name:
        return "torch:fill"
    if "copyBuffer" in name:
        return "runtime:copyBuffer"
    return name[:60]


def stats(path: str, cmd: str | None = None) -> str:
    rows = list(csv.DictReader(open(path)))
    lines = []
    if cmd:
        lines.append(f"command: {cmd}")
    lines.append(f"{'kernel':40s} {'calls':>6s} {'avg us':>10s} {'min us':>10s} {'max us':>10s} {'share':>7s}")
    for r in rows:
        lines.append(f"{_short(r['Name']):40s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:10.2f} "
                     f"{float(r['MinNs'])/1e3:10.2f} {float(r['MaxNs'])/1e3:10.2f} "
                     f"{float(r['Percentage']):6.2f}%")
    return "\n".join(lines)


def evicted(path: str, fill_us: float = 50.0) -> str:
    """Per-kernel durations over the library calls that follow an eviction fill
    (a torch fill of at least fill_us): a kernel seen twice since the last fill
    starts a call without one, and that call is left out."""
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    cold, seen = False, set()
    per = defaultdict(list)
    for r in rows:
        k = _short(r["Kernel_Name"])
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if k == "torch:fill" and us >= fill_us:
            cold, seen = True, set()
            continue
        if k.startswith(("torch:", "runtime:")):
            continue
        if k in seen:
            cold = False
        seen.add(k)
        if cold:
            per[k].append(us)
    lines = [f"{'kernel (after an eviction)':40s} {'calls':>6s} {'avg us':>10s} {'min us':>10s} {'max us':>10s}"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1]) / len(kv[1])):
        lines.append(f"{k:40s} {len(v):6d} {sum(v) / len(v):10.2f} {min(v):10.2f} {max(v):10.2f}")
    return "\n".join(lines)


def _counter_means(path: str, counter: str) -> dict:
    """Mean counter value (KiB) per dispatch, per kernel."""
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        vals[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}


def _copy_entry(means: dict, copy_kib: float):
    """Counter reading of the calibration copy (one elementwise multiply by 1 that
    reads and writes copy_kib KiB)."""
    return means["torch:mul"][0] if "torch:mul" in means else None


def traffic(fetch_csv: str, write_csv: str, copy_mib: float, out: str) -> dict:
    sys.path.insert(0, ROOT)
    from bench import _source_digest  # the digest bench.py checks before reporting
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    f_copy, w_copy = _copy_entry(fetch, copy_kib), _copy_entry(write, copy_kib)
    f_scale = copy_kib / f_copy if f_copy else 1.0
    w_scale = copy_kib / w_copy if w_copy else 1.0
    per = {}
    for k in sorted(set(fetch) | set(write)):
        fk = fetch.get(k, (0.0, 0))[0] * f_scale * 1024
        wk = write.get(k, (0.0, 0))[0] * w_scale * 1024
        per[k] = {"fetch_bytes": fk, "write_bytes": wk}
    both = lambda k: per[k]["fetch_bytes"] + per[k]["write_bytes"]
    prefill = sum(both(k) for k in per
                  if k in ("index_kernel", "prep_kernel") or k.startswith("scan_"))
    decode = sum(both(k) for k in per if k == "decode_kernel")
    # a backward-only run (bench.py --only backward): its index, prep and scans are the backward's
    backward = sum(both(k) for k in per if k in ("index_kernel", "prep_kernel", "grad_kernel")
                   or k.startswith("scan_")) if "grad_kernel" in per else 0
    rec = {"source_digest": _source_digest(), "prefill_bytes": (prefill or None) if not backward else None,
           "decode_bytes": decode or None, "backward_bytes": backward or None, "copy_calibration": {
               "copy_mib": copy_mib, "fetch_scale": f_scale, "write_scale": w_scale},
           "per_kernel": per}
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--command", default=None, help="the command that produced the CSV")
    e = sub.add_parser("evicted")
    e.add_argument("trace_csv")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("--copy-mib", type=float, default=256.0)
    b.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        print(stats(args.csv, args.command))
    elif args.cmd == "evicted":
        print(evicted(args.trace_csv))
    else:
        print(json.dumps(traffic(args.fetch_csv, args.write_csv, args.copy_mib, args.out), indent=1))


if __name__ == "__main__":
    main()
