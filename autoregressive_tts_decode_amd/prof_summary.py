"""Summarise a rocprofv3 --kernel-trace --stats run of bench.py as text.

    python -m autoregressive_tts_decode_amd.prof_summary <prefix> [--frames K]
    python -m autoregressive_tts_decode_amd.prof_summary <prefix> --pmc COUNTER [--kernel NAME]
    python -m autoregressive_tts_decode_amd.prof_summary <prefix> --shapes --run-frames F [--exclude A,B]

With --pmc, <prefix>_counter_collection.csv of a rocprofv3 --pmc run is read instead and the
per-dispatch average of COUNTER is printed for every kernel (or the kernels whose name contains
NAME).

With --shapes, the kernel trace is grouped by kernel and launch shape (grid threads in x and
the grid's z extent, which for the split-K GEMMs is the slice count): launches and kernel time
per frame over the run's F frames, kernels named in --exclude (the prompt pass's) left out.

<prefix> is the path prefix rocprofv3 wrote (…/bench): it reads
<prefix>_kernel_stats.csv and <prefix>_kernel_trace.csv. The frame loop is
identified in the trace as the last K frames' kernels (every frame ends with
the semantic-head GEMV that advances the device counters); the per-frame
kernel-time sum and wall span are reported next to the per-kernel table.
"""
from __future__ import annotations

import argparse
import csv
from collections import defaultdict


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("prefix")
    ap.add_argument("--frames", type=int, default=0, help="timed frames at the end of the trace")
    ap.add_argument("--kernels-per-frame", type=int, default=0)
    ap.add_argument("--top", type=int, default=16)
    ap.add_argument("--pmc", default="")
    ap.add_argument("--kernel", default="")
    ap.add_argument("--shapes", action="store_true")
    ap.add_argument("--run-frames", type=int, default=0, help="frames in the whole run (--shapes)")
    ap.add_argument("--exclude", default="", help="comma-separated kernel name parts to leave out (--shapes)")
    a = ap.parse_args()
    if a.shapes:
        if a.run_frames <= 0:
            raise SystemExit("--shapes needs --run-frames")
        skip = [x for x in a.exclude.split(",") if x]
        busy, cnt = defaultdict(float), defaultdict(int)
        for r in csv.DictReader(open(a.prefix + "_kernel_trace.csv")):
            if any(x in r["Kernel_Name"] for x in skip):
                continue
            key = (r["Kernel_Name"].replace("tts::", "")[:44], int(r["Grid_Size_X"]), int(r["Grid_Size_Z"]))
            busy[key] += int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            cnt[key] += 1
        F = a.run_frames
        print(f"per frame over {F} frames: {sum(cnt.values()) / F:.0f} launches, {sum(busy.values()) / F / 1e3:.1f} us of kernels")
        print(f"{'kernel':44s} {'grid x':>8s} {'z':>3s} {'per frame':>9s} {'avg us':>7s} {'us/frame':>9s}")
        for k in sorted(busy, key=lambda k: -busy[k]):
            print(f"{k[0]:44s} {k[1]:8d} {k[2]:3d} {cnt[k] / F:9.1f} {busy[k] / cnt[k] / 1e3:7.2f} {busy[k] / F / 1e3:9.1f}")
        return
    if a.pmc:
        vals = defaultdict(list)
        for r in csv.DictReader(open(a.prefix + "_counter_collection.csv")):
            if r["Counter_Name"] == a.pmc and a.kernel in r["Kernel_Name"]:
                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        print(f"{'kernel':78s} {'dispatches':>10s} {a.pmc + ' avg':>16s} {'min':>14s} {'max':>14s}")
        for k, v in sorted(vals.items(), key=lambda kv: -sum(kv[1])):
            print(f"{k[:78]:78s} {len(v):10d} {sum(v) / len(v):16.1f} {min(v):14.1f} {max(v):14.1f}")
        return
    rows = list(csv.DictReader(open(a.prefix + "_kernel_stats.csv")))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    print(f"total kernel time in the run: {tot / 1e6:.2f} ms over {sum(int(r['Calls']) for r in rows)} launches")
    print(f"{'kernel':78s} {'calls':>7s} {'avg us':>8s} {'min us':>8s} {'share':>6s}")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"]))[: a.top]:
        print(f"{r['Name'][:78]:78s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:8.2f} "
              f"{float(r['MinNs']) / 1e3:8.2f} {float(r['TotalDurationNs']) / tot * 100:5.1f}%")
    if a.frames and a.kernels_per_frame:
        tr = list(csv.DictReader(open(a.prefix + "_kernel_trace.csv")))
        tr.sort(key=lambda r: int(r["Start_Timestamp"]))
        n = a.frames * a.kernels_per_frame
        tail = tr[-n:]
        busy = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in tail)
        span = int(tail[-1]["End_Timestamp"]) - int(tail[0]["Start_Timestamp"])
        per = defaultdict(float)
        for r in tail:
            per[r["Kernel_Name"]] += int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        print(f"\nlast {a.frames} frames ({a.kernels_per_frame} kernels each): kernel time {busy / a.frames / 1e3:.1f} us/frame, "
              f"wall span {span / a.frames / 1e3:.1f} us/frame")


if __name__ == "__main__":
    main()
