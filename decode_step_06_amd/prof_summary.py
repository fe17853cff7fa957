"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m decode_step_06_amd.prof_summary trace TRACE_CSV --title T --cmd C [--kernel K --last N ...]
    python -m decode_step_06_amd.prof_summary traffic --fetch FETCH_CSV --write WRITE_CSV --kernel K --last N
        --source SRC --calib-bytes B --algorithmic-bytes A --out OUT --cmd C [--cmd C ...]

``trace`` prints a markdown table of a ``--kernel-trace`` CSV (per kernel:
dispatches, mean and total duration), and for each kernel name K given the
mean over its last N dispatches (the benchmark's isolated back-to-back
launches).

``trace`` also splits those last N dispatches by grid size (one line per
grid), which separates launches of one kernel on different shapes.

``counters`` prints, for the last N dispatches of kernel K in one or more
``--pmc`` runs, the mean of every counter per dispatch, and what follows from
them, with the dispatches' mean duration (from their timestamps in the same
run, or ``--duration-us``): GRBM_GUI_ACTIVE is summed over the XCDs, so
GRBM_GUI_ACTIVE / XCDs / duration is the clock the GPU ran at;
SQ_INSTS_VALU_MFMA_MOPS_BF16 counts units of 512 FLOPs, so MOPS x 512 /
duration is the FLOP rate the matrix cores issued; SQ_VALU_MFMA_BUSY_CYCLES
is summed over the SIMDs, so over (GRBM_GUI_ACTIVE / XCDs) x SIMDs it is the
fraction of the time the matrix cores were busy.  The issued FLOP rate over
the peak at the measured clock (1024 bf16 FLOP per cycle per SIMD for the
32x32x16 form) checks the busy fraction.

``traffic`` turns two ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of the
same command into HBM bytes per launch of kernel K (mean over its last N
dispatches).  Each counter is scaled by what it reads for the command's
plain 256 MiB device copy (the first dispatch whose fetch is at least an
eighth of B; B bytes read and B written): the counters' KiB are
converted to bytes and calibrated so that the copy reads and writes exactly
B.  The output file records the kernel's source file and its SHA-256, so a
later change of the kernel invalidates the figure.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import re
import sys


def _short(name: str) -> str:
    n = re.sub(r"\(.*", "", name)
    n = n.replace("unsigned short", "bf16").replace("void ", "")
    return n[:90]


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def trace(args):
    rows = _rows(args.csv)
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    per = collections.defaultdict(list)
    for r in rows:
        per[_short(r["Kernel_Name"])].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = [f"# {args.title}", "", f"Command: `{args.cmd}`", "",
           "rocprofv3 kernel trace; durations from each dispatch's start and end timestamps.", "",
           "| kernel | dispatches | mean us | total ms |", "|---|---:|---:|---:|"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        if "ns::" not in k:
            continue
        out.append(f"| `{k}` | {len(v)} | {sum(v) / len(v) / 1e3:.2f} | {sum(v) / 1e6:.3f} |")
    for i, kern in enumerate(args.kernel):
        last = args.last[i] if i < len(args.last) else 0
        sel = [r for r in rows if kern in r["Kernel_Name"]]
        sel = sel[-last:] if last else sel
        if not sel:
            continue
        d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in sel]
        out += ["", f"Last {len(d)} dispatches of `{kern}` (the isolated back-to-back launches): "
                    f"mean {sum(d) / len(d) / 1e3:.3f} us."]
        grids = collections.OrderedDict()
        for r, dd in zip(sel, d):
            grids.setdefault(r.get("Grid_Size_X", "?"), []).append(dd)
        if len(grids) > 1:
            for g, v in grids.items():
                out.append(f"- grid {g}: {len(v)} dispatches, mean {sum(v) / len(v) / 1e3:.3f} us")
        if len(d) <= 32:
            out.append("- in dispatch order (us): " + ", ".join(f"{x / 1e3:.1f}" for x in d))
    print("\n".join(out))


def counters(args):
    per = collections.OrderedDict()
    dur = {}
    for path in args.csv:
        rows = _rows(path)
        names = sorted({r["Counter_Name"] for r in rows})
        for name in names:
            vals = [v for d, (n, v) in sorted(_counter(rows, name).items()) if args.kernel in n][-args.last:]
            if vals:
                per[name] = sum(vals) / len(vals)
        for r in rows:  # each dispatch's own duration in the counter run, when recorded
            if args.kernel in r["Kernel_Name"] and r.get("Start_Timestamp"):
                dur[int(r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    if not per:
        sys.exit(f"no dispatches of {args.kernel}")
    lines = [f"# Counters of {args.kernel}: mean per dispatch over its last {args.last} dispatches",
             *[f"# command: {c}" for c in args.cmd]]
    lines += [f"{k}: {v:.1f}" for k, v in per.items()]
    if not args.duration_us and dur:
        tail = [v for _, v in sorted(dur.items())][-args.last:]
        args.duration_us = sum(tail) / len(tail) / 1e3
        lines.append(f"duration_us (the same dispatches in this counter run): {args.duration_us:.3f}")
    elif args.duration_us:
        lines.append(f"duration_us (kernel trace): {args.duration_us:.3f}")
    cycles = per["GRBM_GUI_ACTIVE"] / args.xcds if "GRBM_GUI_ACTIVE" in per else None
    mhz = None
    if args.duration_us and cycles is not None:
        mhz = cycles / args.duration_us
        lines.append(f"clock_mhz (GRBM_GUI_ACTIVE / {args.xcds} XCDs / duration): {mhz:.0f}")
    if args.duration_us and "SQ_INSTS_VALU_MFMA_MOPS_BF16" in per:
        tf = per["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / (args.duration_us * 1e-6) / 1e12
        lines.append(f"mfma_bf16_tflops_issued (MOPS x 512 / duration): {tf:.1f}")
        if mhz:
            peak = 1024.0 * args.simds * mhz * 1e6 / 1e12
            lines.append(f"mfma_bf16_peak_tflops_at_this_clock (1024 x {args.simds} SIMDs x clock): {peak:.1f}")
            lines.append(f"issued_over_peak_at_this_clock: {tf / peak:.3f}")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in per and cycles:
        frac = per["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * args.simds)
        lines.append(f"mfma_busy_fraction (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {args.xcds} x {args.simds} "
                     f"SIMDs)): {frac:.3f}")
    # wave-time shares: the SQ wave counters all count in 4-cycle units
    if per.get("SQ_WAVE_CYCLES"):
        for name, what in (("SQ_WAIT_INST_ANY", "waiting to issue an instruction"),
                           ("SQ_WAIT_ANY", "waiting on a counter or barrier"),
                           ("SQ_WAIT_INST_LDS", "waiting to issue an LDS instruction"),
                           ("SQ_ACTIVE_INST_ANY", "issuing instructions")):
            if name in per:
                lines.append(f"share_of_wave_time {what} ({name} / SQ_WAVE_CYCLES): "
                             f"{per[name] / per['SQ_WAVE_CYCLES']:.3f}")
    if "SQ_LDS_BANK_CONFLICT" in per and per.get("SQ_LDS_IDX_ACTIVE"):
        busy = per["SQ_LDS_IDX_ACTIVE"] - per["SQ_LDS_BANK_CONFLICT"]
        if busy > 0:
            lines.append(f"lds_bank_conflict_rate (SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - "
                         f"SQ_LDS_BANK_CONFLICT)): {per['SQ_LDS_BANK_CONFLICT'] / busy:.3f}")
    if args.out:
        with open(args.out, "w") as f:
            f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter(rows, name):
    """Dispatch id -> (kernel name, counter value)."""
    out = {}
    for r in rows:
        if r["Counter_Name"] != name:
            continue
        did = int(r["Dispatch_Id"])
        prev = out.get(did, (r["Kernel_Name"], 0.0))[1]
        out[did] = (r["Kernel_Name"], prev + float(r["Counter_Value"]))
    return out


def traffic(args):
    fetch = _counter(_rows(args.fetch), "FETCH_SIZE")
    write = _counter(_rows(args.write), "WRITE_SIZE")
    # the copy is the first dispatch that reads a substantial part of its
    # bytes (the fill before it reads nothing; kernels drawing inputs come
    # after it)
    big = [d for d, (n, v) in sorted(fetch.items()) if v * 1024.0 >= args.calib_bytes / 8]
    if not big:
        sys.exit("calibration copy not found")
    calib = big[0]
    f_calib_kib = fetch[calib][1]
    w_calib_kib = write.get(calib, (None, 0.0))[1]
    if f_calib_kib <= 0 or w_calib_kib <= 0:
        sys.exit("calibration copy not found in both runs")
    f_scale = args.calib_bytes / (f_calib_kib * 1024.0)
    w_scale = args.calib_bytes / (w_calib_kib * 1024.0)
    kf = [v for d, (n, v) in sorted(fetch.items()) if args.kernel in n][-args.last:]
    kw = [v for d, (n, v) in sorted(write.items()) if args.kernel in n][-args.last:]
    if not kf or not kw:
        sys.exit(f"no dispatches of {args.kernel}")
    fk, wk = sum(kf) / len(kf), sum(kw) / len(kw)
    fb, wb = fk * 1024.0 * f_scale, wk * 1024.0 * w_scale
    digest = hashlib.sha256(open(args.source, "rb").read()).hexdigest()
    lines = [f"# HBM traffic of {args.kernel}: rocprofv3 FETCH_SIZE and WRITE_SIZE, calibrated",
             *[f"# command: {c}" for c in args.cmd],
             f"kernel: {args.kernel}",
             f"source: {os.path.relpath(args.source)}",
             f"source_sha256: {digest}",
             f"dispatches_averaged: {len(kf)}",
             f"fetch_kib_per_dispatch: {fk:.1f}",
             f"write_kib_per_dispatch: {wk:.1f}",
             f"calibration_copy_bytes: {args.calib_bytes}",
             f"calibration_fetch_kib: {f_calib_kib:.1f}",
             f"calibration_write_kib: {w_calib_kib:.1f}",
             f"fetch_scale: {f_scale:.4f}",
             f"write_scale: {w_scale:.4f}",
             f"fetch_bytes_per_launch: {fb:.0f}",
             f"write_bytes_per_launch: {wb:.0f}",
             f"traffic_bytes_per_launch: {fb + wb:.0f}",
             f"algorithmic_bytes_per_launch: {args.algorithmic_bytes}",
             f"traffic_over_algorithmic: {(fb + wb) / max(1, args.algorithmic_bytes):.3f}"]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("--title", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--kernel", action="append", default=[])
    t.add_argument("--last", type=int, action="append", default=[])
    t.set_defaults(fn=trace)
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--last", type=int, required=True)
    c.add_argument("--duration-us", type=float, default=0.0)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--simds", type=int, default=1024)
    c.add_argument("--out", default="")
    c.add_argument("--cmd", action="append", default=[])
    c.set_defaults(fn=counters)
    r = sub.add_parser("traffic")
    r.add_argument("--fetch", required=True)
    r.add_argument("--write", required=True)
    r.add_argument("--kernel", required=True)
    r.add_argument("--last", type=int, required=True)
    r.add_argument("--source", required=True)
    r.add_argument("--calib-bytes", type=int, default=256 << 20)
    r.add_argument("--algorithmic-bytes", type=int, required=True)
    r.add_argument("--out", required=True)
    r.add_argument("--cmd", action="append", default=[])
    r.set_defaults(fn=traffic)
    args = ap.parse_args(argv)
    args.fn(args)


if __name__ == "__main__":
    main()
