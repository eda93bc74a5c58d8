"""Summaries of rocprofv3 output for the benchmark's kernels (measurement
support; nothing here runs on the product path).

Three kinds, each printed as short text with the commands that produced the
raw data, so that a summary under ``profiles/`` can be regenerated:

* ``trace``   -- kernel durations from ``--kernel-trace`` CSV: per kernel the
  call count and the mean / median / min over the last N calls (the
  benchmark's timed steps) and over all calls.
* ``traffic`` -- HBM bytes per launch from two ``--pmc`` runs (FETCH_SIZE,
  then WRITE_SIZE, KiB per dispatch), each scaled by what the same counter
  reads for a plain device copy of known size.
* ``sq``      -- shader-sequencer counters per launch from several ``--pmc``
  passes: cycles alive / issuing / waiting, matrix-core busy, instruction
  counts, LDS bank conflicts, the clock (GRBM_GUI_ACTIVE over the dispatch
  time) and occupancy, plus a cross-check of the MFMA instruction count
  against the workload's algorithmic FLOPs.

Usage (from the repository root):
  python -m io_aware_tiled_flash_amd.profsum trace --dir D --workload W --last N --cmd "..."
  python -m io_aware_tiled_flash_amd.profsum traffic --fetch D1 --write D2 --copy-fetch D3 \\
      --copy-write D4 --copy-mib 256 --workload W --kernel K --cmd "..." --cmd "..."
  python -m io_aware_tiled_flash_amd.profsum sq --dir D1 --dir D2 --workload W --kernel K \\
      --last N --cmd "..."
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

N_CU = 256
N_SIMD = 4 * N_CU
N_XCD = 8
MFMA_FLOPS = {"32x32x16": 2 * 32 * 32 * 16}


def _csv(d: str, suffix: str):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for f in files:
        rows.extend(csv.DictReader(open(f)))
    return rows


def kernel_durations(d: str):
    """{kernel name: [duration ns in dispatch order]} from a kernel trace."""
    rows = _csv(d, "kernel_trace.csv")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    by: dict[str, list[int]] = {}
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) -
                                                   int(r["Start_Timestamp"]))
    return by


def counters(d: str, match: str):
    """[(dispatch id, {counter: value}, duration ns)] for dispatches of kernels
    whose name contains `match`, in dispatch order (values summed over the
    per-die rows of one dispatch)."""
    per: dict[int, dict] = {}
    dur: dict[int, int] = {}
    for r in _csv(d, "counter_collection.csv"):
        if match not in r["Kernel_Name"]:
            continue
        i = int(r["Dispatch_Id"])
        c = per.setdefault(i, {})
        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if r.get("End_Timestamp") and r.get("Start_Timestamp"):
            dur[i] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return [(i, per[i], dur.get(i)) for i in sorted(per)]


def _header(title: str, cmds) -> list[str]:
    out = [f"# {title}", "# commands (each from the repository root, with TMPDIR=/tmp):"]
    out += [f"#   {c}" for c in cmds]
    return out + [""]


def cmd_trace(a) -> list[str]:
    by = kernel_durations(a.dir)
    tot = sum(sum(v) for v in by.values())
    out = _header(f"rocprofv3 kernel-trace summary: {a.workload}", a.cmd)
    for name, d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"kernel: {name}")
        out.append(f"  calls: {len(d)}")
        out.append(f"  average_ns (all calls): {sum(d) / len(d):.0f}")
        out.append(f"  min_ns: {min(d)}  max_ns: {max(d)}  stddev_ns: {statistics.pstdev(d):.0f}")
        out.append(f"  percentage: {100 * sum(d) / tot:.4g}")
        if a.last and len(d) >= a.last:
            last = d[-a.last:]
            out.append(f"  average_ns_last_{a.last}_calls (bench.py timed steps): "
                       f"{sum(last) / len(last):.0f}")
            out.append(f"  median_ns_last_{a.last}_calls: {statistics.median(last):.0f}")
            out.append(f"  min_ns_last_{a.last}_calls: {min(last)}")
    sys.path.insert(0, ROOT)
    import bench
    out.append(f"kernel_source_digest: {bench.kernel_source_digest(tuple(a.sources))}"
               f"  ({' '.join(a.sources)})")
    return out


def _mean_counter(rows, name):
    vals = [c[name] for _, c, _ in rows if name in c]
    return sum(vals) / len(vals), len(vals)


def cmd_traffic(a) -> list[str]:
    sys.path.insert(0, ROOT)
    import bench
    f, nf = _mean_counter(counters(a.fetch, a.kernel), "FETCH_SIZE")
    w, nw = _mean_counter(counters(a.write, a.kernel), "WRITE_SIZE")
    cf, _ = _mean_counter(counters(a.copy_fetch, a.copy_kernel), "FETCH_SIZE")
    cw, _ = _mean_counter(counters(a.copy_write, a.copy_kernel), "WRITE_SIZE")
    copy_kib = a.copy_mib * 1024
    fs, ws = copy_kib / cf, copy_kib / cw
    rd, wr = f * fs * 1024, w * ws * 1024
    out = _header(f"HBM traffic per launch of {a.kernel}: {a.workload}", a.cmd)
    out += [f"fetch_size_kib_per_dispatch: {f:.1f}   (mean over {nf} dispatches)",
            f"write_size_kib_per_dispatch: {w:.1f}   (mean over {nw} dispatches)",
            f"copy_{a.copy_mib}MiB_fetch_size_kib: {cf:.1f}",
            f"copy_{a.copy_mib}MiB_write_size_kib: {cw:.1f}",
            f"fetch_scale: {fs:.4f}",
            f"write_scale: {ws:.4f}",
            f"hbm_read_bytes_per_launch: {rd:.0f}",
            f"hbm_write_bytes_per_launch: {wr:.0f}",
            f"hbm_bytes_per_launch: {rd + wr:.0f}",
            f"kernel_source_digest: {bench.kernel_source_digest(tuple(a.sources))}"
            f"  ({' '.join(a.sources)})"]
    return out


SQ_ORDER = ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_ANY",
            "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
            "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS",
            "SQ_INSTS_SALU", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_SCA",
            "GRBM_GUI_ACTIVE"]


def cmd_sq(a) -> list[str]:
    sys.path.insert(0, ROOT)
    import bench
    from workloads import WORKLOADS
    w = WORKLOADS[a.workload]
    vals: dict[str, float] = {}
    ns: dict[str, int] = {}
    durs = []
    for d in a.dir:
        rows = counters(d, a.kernel)
        if a.last:
            rows = rows[-a.last:]
        durs += [t for _, _, t in rows if t]
        names = sorted({n for _, c, _ in rows for n in c})
        for n in names:
            vals[n], ns[n] = _mean_counter(rows, n)
    out = _header(f"shader-sequencer counters per launch of {a.kernel}: {a.workload}", a.cmd)
    out.append(f"dispatches averaged per pass: last {a.last} of the run (bench.py timed steps)")
    out.append("raw counters (mean per dispatch; SQ_*_CYCLES, SQ_WAIT_* and SQ_ACTIVE_* count "
               "in units of 4 shader cycles; GRBM_GUI_ACTIVE is summed over the 8 dies):")
    for n in SQ_ORDER + sorted(set(vals) - set(SQ_ORDER)):
        if n in vals:
            out.append(f"  {n}: {vals[n]:.6g}")
    out.append("")
    out.append("derived:")
    dur_ns = sum(durs) / len(durs) if durs else None
    if dur_ns:
        out.append(f"  dispatch_ns (counter runs, mean): {dur_ns:.0f}")
    if "GRBM_GUI_ACTIVE" in vals and dur_ns:
        ghz = vals["GRBM_GUI_ACTIVE"] / N_XCD / dur_ns
        note = ""
        if dur_ns < 100e3:
            note = ("  (not a clock: for a dispatch this short the GPU-busy count covers"
                    " more than the kernel's own span)")
        out.append(f"  clock_GHz (GRBM_GUI_ACTIVE / 8 dies / dispatch time): {ghz:.3f}{note}")
    # the kernel's own products per visible pair, 2 d FLOPs each: the forward's
    # S and P V; the backward's dK/dV kernel S, dP, dV, dK; its dQ kernel S,
    # dP, dQ
    products = (("fa_bwd_dkdv", 4, "S, dP, dV, dK"), ("fa_bwd_dq", 3, "S, dP, dQ"))
    n_prod, prod_names = 2, "S, P V"
    for key, n, names in products:
        if key in a.kernel:
            n_prod, prod_names = n, names
    flops = w.flops() * n_prod / 2
    if "SQ_INSTS_MFMA" in vals:
        mf = vals["SQ_INSTS_MFMA"]
        per = MFMA_FLOPS[a.mfma]
        out.append(f"  mfma_instructions: {mf:.6g}  x {per} flop = {mf * per:.4g} flop issued")
        out.append(f"  algorithmic_flop ({2 * n_prod} d per visible pair: {prod_names}): "
                   f"{flops:.4g}")
        out.append(f"  issued / algorithmic: {mf * per / flops:.4f} (any excess is masked work "
                   f"on tiles that straddle a band edge or lie outside a wave's band)")
    if "SQ_WAVES" in vals and "SQ_WAVE_CYCLES" in vals:
        waves = vals["SQ_WAVES"]
        out.append(f"  waves: {waves:.6g}")
        if "GRBM_GUI_ACTIVE" in vals:
            busy = vals["GRBM_GUI_ACTIVE"] / N_XCD
            occ = 4 * vals["SQ_WAVE_CYCLES"] / (busy * N_SIMD)
            out.append(f"  mean resident waves per SIMD over the dispatch: {occ:.3f}")
    if "SQ_WAVE_CYCLES" in vals:
        wc = 4 * vals["SQ_WAVE_CYCLES"]
        for n, label in (("SQ_ACTIVE_INST_ANY", "issuing"), ("SQ_WAIT_INST_ANY",
                         "waiting to issue"), ("SQ_WAIT_ANY", "waiting on counters/barrier"),
                         ("SQ_VALU_MFMA_BUSY_CYCLES", "matrix core busy")):
            if n in vals:
                scale = 1 if n == "SQ_VALU_MFMA_BUSY_CYCLES" else 4
                out.append(f"  {label}: {100 * scale * vals[n] / wc:.1f}% of wave cycles")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in vals and "GRBM_GUI_ACTIVE" in vals:
        busy = vals["GRBM_GUI_ACTIVE"] / N_XCD
        out.append(f"  matrix core busy per SIMD: "
                   f"{100 * vals['SQ_VALU_MFMA_BUSY_CYCLES'] / (busy * N_SIMD):.1f}% of the "
                   f"dispatch's cycles")
    if "SQ_LDS_BANK_CONFLICT" in vals and "SQ_INSTS_LDS" in vals:
        out.append(f"  lds_bank_conflict_cycles per LDS instruction: "
                   f"{vals['SQ_LDS_BANK_CONFLICT'] / max(vals['SQ_INSTS_LDS'], 1):.4f}")
    out.append(f"kernel_source_digest: {bench.kernel_source_digest(tuple(a.sources))}"
               f"  ({' '.join(a.sources)})")
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="kind", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--dir", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--last", type=int, default=0)
    t.add_argument("--sources", nargs="+",
                   default=["fa_fwd_mfma.hip", "fa_gfx950.h", "fa_internal.h"])
    t.add_argument("--cmd", action="append", default=[])
    f = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        f.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    f.add_argument("--copy-mib", type=int, default=256)
    f.add_argument("--copy-kernel", default="copy")
    f.add_argument("--workload", required=True)
    f.add_argument("--kernel", required=True)
    f.add_argument("--sources", nargs="+",
                   default=["fa_fwd_mfma.hip", "fa_gfx950.h", "fa_internal.h"])
    f.add_argument("--cmd", action="append", default=[])
    s = sub.add_parser("sq")
    s.add_argument("--dir", action="append", required=True)
    s.add_argument("--workload", required=True)
    s.add_argument("--kernel", required=True)
    s.add_argument("--last", type=int, default=0)
    s.add_argument("--mfma", default="32x32x16", choices=sorted(MFMA_FLOPS))
    s.add_argument("--sources", nargs="+",
                   default=["fa_fwd_mfma.hip", "fa_gfx950.h", "fa_internal.h"])
    s.add_argument("--cmd", action="append", default=[])
    a = ap.parse_args(argv)
    out = {"trace": cmd_trace, "traffic": cmd_traffic, "sq": cmd_sq}[a.kind](a)
    print("\n".join(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
