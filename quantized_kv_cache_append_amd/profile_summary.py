"""Turn rocprofv3 CSV output of bench.py runs into the short text summaries kept
under profiles/ (and read back by bench.py).

  python -m quantized_kv_cache_append_amd.profile_summary stats DIR OUT --command CMD
      kernel-trace statistics (--kernel-trace --stats): calls and average
      duration of every libkvq kernel.

  python -m quantized_kv_cache_append_amd.profile_summary traffic FETCH_DIR WRITE_DIR COPY_MIB WORKLOAD OUT
        --command CMD
      HBM traffic of the decode-partials kernel from two --pmc runs (FETCH_SIZE,
      then WRITE_SIZE, in KiB per dispatch). Each counter is scaled by what it
      reads for a plain device-to-device copy of COPY_MIB MiB in the same run
      (bench.py --copy-probe-mb), so that the figure is in true bytes.

  python -m quantized_kv_cache_append_amd.profile_summary counters OUT --command CMD DIR [DIR ...]
      SQ/GRBM counters of the decode-partials kernel from --pmc runs (one
      directory per pass): the median per dispatch of each counter (summed
      over the GPU's instances), instructions per wave, and the share of the
      kernel's cycles each SIMD spent issuing VALU and MFMA work.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import re
import statistics
import sys

DECODE = re.compile(r"decode_(mx|mha|fast|generic)_kernel")
COPY = "__amd_rocclr_copyBuffer"


def _csv(d, suffix):
    paths = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not paths:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for p in paths:
        with open(p) as f:
            rows.extend(csv.DictReader(f))
    return rows


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("kvq::", "")
    return re.sub(r"\(.*", "", name)


def stats(d, out, command):
    rows = _csv(d, "kernel_stats.csv")
    lines = [f"# rocprofv3 kernel-trace statistics of: {command}",
             "# kernel | calls | average us | min us | max us | share of GPU time %"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        if "kvq" not in r["Name"]:
            continue
        lines.append(f"{_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _per_dispatch(rows, counter):
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = (r["Dispatch_Id"], r["Kernel_Name"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return per


def traffic(fetch_dir, write_dir, copy_mib, workload, out, command, source_hash):
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _per_dispatch(_csv(d, "counter_collection.csv"), counter)
        dec = [v for (i, n), v in per.items() if DECODE.search(n)]
        cop = sorted((v for (i, n), v in per.items() if COPY in n), reverse=True)[:3]
        if not dec or not cop:
            raise SystemExit(f"{counter}: decode dispatches {len(dec)}, copy dispatches {len(cop)}")
        factor = copy_mib * 1024.0 / statistics.median(cop)
        res[counter] = (statistics.median(dec), statistics.median(cop), factor)
    fk, fc, ff = res["FETCH_SIZE"]
    wk, wc, wf = res["WRITE_SIZE"]
    total = (fk * ff + wk * wf) * 1024.0
    lines = [
        f"# HBM traffic of the decode-partials kernel, rocprofv3 --pmc FETCH_SIZE then WRITE_SIZE of: {command}",
        f"# counters in KiB per dispatch (median over dispatches); each scaled by its reading for a plain",
        f"# device-to-device copy of {copy_mib} MiB (__amd_rocclr_copyBuffer) in the same run",
        f"workload: {workload}",
        f"source_hash: {source_hash}",
        f"fetch_kib_per_dispatch: {fk:.1f}",
        f"copy_fetch_kib: {fc:.1f}",
        f"fetch_scale: {ff:.4f}",
        f"write_kib_per_dispatch: {wk:.1f}",
        f"copy_write_kib: {wc:.1f}",
        f"write_scale: {wf:.4f}",
        f"traffic_bytes_per_launch: {total:.0f}",
    ]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# gfx950: 8 XCDs, 256 compute units of 4 SIMDs
XCDS, SIMDS = 8, 1024


def counters(dirs, out, command):
    med = {}
    kernel = None
    for d in dirs:
        rows = _csv(d, "counter_collection.csv")
        names = sorted({r["Counter_Name"] for r in rows})
        for cn in names:
            per = {k: v for k, v in _per_dispatch(rows, cn).items() if DECODE.search(k[1])}
            if per:
                med[cn] = statistics.median(per.values())
                kernel = kernel or _short(next(iter(per))[1])
    lines = [f"# rocprofv3 --pmc counters of the decode-partials kernel ({kernel}); passes of: {command}",
             "# median per dispatch, each counter summed over its instances (SQ per shader engine,",
             "# GRBM per XCD)"]
    for cn in sorted(med):
        lines.append(f"{cn}: {med[cn]:.0f}")
    waves = med.get("SQ_WAVES")
    if waves:
        for cn, label in (("SQ_INSTS_VALU", "valu_insts_per_wave"), ("SQ_INSTS_MFMA", "mfma_insts_per_wave"),
                          ("SQ_INSTS_LDS", "lds_insts_per_wave")):
            if cn in med:
                lines.append(f"{label}: {med[cn] / waves:.0f}")
    gui = med.get("GRBM_GUI_ACTIVE")
    if gui:
        cyc = gui / XCDS   # the kernel's cycles (each XCD counts its own busy clocks)
        lines.append(f"kernel_cycles_per_xcd: {cyc:.0f}")
        if "SQ_ACTIVE_INST_VALU" in med:   # quad-cycles, summed over the SIMDs
            lines.append(f"valu_issue_share_per_simd: {med['SQ_ACTIVE_INST_VALU'] * 4 / SIMDS / cyc:.3f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med:   # cycles, summed over the SIMDs
            lines.append(f"mfma_busy_share_per_simd: {med['SQ_VALU_MFMA_BUSY_CYCLES'] / SIMDS / cyc:.3f}")
    # shares of the waves' lifetime (all three in quad-cycles per wave, summed):
    # issuing an instruction, ready but waiting to be issued, and stopped at a
    # dependency (a wait counter, a barrier)
    if "SQ_WAVE_CYCLES" in med:
        for cn, label in (("SQ_ACTIVE_INST_ANY", "wave_time_issuing"), ("SQ_WAIT_INST_ANY", "wave_time_waiting_for_issue"),
                          ("SQ_WAIT_ANY", "wave_time_waiting_on_dependencies")):
            if cn in med:
                lines.append(f"{label}: {med[cn] / med['SQ_WAVE_CYCLES']:.3f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    a.add_argument("out")
    a.add_argument("--command", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("fetch_dir")
    b.add_argument("write_dir")
    b.add_argument("copy_mib", type=int)
    b.add_argument("workload")
    b.add_argument("out")
    b.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("out")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--command", required=True)
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        stats(args.dir, args.out, args.command)
    elif args.cmd == "counters":
        counters(args.dirs, args.out, args.command)
    else:
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        sys.path.insert(0, root)
        import bench
        traffic(args.fetch_dir, args.write_dir, args.copy_mib, args.workload, args.out, args.command,
                bench.source_hash())


if __name__ == "__main__":
    main()
