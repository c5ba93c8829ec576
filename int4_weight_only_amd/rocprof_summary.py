"""Summaries of rocprofv3 output for the library's kernels.

    python -m int4_weight_only_amd.rocprof_summary stats DIR [--filter w4::]
    python -m int4_weight_only_amd.rocprof_summary pmc DIR [--filter w4::]
                                                   [--calib bitwise_not BYTES]
    python -m int4_weight_only_amd.rocprof_summary sweep DIR

``DIR`` is a rocprofv3 output directory written with ``--output-format csv``.

* ``stats``: per kernel, the calls and the average / min / max duration
  from the kernel-statistics file (microseconds).
* ``sweep``: the decode products of bench.py's headline sweep from the
  kernel trace: dispatches in order, where the four launches of a step
  (M = 1, 8, 16 by k_decode16, then M = 32 by k_decode32) repeat, each
  attributed to its M; per M the count and the mean / median / min
  duration (microseconds).
* ``pmc``: per kernel, the mean per dispatch of every counter in the
  counter-collection file, plus derived figures where their inputs are
  present:
  - MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs) over
    the dispatch, the MFMA pipe's share of the kernel's cycles on every
    SIMD (rocprofv3's MfmaUtil);
  - MFMA co-exec % = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES,
    the MFMA-busy cycles in which a plain VALU op also issued;
  - VALU and MFMA instructions per wave = SQ_INSTS_VALU / SQ_WAVES and
    SQ_INSTS_MFMA / SQ_WAVES;
  - the clock those cycles imply, where the same run also wrote a kernel
    trace (GRBM_GUI_ACTIVE cycles over the dispatch's duration), which
    checks the per-XCD reading of GRBM_GUI_ACTIVE below;
  - HBM bytes = FETCH_SIZE x f_read + WRITE_SIZE x f_write (KiB -> bytes),
    with the factors taken from a calibration kernel of known traffic
    (``--calib NAME BYTES``: a kernel whose name contains NAME that reads
    and writes BYTES bytes each per dispatch).

GRBM_GUI_ACTIVE is reported by rocprofv3 summed over the XCDs; it is
divided by the XCD count (8 on MI355X) to get the kernel's cycles.
"""

import argparse
import collections
import csv
import glob
import os
import sys

SIMDS = 256 * 4          # MI355X: 256 CUs x 4 SIMDs
XCDS = 8


def _find(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits


def short_name(name):
    """Demangled kernel name without the argument list."""
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def stats(d, flt):
    rows = []
    for path in _find(d, "kernel_stats.csv"):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                name = short_name(r["Name"])
                if flt and flt not in name:
                    continue
                rows.append((name, int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                             float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                             float(r["TotalDurationNs"]) / 1e3))
    rows.sort(key=lambda x: -x[5])
    out = [f"{'kernel':<72} {'calls':>7} {'avg_us':>10} {'min_us':>10} {'max_us':>10} "
           f"{'total_us':>12}"]
    for name, calls, avg, mn, mx, tot in rows:
        out.append(f"{name:<72} {calls:>7} {avg:>10.3f} {mn:>10.3f} {mx:>10.3f} {tot:>12.1f}")
    return "\n".join(out)


def sweep(d):
    disp = []
    for path in _find(d, "kernel_trace.csv"):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                name = short_name(r["Kernel_Name"])
                if "k_decode16" in name or "k_decode32" in name:
                    disp.append((int(r["Start_Timestamp"]), name,
                                 (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    disp.sort()
    kinds = ["k_decode16", "k_decode16", "k_decode16", "k_decode32"]
    ms = (1, 8, 16, 32)
    per = {m: [] for m in ms}
    i = 0
    while i + 4 <= len(disp):
        if all(kinds[j] in disp[i + j][1] for j in range(4)):
            for j in range(4):
                per[ms[j]].append(disp[i + j][2])
            i += 4
        else:
            i += 1
    out = [f"{'M':>4} {'launches':>9} {'mean_us':>9} {'median_us':>10} {'min_us':>8}"]
    for m in ms:
        v = sorted(per[m])
        if v:
            out.append(f"{m:>4} {len(v):>9} {mean(v):>9.3f} {v[len(v) // 2]:>10.3f} {v[0]:>8.3f}")
    allv = [x for m in ms for x in per[m]]
    if allv:
        out.append(f"all  {len(allv):>9} {mean(allv):>9.3f}   (sweep steps: {len(per[1])})")
    return "\n".join(out)


def pmc_table(d):
    """{kernel: {counter: [value per dispatch]}} from counter-collection files."""
    per = collections.defaultdict(lambda: collections.defaultdict(dict))
    for path in _find(d, "counter_collection.csv"):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                name = short_name(r["Kernel_Name"])
                disp = (path, r["Dispatch_Id"])
                c = r["Counter_Name"]
                per[name][c][disp] = per[name][c].get(disp, 0.0) + float(r["Counter_Value"])
    return {k: {c: list(v.values()) for c, v in cs.items()} for k, cs in per.items()}


def mean(xs):
    return sum(xs) / len(xs) if xs else float("nan")


def trace_durations(d):
    """{kernel: [duration us per dispatch]} from kernel-trace files, if any."""
    out = collections.defaultdict(list)
    for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                out[short_name(r["Kernel_Name"])].append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return out


def pmc(d, flt, calib):
    tab = pmc_table(d)
    durs = trace_durations(d)
    f_read = f_write = None
    if calib:
        cname, nbytes = calib[0], float(calib[1])
        cal = [v for k, v in tab.items() if cname in k]
        if cal:
            if "FETCH_SIZE" in cal[0]:
                f_read = nbytes / (mean(cal[0]["FETCH_SIZE"]) * 1024.0)
            if "WRITE_SIZE" in cal[0]:
                f_write = nbytes / (mean(cal[0]["WRITE_SIZE"]) * 1024.0)
    lines = []
    if f_read is not None or f_write is not None:
        lines.append(f"calibration ({calib[0]}, {int(float(calib[1]))} B read and written per "
                     f"dispatch): read factor {f_read}, write factor {f_write}")
    for name in sorted(tab):
        if flt and flt not in name:
            continue
        cs = tab[name]
        n = max(len(v) for v in cs.values())
        parts = [f"{c} {mean(v):.1f}" for c, v in sorted(cs.items())]
        lines.append(f"{name}  (dispatches {n})")
        lines.append("    " + ", ".join(parts))
        g = mean(cs["GRBM_GUI_ACTIVE"]) / XCDS if "GRBM_GUI_ACTIVE" in cs else None
        derived = []
        if g and "SQ_VALU_MFMA_BUSY_CYCLES" in cs:
            busy = mean(cs["SQ_VALU_MFMA_BUSY_CYCLES"])
            derived.append(f"MFMA busy {100.0 * busy / (g * SIMDS):.1f}%")
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in cs and busy > 0:
                derived.append(f"MFMA co-exec {100.0 * mean(cs['SQ_VALU_MFMA_COEXEC_CYCLES']) / busy:.1f}%")
        if "SQ_WAVES" in cs and mean(cs["SQ_WAVES"]) > 0:
            w = mean(cs["SQ_WAVES"])
            for c, label in (("SQ_INSTS_VALU", "VALU"), ("SQ_INSTS_MFMA", "MFMA")):
                if c in cs:
                    derived.append(f"{label} insts/wave {mean(cs[c]) / w:.1f}")
        if g:
            derived.append(f"kernel cycles {g:.0f}")
            if name in durs and durs[name]:
                derived.append(f"mean duration {mean(durs[name]):.2f} us, "
                               f"implied clock {g / mean(durs[name]) / 1e3:.2f} GHz")
        if "FETCH_SIZE" in cs and f_read is not None:
            derived.append(f"HBM read {mean(cs['FETCH_SIZE']) * 1024.0 * f_read / 1e6:.3f} MB")
        if "WRITE_SIZE" in cs and f_write is not None:
            derived.append(f"HBM write {mean(cs['WRITE_SIZE']) * 1024.0 * f_write / 1e6:.3f} MB")
        if derived:
            lines.append("    -> " + "; ".join(derived))
    return "\n".join(lines)


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("mode", choices=("stats", "pmc", "sweep"))
    p.add_argument("dir")
    p.add_argument("--filter", default="")
    p.add_argument("--calib", nargs=2, metavar=("NAME", "BYTES"))
    a = p.parse_args(argv)
    if a.mode == "stats":
        print(stats(a.dir, a.filter))
    elif a.mode == "sweep":
        print(sweep(a.dir))
    else:
        print(pmc(a.dir, a.filter, a.calib))


if __name__ == "__main__":
    sys.exit(main())
