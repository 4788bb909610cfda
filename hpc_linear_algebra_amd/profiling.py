"""Summaries of rocprofv3 output (kernel statistics and PMC counters) as
short markdown, for the committed profiles.

  python -m hpc_linear_algebra_amd.profiling stats DIR --command "..." > out.md
  python -m hpc_linear_algebra_amd.profiling pmc DIR [DIR ...] --command "..." > out.md
  python -m hpc_linear_algebra_amd.profiling traffic --fetch D --write D --copy-fetch D \
         --copy-write D --kernel REGEX --out profiles/stage3_traffic_WORKLOAD.json
  python -m hpc_linear_algebra_amd.profiling mfma DIR --kernel REGEX --out profiles/stage3_mfma_WORKLOAD.json

DIR is a rocprofv3 output directory written with --output-format csv.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import re
import sys
from collections import defaultdict


def _short(name: str) -> str:
    m = re.search(r"(grouped_gemm_kernel<[^>]*>|strip_gemm_kernel<[^>]*>|single_gemm_kernel<[^>]*>|scale_kernel<[^>]*>)", name)
    if m:
        return m.group(1)
    m = re.search(r"(grouped_gemm16_kernel|wide_gemm16_kernel|strip_gemm16_kernel|scale16_kernel)I(DF16b|DF16_)((?:Li\d+E)*)", name)
    if m:
        t = "bfloat16" if m.group(2) == "DF16b" else "half"
        args = re.findall(r"Li(\d+)E", m.group(3))
        return f"{m.group(1)}<{', '.join([t] + args)}>"
    m = re.search(r"(grouped_gemm_kernel|strip_gemm_kernel|single_gemm_kernel|scale_kernel)I([df])((?:Li\d+E)*)", name)
    if m:
        t = "double" if m.group(2) == "d" else "float"
        args = re.findall(r"Li(\d+)E", m.group(3))
        return f"{m.group(1)}<{', '.join([t] + args)}>"
    return name[:90]


def _files(d: str, pattern: str):
    return sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))


def trace_stats(dirs, command: str) -> str:
    """Per-kernel durations from rocprofv3 kernel traces, one row per kernel
    symbol and grid size (the three stages of a plan have distinct grids)."""
    groups = defaultdict(list)
    for d in dirs:
        for f in _files(d, "*kernel_trace.csv"):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])))
                    groups[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    tot_all = sum(sum(v) for v in groups.values()) or 1.0
    out = [f"Command: `{command}`", "",
           "| kernel | workgroups | calls | total ms | avg us | median us | min us | max us | % |",
           "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for (k, wg), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        med = sorted(v)[len(v) // 2]
        out.append(f"| {k} | {wg} | {len(v)} | {sum(v)/1e3:.3f} | {sum(v)/len(v):.1f} | {med:.1f} | {min(v):.1f} | "
                   f"{max(v):.1f} | {100*sum(v)/tot_all:.1f} |")
    return "\n".join(out) + "\n"


def stats(dirs, command: str) -> str:
    if any(_files(d, "*kernel_trace.csv") for d in dirs):
        return trace_stats(dirs, command)
    rows = []
    for d in dirs:
        for f in _files(d, "*kernel_stats.csv"):
            with open(f) as fh:
                rows.extend(csv.DictReader(fh))
    out = [f"Command: `{command}`", "", "| kernel | calls | total ms | avg us | min us | max us | % |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = _short(r.get("Name", r.get("KernelName", "?")))
        calls = int(float(r.get("Calls", 0)))
        tot = float(r.get("TotalDurationNs", r.get("DURATION (nsec)", 0)))
        avg = float(r.get("AverageNs", r.get("AVERAGE (nsec)", 0)))
        mn = float(r.get("MinNs", r.get("MIN (nsec)", 0)))
        mx = float(r.get("MaxNs", r.get("MAX (nsec)", 0)))
        pct = float(r.get("Percentage", r.get("PERCENT (INC)", 0)))
        out.append(f"| {name} | {calls} | {tot/1e6:.3f} | {avg/1e3:.1f} | {mn/1e3:.1f} | {mx/1e3:.1f} | {pct:.1f} |")
    return "\n".join(out) + "\n"


def pmc(dirs, command: str) -> str:
    vals = defaultdict(lambda: defaultdict(list))
    for d in dirs:
        for f in _files(d, "*counter_collection.csv"):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    vals[_short(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = [f"Command: `{command}`", "", "| kernel | counter | dispatches | mean per dispatch |", "|---|---|---:|---:|"]
    for k in sorted(vals):
        for c in sorted(vals[k]):
            v = vals[k][c]
            out.append(f"| {k} | {c} | {len(v)} | {sum(v)/len(v):.6g} |")
    return "\n".join(out) + "\n"


def _counter_means(d: str):
    vals = defaultdict(list)
    for f in _files(d, "*counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                vals[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    return vals


def kernel_source_hash(sixteen_bit: bool = False) -> str:
    """Hash of the kernel sources of one family (32/64-bit: gemm.hip; 16-bit:
    gemm16.hip), so that stored counter results of a changed kernel are not
    reused."""
    import hashlib
    h = hashlib.sha256()
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    for f in ("gemm16.hip" if sixteen_bit else "gemm.hip", "tlr_desc.h"):
        h.update(open(os.path.join(here, f), "rb").read())
    return h.hexdigest()[:16]


def _matches(rx: str, name: str) -> bool:
    """rx found in a kernel name as the profiler wrote it (mangled or not) or
    in its short form (as the summaries print it)."""
    return re.search(rx, name) is not None or re.search(rx, _short(name)) is not None


def traffic(fetch_dir, write_dir, cfetch_dir, cwrite_dir, kernel_regex, copy_bytes=1 << 30):
    """HBM bytes per dispatch of the kernels matching kernel_regex: FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch), each scaled by what the same counter
    reads for a plain device copy of copy_bytes."""
    def mean_for(d, counter, rx):
        v = [x for (k, c), xs in _counter_means(d).items() if c == counter and _matches(rx, k) for x in xs]
        return sum(v) / len(v) if v else None
    cf = mean_for(cfetch_dir, "FETCH_SIZE", "copyBuffer")
    cw = mean_for(cwrite_dir, "WRITE_SIZE", "copyBuffer")
    kf = mean_for(fetch_dir, "FETCH_SIZE", kernel_regex)
    kw = mean_for(write_dir, "WRITE_SIZE", kernel_regex)
    fscale = copy_bytes / (cf * 1024.0)
    wscale = copy_bytes / (cw * 1024.0)
    rd = kf * 1024.0 * fscale
    wr = kw * 1024.0 * wscale
    return {"bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr,
            "fetch_kib_raw": kf, "write_kib_raw": kw, "fetch_scale": fscale, "write_scale": wscale,
            "kernel_regex": kernel_regex, "kernel_hash": kernel_source_hash("gemm16" in kernel_regex)}


SIMDS = 256 * 4     # MI355X: 256 compute units of 4 SIMDs
XCDS = 8            # GRBM_GUI_ACTIVE reads as the sum over the 8 XCDs


def mfma_busy(pmc_dir, kernel_regex):
    """Fraction of the kernel's active cycles in which a SIMD's matrix unit is
    busy: SQ_VALU_MFMA_BUSY_CYCLES (summed over every SIMD) divided by the
    SIMD count times the active cycles of one XCD (GRBM_GUI_ACTIVE / 8), per
    dispatch, averaged over the dispatches matching kernel_regex."""
    vals = _counter_means(pmc_dir)

    def mean_for(counter):
        v = [x for (k, c), xs in vals.items() if c == counter and _matches(kernel_regex, k) for x in xs]
        return sum(v) / len(v) if v else None
    busy, active = mean_for("SQ_VALU_MFMA_BUSY_CYCLES"), mean_for("GRBM_GUI_ACTIVE")
    frac = busy / (SIMDS * active / XCDS) if busy is not None and active else None
    return {"mfma_busy": frac, "mfma_busy_cycles": busy, "gui_active_cycles": active,
            "kernel_regex": kernel_regex, "kernel_hash": kernel_source_hash("gemm16" in kernel_regex)}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["stats", "pmc", "traffic", "mfma"])
    ap.add_argument("dirs", nargs="*")
    ap.add_argument("--command", default="")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--kernel", default=r"grouped_gemm_kernel<double, 3")
    ap.add_argument("--out")
    a = ap.parse_args(argv)
    if a.mode in ("traffic", "mfma"):
        import json
        d = (traffic(a.fetch, a.write, a.copy_fetch, a.copy_write, a.kernel) if a.mode == "traffic"
             else mfma_busy(a.dirs[0], a.kernel))
        d["command"] = a.command
        txt = json.dumps(d, indent=1)
        if a.out:
            open(a.out, "w").write(txt + "\n")
        sys.stdout.write(txt + "\n")
        return
    sys.stdout.write(stats(a.dirs, a.command) if a.mode == "stats" else pmc(a.dirs, a.command))


if __name__ == "__main__":
    main()
