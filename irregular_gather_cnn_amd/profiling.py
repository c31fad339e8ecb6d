"""rocprofv3 summaries for the benchmark: per-kernel durations and HBM traffic.

Two kinds of text summaries live under ``profiles/``:

* kernel statistics of ``rocprofv3 --kernel-trace --stats`` (the
  ``*_kernel_stats.csv`` the tool writes), one row per kernel;
* HBM traffic per dispatch from two ``rocprofv3 --pmc`` runs (``FETCH_SIZE``,
  then ``WRITE_SIZE``, in KiB per dispatch).  Those counters do not read the
  bytes one-to-one, so each is scaled by what it reads for the largest plain
  device copy the same run performs: bench.py's 1 GiB copy that measures the
  device's HBM rate (``--calib-copy-mib`` adds a copy of another size).
  Every traffic row records a hash of the kernel's sources, so a reader can
  tell whether the kernel changed after the counters were taken.

Usage (after the rocprofv3 runs, on any machine)::

    python -m irregular_gather_cnn_amd.profiling stats STATS_CSV OUT_MD "COMMAND"
    python -m irregular_gather_cnn_amd.profiling traffic FETCH_DIR WRITE_DIR COPY_MIB OUT_MD "COMMANDS"
    python -m irregular_gather_cnn_amd.profiling sq OUT_MD TITLE "COMMANDS" PMC_DIR...
    python -m irregular_gather_cnn_amd.profiling tcc ON_DIR OFF_DIR OUT_MD "COMMANDS"
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import re
import sys
from collections import defaultdict

_HERE = os.path.dirname(os.path.abspath(__file__))
_CSRC = os.path.join(_HERE, "csrc")

# benchmark name of a launch -> (pattern of the kernel symbol, source files of the kernel)
KERNELS = {
    "x_channel_minor": (r"k_x_channel_minor", ["deft_sample.hip"]),
    "fused_offset_sample": (r"k_sample_direct<[^,>]*, 1, 0>", ["deft_sample.hip", "deft_device.h"]),
    "fused_offset_sample_lds_halo": (r"k_sample<[^>]*, true", ["deft_sample.hip", "deft_device.h"]),
    "offset_conv": (r"k_sample_direct<[^,>]*, 1, 1>", ["deft_sample.hip", "deft_device.h"]),
    "sample_only": (r"k_sample_direct<[^,>]*, 1, 2>", ["deft_sample.hip", "deft_device.h"]),
    "sample_only_lds_halo": (r"k_sample<[^>]*, false", ["deft_sample.hip", "deft_device.h"]),
    "fused_gather_gemm": (r"k_igemm\b", ["deft_igemm.hip", "deft_device.h"]),
    "dwconv1d": (r"k_dwconv1d\b", ["deft_dwconv.hip"]),
    "dwpw1d": (r"k_dwpw1d\b", ["deft_dwpw.hip"]),
    "gemm_forward": (r"k_gemm_(dl|vd)<.*(DlFwd|FwdBal)|k_gemm<.*FwdOp",
                     ["deft_gemm_dl.hip", "deft_gemm.hip", "deft_device.h"]),
    "gemm_dcol": (r"k_gemm_dl<.*DlDcol|k_dcol_res\b|k_gemm<.*DcolOp", ["deft_gemm_dl.hip", "deft_gemm.hip", "deft_device.h"]),
    "gemm_dw": (r"k_gemm_(dl|ws)<.*DlDw|k_gemm<.*DwOp", ["deft_gemm_dl.hip", "deft_gemm.hip", "deft_device.h"]),
    "sample_backward": (r"k_sample_bwd<|k_sample_bwd_mf\b", ["deft_backward.hip", "deft_device.h"]),
    "sample_backward_miss": (r"k_sample_bwd_miss<", ["deft_backward.hip", "deft_device.h"]),

    "offset_weight_backward": (r"k_woff_bwd<", ["deft_backward.hip", "deft_device.h"]),
    "dx_final": (r"k_dx_final<", ["deft_backward.hip", "deft_device.h"]),
    "bias_partial": (r"k_bias_partial<", ["deft_backward.hip"]),
    "reduce_final": (r"k_reduce_final<", ["deft_backward.hip"]),
    "prep_backward": (r"k_prep_backward<", ["deft_backward.hip"]),
    "prep_forward": (r"k_prep_forward<", ["deft_sample.hip"]),
}


def source_hash(bench_name: str) -> str:
    """sha256 (first 16 hex digits) over the kernel's source files."""
    h = hashlib.sha256()
    for f in KERNELS[bench_name][1]:
        with open(os.path.join(_CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def bench_name_of(symbol: str):
    s = symbol.replace("(anonymous namespace)::", "")
    for name, (pat, _) in KERNELS.items():
        if re.search(pat, s):
            return name
    return None


def _rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError("no counter_collection.csv under %s" % d)
    out = []
    for f in files:
        with open(f) as fh:
            out.extend(csv.DictReader(fh))
    return out


def _per_dispatch(rows, counter):
    """{dispatch id: (kernel symbol, grid size, value summed over dimensions)}"""
    acc = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        k = r["Dispatch_Id"]
        sym, grid, v = acc.get(k, (r["Kernel_Name"], int(r["Grid_Size"]), 0.0))
        acc[k] = (sym, grid, v + float(r["Counter_Value"]))
    return acc


def counter_scale(disp, copy_bytes):
    """Bytes per counted KiB, from the largest plain copy dispatch of the run."""
    copies = [(v, g) for (s, g, v) in disp.values() if "copyBuffer" in s]
    if not copies:
        raise ValueError("no copy dispatch in the counter run")
    v = max(copies)[0]
    return copy_bytes / (v * 1024.0), v


def traffic_table(fetch_dir, write_dir, copy_mib):
    copy_bytes = copy_mib * (1 << 20)
    f = _per_dispatch(_rows(fetch_dir), "FETCH_SIZE")
    w = _per_dispatch(_rows(write_dir), "WRITE_SIZE")
    fs, fcopy = counter_scale(f, copy_bytes)
    ws, wcopy = counter_scale(w, copy_bytes)
    per = defaultdict(lambda: [[], []])
    for disp, idx in ((f, 0), (w, 1)):
        for sym, grid, v in disp.values():
            name = bench_name_of(sym)
            if name:
                per[name][idx].append(v)
    table = {}
    for name, (fv, wv) in per.items():
        if not fv or not wv:
            continue
        fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
        table[name] = dict(fetch_kib=fk, write_kib=wk, fetch_bytes=fk * 1024 * fs, write_bytes=wk * 1024 * ws,
                           traffic=fk * 1024 * fs + wk * 1024 * ws, dispatches=len(fv), src=source_hash(name))
    return table, dict(fetch_scale=fs, write_scale=ws, copy_fetch_kib=fcopy, copy_write_kib=wcopy,
                       copy_bytes=copy_bytes)


def write_traffic_md(path, table, calib, commands):
    lines = ["# HBM traffic per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Commands (from the repository root, on the GPU machine):", "", "```"] + commands + ["```", "",
             "Calibration: a plain device copy of %d bytes reads FETCH_SIZE %.1f KiB and WRITE_SIZE %.1f KiB per "
             "dispatch, so one counted KiB is %.4f bytes fetched and %.4f bytes written."
             % (calib["copy_bytes"], calib["copy_fetch_kib"], calib["copy_write_kib"], calib["fetch_scale"],
                calib["write_scale"]), "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched MB | written MB | traffic bytes "
             "| source hash |",
             "|---|---|---|---|---|---|---|---|"]
    for name in sorted(table):
        t = table[name]
        lines.append("| %s | %d | %.1f | %.1f | %.2f | %.2f | %d | %s |" % (
            name, t["dispatches"], t["fetch_kib"], t["write_kib"], t["fetch_bytes"] / 1e6, t["write_bytes"] / 1e6,
            int(t["traffic"]), t["src"]))
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def read_traffic(path):
    """{kernel: (traffic bytes per dispatch, source hash)} from a summary written above."""
    out = {}
    if not os.path.exists(path):
        return out
    with open(path) as fh:
        for line in fh:
            m = re.match(r"\|\s*(\w+)\s*\|\s*\d+\s*\|[^|]*\|[^|]*\|[^|]*\|[^|]*\|\s*(\d+)\s*\|\s*(\w+)\s*\|", line)
            if m:
                out[m.group(1)] = (int(m.group(2)), m.group(3))
    return out


def write_stats_md(stats_csv, path, command):
    with open(stats_csv) as fh:
        rows = list(csv.DictReader(fh))
    lines = ["# Kernel statistics (rocprofv3 --kernel-trace --stats)", "", "Command (from the repository root):", "",
             "```", command, "```", "",
             "| kernel | bench name | calls | total ms | average us | min us | max us | share % |",
             "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r.get("Name") or r.get("KernelName") or ""
        calls = int(float(r.get("Calls", 0)))
        tot = float(r.get("TotalDurationNs", 0)) / 1e6
        avg = float(r.get("AverageNs", 0)) / 1e3
        mn = float(r.get("MinNs", 0)) / 1e3
        mx = float(r.get("MaxNs", 0)) / 1e3
        pct = float(r.get("Percentage", 0))
        short = re.sub(r"\(.*", "", name.replace("(anonymous namespace)::", ""))[:70]
        lines.append("| `%s` | %s | %d | %.3f | %.1f | %.1f | %.1f | %.2f |" % (
            short, bench_name_of(name) or "", calls, tot, avg, mn, mx, pct))
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def counters_table(dirs):
    """{kernel: {counter: value per dispatch averaged over its dispatches}} from pmc runs."""
    out = defaultdict(lambda: defaultdict(list))
    for d in dirs:
        rows = _rows(d)
        names = sorted({r["Counter_Name"] for r in rows})
        for c in names:
            for sym, grid, v in _per_dispatch(rows, c).values():
                name = bench_name_of(sym)
                if name:
                    out[name][c].append(v)
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in out.items()}


SQ_COLS = ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS",
           "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VMEM", "SQ_LDS_IDX_ACTIVE",
           "SQ_LDS_BANK_CONFLICT", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]


def write_sq_md(path, table, title, commands, simds=1024, xcds=8):
    def g(t, c):
        return t.get(c)

    def pct(a, b):
        return "%.0f %%" % (100.0 * a / b) if a is not None and b else "-"

    cols = [c for c in SQ_COLS if any(c in t for t in table.values())]
    lines = ["# " + title, "", "Commands (from the repository root, on the GPU machine; R = the repository root):", "",
             "```"] + commands + ["```", "",
             "Each value is the counter summed over its hardware instances for one dispatch, averaged over the "
             "dispatches of the kernel in the run. MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / %d "
             "XCDs x %d SIMDs): GRBM_GUI_ACTIVE is summed over the %d XCDs and SQ_VALU_MFMA_BUSY_CYCLES over the "
             "SIMDs (32 busy cycles per 32x32x16 bf16 MFMA), so this is the share of the dispatch's active cycles "
             "in which an average SIMD's matrix unit was busy (MFMAs on padded rows count as busy)."
             % (xcds, simds, xcds), "",
             "| kernel | " + " | ".join(c.replace("SQ_", "") for c in cols) + " |",
             "|---|" + "---|" * len(cols)]
    order = sorted(table, key=lambda k: -(table[k].get("GRBM_GUI_ACTIVE") or table[k].get("SQ_WAVE_CYCLES") or 0))
    for k in order:
        t = table[k]
        lines.append("| %s | " % k + " | ".join("%d" % t[c] if c in t else "-" for c in cols) + " |")
    lines += ["", "Derived ratios:", "",
              "| kernel | waiting / wave cycles | waiting on a dependency / wave cycles | LDS bank-conflict cycles / "
              "LDS active cycles | VALU instructions per MFMA | MFMA busy |", "|---|---|---|---|---|---|"]
    for k in order:
        t = table[k]
        mf = g(t, "SQ_INSTS_MFMA")
        vpm = "%.0f" % (g(t, "SQ_INSTS_VALU") / mf) if mf and g(t, "SQ_INSTS_VALU") is not None else "-"
        busy = g(t, "SQ_VALU_MFMA_BUSY_CYCLES")
        act = g(t, "GRBM_GUI_ACTIVE")
        lines.append("| %s | %s | %s | %s | %s | %s |" % (
            k, pct(g(t, "SQ_WAIT_ANY"), g(t, "SQ_WAVE_CYCLES")), pct(g(t, "SQ_WAIT_INST_ANY"), g(t, "SQ_WAVE_CYCLES")),
            pct(g(t, "SQ_LDS_BANK_CONFLICT"), g(t, "SQ_LDS_IDX_ACTIVE")), vpm,
            pct(busy, act / xcds * simds if act else None)))
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def write_tcc_md(path, on, off, commands):
    lines = ["# L2 (TCC) hits and misses per dispatch, XCD-aware block order on and off", "",
             "Commands (from the repository root, on the GPU machine; R = the repository root):", "", "```"] + \
            commands + ["```", "",
                        "Each value is TCC_HIT_sum / TCC_MISS_sum for one dispatch, averaged over the kernel's "
                        "dispatches. 'off' is a build whose workgroup order is the hardware's (consecutive "
                        "workgroups on different XCDs); everything else is identical.", "",
                        "| kernel | hits (on) | misses (on) | hit rate (on) | hits (off) | misses (off) | "
                        "hit rate (off) |", "|---|---|---|---|---|---|---|"]
    for k in sorted(set(on) | set(off)):
        a, b = on.get(k, {}), off.get(k, {})

        def hr(t):
            h, m = t.get("TCC_HIT_sum"), t.get("TCC_MISS_sum")
            return "%.1f %%" % (100.0 * h / (h + m)) if h is not None and m is not None and h + m else "-"
        lines.append("| %s | %s | %s | %s | %s | %s | %s |" % (
            k, "%d" % a["TCC_HIT_sum"] if "TCC_HIT_sum" in a else "-",
            "%d" % a["TCC_MISS_sum"] if "TCC_MISS_sum" in a else "-", hr(a),
            "%d" % b["TCC_HIT_sum"] if "TCC_HIT_sum" in b else "-",
            "%d" % b["TCC_MISS_sum"] if "TCC_MISS_sum" in b else "-", hr(b)))
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def main(argv):
    if len(argv) >= 4 and argv[0] == "stats":
        write_stats_md(argv[1], argv[2], argv[3])
    elif len(argv) >= 6 and argv[0] == "traffic":
        table, calib = traffic_table(argv[1], argv[2], int(argv[3]))
        write_traffic_md(argv[4], table, calib, argv[5].split("\n"))
    elif len(argv) >= 5 and argv[0] == "sq":
        # sq OUT_MD TITLE COMMANDS DIR...
        write_sq_md(argv[1], counters_table(argv[4:]), argv[2], argv[3].split("\n"))
    elif len(argv) == 5 and argv[0] == "tcc":
        # tcc ON_DIR OFF_DIR OUT_MD COMMANDS
        write_tcc_md(argv[3], counters_table([argv[1]]), counters_table([argv[2]]), argv[4].split("\n"))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
