"""Summaries of rocprofv3 output for the attention kernels.

``python -m tiled_online_softmax_02_amd.profiling stats <kernel_stats.csv> <out.txt> "<command>"``
    writes the per-kernel average durations of a ``rocprofv3 --kernel-trace --stats`` run.

``python -m tiled_online_softmax_02_amd.profiling traffic <fetch.csv> <write.csv> <workload> <out_dir> "<commands>"``
    turns two ``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of ``bench.py`` into
    HBM bytes per launch for each attention kernel.  Both counters are scaled by what they read
    for the plain device-to-device copy that bench.py performs before its timed region (its
    size is known: 256 MiB read, 256 MiB written), which calibrates the counter units.
    One file ``hbm_traffic_<kernel>_<workload>.txt`` is written per kernel; bench.py reports it
    as ``roofline.traffic`` while the kernel sources are unchanged.

``python -m tiled_online_softmax_02_amd.profiling sq <out.txt> "<commands>" <pass1.csv> <pass2.csv> ...``
    averages ``rocprofv3 --pmc`` SQ counters per dispatch for each attention kernel and derives
    the matrix-core busy fraction and the vector and LDS instruction activity per SIMD.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["attn_device.h", "attn_sched.h", "attn_fwd.hip", "attn_bwd.hip", "attn_fwd_fp8.hip"]
CALIBRATION_BYTES = 256 << 20   # bench.py copies 64 Mi int32 values before timing
SHORT = {"fwd_kernel": "fwd", "fwd_decode_kernel": "fwd_decode", "fwd_fp8_kernel": "fwd_fp8",
         "fwd_combine_kernel": "combine", "bwd_dkdv2_kernel": "dkdv",
         "bwd_dkdv4_kernel": "dkdv", "bwd_dq_kernel": "dq",
         "bwd_preprocess_kernel": "preprocess"}


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(PKG, "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(full: str) -> str | None:
    for key, short in SHORT.items():
        if key in full:
            return short
    return None


def stats_summary(stats_csv: str, command: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = ["rocprofv3 --kernel-trace --stats summary", "command: " + command, "",
             "%-12s %6s %12s %12s %12s %7s" % ("kernel", "calls", "avg_us", "min_us", "max_us", "pct")]
    for r in rows:
        name = short_name(r["Name"]) or r["Name"][:40]
        lines.append("%-12s %6s %12.2f %12.2f %12.2f %7.2f" % (
            name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            100.0 * float(r["TotalDurationNs"]) / total))
    lines.append("")
    lines.append("kernel source sha (%s): %s" % (", ".join(KERNEL_SOURCES), kernel_source_sha()))
    return "\n".join(lines) + "\n"


def counter_per_kernel(path: str, counter: str):
    """Average counter value (KiB) per dispatch for each attention kernel, and for "copy" the
    largest copy dispatch (the calibration copy; the runtime may add small copies of its own)."""
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        key = short_name(name) or ("copy" if "copyBuffer" in name else None)
        if key:
            vals[key].append(float(r["Counter_Value"]))
    return {k: (max(v) if k == "copy" else sum(v) / len(v)) for k, v in vals.items()}


def traffic_summaries(fetch_csv: str, write_csv: str, workload: str, out_dir: str, commands: str) -> list[str]:
    fetch = counter_per_kernel(fetch_csv, "FETCH_SIZE")
    write = counter_per_kernel(write_csv, "WRITE_SIZE")
    f_factor = CALIBRATION_BYTES / (fetch["copy"] * 1024.0)
    w_factor = CALIBRATION_BYTES / (write["copy"] * 1024.0)
    sha = kernel_source_sha()
    written = []
    for k in sorted(set(fetch) & set(write)):
        if k == "copy":
            continue
        fb = fetch[k] * 1024.0 * f_factor
        wb = write[k] * 1024.0 * w_factor
        rec = {"kernel": k, "workload": workload, "hbm_bytes_per_launch": fb + wb, "fetch_bytes": fb,
               "write_bytes": wb, "fetch_kib_raw": fetch[k], "write_kib_raw": write[k],
               "fetch_scale": f_factor, "write_scale": w_factor, "kernel_source_sha": sha}
        text = "\n".join([
            "HBM traffic per launch of the %s kernel, workload %s" % (k, workload),
            "commands: " + commands,
            "calibration: device copy of %d bytes reads FETCH_SIZE=%.1f KiB, WRITE_SIZE=%.1f KiB"
            % (CALIBRATION_BYTES, fetch["copy"], write["copy"]),
            "scale factors: fetch x%.4f, write x%.4f" % (f_factor, w_factor),
            "fetch %.1f MiB + write %.1f MiB = %.1f MiB per launch" % (fb / 2**20, wb / 2**20, (fb + wb) / 2**20),
            "JSON: " + json.dumps(rec), ""])
        path = os.path.join(out_dir, "hbm_traffic_%s_%s.txt" % (k, workload))
        with open(path, "w") as f:
            f.write(text)
        written.append(path)
    return written


# MI355X: 256 CUs of 4 SIMDs in 32 shader engines; the SQ cycle counters are summed over the
# engines, the wave-level activity counters count 4-cycle units summed over waves.
N_SE, N_SIMD = 32, 1024


def sq_summary(csvs: list[str], commands: str) -> str:
    vals = defaultdict(lambda: defaultdict(list))
    for path in csvs:
        for r in csv.DictReader(open(path)):
            k = short_name(r["Kernel_Name"])
            if k:
                vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = ["rocprofv3 SQ counters, average per dispatch", "commands: " + commands, ""]
    for k in sorted(vals):
        c = {n: sum(v) / len(v) for n, v in vals[k].items()}
        lines.append("== %s" % k)
        for n in sorted(c):
            lines.append("  %-28s %16.0f" % (n, c[n]))
        if "SQ_CYCLES" in c:
            cyc = c["SQ_CYCLES"] / N_SE  # kernel cycles (per engine)
            derived = []
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                derived.append("matrix cores busy %.1f%% of SIMD cycles" % (100 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * cyc)))
            if "SQ_ACTIVE_INST_VALU" in c:
                derived.append("vector instructions active %.1f%%" % (100 * 4 * c["SQ_ACTIVE_INST_VALU"] / (N_SIMD * cyc)))
            if "SQ_ACTIVE_INST_LDS" in c:
                derived.append("LDS instructions active %.1f%%" % (100 * 4 * c["SQ_ACTIVE_INST_LDS"] / (N_SIMD * cyc)))
            if "SQ_WAIT_INST_ANY" in c and "SQ_WAVE_CYCLES" in c:
                derived.append("waves waiting to issue %.1f%% of their cycles" % (100 * c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]))
            lines.append("  derived (kernel %.0f cycles): %s" % (cyc, "; ".join(derived)))
        lines.append("")
    lines.append("kernel source sha (%s): %s" % (", ".join(KERNEL_SOURCES), kernel_source_sha()))
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        with open(sys.argv[3], "w") as f:
            f.write(stats_summary(sys.argv[2], sys.argv[4]))
    elif sys.argv[1] == "sq":
        with open(sys.argv[2], "w") as f:
            f.write(sq_summary(sys.argv[4:], sys.argv[3]))
    elif sys.argv[1] == "traffic":
        for p in traffic_summaries(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6]):
            print(p)
    else:
        raise SystemExit(__doc__)
