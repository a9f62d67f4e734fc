"""Summaries of rocprofv3 output for the decode kernel (text, for profiles/).

    python -m sparse_mla_decode_gather_amd.rocprof_summary stats <dir> <cmd>
    python -m sparse_mla_decode_gather_amd.rocprof_summary traffic \\
        <fetch_dir> <write_dir> <copy_bytes> <cmd>

``stats`` condenses a --kernel-trace --stats run (kernel_stats.csv).
``traffic`` turns a FETCH_SIZE run and a WRITE_SIZE run (KiB per dispatch)
into HBM bytes per decode launch, calibrated by the same counters on a
plain device copy of known size taken in the same process: the factor is
counter bytes / true bytes of the copy, and decode traffic = counter
bytes / factor.  The result is tagged with a digest of the kernel sources,
so a stale figure is ignored once the kernel changes.
"""

from __future__ import annotations

import csv
import glob
import hashlib
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
DECODE = "decode_kernel"
COPY_PATTERNS = ("copy", "Copy")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in ("kernels.hip", "api.cpp", "internal.h"):
        with open(os.path.join(PKG, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _csv(directory: str, suffix: str):
    files = glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def stats(directory: str, cmd: str) -> str:
    rows = _csv(directory, "kernel_stats.csv")
    lines = [f"# rocprofv3 --kernel-trace --stats summary", f"# command: {cmd}",
             "kernel | calls | average_ns | min_ns | max_ns | percent"]
    for r in rows:
        name = r["Name"]
        if DECODE in name or "combine_kernel" in name:
            short = name.replace("smla::(anonymous namespace)::", "")
            short = short.replace("void ", "").split("(smla::")[0]
            lines.append(f"{short} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                         f"{r['MinNs']} | {r['MaxNs']} | {float(r['Percentage']):.2f}")
    return "\n".join(lines) + "\n"


def _per_dispatch(rows, counter, pattern_ok):
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter or not pattern_ok(r["Kernel_Name"]):
            continue
        per.setdefault(r["Dispatch_Id"], 0.0)
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    return list(per.values())


def traffic(fetch_dir: str, write_dir: str, copy_bytes: int, cmd: str) -> str:
    is_decode = lambda n: DECODE in n
    is_copy = lambda n: any(p in n for p in COPY_PATTERNS) and DECODE not in n
    f_rows = _csv(fetch_dir, "counter_collection.csv")
    w_rows = _csv(write_dir, "counter_collection.csv")
    fd = _per_dispatch(f_rows, "FETCH_SIZE", is_decode)
    wd = _per_dispatch(w_rows, "WRITE_SIZE", is_decode)
    fc = _per_dispatch(f_rows, "FETCH_SIZE", is_copy)
    wc = _per_dispatch(w_rows, "WRITE_SIZE", is_copy)
    # the calibration copies are the last (largest) copy dispatches
    fc = sorted(fc)[-3:]
    wc = sorted(wc)[-3:]
    f_factor = statistics.median(fc) * 1024 / copy_bytes
    w_factor = statistics.median(wc) * 1024 / copy_bytes
    fetch = statistics.median(fd) * 1024 / f_factor
    write = statistics.median(wd) * 1024 / w_factor
    return "\n".join([
        "# HBM traffic of the decode kernel from rocprofv3 --pmc counters",
        f"# command: {cmd}",
        "# FETCH_SIZE and WRITE_SIZE are KiB per dispatch; each is divided by",
        "# the factor the same counter shows on a plain device copy of",
        f"# {copy_bytes} bytes read and written in the same process.",
        f"decode_dispatches: {len(fd)}",
        f"decode_fetch_kib_median: {statistics.median(fd):.1f}",
        f"decode_write_kib_median: {statistics.median(wd):.1f}",
        f"copy_fetch_kib_median: {statistics.median(fc):.1f}",
        f"copy_write_kib_median: {statistics.median(wc):.1f}",
        f"fetch_calibration_factor: {f_factor:.4f}",
        f"write_calibration_factor: {w_factor:.4f}",
        f"fetch_bytes_per_launch: {fetch:.0f}",
        f"write_bytes_per_launch: {write:.0f}",
        f"traffic_bytes_per_launch: {fetch + write:.0f}",
        f"kernel_source_digest: {kernel_source_digest()}",
    ]) + "\n"


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "stats":
        print(stats(sys.argv[2], sys.argv[3]), end="")
    elif mode == "traffic":
        print(traffic(sys.argv[2], sys.argv[3], int(sys.argv[4]), sys.argv[5]),
              end="")
    else:
        raise SystemExit(__doc__)
