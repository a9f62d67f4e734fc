"""Summaries of rocprofv3 output for the decode kernel (text, for profiles/).

    python -m sparse_mla_decode_gather_amd.rocprof_summary stats <dir> <cmd> [<K>]
    python -m sparse_mla_decode_gather_amd.rocprof_summary traffic \\
        <fetch_dir> <write_dir> <copy_bytes> <cmd> [<request_dir>]
    python -m sparse_mla_decode_gather_amd.rocprof_summary sq <cmd> <dir>...

``stats`` condenses a --kernel-trace --stats run (kernel_stats.csv): the
decode, combine and combined-table builder kernels.  With K it adds, from
kernel_trace.csv, the duration statistics of the last K dispatches of the
most-dispatched decode kernel (and of the combine kernel, if it ran): under
``bench.py --headline-only --steps K`` those are the K timed launches (the
earlier dispatches are the settling and warmup launches); under
``bench.py --only-workload NAME`` the last 100 are its HIP-graph replays.
``sq`` gives the median per dispatch of every counter in one or more
--pmc runs over the decode kernels, with the MFMA-busy and waiting
fractions derived from them.
``traffic`` turns a FETCH_SIZE run and a WRITE_SIZE run (KiB per dispatch)
into HBM bytes per decode launch, calibrated by the same counters on a
plain device copy of known size taken in the same process: the factor is
counter bytes / true bytes of the copy, and decode traffic = counter
bytes / factor.  The result is tagged with a digest of the kernel sources
as code (comments and layout excluded), so a stale figure is ignored once
the kernel code changes.  With a third run of
the EA read-request counters by size (TCC_EA0_RDREQ_sum, _128B_sum,
_32B_sum) the summary adds an uncalibrated cross-check of the read bytes.
"""

from __future__ import annotations

import csv
import glob
import hashlib
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
DECODE = ("decode_h64_kernel", "decode_hd_kernel")   # the decode kernels (not gather_only)
COPY_PATTERNS = ("copy", "Copy")


def _code_only(text: str) -> str:
    """C++ source with its comments removed and whitespace runs collapsed
    (string and character literals kept as written), so that an edit of a
    comment or of the layout does not count as a change of the kernels."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_digest() -> str:
    """Digest of the kernel and host-layer sources as code (comments and
    layout excluded): a traffic figure is only used on the code it was
    measured on."""
    h = hashlib.sha256()
    for f in ("kernels.hip", "api.cpp", "internal.h"):
        with open(os.path.join(PKG, "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
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
        if any(d in name for d in DECODE) or "combine_kernel" in name or \
                "build_indices_kernel" in name:
            short = name.replace("smla::(anonymous namespace)::", "")
            short = short.replace("void ", "").split("(smla::")[0]
            lines.append(f"{short} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                         f"{r['MinNs']} | {r['MaxNs']} | {float(r['Percentage']):.2f}")
    return "\n".join(lines) + "\n"


def timed_tail(directory: str, k: int) -> str:
    """Duration statistics of the last k dispatches (by start time) of the
    most-dispatched decode kernel in kernel_trace.csv, and of the combine
    kernel's last k when it ran."""
    rows = _csv(directory, "kernel_trace.csv")
    dec = [r for r in rows if any(d in r["Kernel_Name"] for d in DECODE)]
    if not dec:
        raise ValueError("no decode kernel dispatches in the trace")
    counts = {}
    for r in dec:
        counts[r["Kernel_Name"]] = counts.get(r["Kernel_Name"], 0) + 1
    names = [max(counts, key=counts.get)]
    names += sorted({r["Kernel_Name"] for r in rows if "combine_kernel" in r["Kernel_Name"]})
    out = []
    for name in names:
        mine = sorted((r for r in rows if r["Kernel_Name"] == name),
                      key=lambda r: int(r["Start_Timestamp"]))
        if len(mine) < k:
            raise ValueError(f"{len(mine)} dispatches of {name}, fewer than {k}")
        dur = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in mine[-k:]]
        short = name.replace("smla::(anonymous namespace)::", "")
        short = short.replace("void ", "").split("(smla::")[0]
        tag = "combine_" if "combine_kernel" in name else ""
        out += [f"# the last {k} of {len(mine)} dispatches of {short}",
                f"{tag}tail_dispatches: {k}",
                f"{tag}tail_average_ns: {statistics.fmean(dur):.0f}",
                f"{tag}tail_median_ns: {statistics.median(dur):.0f}",
                f"{tag}tail_min_ns: {min(dur)}",
                f"{tag}tail_max_ns: {max(dur)}"]
    return "\n".join(out) + "\n"


def _per_dispatch(rows, counter, pattern_ok):
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter or not pattern_ok(r["Kernel_Name"]):
            continue
        per.setdefault(r["Dispatch_Id"], 0.0)
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    return list(per.values())


def _req_bytes(rows, pattern_ok):
    """Read bytes per dispatch from the EA read-request counters: 128-byte,
    32-byte and (the rest) 64-byte requests."""
    tot = _per_dispatch(rows, "TCC_EA0_RDREQ_sum", pattern_ok)
    r128 = _per_dispatch(rows, "TCC_EA0_RDREQ_128B_sum", pattern_ok)
    r32 = _per_dispatch(rows, "TCC_EA0_RDREQ_32B_sum", pattern_ok)
    n = min(len(tot), len(r128), len(r32))
    return [128 * r128[i] + 32 * r32[i] + 64 * (tot[i] - r128[i] - r32[i])
            for i in range(n)], tot, r128, r32


def traffic(fetch_dir: str, write_dir: str, copy_bytes: int, cmd: str,
            req_dir: str = None) -> str:
    is_decode = lambda n: any(d in n for d in DECODE)
    is_copy = lambda n: any(p in n for p in COPY_PATTERNS) and not is_decode(n)
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
    ] + ([] if req_dir is None else _req_check(req_dir, is_decode, is_copy, copy_bytes,
                                               fetch))) + "\n"


def _req_check(req_dir, is_decode, is_copy, copy_bytes, fetch):
    """Cross-check of the calibrated FETCH_SIZE with a second counter set:
    the EA read requests by size (TCC_EA0_RDREQ_sum, _128B_sum, _32B_sum),
    uncalibrated, on the decode and on the same plain copy."""
    rows = _csv(req_dir, "counter_collection.csv")
    dec, tot, r128, r32 = _req_bytes(rows, is_decode)
    cpy, _, _, _ = _req_bytes(rows, is_copy)
    cpy = sorted(cpy)[-3:]
    d = statistics.median(dec)
    c = statistics.median(cpy)
    return [
        "# cross-check: read bytes from EA read requests by size",
        "# (128 x RDREQ_128B + 32 x RDREQ_32B + 64 x the other RDREQ), no calibration",
        f"decode_rdreq_median: {statistics.median(tot):.0f}",
        f"decode_rdreq_128b_median: {statistics.median(r128):.0f}",
        f"decode_rdreq_32b_median: {statistics.median(r32):.0f}",
        f"decode_request_read_bytes: {d:.0f}",
        f"copy_request_read_bytes_over_true_bytes: {c / copy_bytes:.4f}",
        f"decode_request_bytes_over_calibrated_fetch: {d / fetch:.4f}",
    ]


def sq(dirs, cmd: str, simds: int = 1024, xcds: int = 8) -> str:
    is_decode = lambda n: any(d in n for d in DECODE)
    med = {}
    for d in dirs:
        rows = _csv(d, "counter_collection.csv")
        for name in sorted({r["Counter_Name"] for r in rows}):
            vals = _per_dispatch(rows, name, is_decode)
            if vals:
                med[name] = statistics.median(vals)
    lines = ["# SQ counters of the decode kernel (median per dispatch; summed over the chip)",
             f"# command: {cmd}"]
    lines += [f"{k}: {v:.4g}" for k, v in sorted(med.items())]
    if "SQ_VALU_MFMA_BUSY_CYCLES" in med and "GRBM_GUI_ACTIVE" in med:
        # GRBM_GUI_ACTIVE is summed over the XCDs; SQ_VALU_MFMA_BUSY_CYCLES
        # over all SIMDs
        busy = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (med["GRBM_GUI_ACTIVE"] / xcds * simds)
        lines.append(f"# derived: MFMA busy fraction of SIMD cycles = {busy:.3f}")
    if "SQ_WAIT_ANY" in med and "SQ_WAVE_CYCLES" in med:
        lines.append("# derived: wave-time waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES) = "
                     f"{med['SQ_WAIT_ANY'] / med['SQ_WAVE_CYCLES']:.3f}")
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "stats":
        print(stats(sys.argv[2], sys.argv[3]), end="")
        if len(sys.argv) > 4:
            print(timed_tail(sys.argv[2], int(sys.argv[4])), end="")
    elif mode == "traffic":
        print(traffic(sys.argv[2], sys.argv[3], int(sys.argv[4]), sys.argv[5],
                      sys.argv[6] if len(sys.argv) > 6 else None), end="")
    elif mode == "sq":
        print(sq(sys.argv[3:], sys.argv[2]), end="")
    else:
        raise SystemExit(__doc__)
