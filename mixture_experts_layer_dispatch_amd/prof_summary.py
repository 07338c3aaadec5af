"""Summarise a rocprofv3 kernel trace (``--kernel-trace --output-format csv``)
of ``bench.py`` into a per-kernel table.

    python -m mixture_experts_layer_dispatch_amd.prof_summary TRACE.csv [--counters FETCH.csv WRITE.csv
        --calib CFETCH.csv CWRITE.csv] [--mfma MFMA.csv]

Kernels of this library are grouped by name and grid size (one kernel can
serve two shapes, e.g. both MXFP8 weight gradients); everything else (torch's
input generation) is summed in one line.  With counter files, each group also
gets its HBM bytes per launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
each scaled by what that counter reads for torch's copy kernel of known size
in the calibration files (``bench.py --calibrate`` copies 4 GiB).  With an
MFMA counter file (``--pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16
SQ_INSTS_VALU_MFMA_MOPS_F8``), each group gets the percentage of cycles the
MFMA units were busy (rocprofv3's MfmaUtil: busy cycles summed over SIMDs over
active GPU cycles times the SIMD count) and the matrix TFLOP/s the counters
saw (MOPS x 512 flops, padded rows included) over the traced average duration.

``--traffic-json OUT`` also writes the counter bytes per launch of every
kernel that ran with a single grid size, keyed by kernel name, together with
``sources_sha256()`` of the HIP sources they were measured on; ``bench.py``
reports a kernel's counter traffic only while that hash still matches.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re

COPY_BYTES = 4 << 30          # bench.py --calibrate: 4 GiB read and 4 GiB written
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def sources_sha256() -> str:
    """Hash of every HIP source and header the library is built from."""
    h = hashlib.sha256()
    for fn in sorted(os.listdir(CSRC)):
        if fn.endswith((".hip", ".h")):
            h.update(fn.encode())
            with open(os.path.join(CSRC, fn), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def _short(name: str):
    """The kernel's name without namespace and template arguments; the MXFP4
    instantiations of the MX GEMMs (second template argument true) are told
    apart as k_gemm_*_mx4, the names their launches time under."""
    m = re.match(r".*moe::(k_\w+)(<[^>]*>)?", name)
    if not m:
        return None
    n, targs = m.group(1), m.group(2) or ""
    if n in ("k_gemm_gate_up_mx", "k_gemm_down_mx") and targs.replace(" ", "").endswith(",true>"):
        n += "4"
    return n


def trace_table(path):
    groups = collections.defaultdict(list)
    other_ns, other_calls = 0, 0
    for r in csv.DictReader(open(path)):
        n = _short(r["Kernel_Name"])
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if n is None:
            other_ns += dur
            other_calls += 1
            continue
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        groups[(n, grid)].append(dur)
    return groups, other_ns, other_calls


def counter_table(path, counter):
    vals = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        n = _short(r["Kernel_Name"])
        key = (n, int(r["Grid_Size"])) if n else r["Kernel_Name"]
        vals[key].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def copy_factor(path, counter):
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]]
    kib = sorted(vals)[len(vals) // 2]                      # median launch
    return COPY_BYTES / (kib * 1024.0)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("trace")
    ap.add_argument("--counters", nargs=2, metavar=("FETCH", "WRITE"))
    ap.add_argument("--calib", nargs=2, metavar=("CFETCH", "CWRITE"))
    ap.add_argument("--mfma", metavar="MFMA")
    ap.add_argument("--traffic-json", metavar="OUT")
    ap.add_argument("--workload", default="", help="workload name recorded in the traffic file")
    ap.add_argument("--command", default="", help="command line recorded in the traffic file")
    args = ap.parse_args()
    groups, other_ns, other_calls = trace_table(args.trace)
    fetch = write = None
    if args.counters and args.calib:
        ff = copy_factor(args.calib[0], "FETCH_SIZE")
        fw = copy_factor(args.calib[1], "WRITE_SIZE")
        fetch = {k: v * 1024 * ff for k, v in counter_table(args.counters[0], "FETCH_SIZE").items()}
        write = {k: v * 1024 * fw for k, v in counter_table(args.counters[1], "WRITE_SIZE").items()}
        print(f"copy calibration: FETCH_SIZE x{ff:.3f}, WRITE_SIZE x{fw:.3f}")
    util = mops = None
    if args.mfma:
        util = counter_table(args.mfma, "MfmaUtil")
        bf = counter_table(args.mfma, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        f8 = counter_table(args.mfma, "SQ_INSTS_VALU_MFMA_MOPS_F8")
        mops = {k: bf.get(k, 0.0) + f8.get(k, 0.0) for k in set(bf) | set(f8)}
    head = f"{'kernel':24s} {'grid':>9s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'total_ms':>10s}"
    if fetch is not None:
        head += f" {'read_MB':>10s} {'write_MB':>10s} {'GB/s':>8s}"
    if util is not None:
        head += f" {'mfma_busy%':>10s} {'mfma_TF/s':>10s}"
    print(head)
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))
    for (n, grid), d in rows:
        avg = sum(d) / len(d)
        line = (f"{n:24s} {grid:9d} {len(d):6d} {avg / 1e3:10.1f} {min(d) / 1e3:10.1f} "
                f"{max(d) / 1e3:10.1f} {sum(d) / 1e6:10.3f}")
        if fetch is not None:
            rd, wr = fetch.get((n, grid)), write.get((n, grid))
            if rd is not None and wr is not None:
                line += f" {rd / 1e6:10.1f} {wr / 1e6:10.1f} {(rd + wr) / avg:8.1f}"
            elif util is not None:
                line += f" {'':>10s} {'':>10s} {'':>8s}"
        if util is not None and (n, grid) in util:
            line += f" {util[(n, grid)]:10.1f} {mops.get((n, grid), 0.0) * 512 / avg / 1e3:10.1f}"
        print(line)
    print(f"{'(torch input generation)':24s} {'':>9s} {other_calls:6d} {'':>10s} {'':>10s} {'':>10s} "
          f"{other_ns / 1e6:10.3f}")
    if args.traffic_json and fetch is not None:
        grids = collections.Counter(n for (n, _) in groups)
        kern = {}
        for (n, grid), d in groups.items():
            rd, wr = fetch.get((n, grid)), write.get((n, grid))
            if grids[n] == 1 and rd is not None and wr is not None:
                kern[n] = {"grid": grid, "read_bytes": round(rd), "write_bytes": round(wr),
                           "avg_us": round(sum(d) / len(d) / 1e3, 1)}
        with open(args.traffic_json, "w") as f:
            json.dump({"workload": args.workload, "sources_sha256": sources_sha256(),
                       "command": args.command, "kernels": kern}, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main()
