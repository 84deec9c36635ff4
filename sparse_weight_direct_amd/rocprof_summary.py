"""Summaries of rocprofv3 output (CSV format) for the files kept under profiles/.

    python3 -m sparse_weight_direct_amd.rocprof_summary trace DIR
        per-kernel launch statistics from DIR/**/*_kernel_stats.csv, with grid, workgroup
        and LDS size from *_kernel_trace.csv
    python3 -m sparse_weight_direct_amd.rocprof_summary counters DIR
        per-kernel mean of every counter per dispatch from DIR/**/*_counter_collection.csv
    python3 -m sparse_weight_direct_amd.rocprof_summary traffic --fetch DIR --write DIR \
            --kernel NAME --copy-bytes B --workload LAYER
        HBM bytes per launch of kernel NAME: FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
        each scaled by what the same counter reads for the copy kernel of B bytes that ran in
        the same process (bench.py --copy-mb), printed in the key: value form bench.py reads.

Reads only the profiler's CSV output; no GPU access.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_CSRC = os.path.join(ROOT, "sparse_weight_direct_amd", "csrc")
# the sources each kernel is built from; a weights-in-code kernel is generated at pack time
# from the generator and the layer's weights, which the seeded workloads fix
KERNEL_SOURCES = {
    "sparse_direct_fwd": [os.path.join(_CSRC, f) for f in ("kernels.hip", "xcd.h", "plan.h", "pack.cpp", "api.cpp")],
    "escoin_sconv": [os.path.join(_CSRC, f) for f in ("escoin.hip", "xcd.h", "plan.h", "api.cpp")],
    "sc_baked": [os.path.join(_CSRC, f) for f in ("bake.cpp", "bake.h", "plan.h", "pack.cpp", "api.cpp")] +
                [os.path.join(ROOT, "workloads.py")],
}
COPY_KERNELS = ("__amd_rocclr_copyBuffer", "copy", "Copy")


def _code_only(path: str) -> bytes:
    """A source file's code: comments (C++ ``//`` and ``/* */``, Python ``#``), trailing blanks
    and empty lines removed, so that editing a comment keeps the digest."""
    text = open(path, encoding="utf-8").read()
    if path.endswith(".py"):
        lines = [ln.split("#", 1)[0] if ln.lstrip().startswith("#") else ln for ln in text.splitlines()]
    else:
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"(^|\s)//.*$", "", ln) for ln in text.splitlines()]
    return "\n".join(ln.rstrip() for ln in lines if ln.strip()).encode()


def kernel_digest(kernel: str = "sc_baked") -> str:
    """Digest of the code a kernel is built from, comments left out (ties stored counters to
    the code they were taken with)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel]:
        h.update(_code_only(p))
    return h.hexdigest()[:16]


def _find(d: str, suffix: str) -> list[str]:
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        sys.exit(f"no *{suffix} under {d}")
    return files


def _short(name: str) -> str:
    return name if len(name) <= 110 else name[:107] + "..."


def trace(d: str) -> None:
    shape = {}
    for f in _find(d, "_kernel_trace.csv"):
        for r in csv.DictReader(open(f)):
            shape.setdefault(r["Kernel_Name"], (r.get("Grid_Size_X") or r.get("Grid_Size"),
                                                r.get("Workgroup_Size_X") or r.get("Workgroup_Size"),
                                                r.get("LDS_Block_Size") or r.get("Group_Segment_Size")))
    print("# kernel | calls | avg_us | min_us | max_us | total_ms | grid_x | wg_x | lds_bytes")
    for f in _find(d, "_kernel_stats.csv"):
        for r in csv.DictReader(open(f)):
            g, w, l = shape.get(r["Name"], ("?", "?", "?"))
            print(f"{_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                  f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | "
                  f"{float(r['TotalDurationNs']) / 1e6:.3f} | {g} | {w} | {l}")


def _counters(d: str) -> dict:
    """{kernel: {counter: [value per dispatch]}} (values of one dispatch summed over rows)."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for f in _find(d, "_counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            key = (f, r["Dispatch_Id"])
            names[key] = r["Kernel_Name"]
            per[key][r["Counter_Name"]] += float(r["Counter_Value"])
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for key, cs in per.items():
        for c, v in cs.items():
            out[names[key]][c].append(v)
    return out


def counters(d: str) -> None:
    print("# kernel | dispatches | counter = mean per dispatch (min..max)")
    for k, cs in _counters(d).items():
        for c, vs in sorted(cs.items()):
            print(f"{_short(k)} | {len(vs)} | {c} = {statistics.fmean(vs):.6g} ({min(vs):.6g}..{max(vs):.6g})")


def _pick(cs: dict, pred) -> list:
    return [v for k, v in cs.items() if pred(k)]


def traffic(fetch_dir: str, write_dir: str, kernel: str, copy_bytes: int, workload: str) -> None:
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        cs = _counters(d)
        kern = [v[counter] for k, v in cs.items() if kernel in k and counter in v]
        copy = [v[counter] for k, v in cs.items() if any(c in k for c in COPY_KERNELS) and kernel not in k
                and counter in v]
        if not kern or not copy:
            sys.exit(f"{counter}: kernel or copy dispatches missing under {d}")
        kib = statistics.median([x for xs in kern for x in xs])
        # the copy of copy_bytes reads and writes copy_bytes: keep the dispatches of that size
        cvals = [x for xs in copy for x in xs]
        ckib = max(cvals)
        factor = (copy_bytes / 1024.0) / ckib
        res[counter] = (kib, ckib, factor, len(kern[0]) if kern else 0)
    fb = res["FETCH_SIZE"][0] * 1024 * res["FETCH_SIZE"][2]
    wb = res["WRITE_SIZE"][0] * 1024 * res["WRITE_SIZE"][2]
    print(f"kernel_digest: {kernel_digest(kernel) if kernel in KERNEL_SOURCES else '?'}")
    print(f"workload: {workload}")
    print(f"kernel: {kernel}")
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        kib, ckib, factor, n = res[c]
        print(f"{c.lower()}_kib_per_launch: {kib:.1f}")
        print(f"{c.lower()}_copy_kib: {ckib:.1f}  (copy of {copy_bytes} B; scale factor {factor:.4f})")
    print(f"fetch_bytes_per_launch: {fb:.0f}")
    print(f"write_bytes_per_launch: {wb:.0f}")
    print(f"traffic_bytes_per_launch: {fb + wb:.0f}")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    c = sub.add_parser("counters")
    c.add_argument("dir")
    tr = sub.add_parser("traffic")
    tr.add_argument("--fetch", required=True)
    tr.add_argument("--write", required=True)
    tr.add_argument("--kernel", default="sc_baked")
    tr.add_argument("--copy-bytes", type=int, required=True)
    tr.add_argument("--workload", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        trace(a.dir)
    elif a.cmd == "counters":
        counters(a.dir)
    else:
        traffic(a.fetch, a.write, a.kernel, a.copy_bytes, a.workload)


if __name__ == "__main__":
    main()
