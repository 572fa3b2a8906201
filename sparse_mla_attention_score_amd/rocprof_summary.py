"""Summaries of rocprofv3 CSV output for this library's kernels.

    python -m sparse_mla_attention_score_amd.rocprof_summary stats DIR
        per-kernel launch statistics from a `rocprofv3 --kernel-trace --stats -f csv` run
    python -m sparse_mla_attention_score_amd.rocprof_summary pmc DIR [DIR ...]
        per-kernel mean of each counter from `rocprofv3 --pmc ... -f csv` runs
    python -m sparse_mla_attention_score_amd.rocprof_summary traffic --fetch DIR --write DIR \
            --kernel REGEX [--fetch-scale F] [--write-scale W]
        HBM bytes per dispatch of one kernel from a FETCH_SIZE run and a WRITE_SIZE run, each
        scaled by the factor a copy kernel of known size gives, in the `key: value` format that
        bench.py reads (with the fingerprint of the kernel's sources)

The fingerprint ties a stored traffic figure to the exact kernel sources it was measured on:
bench.py reports it only while the sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

# Sources each kernel is compiled from (its own file, the shared headers, and the build script
# that holds the compiler flags).
_SHARED = ["csrc/hs_device.h", "csrc/hs_internal.h", "../include/hisparse.h", "build.py"]
KERNEL_SOURCES = {
    "index_score_kernel": ["csrc/hs_index_topk.hip"] + _SHARED,
    "topk_select_kernel": ["csrc/hs_index_topk.hip"] + _SHARED,
    "resolve_kernel": ["csrc/hs_resolve.hip"] + _SHARED,
    "miss_copy_kernel": ["csrc/hs_resolve.hip"] + _SHARED,
    "sparse_mla_decode_kernel": ["csrc/hs_decode.hip"] + _SHARED,
}


def source_fingerprint(kernel: str) -> str:
    """sha256 over the kernel's source files (names and contents), first 16 hex digits."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        path = os.path.normpath(os.path.join(PKG, rel))
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    """`void hs::(anonymous namespace)::index_score_kernel<4, true>(...)` -> `index_score_kernel<4, true>`"""
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    n = re.sub(r"^hs::", "", n.strip())
    depth, out = 0, []
    for ch in n:  # drop the parameter list, keep template arguments
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out).strip()


def _rows(directory: str, suffix: str):
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    for path in files:
        with open(path, newline="") as f:
            yield from csv.DictReader(f)


def _col(row: dict, *names: str):
    low = {k.lower(): v for k, v in row.items()}
    for n in names:
        if n.lower() in low:
            return low[n.lower()]
    raise KeyError(f"none of {names} in {sorted(row)}")


def kernel_stats(directory: str) -> list:
    """[(kernel, calls, avg_us, min_us, max_us, total_us)] from the kernel trace, longest first."""
    durs = defaultdict(list)
    for r in _rows(directory, "kernel_trace.csv"):
        k = short_name(_col(r, "Kernel_Name"))
        durs[k].append((int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))) / 1e3)
    out = [(k, len(v), sum(v) / len(v), min(v), max(v), sum(v)) for k, v in durs.items()]
    return sorted(out, key=lambda t: -t[5])


def counter_means(directories) -> dict:
    """{(kernel, counter): (dispatches, mean value)}."""
    acc = defaultdict(list)
    for d in directories:
        for r in _rows(d, "counter_collection.csv"):
            k = short_name(_col(r, "Kernel_Name"))
            acc[(k, _col(r, "Counter_Name"))].append(float(_col(r, "Counter_Value")))
    return {key: (len(v), sum(v) / len(v)) for key, v in sorted(acc.items())}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("stats").add_argument("dir")
    p = sub.add_parser("pmc")
    p.add_argument("dirs", nargs="+")
    p = sub.add_parser("traffic")
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--kernel", required=True, help="regex on the short kernel name")
    p.add_argument("--fetch-scale", type=float, default=2.0)
    p.add_argument("--write-scale", type=float, default=1.0)
    a = ap.parse_args(argv)

    if a.cmd == "stats":
        print("| kernel | launches | avg us | min us | max us | total us |")
        print("|---|---|---|---|---|---|")
        for k, n, avg, lo, hi, tot in kernel_stats(a.dir):
            print(f"| {k} | {n} | {avg:.1f} | {lo:.1f} | {hi:.1f} | {tot:.1f} |")
    elif a.cmd == "pmc":
        print("| kernel | counter | dispatches | mean per dispatch |")
        print("|---|---|---|---|")
        for (k, c), (n, v) in counter_means(a.dirs).items():
            print(f"| {k} | {c} | {n} | {v:.1f} |")
    else:
        rx = re.compile(a.kernel)

        def pick(d, counter):
            hits = [(k, nv) for (k, c), nv in counter_means([d]).items() if c == counter and rx.search(k)]
            if len(hits) != 1:
                raise SystemExit(f"{counter}: expected one kernel matching {a.kernel}, got {[h[0] for h in hits]}")
            return hits[0]

        kf, (nf, fetch_kb) = pick(a.fetch, "FETCH_SIZE")
        kw, (nw, write_kb) = pick(a.write, "WRITE_SIZE")
        base = re.sub(r"<.*$", "", kf)
        print(f"kernel: {kf}")
        print(f"source_fingerprint: {source_fingerprint(base)}")
        print(f"fetch_size_kb: {fetch_kb:.1f}")
        print(f"write_size_kb: {write_kb:.1f}")
        print(f"fetch_scale: {a.fetch_scale}")
        print(f"write_scale: {a.write_scale}")
        print(f"dispatches: {min(nf, nw)}")
        print(f"traffic_bytes: {int(round(fetch_kb * 1024 * a.fetch_scale + write_kb * 1024 * a.write_scale))}")
    return 0


def read_traffic(path: str):
    """The `key: value` traffic file; None if missing or measured on other kernel sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    base = re.sub(r"<.*$", "", kv.get("kernel", ""))
    if base not in KERNEL_SOURCES or kv.get("source_fingerprint") != source_fingerprint(base):
        return None
    return int(kv["traffic_bytes"])


if __name__ == "__main__":
    sys.exit(main())
