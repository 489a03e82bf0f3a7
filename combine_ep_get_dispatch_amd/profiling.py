"""HBM traffic of the kernels from rocprofv3 hardware counters.

Two counter runs of the same benchmark command (one with FETCH_SIZE, one with
WRITE_SIZE; rocprofv3 reports both in KiB per kernel dispatch) give the bytes
each kernel moved between L2 and the memory side.  Each is scaled by what the
same counter reads for the library's plain copy kernel (ep_probe_copy) of a
known size in the same run, so the figures are in bytes.  The result is stored
with a hash of the kernel sources; the benchmark reports it only while the
sources still match, i.e. only for the kernels the counters were taken on.

    python -m combine_ep_get_dispatch_amd.profiling FETCH_DIR WRITE_DIR OUT_JSON PROBE_BYTES WORKLOAD

With --by-launch first, the kernels are told apart by their launch geometry
as well (grid and workgroup size), for runs in which one kernel instance
serves several calls (the flat and the group combine, the group dispatch and
a push permutation):

    python -m combine_ep_get_dispatch_amd.profiling --by-launch FETCH_DIR WRITE_DIR OUT_JSON PROBE_BYTES WORKLOAD
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

KERNELS = ("moedisp_layout", "moedisp_layout_sort", "moedisp_layout_reduce", "moedisp_count", "moedisp_notify",
           "moedisp_scatter", "moedisp_scatter_pull", "moedisp_scatter_pull_compact", "moedisp_scatter_quant",
           "moedisp_combine",
           "moedisp_dispatch_fused", "moedisp_probe_read", "moedisp_probe_copy", "moedisp_probe_fill")
_NAME = re.compile(r"\b(moedisp_\w+?)(<[^>(]*>)?\(")


def source_hash() -> str:
    files = sorted(glob.glob(os.path.join(HERE, "csrc", "*"))) + sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def short_name(kernel_name: str) -> str:
    """Kernel instance as `name<template args>` (e.g. moedisp_scatter<1>), or
    "" for kernels that are not the library's."""
    m = _NAME.search(kernel_name)
    if not m or m.group(1) not in KERNELS:
        return ""
    return m.group(1) + (m.group(2) or "").replace(" ", "")


def base_name(instance: str) -> str:
    return instance.split("<", 1)[0]


def kernel_traffic(measured: dict, kernel: str):
    """Bytes of the instance of `kernel` with the most counted dispatches."""
    cands = [(v["dispatches"][0], v) for k, v in measured.get("kernels", {}).items()
             if base_name(k.split(" ", 1)[0]) == kernel]
    return max(cands, key=lambda c: c[0])[1] if cands else None


def read_counter(run_dir: str, counter: str, by_launch: bool = False) -> dict:
    """{kernel: [per-dispatch value in KiB, ...]} from a rocprofv3 --pmc csv
    run; with by_launch the key is `kernel grid/workgroup` (work-items)."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    out = defaultdict(list)
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                k = short_name(row.get("Kernel_Name", ""))
                if k and by_launch and base_name(k) != "moedisp_probe_copy":
                    k = f"{k} {row.get('Grid_Size', '?')}/{row.get('Workgroup_Size', '?')}"
                if k:
                    out[k].append(float(row["Counter_Value"]))
    return out


def summarise(fetch_dir: str, write_dir: str, probe_bytes: int, workload: str, by_launch: bool = False) -> dict:
    fetch = read_counter(fetch_dir, "FETCH_SIZE", by_launch)
    write = read_counter(write_dir, "WRITE_SIZE", by_launch)
    med = lambda v: sorted(v)[len(v) // 2]
    f_probe, w_probe = med(fetch["moedisp_probe_copy"]), med(write["moedisp_probe_copy"])
    f_scale = probe_bytes / f_probe   # bytes per counter unit
    w_scale = probe_bytes / w_probe
    kernels = {}
    for k in sorted(set(fetch) & set(write)):
        kernels[k] = {"fetch_bytes": med(fetch[k]) * f_scale, "write_bytes": med(write[k]) * w_scale,
                      "fetch_kib_raw": med(fetch[k]), "write_kib_raw": med(write[k]),
                      "dispatches": [len(fetch[k]), len(write[k])]}
    return {"source_sha256": source_hash(), "workload": workload, "probe_bytes": probe_bytes,
            "calibration": {"fetch_bytes_per_unit": f_scale, "write_bytes_per_unit": w_scale},
            "kernels": kernels}


def load_traffic(path: str):
    """Per-kernel traffic if it was measured on the current kernel sources, else None."""
    try:
        with open(path) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    return d if d.get("source_sha256") == source_hash() else None


if __name__ == "__main__":
    args = sys.argv[1:]
    by_launch = bool(args) and args[0] == "--by-launch"
    if by_launch:
        args = args[1:]
    fetch_dir, write_dir, out, probe, workload = args[0], args[1], args[2], int(args[3]), args[4]
    res = summarise(fetch_dir, write_dir, probe, workload, by_launch)
    with open(out, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res, indent=1))
