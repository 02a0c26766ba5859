"""Measured HBM traffic of the decode call, from rocprofv3 counter runs.

rocprofv3 collects one counter per pass here: ``--pmc FETCH_SIZE`` and
``--pmc WRITE_SIZE`` (KiB per dispatch) over the benchmark, and the same two
counters over a plain device copy of known size (``bench.py --copy-probe``),
which calibrates what each counter reads per byte actually moved.  This module
turns the four counter CSVs into a small JSON summary keyed by a hash of the
kernel sources, and reads it back for the benchmark, which reports the traffic
only while the sources are unchanged.

    python -m paged_mla_decode_04_amd.traffic summarize \\
        --copy-fetch C1.csv --copy-write C2.csv --fetch F.csv --write W.csv \\
        --workload wide --out profiles/decode_wide_b128_h128_traffic.json
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30                     # bench.py --copy-probe copies 1 GiB
DECODE_KERNELS = ("decode", "combine")  # name parts of the kernels a decode call launches


def source_hash() -> str:
    """sha256 over the HIP sources and headers the decode call is built from."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")) +
                   glob.glob(os.path.join(HERE, "csrc", "*.h")))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _per_dispatch_kib(path: str, counter: str) -> dict:
    """Mean value of `counter` per dispatch, by kernel name."""
    vals = defaultdict(list)
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter:
                vals[row["Kernel_Name"]].append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def _pick(kib: dict, key: str) -> float:
    hits = [v for k, v in kib.items() if key in k]
    if len(hits) != 1:
        raise ValueError(f"expected one kernel matching {key!r}, found {sorted(kib)}")
    return hits[0]


def summarize(copy_fetch: str, copy_write: str, fetch: str, write: str, workload: str) -> dict:
    cf = _pick(_per_dispatch_kib(copy_fetch, "FETCH_SIZE"), "copyBuffer")
    cw = _pick(_per_dispatch_kib(copy_write, "WRITE_SIZE"), "copyBuffer")
    fetch_scale = COPY_BYTES / (cf * 1024.0)
    write_scale = COPY_BYTES / (cw * 1024.0)
    f = _per_dispatch_kib(fetch, "FETCH_SIZE")
    w = _per_dispatch_kib(write, "WRITE_SIZE")
    kernels = {}
    for name in sorted(f):
        if any(k in name for k in DECODE_KERNELS) and name in w:
            short = name.rsplit("(", 1)[0].replace("void ", "").replace("(anonymous namespace)::", "")
            short = short.replace("mla::", "")
            kernels[short] = {"fetch_bytes": f[name] * 1024.0 * fetch_scale,
                              "write_bytes": w[name] * 1024.0 * write_scale}
    if not kernels:
        raise ValueError(f"no decode or combine kernel among {sorted(f)}")
    total = sum(v["fetch_bytes"] + v["write_bytes"] for v in kernels.values())
    return {
        "workload": workload,
        "source_sha256": source_hash(),
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "kernels": kernels,
        "bytes_per_call": total,
    }


def load(workload: str):
    """Traffic summary for `workload` if it was measured on the current sources."""
    for path in glob.glob(os.path.join(PROFILES, "*_traffic.json")):
        with open(path) as f:
            d = json.load(f)
        if d.get("workload") == workload and d.get("source_sha256") == source_hash():
            return d
    return None


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--copy-fetch", required=True)
    s.add_argument("--copy-write", required=True)
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--workload", required=True)
    s.add_argument("--out", required=True)
    sub.add_parser("hash")
    args = ap.parse_args()
    if args.cmd == "hash":
        print(source_hash())
        return
    d = summarize(args.copy_fetch, args.copy_write, args.fetch, args.write, args.workload)
    with open(args.out, "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    print(json.dumps(d))


if __name__ == "__main__":
    main()
