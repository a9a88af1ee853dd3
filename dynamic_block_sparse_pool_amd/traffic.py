"""HBM traffic of the attention kernel from rocprofv3 counter runs.

    python -m dynamic_block_sparse_pool_amd.traffic \\
        --fetch A.csv --write B.csv --copy-fetch C.csv --copy-write D.csv \\
        --workload final_720p_clip2 --out profiles/attn_traffic_final_720p.json \\
        --command "<the commands that produced the four files>"

A, B: `rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE` counter collections of bench.py (one
counter per run). C, D: the same counters over `bench.py --only-copy`, whose 1 GiB device copy
reads and writes known byte counts; the ratio known / counted is the scale applied to the
attention kernel's per-dispatch means (FETCH_SIZE and WRITE_SIZE are in KiB). The JSON written
carries the sha256 of the kernel sources, so bench.py only reports the figure while the kernel is
the one that was measured.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL = "attn_fwd_bf16_kernel"
COPY_KERNEL = "copyBuffer"
COPY_BYTES = 1 << 30


def mean_counter(path: str, counter: str, kernel_substr: str) -> float:
    vals = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"{path}: no {counter} rows for a kernel named like {kernel_substr!r}")
    return sum(vals) / len(vals)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--out", "--workload",
              "--command"):
        ap.add_argument(a, required=True)
    args = ap.parse_args(argv)
    sys.path.insert(0, ROOT)
    import bench  # noqa: E402  (the source hash must be the one bench.py checks)

    fetch_kib = mean_counter(args.fetch, "FETCH_SIZE", KERNEL)
    write_kib = mean_counter(args.write, "WRITE_SIZE", KERNEL)
    copy_fetch_kib = mean_counter(args.copy_fetch, "FETCH_SIZE", COPY_KERNEL)
    copy_write_kib = mean_counter(args.copy_write, "WRITE_SIZE", COPY_KERNEL)
    fetch_scale = COPY_BYTES / (copy_fetch_kib * 1024)
    write_scale = COPY_BYTES / (copy_write_kib * 1024)
    traffic = fetch_kib * 1024 * fetch_scale + write_kib * 1024 * write_scale
    out = {
        "kernel": KERNEL,
        "workload": args.workload,
        "source_sha256": bench.attn_source_hash(),
        "fetch_kib_per_dispatch": round(fetch_kib, 1),
        "write_kib_per_dispatch": round(write_kib, 1),
        "copy_fetch_kib_per_GiB": round(copy_fetch_kib, 1),
        "copy_write_kib_per_GiB": round(copy_write_kib, 1),
        "fetch_scale": round(fetch_scale, 4),
        "write_scale": round(write_scale, 4),
        "traffic_bytes": int(round(traffic)),
        "command": args.command,
    }
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


if __name__ == "__main__":
    main()
