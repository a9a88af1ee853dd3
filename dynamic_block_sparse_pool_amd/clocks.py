"""Effective shader clock of kernels from a rocprofv3 counter run.

    python -m dynamic_block_sparse_pool_amd.clocks --prefix DIR/NAME [--kernel SUBSTR ...]

DIR/NAME is the output prefix of one
`rocprofv3 --kernel-trace --pmc GRBM_GUI_ACTIVE SQ_CYCLES -d DIR -o NAME --output-format csv`
run: NAME_counter_collection.csv, NAME_kernel_trace.csv and NAME_agent_info.csv. Each counter is
the sum over the GPU's accelerator complexes (GRBM_GUI_ACTIVE) or shader engines (SQ_CYCLES)
of the cycles a dispatch kept them busy, so counter / units / kernel duration is the clock the
kernel ran at (the unit counts come from the agent info). Prints one line per kernel matched:
dispatches, mean duration, and both clock estimates against the agent's maximum engine clock.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob


def _one(pattern: str) -> str:
    hits = glob.glob(pattern, recursive=True)
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def gpu_agent(path: str) -> dict:
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if int(r.get("Simd_Count", "0") or 0) > 0:
                return r
    raise SystemExit(f"{path}: no GPU agent")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--prefix", required=True, help="DIR/NAME of the rocprofv3 output")
    ap.add_argument("--kernel", action="append", default=None,
                    help="substring of the kernel names to report (repeatable; default: all)")
    args = ap.parse_args(argv)
    agent = gpu_agent(_one(args.prefix + "_agent_info.csv"))
    xcc = int(agent["Num_Xcc"])
    se = int(agent["Num_Shader_Banks"])
    fmax = float(agent["Max_Engine_Clk_Fcompute"]) * 1e6
    durs = collections.defaultdict(list)
    with open(_one(args.prefix + "_kernel_trace.csv"), newline="") as f:
        for r in csv.DictReader(f):
            durs[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    cnt = collections.defaultdict(list)
    with open(_one(args.prefix + "_counter_collection.csv"), newline="") as f:
        for r in csv.DictReader(f):
            cnt[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    print(f"agent: {xcc} XCC, {se} shader engines, max engine clock {fmax / 1e9:.2f} GHz")
    for name, d in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        if args.kernel and not any(k in name for k in args.kernel):
            continue
        mean_s = sum(d) / len(d)
        g = cnt.get((name, "GRBM_GUI_ACTIVE"))
        s = cnt.get((name, "SQ_CYCLES"))
        g_hz = sum(g) / len(g) / xcc / mean_s if g else float("nan")
        s_hz = sum(s) / len(s) / se / mean_s if s else float("nan")
        short = name.split("(")[0]
        print(f"{short}: {len(d)} dispatches, mean {mean_s * 1e3:.3f} ms, clock "
              f"{g_hz / 1e9:.3f} GHz (GRBM_GUI_ACTIVE) / {s_hz / 1e9:.3f} GHz (SQ_CYCLES), "
              f"{g_hz / fmax:.1%} of {fmax / 1e9:.2f} GHz")


if __name__ == "__main__":
    main()
