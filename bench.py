"""Benchmark of the block-sparse attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch of resident synthetic input:
dbsp_sparse_select (pool Q and K, score, select, CSR) followed by dbsp_sparse_attn_fwd.
Default workload: the 720p final scale (32 heads, d = 128, bf16, Lq = 72,192 queries against
Lk = 144,896 keys = 512 text + 72,192 reference + 72,192 current tokens, text forced, Top-K
density 0.09375). Prints one JSON line.

Reported numbers:
  value           executed attention FLOP of the step / step time (TFLOP/s)
  select_ms       per-step time of the selection kernels (HIP events on the launch stream)
  select_GBps     selection's algorithmic bytes (Q + K read once, CSR written) / select_ms
  attn_ms         per-step time of the attention kernel (HIP events on the launch stream)
  roofline        the attention kernel (dominant): executed FLOP / its average launch time,
                  against the bf16 dense MFMA peak
  cpu_baseline    the float64 NumPy oracle on the host cores, on a bounded sample of the same
                  workload, extrapolated to the whole step in the same unit
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-attn fwd ms + MFMA util @72k-token scale; select ms + HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle's attention sample")
    return ap.parse_args()


def cpu_baseline(w, q, k, v, row_ptr, col_idx, nnz, flop_per_pair, budget_s):
    """Time the oracle (as it is) on one head's selection and on sampled attention rows of the
    same head, then extrapolate to the whole step: selection x heads, attention x nnz."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    h = w.heads // 2
    qh = q[:, h:h + 1].float().cpu().numpy()
    kh = k[:, h:h + 1].float().cpu().numpy()
    vh = v[:, h:h + 1].float().cpu().numpy()
    t0 = time.perf_counter()
    oracle.sparse_select(qh, kh, w.text, w.extra, w.mode, w.param)
    t_sel = time.perf_counter() - t0
    nqb = w.n_q_blocks
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx.cpu().numpy().astype(np.int64)
    base = h * nqb  # batch 0
    rng = np.random.default_rng(7)
    order = rng.permutation(nqb)
    done_pairs = 0
    t_att = 0.0
    n_rows = 0
    for i in order:
        r = base + int(i)
        cols = ci[rp[r]:rp[r + 1]]
        rp_h = np.zeros(nqb + 1, np.int64)
        rp_h[i + 1:] = cols.size
        t0 = time.perf_counter()
        oracle.attention_rows(qh, kh, vh, rp_h, cols, rows=[int(i)])
        t_att += time.perf_counter() - t0
        done_pairs += cols.size
        n_rows += 1
        if t_att >= budget_s and n_rows >= 4:
            break
    est_total_s = t_sel * w.heads * w.batch + t_att * (nnz / max(done_pairs, 1))
    exec_flop = nnz * flop_per_pair
    return {
        "value": exec_flop / est_total_s / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"float64 NumPy oracle: selection of 1 of {w.heads} heads ({t_sel:.2f} s) and "
                   f"attention of {n_rows} query blocks of that head ({done_pairs} kept blocks, "
                   f"{t_att:.2f} s), extrapolated x{w.heads} heads and x nnz/sampled blocks to "
                   f"one step ({est_total_s:.1f} s)"),
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the work shards by head with no communication; see the design notes).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import dynamic_block_sparse_pool_amd as dbsp
    from synth import BENCH_WORKLOAD, WORKLOADS, make_qkv

    name = args.workload or BENCH_WORKLOAD
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = make_qkv(w, device=dev, seed=args.seed)
    kw = dict(density=w.param) if w.mode == "topk" else dict(mass=w.param)
    plan = dbsp.SelectPlan(q, k, w.text, w.extra, **kw)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    idx = plan.run(q, k)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    n_ev = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]

    def step(e=None):
        if e is not None:
            e[0].record(stream)
        plan.run(q, k)
        if e is not None:
            e[1].record(stream)
        dbsp.sparse_attn_fwd(q, k, v, idx, out=out)
        if e is not None:
            e[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    sel_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / n_ev
    att_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / n_ev
    ms_per_step = wall * 1e3 / args.steps

    nnz = idx.nnz()
    rows = w.rows
    flop_per_pair = 4 * 128 * 128 * w.head_dim
    exec_flop = nnz * flop_per_pair
    elt = 2 if w.dtype == "bf16" else 4
    sel_bytes = (w.batch * w.heads * (w.lq + w.lk) * w.head_dim * elt) + 4 * (rows + 1) + 4 * nnz
    att_tflops = exec_flop / (att_ms * 1e-3) / 1e12
    sel_gbps = sel_bytes / (sel_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(exec_flop / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.batch, "heads": w.heads, "lq": w.lq, "lk": w.lk,
            "head_dim": w.head_dim, "mode": w.mode, "param": w.param,
            "forced_text_blocks": list(w.text), "forced_extra_blocks": list(w.extra),
            "nnz": nnz, "executed_density": round(nnz / (rows * w.n_k_blocks), 5),
            "output_dtype": "bf16",
        },
        "select_ms": round(sel_ms, 4),
        "select_GBps": round(sel_gbps, 1),
        "select_hbm_frac": round(sel_gbps / PEAK_HBM_GBPS, 4),
        "attn_ms": round(att_ms, 4),
        "attn_TFLOPs": round(att_tflops, 2),
        "attn_mfma_frac": round(att_tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(att_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(att_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "attn_fwd_bf16_kernel",
                     "per_launch_flop": exec_flop},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, q, k, v, idx.row_ptr, idx.col_idx, nnz,
                                           flop_per_pair, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
