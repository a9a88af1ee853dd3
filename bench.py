"""Benchmark of the block-sparse attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch of resident synthetic input:
dbsp_sparse_select (pool Q and K, score, select, CSR) followed by dbsp_sparse_attn_fwd.
Default workload: the 720p final scale (32 heads, d = 128, bf16, Lq = 72,192 queries against
Lk = 144,896 keys = 512 text + 72,192 reference + 72,192 current tokens, text forced, Top-K
density 0.09375). Prints one JSON line.

Reported numbers (the measurement protocol: HIP events on the launch stream; the headline
kernel times are medians over iterations that each start with the 256 MiB last-level cache
flushed; warm figures are labelled *_warm):
  value           executed attention FLOP of the step / step time (TFLOP/s), over the K timed
                  back-to-back steps (ms_per_step)
  select_ms       selection kernels (pool Q and K, score, select, CSR; in mass mode also the
                  longest-first row order the attention launch then follows, --row-order),
                  timed alone after a cache flush: median of --cold-iters iterations, with
                  select_ms_p10 / _p90; select_ms_warm is the mean over the timed steps
  select_GBps     selection's algorithmic bytes (Q + K read once, CSR written) / select_ms, and
                  select_hbm_frac against 8 TB/s
  attn_ms         the attention kernel timed alone after a cache flush: median (p10 / p90
                  beside it); attn_ms_warm is the mean over the timed steps
  attn_TFLOPs     executed attention FLOP / attn_ms, and attn_mfma_frac against the bf16 dense
                  peak
  attn_kv_gathered_GBps
                  K and V bytes of every kept (row, key block) pair plus Q and O once, per
                  second of attn_ms: the bytes the kernel gathers into LDS, most of them served
                  by the caches (not an HBM figure)
  copy_GBps       a plain device-to-device copy of 1 GiB (read + write bytes / time) and
  read_GBps       a read-only streaming pass over 1 GiB (bytes read / time; the probe kernel of
                  libdbsp_probe.so): achievable HBM ceilings
                  measured on the same GPU, with select_copy_frac and select_read_frac
  roofline        the attention kernel (dominant): executed FLOP / its mean launch time over the
                  timed steps, against the bf16 dense MFMA peak; traffic = its L2-miss bytes per
                  launch (FETCH_SIZE and WRITE_SIZE counters, scaled by a copy calibration) from
                  the committed counter summary when that summary was taken on the current
                  kernel source (else null). Those bytes leave the L2 for the fabric; part of
                  them is served by the last-level cache rather than HBM
  gemm_ceiling    context for the MFMA fraction, measured after the timed region: a dense
                  bf16 16384^3 GEMM through torch.matmul (the vendor's hipBLASLt) on the same
                  GPU, its TFLOP/s, fraction of the nominal peak, and attention's throughput as
                  a fraction of it (--no-ceiling skips it)
  cpu_baseline    the float64 NumPy oracle on the host cores, on a bounded sample of the same
                  workload, extrapolated to the whole step in the same unit

Other suites (--suite): energy (token-level block energies), calibrate (energies + vote),
anchor (the anchor-row path), ceiling (a dense 16384^3 bf16 GEMM through torch.matmul: the
matrix-core throughput a tuned dense kernel sustains on this GPU, as context for the MFMA
fraction).
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic_final_720p.json")
ATTN_SOURCES = ("attn.hip", "tile.hpp", "common.hpp", "kernels.hpp")
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_VALU_TFLOPS = 157.3   # MI355X fp32 vector (the fp32 attention kernel is plain FMA)
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the dense-GEMM context figure (gemm_ceiling) of the hot suite")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle's attention sample")
    ap.add_argument("--suite", choices=("hot", "energy", "calibrate", "anchor", "ceiling"),
                    default="hot",
                    help="hot: the selection + attention step (default); energy: the token-level "
                         "block energy, energy-driven selection and retained mass; calibrate: "
                         "per-input token-level masks voted into one static CSR, reused on a "
                         "held-out input; anchor: the anchor-row path of repeating heads on "
                         "the DiT geometry (one JSON line each)")
    ap.add_argument("--inputs", type=int, default=16, help="calibrate: calibration inputs")
    ap.add_argument("--bound-rows", type=int, default=8,
                    help="energy: sampled rows for the token-wise upper bound, computed by the "
                         "oracle with the CPU baseline (0, or --no-cpu-baseline, skips it)")
    ap.add_argument("--row-order", choices=("auto", "row", "lpt"), default="auto",
                    help="attention row order: longest first (lpt, built after each selection "
                         "and timed with it) or row order; auto = lpt in mass mode")
    ap.add_argument("--only-copy", action="store_true",
                    help="run only the 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--cold-iters", type=int, default=20,
                    help="iterations of the cache-flushed timing of each kernel (at least 1)")
    return ap.parse_args()


def attn_source_hash() -> str:
    """sha256 over the attention kernel's sources, to tell whether a stored counter summary
    still describes the kernel that runs."""
    import hashlib
    h = hashlib.sha256()
    for name in ATTN_SOURCES:
        with open(os.path.join(ROOT, "dynamic_block_sparse_pool_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(workload: str):
    """HBM bytes per attention launch from the committed counter summary, or None when it is
    missing, for another workload, or taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("source_sha256") != attn_source_hash():
        return None
    return int(t["traffic_bytes"])


def percentiles(xs):
    ys = sorted(xs)
    pick = lambda f: ys[min(len(ys) - 1, max(0, int(round(f * (len(ys) - 1)))))]
    return pick(0.1), pick(0.5), pick(0.9)


def copy_ceiling(torch, dev, reps: int = 5) -> float:
    """Read + write GB/s of a plain 1 GiB device-to-device copy."""
    n = 1 << 28  # float32 elements = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def read_ceiling(torch, dev, reps: int = 5):
    """Bytes read / time of a read-only pass over 1 GiB by the read-bandwidth probe
    (libdbsp_probe.so: 16-byte non-temporal loads, one word written per workgroup), the best of
    a few launch sizes: the HBM read ceiling a streaming kernel reaches on this GPU. None when
    the probe library is not built."""
    import ctypes
    path = os.path.join(ROOT, "dynamic_block_sparse_pool_amd", "libdbsp_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.dbsp_probe_read.restype = ctypes.c_int32
    lib.dbsp_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                    ctypes.c_int32, ctypes.c_void_p]
    n = 1 << 30
    x = torch.ones(n // 4, dtype=torch.float32, device=dev)
    out = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    best = 0.0
    for grid in (2048, 4096, 8192, 16384):
        run = lambda: lib.dbsp_probe_read(ctypes.c_void_p(x.data_ptr()), n,
                                          ctypes.c_void_p(out.data_ptr()), grid, stream)
        if run() != 0:
            return None
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        best = max(best, n / (ms * 1e-3) / 1e9)
    del x, out
    return best


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


def energy_suite(args, torch):
    """Token-level block energy (one dense sweep of Q K^T per row in bf16), the cumulative-mass
    selection on those energies, and the retained mass of that mask and of the pooled
    selection's mask. Default workload: the DiT mass-mode configuration, where the token-level
    energy is the pages' own calibration quantity."""
    import numpy as np
    import dynamic_block_sparse_pool_amd as dbsp
    from synth import WORKLOADS, make_qkv

    w = WORKLOADS[args.workload or "dit_mass"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, _ = make_qkv(w, device=dev, seed=args.seed)
    rows, nkb = w.rows, w.n_k_blocks
    energy = torch.empty((rows, nkb), dtype=torch.float32, device=dev)
    tau = w.param if w.mode == "mass" else 0.9
    kw = dict(density=w.param) if w.mode == "topk" else dict(mass=w.param)
    pooled = dbsp.sparse_select(q, k, w.text, w.extra, **kw)
    ews = torch.empty(max(dbsp.block_energy_workspace_bytes(q, k), 1), dtype=torch.uint8,
                      device=dev)
    for _ in range(max(args.warmup, 1)):
        dbsp.block_energy(q, k, out=energy, workspace=ews)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in ev:
        e[0].record()
        dbsp.block_energy(q, k, out=energy, workspace=ews)
        e[1].record()
        idx = dbsp.select_energy(energy, tau, w.text, w.extra, batch=w.batch, heads=w.heads)
        e[2].record()
        mass_tok = dbsp.retained_mass(energy, idx, batch=w.batch, heads=w.heads)
        e[3].record()
    torch.cuda.synchronize()
    e_ms = [e[0].elapsed_time(e[1]) for e in ev]
    s_ms = [e[1].elapsed_time(e[2]) for e in ev]
    m_ms = [e[2].elapsed_time(e[3]) for e in ev]
    mass_pooled = dbsp.retained_mass(energy, pooled, batch=w.batch, heads=w.heads)
    nnz_tok, nnz_pool = idx.nnz(), pooled.nnz()
    # bf16: the dense Q K^T product once per row (one sweep); float32: twice (two sweeps)
    flop = rows * nkb * (2 if w.dtype == "bf16" else 4) * 128 * 128 * w.head_dim
    e_mean = sum(e_ms) / len(e_ms)
    tflops = flop / (e_mean * 1e-3) / 1e12
    res = {
        "metric": "token-level block energy TFLOP/s (the dense Q K^T product per row); energy-driven "
                  "selection ms; retained mass",
        "value": round(tflops, 2), "unit": "TFLOP/s", "higher_is_better": True,
        "n_gpus": 1, "steps": args.steps, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "lq": w.lq,
                   "lk": w.lk, "head_dim": w.head_dim, "rows": rows, "n_k_blocks": nkb,
                   "tau": tau},
        "energy_ms": round(e_mean, 4),
        "energy_ms_p10_p50_p90": [round(x, 4) for x in percentiles(e_ms)],
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "block_energy_bf16_kernel",
                     "per_launch_flop": flop},
        "select_energy_ms": round(sum(s_ms) / len(s_ms), 4),
        "retained_mass_ms": round(sum(m_ms) / len(m_ms), 4),
        "token_mask": {"nnz": nnz_tok, "density": round(nnz_tok / (rows * nkb), 5),
                       "mean_retained_mass": round(float(mass_tok.mean()), 5)},
        "pooled_mask": {"mode": w.mode, "param": w.param, "nnz": nnz_pool,
                        "density": round(nnz_pool / (rows * nkb), 5),
                        "mean_retained_mass": round(float(mass_pooled.mean()), 5),
                        "min_retained_mass": round(float(mass_pooled.min()), 5)},
    }
    if not args.no_cpu_baseline:  # the oracle leg: its timing, and the token-wise bound
        res["cpu_baseline"] = energy_cpu_baseline(w, q, k, flop, args.cpu_seconds)
        if args.bound_rows > 0:
            res["token_upper_bound"] = token_bound_sample(w, q, k, pooled, mass_pooled,
                                                          args.bound_rows, args.seed)
    print(json.dumps(res), flush=True)


def token_bound_sample(w, q, k, index, mass_gpu, n_rows, seed):
    """The comparison behind SparSTAR's Figure 3: on sampled rows of one head, the attention mass
    the hot path's block mask keeps (from the GPU's token-level energies) against the token-wise
    upper bound for the same token budget (the oracle: each query keeps its own largest
    probabilities, as many keys as the block mask gives it). The gap is bound - block mass.
    Part of the suite's oracle leg: it runs with the CPU baseline, never without it."""
    import numpy as np
    import oracle
    h = w.heads // 2
    nqb = w.n_q_blocks
    rng = np.random.default_rng(seed + 11)
    qi = sorted(rng.choice(nqb, size=min(n_rows, nqb), replace=False).tolist())
    rp = index.row_ptr.cpu().numpy().astype(np.int64)
    rows = [h * nqb + i for i in qi]                        # batch 0, head h
    kept = [int(rp[r + 1] - rp[r]) for r in rows]
    budgets = [128 * n for n in kept]
    qh = q[0:1, h:h + 1].double().cpu().numpy()
    kh = k[0:1, h:h + 1].double().cpu().numpy()
    t0 = time.perf_counter()
    bound = oracle.token_upper_bound(qh, kh, qi, budgets)
    t = time.perf_counter() - t0
    block = mass_gpu.cpu().numpy()[rows]
    gap = bound - block
    return {"head": h, "rows": qi, "kept_blocks": kept,
            "block_mass": [round(float(x), 5) for x in block],
            "bound": [round(float(x), 5) for x in bound],
            "mean_block_mass": round(float(block.mean()), 5),
            "mean_bound": round(float(bound.mean()), 5),
            "mean_gap": round(float(gap.mean()), 5), "max_gap": round(float(gap.max()), 5),
            "oracle_s": round(t, 1)}


def calibrate_suite(args, torch):
    """The offline calibration path: for each of N seeded synthetic inputs, token-level energies
    -> a mask at tau -> added to the vote; the vote at rho gives one static CSR, which then
    drives the sparse attention of a held-out input. Reports the per-stage times and how much
    of the held-out input's token-level attention mass the static mask keeps, next to the mask
    chosen on that input itself."""
    import dynamic_block_sparse_pool_amd as dbsp
    from synth import PROMPT_SHARED, WORKLOADS, make_prompt_qkv

    w = WORKLOADS[args.workload or "star_mid_clip2"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tau, rho, n = 0.9, 0.5, args.inputs
    rows, nkb = w.rows, w.n_k_blocks
    vote = dbsp.MaskVote(w.batch, w.heads, w.n_q_blocks, nkb, dev)
    energy = torch.empty((rows, nkb), dtype=torch.float32, device=dev)
    t_e, t_s, t_a = [], [], []
    for p in range(n):
        q, k, _ = make_prompt_qkv(w, p, device=dev)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        dbsp.block_energy(q, k, out=energy)
        ev[1].record()
        idx = dbsp.select_energy(energy, tau, w.text, w.extra, batch=w.batch, heads=w.heads)
        ev[2].record()
        vote.add(idx)
        ev[3].record()
        torch.cuda.synchronize()
        if p > 0:  # the first input warms up
            t_e.append(ev[0].elapsed_time(ev[1]))
            t_s.append(ev[1].elapsed_time(ev[2]))
            t_a.append(ev[2].elapsed_time(ev[3]))
        del q, k
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    static = vote.select(rho)
    e1.record()
    torch.cuda.synchronize()
    t_vote = e0.elapsed_time(e1)
    # held-out input: the static mask against its own token-level mask
    q, k, v = make_prompt_qkv(w, n + 1000, device=dev)
    dbsp.block_energy(q, k, out=energy)
    own = dbsp.select_energy(energy, tau, w.text, w.extra, batch=w.batch, heads=w.heads)
    m_static = dbsp.retained_mass(energy, static, batch=w.batch, heads=w.heads)
    m_own = dbsp.retained_mass(energy, own, batch=w.batch, heads=w.heads)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    dbsp.sparse_attn_fwd(q, k, v, static, out=out)
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for _ in range(5):
        dbsp.sparse_attn_fwd(q, k, v, static, out=out)
    a1.record()
    torch.cuda.synchronize()
    nnz_s, nnz_o = static.nnz(), own.nnz()
    mean = lambda xs: sum(xs) / max(len(xs), 1)
    res = {
        "metric": "calibration: per-input energy + selection + vote ms; static-mask density and "
                  "retained mass on a held-out input",
        "value": round(mean(t_e) + mean(t_s) + mean(t_a), 4), "unit": "ms per calibration input",
        "higher_is_better": False, "n_gpus": 1, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "heads": w.heads, "lq": w.lq, "lk": w.lk, "rows": rows,
                   "n_k_blocks": nkb, "inputs": n, "tau": tau, "rho": rho,
                   "prompt_shared_variance": PROMPT_SHARED},
        "energy_ms": round(mean(t_e), 4), "select_energy_ms": round(mean(t_s), 4),
        "vote_accumulate_ms": round(mean(t_a), 4), "vote_select_ms": round(t_vote, 4),
        "static_mask": {"nnz": nnz_s, "density": round(nnz_s / (rows * nkb), 5),
                        "heldout_mean_retained_mass": round(float(m_static.mean()), 5),
                        "heldout_min_retained_mass": round(float(m_static.min()), 5),
                        "attn_ms": round(a0.elapsed_time(a1) / 5, 4)},
        "heldout_own_mask": {"nnz": nnz_o, "density": round(nnz_o / (rows * nkb), 5),
                             "mean_retained_mass": round(float(m_own.mean()), 5)},
    }
    print(json.dumps(res), flush=True)


def anchor_suite(args, torch):
    """The anchor-row path on the DiT shape: 21 latent frames of 45 rows x 80 tokens plus 48
    trailing tokens, 5 anchors per frame, all 40 heads; executed FLOP = packed query blocks x
    key blocks x 4 * 128^2 * d."""
    import dynamic_block_sparse_pool_amd as dbsp
    from synth import WORKLOADS, make_qkv

    w = WORKLOADS[args.workload or "dit_mass"]
    frames, rows, width, k_anchors = 21, 45, 80, 5
    if frames * rows * width > w.lq:
        raise SystemExit("workload shorter than the 21 x 45 x 80 geometry")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = make_qkv(w, device=dev, seed=args.seed)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    la = frames * k_anchors * width + (w.lq - frames * rows * width)
    la_pad = -(-la // 128) * 128
    ws = None
    for _ in range(max(args.warmup, 1)):
        dbsp.anchor_attn_fwd(q, k, v, frames, rows, width, k_anchors, out=out)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in ev:
        e[0].record()
        dbsp.anchor_attn_fwd(q, k, v, frames, rows, width, k_anchors, out=out, workspace=ws)
        e[1].record()
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in ev]
    mean = sum(ms) / len(ms)
    pairs = w.batch * w.heads * (la_pad // 128) * w.n_k_blocks
    flop = pairs * 4 * 128 * 128 * w.head_dim
    dense_flop = w.rows * w.n_k_blocks * 4 * 128 * 128 * w.head_dim
    tflops = flop / (mean * 1e-3) / 1e12
    res = {
        "metric": "anchor-row attention ms and executed TFLOP/s (repeating heads)",
        "value": round(mean, 4), "unit": "ms", "higher_is_better": False, "n_gpus": 1,
        "steps": args.steps, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "heads": w.heads, "lq": w.lq, "lk": w.lk,
                   "frames": frames, "rows_per_frame": rows, "row_width": width,
                   "anchors": k_anchors, "packed_queries": la, "packed_padded": la_pad},
        "ms_p10_p50_p90": [round(x, 4) for x in percentiles(ms)],
        "executed_TFLOPs": round(tflops, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "attn_fwd_bf16_kernel (packed anchor queries)",
                     "per_launch_flop": flop},
        "interaction_sparsity": round(1 - k_anchors / rows, 4),
        "executed_vs_dense_flop": round(flop / dense_flop, 4),
    }
    print(json.dumps(res), flush=True)


GEMM_N = 16384


def gemm_ceiling(torch, dev, seed, steps, warmup):
    """Mean time and TFLOP/s of a dense bf16 GEMM of GEMM_N^3 through torch.matmul (the vendor's
    hipBLASLt kernels), timed with HIP events: the matrix-core throughput a tuned dense kernel
    sustains on this GPU under load. Context for the MFMA fraction, not part of the hot path."""
    n = GEMM_N
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(max(warmup, 1)):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        torch.matmul(a, b, out=c)
        e[1].record()
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in ev]
    mean = sum(ms) / len(ms)
    del a, b, c
    return mean, 2.0 * n ** 3 / (mean * 1e-3) / 1e12


def ceiling_suite(args, torch):
    """Context for the MFMA fraction: the dense bf16 GEMM of gemm_ceiling as its own line."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mean, tflops = gemm_ceiling(torch, dev, args.seed, args.steps, args.warmup)
    res = {"metric": "dense bf16 GEMM TFLOP/s (torch.matmul, 16384^3): sustained MFMA context",
           "value": round(tflops, 1), "unit": "TFLOP/s", "higher_is_better": True, "n_gpus": 1,
           "steps": args.steps, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "gemm_16384_cubed"}, "ms_mean": round(mean, 4),
           "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4)}
    print(json.dumps(res), flush=True)


def energy_cpu_baseline(w, q, k, flop, budget_s):
    """The oracle's Eq. (5) on as many rows of one head as fit in the budget, extrapolated."""
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
    n, t = 0, 0.0
    for i in np.random.default_rng(7).permutation(w.n_q_blocks):
        t0 = time.perf_counter()
        oracle.block_energy_rows(qh, kh, rows=[int(i)])
        t += time.perf_counter() - t0
        n += 1
        if t >= budget_s and n >= 2:
            break
    total_s = t * w.rows / n
    return {"value": flop / total_s / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"float64 NumPy oracle: Eq. (5) for {n} query blocks of 1 head ({t:.2f} s), "
                      f"extrapolated x{w.rows / n:.0f} to all rows ({total_s:.0f} s)"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the work shards by head with no communication; see the design notes).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.only_copy:
        torch.cuda.set_device(0)
        print(json.dumps({"copy_GBps": round(copy_ceiling(torch, torch.device("cuda:0")), 1)}))
        return
    if args.suite == "energy":
        return energy_suite(args, torch)
    if args.suite == "calibrate":
        return calibrate_suite(args, torch)
    if args.suite == "anchor":
        return anchor_suite(args, torch)
    if args.suite == "ceiling":
        return ceiling_suite(args, torch)
    import dynamic_block_sparse_pool_amd as dbsp
    from synth import BENCH_WORKLOAD, WORKLOADS, make_qkv

    name = args.workload or BENCH_WORKLOAD
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = make_qkv(w, device=dev, seed=args.seed)
    kw = dict(density=w.param) if w.mode == "topk" else dict(mass=w.param)
    plan = dbsp.SelectPlan(q, k, w.text, w.extra, **kw)
    bf16 = w.dtype == "bf16"
    out = torch.empty(q.shape, dtype=torch.bfloat16 if bf16 else torch.float32, device=dev)
    idx = plan.run(q, k)
    lpt = args.row_order == "lpt" or (args.row_order == "auto" and w.mode == "mass")
    order = dbsp.lpt_order(q, k, idx) if lpt else None
    order_ws = (torch.empty(8 * w.batch * w.heads * (w.n_k_blocks + 1) + 512, dtype=torch.uint8,
                            device=dev) if lpt else None)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    n_ev = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]

    def step(e=None):
        if e is not None:
            e[0].record(stream)
        plan.run(q, k)
        if lpt:  # part of building the index: timed with the selection
            dbsp.lpt_order(q, k, idx, out=order, workspace=order_ws)
        if e is not None:
            e[1].record(stream)
        dbsp.sparse_attn_fwd(q, k, v, idx, out=out, row_order=order)
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

    sel_list = [e[0].elapsed_time(e[1]) for e in ev]
    att_list = [e[1].elapsed_time(e[2]) for e in ev]
    sel_warm = sum(sel_list) / n_ev
    att_warm = sum(att_list) / n_ev
    ms_per_step = wall * 1e3 / args.steps

    # the protocol's headline times: each kernel alone, after overwriting a 512 MiB scratch
    # buffer (outside the timed region) so that the 256 MiB last-level cache holds none of its
    # inputs; medians over the iterations
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cs, ca = [], []
    for it in range(max(args.cold_iters, 1)):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        scratch.fill_(it & 0xFF)
        e[0].record(stream)
        plan.run(q, k)
        if lpt:
            dbsp.lpt_order(q, k, idx, out=order, workspace=order_ws)
        e[1].record(stream)
        scratch.fill_((it + 128) & 0xFF)
        e[2].record(stream)
        dbsp.sparse_attn_fwd(q, k, v, idx, out=out, row_order=order)
        e[3].record(stream)
        torch.cuda.synchronize()
        cs.append(e[0].elapsed_time(e[1]))
        ca.append(e[2].elapsed_time(e[3]))
    del scratch
    sp, ap_ = percentiles(cs), percentiles(ca)
    sel_ms, att_ms = sp[1], ap_[1]
    copy_gbps = copy_ceiling(torch, dev)
    read_gbps = read_ceiling(torch, dev)

    nnz = idx.nnz()
    rows = w.rows
    flop_per_pair = 4 * 128 * 128 * w.head_dim
    exec_flop = nnz * flop_per_pair
    elt = 2 if w.dtype == "bf16" else 4
    sel_bytes = (w.batch * w.heads * (w.lq + w.lk) * w.head_dim * elt) + 4 * (rows + 1) + 4 * nnz
    att_tflops = exec_flop / (att_ms * 1e-3) / 1e12
    att_tflops_warm = exec_flop / (att_warm * 1e-3) / 1e12
    sel_gbps = sel_bytes / (sel_ms * 1e-3) / 1e9
    tok_bytes = 128 * w.head_dim * elt  # one block of K or V
    att_bytes = nnz * 2 * tok_bytes + 2 * w.batch * w.heads * w.lq * w.head_dim * elt
    att_gbps = att_bytes / (att_ms * 1e-3) / 1e9
    sw, aw = percentiles(sel_list), percentiles(att_list)
    traffic = stored_traffic(w.name)
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
            "output_dtype": "bf16" if bf16 else "f32", "row_order": "lpt" if lpt else "row",
        },
        "timing": f"select_ms / attn_ms: each kernel alone after a 512 MiB cache flush, median "
                  f"of {len(cs)}; *_warm: the {n_ev} back-to-back timed steps",
        "select_ms": round(sel_ms, 4),
        "select_ms_p10": round(sp[0], 4), "select_ms_p90": round(sp[2], 4),
        "select_GBps": round(sel_gbps, 1),
        "select_hbm_frac": round(sel_gbps / PEAK_HBM_GBPS, 4),
        "select_ms_warm": round(sel_warm, 4), "select_ms_warm_p50": round(sw[1], 4),
        "select_hbm_frac_warm": round(sel_bytes / (sel_warm * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "copy_GBps": round(copy_gbps, 1),
        "read_GBps": round(read_gbps, 1) if read_gbps else None,
        "select_copy_frac": round(sel_gbps / copy_gbps, 4),
        "select_read_frac": round(sel_gbps / read_gbps, 4) if read_gbps else None,
        "attn_ms": round(att_ms, 4),
        "attn_ms_p10": round(ap_[0], 4), "attn_ms_p90": round(ap_[2], 4),
        "attn_TFLOPs": round(att_tflops, 2),
        "attn_mfma_frac": round(att_tflops / PEAK_BF16_TFLOPS, 4) if bf16 else None,
        "attn_ms_warm": round(att_warm, 4), "attn_ms_warm_p50": round(aw[1], 4),
        "attn_mfma_frac_warm": round(att_tflops_warm / PEAK_BF16_TFLOPS, 4) if bf16 else None,
        "attn_kv_gathered_GBps": round(att_gbps, 1),
        "roofline": ({"bound": "mfma", "achieved": round(att_tflops_warm, 2),
                      "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(att_tflops_warm / PEAK_BF16_TFLOPS, 4),
                      "traffic": traffic, "kernel": "attn_fwd_bf16_kernel",
                      "per_launch_flop": exec_flop,
                      "traffic_what": "L2-miss bytes per launch (FETCH_SIZE and WRITE_SIZE, "
                                      "copy-calibrated); part is served by the last-level cache"}
                     if bf16 else
                     {"bound": "alu", "achieved": round(att_tflops_warm, 4),
                      "peak": PEAK_F32_VALU_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(att_tflops_warm / PEAK_F32_VALU_TFLOPS, 6), "traffic": None,
                      "kernel": "attn_fwd_f32_kernel", "per_launch_flop": exec_flop}),
    }
    if bf16 and not args.no_ceiling:
        g_ms, g_tflops = gemm_ceiling(torch, dev, args.seed, 5, 1)
        res["gemm_ceiling"] = {
            "what": f"dense bf16 GEMM {GEMM_N}^3 through torch.matmul (hipBLASLt) on this GPU",
            "TFLOPs": round(g_tflops, 1), "frac_of_peak": round(g_tflops / PEAK_BF16_TFLOPS, 4),
            "attn_frac_of_gemm": round(att_tflops / g_tflops, 4)}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, q, k, v, idx.row_ptr, idx.col_idx, nnz,
                                           flop_per_pair, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
