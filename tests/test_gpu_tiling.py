"""GPU parity of the selection on shapes that take each branch of the scoring kernel's tiling.

The scoring and selection kernel cuts every (batch, head) into 16-block tiles and 8-block tiles
depending on how full the last generation of workgroups would be: all short (every long tile
fits in one generation), the last generation cut into short tiles (at most half full), or long
tiles with only the head's remainder short; heads are spread over the 8 XCDs, unevenly when their
number is not a multiple of 8. Each case checks every row: the pooled scores against the
oracle's pooling of that head, and the mask bit-exact against the oracle selecting from the
GPU's own scores. Few key blocks keep the cases fast; query lengths are ragged.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, make_qkv
from tests import parity as P

pytestmark = pytest.mark.gpu

CASES = {
    # name: (batch, heads, query blocks, mode, param)
    "all_short": (1, 8, 20, "topk", 0.25),
    "last_generation_cut": (1, 8, 1100, "topk", 0.25),
    "long_tiles": (1, 8, 1600, "topk", 0.25),
    "uneven_heads": (1, 3, 1100, "topk", 0.25),
    "batch_two_long": (2, 5, 900, "topk", 0.25),
    "mass_cut": (1, 8, 1100, "mass", 0.9),
}


def say(msg):
    print(f"[gpu-tiling] {msg}", flush=True)


@pytest.mark.parametrize("case", sorted(CASES))
def test_selection_tiling_branches(case):
    import dynamic_block_sparse_pool_amd as dbsp
    batch, heads, nqb, mode, param = CASES[case]
    w = WORKLOADS["star_mid_clip2"].with_(name=case, batch=batch, heads=heads,
                                          lq=nqb * 128 - 5, lk=16 * 128 + 37, text=(0, 1),
                                          extra=(0, 0), mode=mode, param=param)
    say(f"case {case}: B={batch} H={heads} nqb={w.n_q_blocks} nkb={w.n_k_blocks} {mode}={param}")
    q, k, _ = make_qkv(w, device="cuda", seed=3)
    kw = dict(density=param) if mode == "topk" else dict(mass=param)
    idx = dbsp.SelectPlan(q, k, w.text, w.extra, return_scores=True, **kw).run(q, k)
    torch.cuda.synchronize()
    nkb = w.n_k_blocks
    rp = idx.row_ptr.cpu().numpy().astype(np.int64)
    ci = idx.col_idx.cpu().numpy().astype(np.int64)
    gpu_out = idx.scores.cpu().numpy().astype(np.float64)  # S (Top-K) or p (mass), [rows, nkb]

    # pooled scores of every row, head by head, against the oracle's pooling
    scale = 1.0 / np.sqrt(w.head_dim)
    s4 = gpu_out.reshape(batch, heads, nqb, nkb)
    for b in range(batch):
        for h in range(heads):
            qbar = oracle.pool(P.host(q[b:b + 1, h:h + 1]))[0, 0]
            kbar = oracle.pool(P.host(k[b:b + 1, h:h + 1]))[0, 0]
            if mode == "topk":
                P.check_scores(s4[b, h], qbar, kbar, scale)
            else:
                P.check_energies(s4[b, h], oracle.block_softmax(oracle.block_scores(qbar, kbar,
                                                                                    scale)))
    say("  scores (or energies) of every row match the oracle's pooling")

    # every mask row bit-exact on the GPU's own scores
    forced = oracle.forced_blocks(nkb, w.text, w.extra)
    kept_gpu = P.csr_to_kept_fast(rp, ci, nkb)
    if mode == "topk":
        kk = oracle.topk_budget(param, int((~forced).sum()))
        kept_ora = oracle.select_topk(gpu_out, forced, kk)
    else:
        kept_ora = oracle.select_mass(gpu_out, forced, param)
    np.testing.assert_array_equal(kept_gpu, kept_ora)
    say(f"  masks bit-exact on all {w.rows} rows, nnz {int(rp[-1])}")
