"""Oracle for per-head dynamic block-sparse attention: plain, slow, float64 NumPy.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path (the HIP library and its Python binding) never calls it,
and this package imports nothing from the product.

What it computes, step by step, in the order the pages describe:

  select.py     partition into 128-token blocks, mean-pool Q and K per block, score pooled
                block pairs, force the conditioning blocks, pick the rest by Top-K at a density
                or by the shortest cumulative-mass prefix, encode the kept set as CSR
  attention.py  softmax attention of each query block over all tokens of its kept key blocks
                (two independent formulations), and the dense reference
  energy.py     token-level block energy (CalibAtt Eq. (5)) and retained mass of a mask
  vote.py       cross-input vote of binary masks (CalibAtt Eq. (8)/(9))
  anchor.py     the anchor-row path of spatially repeating heads (CalibAtt key designs 3, 4)

Every function cites the passage it follows by page title and section. Readings taken where the
pages are silent are listed in the docstrings of the functions that make them.

Parity unpinned against the pages: every function here is pinned by tests to closed forms,
brute force, library routines or hand-worked rows of its own definition, but for these readings
no value printed on the pages confirms that the definition is the pages' intent:
  topk_budget     K = ceil(density * |C|) over the non-forced blocks (floor or round would keep
                  one block fewer on some configurations)
  select_mass     forced blocks counted toward the threshold first (no configuration on the
                  pages has forced blocks in mass mode)
  anchor_rows     equally spaced anchors read as band centres floor((2 j + 1) H / (2 k))
and, for the workloads rather than a function, the 48 padding tokens of the 21 x 3,600 DiT
sequence read as ordinary tokens.
"""
from .select import (BLOCK, MASS_BITS, block_scores, block_softmax, forced_blocks, mass_threshold_units,
                     mass_units, n_blocks, pool, select_mass, select_topk, sparse_select, to_csr, to_intervals,
                     topk_budget)
from .attention import attention_dense, attention_masked, attention_rows
from .energy import block_energy_rows, retained_mass, token_upper_bound
from .vote import vote_masks
from .anchor import anchor_attention, anchor_rows, nearest_anchor

__all__ = [
    "BLOCK", "MASS_BITS", "n_blocks", "pool", "block_scores", "block_softmax", "forced_blocks",
    "topk_budget", "select_topk", "mass_units", "mass_threshold_units", "select_mass", "to_csr",
    "to_intervals",
    "sparse_select", "attention_rows", "attention_masked", "attention_dense", "block_energy_rows",
    "token_upper_bound", "retained_mass", "vote_masks", "anchor_rows", "nearest_anchor",
    "anchor_attention",
]
