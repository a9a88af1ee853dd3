"""Oracle: cross-input vote over binary block masks.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: [CalibAtt] "Accelerating Text-to-Video Generation with Calibrated Sparse Attention",
key design 2, Eq. (8) and the description of Eq. (9): the masks of all calibration inputs are
averaged element-wise into a keep frequency, and a block is kept when that frequency is at
least rho. The page's worked example: rho = 0.5 over 64 inputs keeps blocks chosen 32 or more
times.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def vote_masks(masks, rho: float) -> np.ndarray:
    """masks [n_inputs, ...] bool -> kept [...] bool with mean(masks) >= rho. The comparison is
    done exactly on the rational count / n_inputs."""
    masks = np.asarray(masks, dtype=bool)
    n = masks.shape[0]
    if n == 0:
        raise ValueError("need at least one mask")
    counts = masks.sum(axis=0)
    r = Fraction(rho)
    # count / n >= rho  <=>  count * den >= num * n   (all integers)
    return (counts.astype(object) * r.denominator >= r.numerator * n).astype(bool)
