"""Seeded synthetic inputs and the workload registry for the block-sparse attention path.

This module is shared by the oracle tests, the GPU parity tests and the benchmark. It only
describes shapes, forced key-block ranges and selection parameters, and draws random tensors.
It holds no step of the method's arithmetic (no pooling, scoring, selection or attention).

Workloads (shapes from the SparSTAR pages: ~72k tokens at the 720p final scale and 32 heads,
"SparSTAR：为什么视频自回归的稀疏注意力不能跨尺度复用？", problem statement and Figure 3
caption; densities from the decreasing density schedule in its method overview; the DiT-style
mass-threshold case takes the Wan 2.1 720p shape the CalibAtt page
"Accelerating Text-to-Video Generation with Calibrated Sparse Attention" evaluates on):

  toy               1 head, d=64, fp32, Lq=Lk=1024, Q/K/V iid N(0,1); block 0 forced; density 0.5
  toy_dense         same inputs, density 1.0 (must equal dense attention)
  star_mid_clip2    32 heads, d=128, bf16, Lq=8192, KV = 512 text + 8192 reference + 8192 current
  clip1_early       32 heads, d=128, bf16, Lq=18048, KV = 512 text + 4096 pyramid + 18048 current
  final_720p_clip2  32 heads, d=128, bf16, Lq=72192, KV = 512 text + 72192 reference + 72192 current
  dit_mass          40 heads, d=128, bf16, L=75648 (21 frames x 3600 tokens padded), mass 0.9

Block-structured tensors: for every (tensor, batch, head, 128-token block) a centroid is drawn
from N(0, 2^2 I_d) and every token of the block is centroid + N(0, 0.5^2 I_d) noise.  All
segments (text, reference, pyramid, current, pad) use the same recipe.

Random numbers come from torch generators seeded from (seed, workload id, tensor id), on the
device the tensors are made on.  A CUDA generator and a CPU generator give different values
for the same seed; a test draws its inputs once and hands the same tensors to both sides.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import torch

BLOCK = 128

TENSOR_IDS = {"q": 0, "k": 1, "v": 2}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # stable id mixed into the seeds
    batch: int
    heads: int
    lq: int
    lk: int
    head_dim: int
    dtype: str               # "f32" or "bf16"
    text: Tuple[int, int]    # forced key-block range [begin, end), text tokens
    extra: Tuple[int, int]   # forced key-block range [begin, end), Clip-1 image pyramid
    mode: str                # "topk" or "mass"
    param: float             # density (topk) or cumulative-mass threshold (mass)
    structure: str           # "iid" or "centroid"

    @property
    def n_q_blocks(self) -> int:
        return -(-self.lq // BLOCK)

    @property
    def n_k_blocks(self) -> int:
        return -(-self.lk // BLOCK)

    @property
    def rows(self) -> int:
        return self.batch * self.heads * self.n_q_blocks

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "toy": Workload("toy", 1, 1, 1, 1024, 1024, 64, "f32", (0, 1), (0, 0), "topk", 0.5, "iid"),
    "toy_dense": Workload("toy_dense", 1, 1, 1, 1024, 1024, 64, "f32", (0, 1), (0, 0), "topk", 1.0,
                          "iid"),
    "star_mid_clip2": Workload("star_mid_clip2", 2, 1, 32, 8192, 16896, 128, "bf16", (0, 4), (0, 0),
                               "topk", 0.1875, "centroid"),
    "clip1_early": Workload("clip1_early", 3, 1, 32, 18048, 22656, 128, "bf16", (0, 4), (4, 36),
                            "topk", 0.625, "centroid"),
    "final_720p_clip2": Workload("final_720p_clip2", 4, 1, 32, 72192, 144896, 128, "bf16", (0, 4),
                                 (0, 0), "topk", 0.09375, "centroid"),
    "dit_mass": Workload("dit_mass", 5, 1, 40, 75648, 75648, 128, "bf16", (0, 0), (0, 0), "mass",
                         0.9, "centroid"),
}

# The workload the benchmark times: the ~72k-token final scale.
BENCH_WORKLOAD = "final_720p_clip2"


def _seed(seed: int, wid: int, tensor: str) -> int:
    # splitmix-style mixing so neighbouring ids give unrelated streams
    x = (seed * 0x9E3779B97F4A7C15 + wid * 0xBF58476D1CE4E5B9 + TENSOR_IDS[tensor] * 0x94D049BB133111EB)
    x &= (1 << 64) - 1
    x ^= x >> 31
    x = (x * 0xD6E8FEB86659FD93) & ((1 << 64) - 1)
    x ^= x >> 32
    return x & ((1 << 63) - 1)


def make_tensor(w: Workload, tensor: str, device="cpu", seed: int = 0,
                heads: Optional[int] = None) -> torch.Tensor:
    """Draw Q, K or V of workload `w` as a contiguous [batch, heads, L, d] tensor in w's dtype."""
    h = w.heads if heads is None else heads
    length = w.lq if tensor == "q" else w.lk
    d = w.head_dim
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(_seed(seed, w.wid, tensor))
    if w.structure == "iid":
        x = torch.randn((w.batch, h, length, d), generator=g, device=dev, dtype=torch.float32)
    elif w.structure == "centroid":
        # a partial last block (length not a multiple of 128) takes the first tokens of a
        # block drawn whole
        nb = -(-length // BLOCK)
        cent = torch.randn((w.batch, h, nb, 1, d), generator=g, device=dev, dtype=torch.float32)
        cent.mul_(2.0)
        x = torch.randn((w.batch, h, nb, BLOCK, d), generator=g, device=dev, dtype=torch.float32)
        x.mul_(0.5).add_(cent)
        x = x.view(w.batch, h, nb * BLOCK, d)[:, :, :length]
        del cent
    else:
        raise ValueError(f"unknown structure {w.structure!r}")
    return x.to(w.torch_dtype).contiguous()


def make_qkv(w: Workload, device="cpu", seed: int = 0, heads: Optional[int] = None):
    return tuple(make_tensor(w, t, device, seed, heads) for t in ("q", "k", "v"))


PROMPT_SHARED = 0.75  # share of the centroid variance common to every calibration prompt


def make_prompt_tensor(w: Workload, tensor: str, prompt: int, device="cpu",
                       shared: float = PROMPT_SHARED) -> torch.Tensor:
    """Q, K or V of one synthetic calibration "prompt" of a centroid workload. The centroid of
    every (tensor, batch, head, block) is sqrt(shared) * a + sqrt(1 - shared) * b with a drawn
    once for the workload (common to all prompts) and b per prompt, both N(0, 2^2 I_d), so the
    centroid keeps the N(0, 2^2 I_d) law of make_tensor while prompts of one head share most of
    their block structure; tokens add per-prompt N(0, 0.5^2 I_d) noise."""
    if w.structure != "centroid":
        raise ValueError("prompts are defined for centroid workloads")
    length = w.lq if tensor == "q" else w.lk
    nb, d = length // BLOCK, w.head_dim
    dev = torch.device(device)
    g_common = torch.Generator(device=dev)
    g_common.manual_seed(_seed(0x5EED, w.wid, tensor))
    g_prompt = torch.Generator(device=dev)
    g_prompt.manual_seed(_seed(0x1000 + prompt, w.wid, tensor))
    cent = torch.randn((w.batch, w.heads, nb, 1, d), generator=g_common, device=dev,
                       dtype=torch.float32).mul_(2.0 * shared ** 0.5)
    cent.add_(torch.randn((w.batch, w.heads, nb, 1, d), generator=g_prompt, device=dev,
                          dtype=torch.float32), alpha=2.0 * (1.0 - shared) ** 0.5)
    x = torch.randn((w.batch, w.heads, nb, BLOCK, d), generator=g_prompt, device=dev,
                    dtype=torch.float32)
    x.mul_(0.5).add_(cent)
    return x.view(w.batch, w.heads, length, d).to(w.torch_dtype).contiguous()


def make_prompt_qkv(w: Workload, prompt: int, device="cpu", shared: float = PROMPT_SHARED):
    return tuple(make_prompt_tensor(w, t, prompt, device, shared) for t in ("q", "k", "v"))


def small_variants():
    """Reduced shapes for parity tests the oracle finishes in seconds.

    They keep each workload's segment structure and selection rule but shrink the token counts,
    choosing block counts that are not multiples of the kernels' tile sizes (ragged tails).
    """
    W = WORKLOADS
    return {
        "toy": W["toy"],
        "toy_dense": W["toy_dense"],
        "star_mid_small": W["star_mid_clip2"].with_(heads=3, lq=9 * BLOCK, lk=(4 + 9 + 9) * BLOCK),
        "clip1_small": W["clip1_early"].with_(heads=2, lq=11 * BLOCK, lk=(4 + 8 + 11) * BLOCK,
                                              extra=(4, 12)),
        "final_small": W["final_720p_clip2"].with_(heads=2, lq=17 * BLOCK, lk=(4 + 33 + 33) * BLOCK),
        "dit_mass_small": W["dit_mass"].with_(heads=2, lq=19 * BLOCK, lk=19 * BLOCK),
    }
