"""The seeded input generators: shapes, dtypes, reproducibility, and the block structure the
workload recipes state (centroid law, shared share of calibration prompts)."""
import torch

from synth import BLOCK, PROMPT_SHARED, make_prompt_qkv, make_qkv, small_variants


def test_reproducible_and_shaped():
    w = small_variants()["star_mid_small"]
    a = make_qkv(w, seed=3)
    b = make_qkv(w, seed=3)
    c = make_qkv(w, seed=4)
    for x, y, z, length in zip(a, b, c, (w.lq, w.lk, w.lk)):
        assert x.shape == (w.batch, w.heads, length, w.head_dim) and x.dtype == torch.bfloat16
        assert torch.equal(x, y) and not torch.equal(x, z)


def test_prompt_centroids_share_the_stated_variance():
    w = small_variants()["final_small"]
    ka = make_prompt_qkv(w, 0)[1].float()
    kb = make_prompt_qkv(w, 1)[1].float()
    # block means estimate the centroids (token noise variance 0.25 / 128 per coordinate)
    ca = ka.view(-1, BLOCK, w.head_dim).mean(1)
    cb = kb.view(-1, BLOCK, w.head_dim).mean(1)
    var = float(ca.var())
    corr = float(((ca - ca.mean()) * (cb - cb.mean())).mean() / (ca.std() * cb.std()))
    assert abs(var - 4.0) < 0.25
    assert abs(corr - PROMPT_SHARED) < 0.05
    # token noise around the centroid: N(0, 0.5^2)
    noise = ka.view(-1, BLOCK, w.head_dim) - ca[:, None, :]
    assert abs(float(noise.std()) - 0.5) < 0.02
