"""Seeded random layers through the C ABI against the oracle.

Each layer draws the expert format (bf16, E4M3, MXFP4, fp32), E, k, d, f, T, the score, the
renormalisation, the scale, the selection bias, the load skew and zero to two (gated) shared
experts, and is checked like the fixed small layers (every token) and for repeatability (the
same inputs give the same bits on every forward).  Shapes between the fixed cases catch what
those miss: a race in the LDS ring showed only on one such layer (16-row tiles, about 12 rows
per expert)."""
import random

import pytest
import torch

from mixture_experts_ffn_softplus_amd import PRESETS, api
from mixture_experts_ffn_softplus_amd.configs import SIGMOID, SOFTMAX, SQRT_SOFTPLUS, MoEConfig

SEED, COUNT = 7, 30


def random_layers(seed: int, n: int) -> list:
    rng = random.Random(seed)
    out = []
    for i in range(n):
        kind = rng.choice(["bf16", "bf16", "fp8", "fp8", "mx", "f32"])
        base = {"bf16": "softmax_bf16", "fp8": "fp8_block", "mx": "mxfp4_block",
                "f32": "tiny_fp32"}[kind]
        e4m3 = kind in ("fp8", "mx")
        E = rng.choice([4, 8, 16, 24, 40, 64, 96, 130])
        k = rng.randint(1, min(E, 12))
        d = rng.choice([128, 256]) if kind == "f32" else rng.choice([128, 256, 384])
        f = rng.choice([512, 768]) if e4m3 else rng.choice([128, 256, 512])
        T = rng.choice([1, 3, 17, 64, 130, 257, 400])
        S = rng.randint(0, 2)
        fs = (512 if e4m3 else rng.choice([128, 256, 512])) if S else 0
        out.append(PRESETS[base].with_(
            name=f"random{i}_{kind}", num_tokens=T, d_model=d, num_experts=E, top_k=k, d_ff=f,
            num_shared=S, d_ff_shared=fs, score=rng.choice([SOFTMAX, SIGMOID, SQRT_SOFTPLUS]),
            renormalize=rng.randint(0, 1), routed_scale=rng.choice([1.0, 2.5]), seed=1000 + i,
            select_bias_range=rng.choice([0.0, 0.1]), zipf_s=rng.choice([0.0, 0.0, 1.1]),
            shared_gate=rng.randint(0, 1) if S else 0))
    return out


LAYERS = random_layers(SEED, COUNT)


def test_random_layers_are_valid_configs():
    # host-side only: every drawn layer passes the library's config check
    assert len({c.name for c in LAYERS}) == COUNT
    for cfg in LAYERS:
        assert isinstance(cfg, MoEConfig)
        assert api.moe_workspace_size(cfg) > 0, cfg.describe()
    kinds = {c.name.split("_")[-1] for c in LAYERS}
    assert kinds == {"bf16", "fp8", "mx", "f32"}


@pytest.mark.gpu
@pytest.mark.parametrize("index", range(COUNT))
def test_random_layer_matches_oracle_and_repeats(index):
    from tests._gpu import Layer, check_layer

    cfg = LAYERS[index]
    layer = Layer(cfg)
    check_layer(layer)
    first = layer.forward()
    for _ in range(4):
        assert torch.equal(layer.forward(), first)
    del layer
    torch.cuda.empty_cache()
