"""moe_forward_noalloc (the block on the library's own static workspace, for callers that cannot
allocate) against moe_forward with a caller workspace, through the C ABI: two calls in a row,
the second with fewer tokens, each equal to moe_forward bit for bit (same kernels, same
inputs; the block is deterministic) and within the layer tolerance of the oracle."""
import numpy as np
import pytest
import torch

from mixture_experts_ffn_softplus_amd import PRESETS, api
from tests._gpu import TOL, Layer, oracle_block, oracle_route_on

pytestmark = pytest.mark.gpu

CASES = {
    # decode-shaped bf16 and FP8 layers (the callers this entry point is for)
    "bf16_decode": PRESETS["decode_bf16"].with_(name="noalloc_bf16_decode", num_tokens=64,
                                                d_model=1024, num_experts=64, top_k=8,
                                                d_ff=512, num_shared=1, d_ff_shared=512,
                                                seed=31),
    "fp8_decode": PRESETS["fp8_block"].with_(name="noalloc_fp8_decode", num_tokens=48,
                                             d_model=512, num_experts=32, top_k=6, d_ff=512,
                                             num_shared=1, d_ff_shared=512, seed=32),
}


def _both(cfg, layer, x):
    """out of moe_forward (caller workspace) and of moe_forward_noalloc, with the latter's
    logits for the oracle's routing."""
    dev = x.device
    T, E = cfg.num_tokens, cfg.num_experts
    ref = torch.empty(T, cfg.d_model, dtype=api.out_dtype(cfg), device=dev)
    api.moe_forward(cfg, x, layer.w, ref, layer.ws)
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    got = torch.full_like(ref, float("nan"))
    api.moe_forward_noalloc(cfg, x, layer.w, got, {"logits": logits})
    torch.cuda.synchronize()
    return ref, got, logits


@pytest.mark.parametrize("name", sorted(CASES))
def test_noalloc_forward_matches_forward_twice(name):
    cfg = CASES[name]
    assert api.moe_workspace_size(cfg) <= api.NOALLOC_SCRATCH_BYTES
    layer = Layer(cfg)
    x = layer.inp["x"]
    # first call: the whole batch; second call: fewer tokens on the same (now dirty) scratch
    for T in (cfg.num_tokens, cfg.num_tokens // 3 + 1):
        c = cfg.with_(num_tokens=T)
        print(f"[noalloc] {name}: T={T}", flush=True)
        xs = x[:T].contiguous()
        ref, got, logits = _both(c, layer, xs)
        assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), \
            f"T={T}: moe_forward_noalloc differs from moe_forward"
        ids, w, _ = oracle_route_on(c, logits, layer.inp["select_bias"])
        inp = dict(layer.inp, x=xs)
        want = oracle_block(c, inp, np.arange(T), ids, w)
        err = float(np.max(np.abs(got.double().cpu().numpy() - want)) /
                    np.sqrt(np.mean(want ** 2)))
        print(f"[noalloc] {name}: T={T} max-abs/RMS vs oracle {err:.3g}", flush=True)
        assert err <= TOL[cfg.expert_dtype]


def test_noalloc_forward_refuses_a_prefill_shape_on_the_gpu():
    cfg = PRESETS["softmax_bf16"].with_(num_tokens=4096)
    out = torch.empty(1, dtype=torch.float32, device="cuda")
    w = api.moe_weights_t(*([1] * len(api.moe_weights_t._fields_)))
    with pytest.raises(api.MoEError) as ei:
        api.moe_forward_noalloc(api.config_struct(cfg), out, w, out)
    assert ei.value.status == api.MOE_ERR_WORKSPACE_TOO_SMALL
