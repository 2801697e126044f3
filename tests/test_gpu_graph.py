"""The block under HIP-graph capture.

moe_forward and moe_forward_noalloc make no allocation, memset or host synchronisation and read
every size they launch with from the device (tile lists, offsets), so one forward can be captured
once and replayed on new inputs written into the same buffers.  Each replay is checked bit for
bit against an eager forward of the same inputs on a workspace of its own, with eager work and
synchronisations between the replays; the inputs change between replays, so the routing, the
tile lists and the grid's share of tiles all differ from the captured call's.
"""
import pytest
import torch

from mixture_experts_ffn_softplus_amd import PRESETS, api
from tests._gpu import Layer

pytestmark = pytest.mark.gpu

BF = PRESETS["softmax_bf16"]
CASES = {
    # ragged bf16 tiles, softmax router
    "bf16_ragged": BF.with_(name="graph_bf16_ragged", num_tokens=300, d_model=256,
                            num_experts=24, top_k=4, d_ff=128, num_shared=1, d_ff_shared=256,
                            seed=41),
    # block-scaled FP8 experts, fp32 router, gated shared expert
    "fp8_gated": PRESETS["fp8_block"].with_(name="graph_fp8_gated", num_tokens=170, d_model=256,
                                            num_experts=8, top_k=2, d_ff=512, num_shared=1,
                                            d_ff_shared=512, shared_gate=1, seed=42),
    # decode-sized batch: shared experts inside the routed launches, one-workgroup permutation
    "decode_bf16": PRESETS["decode_bf16"].with_(name="graph_decode_bf16", num_tokens=16,
                                                d_model=512, num_experts=64, top_k=4,
                                                d_ff=256, num_shared=1, d_ff_shared=256,
                                                seed=43),
    # MXFP4 experts at decode size
    "mxfp4_decode": PRESETS["mxfp4_decode"].with_(name="graph_mxfp4_decode", num_tokens=24,
                                                  d_model=512, num_experts=32, top_k=4,
                                                  d_ff=512, num_shared=1, d_ff_shared=512,
                                                  seed=44),
}


def _new_inputs(x0: torch.Tensor, r: int) -> torch.Tensor:
    # a different, deterministic input per replay: the rows of x0 rotated and rescaled
    return (torch.roll(x0.float(), shifts=7 * r + 1, dims=0) * (1.0 + 0.125 * r)).to(x0.dtype)


def _capture(fn):
    # first calls (per-device set-up, cached occupancy queries) run eagerly on a side stream
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager_forwards(name, noalloc):
    cfg = CASES[name]
    print(f"[graph] {name} noalloc={noalloc}", flush=True)
    layer = Layer(cfg, keep_logical=False)
    x, w = layer.inp["x"], layer.w
    T, d = cfg.num_tokens, cfg.d_model
    out = torch.empty(T, d, dtype=api.out_dtype(cfg), device="cuda")
    if noalloc:
        g = _capture(lambda: api.moe_forward_noalloc(cfg, x, w, out))
    else:
        g = _capture(lambda: api.moe_forward(cfg, x, w, out, layer.ws))
    ws_ref = api.workspace(cfg)
    ref = torch.empty_like(out)
    x0 = x.clone()
    for r in range(4):
        x.copy_(_new_inputs(x0, r))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        # eager work between the replays: the reference forward on its own workspace
        api.moe_forward(cfg, x, w, ref, ws_ref)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay {r} differs from the eager forward"
        if r > 0:
            assert not torch.equal(got, prev), "the replay did not follow the new inputs"
        prev = got
