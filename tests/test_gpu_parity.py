"""GPU parity of the HIP path against the oracle, through the C ABI.

Graded (archdiff.com pages' block; tolerances are the layer's contract): router logits within
1e-4 RMS; expert ids bit-exact and weights within 1e-6 when the oracle routes on the GPU's
fp32 logits; expert offsets / permutation bit-exact; block output max-abs error / RMS(ref) at
most 1e-5 (fp32), 2e-2 (bf16), 6e-2 (block-scaled fp8).  Small layers check every token over
several tiles with ragged tails; the full-size workloads check a seeded token sample.

FP8 expert widths.  The 16x16x128 E4M3 MFMA of gfx950 does not sum its 128 products exactly
(measured against exact sums: median error 1.2e-5 of the result, at most about 2e-5 of the sum
of the products' magnitudes), so h = SiLU(g) * u carries that much relative error into its
re-quantisation and about 0.2% of the h codes land one E4M3 step from the oracle's.  One such
step moves an output row by (step) * scale * |W_down row|, which shrinks as 1/sqrt(F): at F = 128
a single step on a large h value can reach 0.1 * RMS, at F = 512 (the narrowest expert of the
FP8 workload) about half the 6e-2 bar.  The small FP8 layers therefore use F >= 512.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_ffn_softplus_amd import PRESETS, api, synth
from mixture_experts_ffn_softplus_amd.configs import BF16, F32, FP8_E4M3, MXFP4, SIGMOID, SOFTMAX, \
    SQRT_SOFTPLUS
from tests._common import exact64, np_storage, rel_err
from tests._gpu import Layer, check_layer, oracle_block, oracle_route_on

pytestmark = pytest.mark.gpu

BF = PRESETS["softmax_bf16"]
SMALL = {
    "bf16_softmax_ragged": BF.with_(name="bf16_softmax_ragged", num_tokens=300, d_model=256,
                                    num_experts=24, top_k=4, d_ff=128, num_shared=1,
                                    d_ff_shared=256, seed=11),
    "bf16_sqrt_softplus_zipf": PRESETS["softplus_bf16"].with_(
        name="bf16_sqrt_softplus_zipf", num_tokens=200, d_model=384, num_experts=20, top_k=3,
        d_ff=256, num_shared=2, d_ff_shared=128, seed=12),
    "bf16_sigmoid_norenorm": BF.with_(name="bf16_sigmoid_norenorm", num_tokens=130,
                                      d_model=256, num_experts=40, top_k=5, d_ff=128,
                                      num_shared=1, d_ff_shared=128, score=SIGMOID,
                                      renormalize=0, routed_scale=1.5, select_bias_range=0.05,
                                      seed=13),
    "bf16_many_rows": BF.with_(name="bf16_many_rows", num_tokens=1000, d_model=256,
                               num_experts=8, top_k=2, d_ff=256, num_shared=1, d_ff_shared=128,
                               seed=14),
    # FP8 cases keep the FP8 workload's expert widths (F >= 512, see the module docstring)
    "fp8_f32_router": PRESETS["fp8_block"].with_(name="fp8_f32_router", num_tokens=150,
                                                 d_model=256, num_experts=10, top_k=3,
                                                 d_ff=512, num_shared=1, d_ff_shared=512,
                                                 seed=15),
    "fp8_bf16_router": PRESETS["fp8_block"].with_(name="fp8_bf16_router", num_tokens=333,
                                                  d_model=384, num_experts=6, top_k=2,
                                                  d_ff=512, num_shared=2, d_ff_shared=256,
                                                  router_dtype=BF16, seed=16),
    "f32_softplus": PRESETS["tiny_fp32"].with_(name="f32_softplus", num_tokens=77,
                                               score=SQRT_SOFTPLUS, routed_scale=2.5,
                                               select_bias_range=0.1, num_shared=2, seed=17),
    # gated shared expert (Qwen3.5 cell of the shared-expert row): sigmoid(x~ . w_sg) per token
    "bf16_gated_shared": BF.with_(name="bf16_gated_shared", num_tokens=210, d_model=384,
                                  num_experts=16, top_k=4, d_ff=128, num_shared=2,
                                  d_ff_shared=128, shared_gate=1, seed=18),
    "fp8_gated_shared": PRESETS["fp8_block"].with_(name="fp8_gated_shared", num_tokens=170,
                                                   d_model=256, num_experts=8, top_k=2,
                                                   d_ff=512, num_shared=1, d_ff_shared=512,
                                                   shared_gate=1, seed=19),
    "fp8_gated_bf16_router": PRESETS["fp8_block"].with_(
        name="fp8_gated_bf16_router", num_tokens=95, d_model=384, num_experts=6, top_k=2,
        d_ff=512, num_shared=1, d_ff_shared=512, router_dtype=BF16, shared_gate=1, seed=20),
    "f32_gated_shared": PRESETS["tiny_fp32"].with_(name="f32_gated_shared", num_tokens=90,
                                                   num_shared=1, shared_gate=1, seed=21),
    # decode-like rows per expert: the E4M3-activation GEMMs take 16-row tiles
    "fp8_decode_rows": PRESETS["fp8_block"].with_(name="fp8_decode_rows", num_tokens=24,
                                                  d_model=384, num_experts=32, top_k=4,
                                                  d_ff=512, num_shared=1, d_ff_shared=512,
                                                  seed=22),
    # MXFP4 experts (E2M1 weights, E8M0 scales per 32 along K; E4M3 activations)
    "mxfp4_f32_router": PRESETS["mxfp4_block"].with_(name="mxfp4_f32_router", num_tokens=150,
                                                     d_model=256, num_experts=10, top_k=3,
                                                     d_ff=512, num_shared=1, d_ff_shared=512,
                                                     seed=23),
    "mxfp4_decode_rows": PRESETS["mxfp4_decode"].with_(name="mxfp4_decode_rows", num_tokens=40,
                                                       d_model=384, num_experts=24, top_k=4,
                                                       d_ff=512, num_shared=2, d_ff_shared=256,
                                                       seed=24),
    "mxfp4_many_rows": PRESETS["mxfp4_block"].with_(name="mxfp4_many_rows", num_tokens=600,
                                                    d_model=512, num_experts=4, top_k=2,
                                                    d_ff=768, num_shared=1, d_ff_shared=512,
                                                    router_dtype=BF16, seed=25),
    # one 128-deep K step per gate/up tile: with the deep LDS ring of the row-light E4M3 tiles
    # the loads run several tiles ahead of the MFMAs
    "fp8_decode_k128": PRESETS["fp8_block"].with_(name="fp8_decode_k128", num_tokens=20,
                                                  d_model=128, num_experts=16, top_k=2,
                                                  d_ff=512, num_shared=1, d_ff_shared=512,
                                                  seed=26),
    "mxfp4_decode_k128": PRESETS["mxfp4_decode"].with_(name="mxfp4_decode_k128", num_tokens=20,
                                                       d_model=128, num_experts=16, top_k=2,
                                                       d_ff=512, num_shared=1, d_ff_shared=256,
                                                       seed=27),
    # about 12 rows per expert: 16-row bf16 tiles, nearly all of them ragged, whose refills of
    # the zero rows past a tile's end return early (the LDS ring must not refill a slot before
    # every wave's fragment reads of it have executed)
    "bf16_short_tiles": BF.with_(name="bf16_short_tiles", num_tokens=130, d_model=256,
                                 num_experts=96, top_k=9, d_ff=512, num_shared=1,
                                 d_ff_shared=128, score=SQRT_SOFTPLUS, renormalize=0,
                                 routed_scale=2.5, select_bias_range=0.1, shared_gate=1,
                                 seed=1011),
    # decode-sized batches whose shared experts are as wide as a routed expert (S * f_s = f):
    # moe_forward runs them as one extra group of the routed GEMMs (the split calls do not)
    "bf16_decode_merged_shared": BF.with_(name="bf16_decode_merged_shared", num_tokens=48,
                                          d_model=256, num_experts=32, top_k=4, d_ff=256,
                                          num_shared=2, d_ff_shared=128, score=SQRT_SOFTPLUS,
                                          routed_scale=2.5, select_bias_range=0.1,
                                          shared_gate=1, seed=1012),
    "bf16_decode_merged_one_tile": BF.with_(name="bf16_decode_merged_one_tile", num_tokens=13,
                                            d_model=384, num_experts=40, top_k=3, d_ff=128,
                                            num_shared=1, d_ff_shared=128, seed=1013),
}


def test_tiny_fp32_end_to_end():
    check_layer(Layer(PRESETS["tiny_fp32"]))


@pytest.mark.parametrize("name", list(SMALL))
def test_small_layers(name):
    check_layer(Layer(SMALL[name]))


@pytest.mark.parametrize("name", ["fp8_f32_router", "fp8_bf16_router", "mxfp4_f32_router"])
def test_fp8_activation_codes_bit_exact(name):
    cfg = SMALL[name]
    layer = Layer(cfg)
    T, d, k = cfg.num_tokens, cfg.d_model, cfg.top_k
    dev = layer.ws.device
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    xq = torch.empty(T, d, dtype=torch.uint8, device=dev)
    xs = torch.empty(T, d // 128, dtype=torch.float32, device=dev)
    api.moe_route(cfg, layer.inp["x"], layer.w, None, ids, w, xq, xs, layer.ws)
    torch.cuda.synchronize()
    codes, scales, _ = oracle.quant_rows(exact64(layer.inp["x"]), 128)
    assert np.array_equal(xs.cpu().numpy(), scales)
    assert np.array_equal(xq.cpu().numpy(), codes)


def _crafted_fp8_rows(T: int, d: int, seed: int) -> torch.Tensor:
    """bf16 activation rows whose 128-value groups probe the quantiser's edges: all-zero groups,
    -0, one spike over values in (and below) E4M3's subnormal range, values exactly on code
    rounding midpoints (scale 1: amax = 448), a group whose maximum is the smallest bf16
    normal, and ordinary Gaussian groups."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, d, generator=g)
    groups = d // 128
    mids = torch.tensor([1.0625, 1.1875, 2.125, 2.375, 0.0068359375, 0.013671875, 208.0, 432.0,
                         -1.0625, -2.125, -0.0068359375, -208.0])
    for t in range(T):
        for gi in range(groups):
            kind = (t * groups + gi) % 6
            sl = slice(gi * 128, gi * 128 + 128)
            if kind == 0:
                x[t, sl] = 0.0
                x[t, gi * 128] = -0.0
            elif kind == 1:
                x[t, sl] = torch.randn(128, generator=g) * 1e-4
                x[t, gi * 128 + (t % 128)] = 3.0e3
            elif kind == 2:
                x[t, sl] = mids[torch.randint(0, len(mids), (128,), generator=g)]
                x[t, gi * 128 + 5] = 448.0
            elif kind == 3:
                x[t, sl] = torch.randn(128, generator=g).abs() * 2.0 ** -126
                x[t, gi * 128 + 3] = 2.0 ** -126
    return x.to(torch.bfloat16)


def test_fp8_activation_codes_bit_exact_on_crafted_rows():
    cfg = SMALL["fp8_bf16_router"].with_(num_tokens=97)
    layer = Layer(cfg)
    T, d, k = cfg.num_tokens, cfg.d_model, cfg.top_k
    dev = layer.ws.device
    x = _crafted_fp8_rows(T, d, 31).to(dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    xq = torch.empty(T, d, dtype=torch.uint8, device=dev)
    xs = torch.empty(T, d // 128, dtype=torch.float32, device=dev)
    api.moe_route(cfg, x, layer.w, None, ids, w, xq, xs, layer.ws)
    torch.cuda.synchronize()
    codes, scales, _ = oracle.quant_rows(exact64(x), 128)
    assert np.array_equal(xs.cpu().numpy(), scales)
    assert np.array_equal(xq.cpu().numpy(), codes)
    # the crafted groups did reach the edges: zero groups, subnormal codes, rounding ties
    assert (scales == 1.0).any() and ((codes & 0x78) == 0).any()


# The split calls run the shared experts in launches of their own; moe_forward of the
# decode-sized layers here runs them as an extra group of the routed GEMMs: the same bits.
@pytest.mark.parametrize("name", ["bf16_sqrt_softplus_zipf", "bf16_gated_shared",
                                  "bf16_decode_merged_shared", "bf16_decode_merged_one_tile",
                                  "fp8_decode_rows", "mxfp4_decode_rows"])
def test_split_api_matches_forward_bit_exact(name):
    cfg = SMALL[name]
    layer = Layer(cfg)
    out_f = layer.forward()
    T, E, k, A, d = cfg.num_tokens, cfg.num_experts, cfg.top_k, cfg.assignments, cfg.d_model
    dev = layer.ws.device
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(A, dtype=torch.int32, device=dev)
    inv = torch.empty(A, dtype=torch.int32, device=dev)
    y = torch.empty(A, d, dtype=api.y_dtype(cfg), device=dev)
    out = torch.empty(T, d, dtype=api.out_dtype(cfg), device=dev)
    x = layer.inp["x"]
    xq = xs = None
    if cfg.expert_dtype in (FP8_E4M3, MXFP4):  # block-scaled E4M3 activations from the router
        xq = torch.empty(T, d, dtype=torch.uint8, device=dev)
        xs = torch.empty(T, d // 128, dtype=torch.float32, device=dev)
    api.moe_route(cfg, x, layer.w, logits, ids, w, xq, xs, ws=layer.ws)
    # route_from_logits on the same logits gives the same ids and weights
    ids2 = torch.empty_like(ids)
    w2 = torch.empty_like(w)
    api.moe_route_from_logits(cfg, logits, layer.inp["select_bias"], ids2, w2)
    api.moe_permute(cfg, ids, off, perm, inv, layer.ws)
    xa = x if xq is None else xq
    api.moe_expert_ffn(cfg, xa, xs, off, perm, layer.w, y, layer.ws)
    api.moe_combine(cfg, xa, xs, y, inv, w, layer.w, out, layer.ws)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(w, w2)
    assert torch.equal(out, out_f)


@pytest.mark.parametrize("name", ["bf16_softmax_ragged", "bf16_short_tiles", "fp8_decode_rows"])
def test_forward_is_deterministic(name):
    # repeated forwards: a race inside a kernel shows as an occasional different result (a
    # slot refilled too early once changed a whole row tile in about one forward in seven of
    # bf16_short_tiles)
    layer = Layer(SMALL[name])
    first = layer.forward()
    for _ in range(40):
        assert torch.equal(layer.forward(), first)


@pytest.mark.parametrize("name", ["bf16_softmax_ragged", "bf16_short_tiles", "fp8_f32_router",
                                  "mxfp4_decode_rows"])
def test_bf16_output_is_the_rounded_fp32_output(name):
    # out_f32 changes only the store of the combine's fp32 sum: the bf16 output is that sum
    # rounded to nearest even, bit for bit (so its parity follows from the fp32 output's)
    base = SMALL[name]
    layer = Layer(base.with_(out_f32=1))
    full = layer.forward()
    cfg16 = base.with_(out_f32=0)
    out = torch.empty(cfg16.num_tokens, cfg16.d_model, dtype=torch.bfloat16, device="cuda")
    api.moe_forward(cfg16, layer.inp["x"], layer.w, out, layer.ws)
    torch.cuda.synchronize()
    assert full.dtype == torch.float32
    assert torch.equal(out, full.to(torch.bfloat16))


def test_route_from_logits_with_ties_bit_exact():
    # integer-valued logits give many exactly equal keys: the lower expert index must win
    cfg = BF.with_(num_tokens=257, num_experts=96, top_k=7)
    g = torch.Generator().manual_seed(5)
    logits = torch.randint(-3, 4, (257, 96), generator=g).float().cuda()
    for score, gamma, sb in [(SOFTMAX, 1.0, None),
                             (SQRT_SOFTPLUS, 2.5, torch.linspace(-0.1, 0.1, 96).cuda()),
                             (SIGMOID, 1.0, torch.zeros(96).cuda())]:
        c = cfg.with_(score=score, routed_scale=gamma)
        ids = torch.empty(257, 7, dtype=torch.int32, device="cuda")
        w = torch.empty(257, 7, dtype=torch.float32, device="cuda")
        api.moe_route_from_logits(c, logits, sb, ids, w)
        torch.cuda.synchronize()
        ids_ref, w_ref, _ = oracle_route_on(c, logits, sb)
        assert np.array_equal(ids.cpu().numpy(), ids_ref)
        assert np.max(np.abs(w.cpu().double().numpy() - w_ref)) <= 1e-6 * max(gamma, 1)


@pytest.mark.parametrize("k", [64, 22, 1])
def test_route_from_logits_with_ties_at_1024_experts(k):
    # the library's largest expert count (16 experts a lane) and top-k: integer-valued logits
    # make most heads tie in every round, across lanes and within a lane
    T, E = 193, 1024
    cfg = BF.with_(num_tokens=T, num_experts=E, top_k=k)
    g = torch.Generator().manual_seed(6 + k)
    logits = torch.randint(-2, 3, (T, E), generator=g).float().cuda()
    for score, gamma, sb in [(SOFTMAX, 1.0, None),
                             (SQRT_SOFTPLUS, 2.5, (torch.arange(E) % 3 - 1).float().cuda() * 0.25)]:
        c = cfg.with_(score=score, routed_scale=gamma)
        ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
        w = torch.empty(T, k, dtype=torch.float32, device="cuda")
        api.moe_route_from_logits(c, logits, sb, ids, w)
        torch.cuda.synchronize()
        ids_ref, w_ref, _ = oracle_route_on(c, logits, sb)
        assert np.array_equal(ids.cpu().numpy(), ids_ref)
        assert np.max(np.abs(w.cpu().double().numpy() - w_ref)) <= 1e-6 * max(gamma, 1)


# The library's limits: 1024 experts, top-64 (every routing lane and combine slot in use).
LIMITS = {
    "max_E_max_k_softmax": BF.with_(name="max_E_max_k_softmax", num_tokens=40, d_model=256,
                                    num_experts=1024, top_k=64, d_ff=128, num_shared=1,
                                    d_ff_shared=128, seed=51),
    "max_E_max_k_sqrt_softplus": PRESETS["softplus_bf16"].with_(
        name="max_E_max_k_sqrt_softplus", num_tokens=33, d_model=256, num_experts=1024,
        top_k=64, d_ff=128, num_shared=1, d_ff_shared=128, seed=52),
    "max_E_max_k_fp8": PRESETS["fp8_block"].with_(name="max_E_max_k_fp8", num_tokens=24,
                                                  d_model=256, num_experts=1024, top_k=64,
                                                  d_ff=512, num_shared=1, d_ff_shared=512,
                                                  seed=53),
    "max_E_top1_many_tokens": BF.with_(name="max_E_top1_many_tokens", num_tokens=3000,
                                       d_model=256, num_experts=1024, top_k=1, d_ff=128,
                                       num_shared=1, d_ff_shared=128, seed=54),
}


@pytest.mark.parametrize("name", list(LIMITS))
def test_layers_at_the_limits(name):
    check_layer(Layer(LIMITS[name]))


# Decode-sized batches with a deep reduction split the router GEMM's K into ranges whose partial
# logits the top-k waves add (2, 8 and 4 ranges here: bf16, the fp32 router's bf16 hi + lo
# planes, fp32); the logits, ids and block output are checked as everywhere, and repeated
# forwards must agree bit for bit.
ROUTER_SPLIT = {
    "router_split_bf16": BF.with_(name="router_split_bf16", num_tokens=8, d_model=1024,
                                  num_experts=32, top_k=2, d_ff=128, num_shared=1,
                                  d_ff_shared=128, seed=71),
    "router_split_fp8_f32_router": PRESETS["fp8_block"].with_(
        name="router_split_fp8_f32_router", num_tokens=16, d_model=2048, num_experts=64,
        top_k=4, d_ff=512, num_shared=1, d_ff_shared=512, seed=72),
    "router_split_f32": PRESETS["tiny_fp32"].with_(name="router_split_f32", num_tokens=8,
                                                   d_model=1024, num_experts=16, top_k=2,
                                                   d_ff=128, num_shared=1, d_ff_shared=256,
                                                   seed=73),
}


@pytest.mark.parametrize("name", list(ROUTER_SPLIT))
def test_split_router_layers(name):
    layer = Layer(ROUTER_SPLIT[name])
    check_layer(layer)
    first = layer.forward()
    for _ in range(5):
        assert torch.equal(layer.forward(), first)


# Batches of at most 4096 assignments over at most 768 experts are permuted by one workgroup
# (rounds of 1024 assignments), larger ones by the multi-kernel counting sort: both sides of
# each limit are here, with one expert taking every assignment across all four rounds.
@pytest.mark.parametrize("T,k,E,mode", [(4096, 10, 512, "uniform"), (1000, 3, 64, "skewed"),
                                        (3, 2, 1000, "uniform"), (1, 1, 1, "uniform"),
                                        (16384, 22, 896, "uniform"), (513, 4, 300, "one_hot"),
                                        (1024, 4, 768, "uniform"), (1365, 3, 768, "uniform"),
                                        (1024, 4, 769, "uniform"), (683, 6, 300, "uniform"),
                                        (4096, 1, 700, "one_hot"), (64, 8, 256, "uniform")])
def test_permute_external_ids_bit_exact(T, k, E, mode):
    rng = np.random.default_rng(T + k + E)
    if mode == "uniform":
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    elif mode == "skewed":
        ids = np.stack([np.concatenate([[0], 1 + rng.permutation(7)[:k - 1]]) for _ in range(T)])
    else:  # every token uses experts 5..5+k-1: one hot block, all others empty
        ids = np.tile(np.arange(5, 5 + k), (T, 1))
    ids = ids.astype(np.int32)
    cfg = BF.with_(num_tokens=T, num_experts=E, top_k=k)
    ws = api.workspace(cfg)
    d_ids = torch.from_numpy(ids).cuda()
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    api.moe_permute(cfg, d_ids, off, perm, inv, ws)
    torch.cuda.synchronize()
    o, p, i = oracle.permute(ids, E)
    assert np.array_equal(off.cpu().numpy(), o)
    assert np.array_equal(perm.cpu().numpy(), p)
    assert np.array_equal(inv.cpu().numpy(), i)


@pytest.mark.parametrize("case", ["k_equals_E", "single_expert", "single_token", "no_shared",
                                  "gated_single_token", "gated_no_shared"])
def test_degenerate_layers(case):
    base = SMALL["bf16_softmax_ragged"]
    cfg = {"k_equals_E": base.with_(num_experts=6, top_k=6, num_tokens=50),
           "single_expert": base.with_(num_experts=1, top_k=1, num_tokens=40),
           "single_token": base.with_(num_tokens=1),
           "no_shared": base.with_(num_shared=0, num_tokens=70),
           "gated_single_token": base.with_(num_tokens=1, shared_gate=1),
           # a gate with no shared expert to scale is ignored (no gate vector is passed)
           "gated_no_shared": base.with_(num_shared=0, num_tokens=70, shared_gate=1)}[case]
    check_layer(Layer(cfg.with_(name=case)))


@pytest.mark.parametrize("name", ["bf16_gated_shared", "fp8_gated_shared",
                                  "fp8_gated_bf16_router", "f32_gated_shared"])
def test_shared_gate_factor(name):
    """The gate alone: with the routed experts' down projections zeroed, the gated output over
    the ungated one is G[t] = sigmoid(x~[t] . w_sg) on every column of token t.  No FP8 h
    rounding enters (both runs share the shared experts' output S), so G is checked far
    below the block tolerance: out = round(G S) and round(S) in the output dtype, and the
    least-squares ratio over the d columns is off by at most the two roundings (2^-8 relative
    for bf16 worst case; 1e-3 allowed) -- or 1e-5 for fp32 outputs."""
    cfg = SMALL[name]
    inp = synth.inputs(cfg, "cuda")
    routed = dict(inp["routed"])
    routed["down"] = routed["down"].clone()
    routed["down"].view(torch.uint8).zero_()
    pw = api.pack(cfg, inp["w_router"], routed, inp["shared"], inp["logit_bias"],
                  inp["select_bias"], shared_gate=inp["shared_gate"])
    ws = api.workspace(cfg)
    T, d = cfg.num_tokens, cfg.d_model
    outs = []
    for gated in (1, 0):
        out = torch.empty(T, d, dtype=api.out_dtype(cfg), device="cuda")
        api.moe_forward(cfg.with_(shared_gate=gated), inp["x"], pw.struct(), out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    g_out, s_out = (o.double().cpu().numpy() for o in outs)
    g_fit = np.sum(g_out * s_out, axis=1) / np.sum(s_out * s_out, axis=1)
    x = exact64(inp["x"])
    if cfg.expert_dtype == FP8_E4M3:
        x = oracle.quant_rows(x, cfg.quant_block)[2]
    g_ref = 1.0 / (1.0 + np.exp(-(x @ exact64(inp["shared_gate"]))))
    tol = 1e-5 if cfg.act_dtype == F32 else 1e-3
    err = float(np.max(np.abs(g_fit - g_ref)))
    print(f"[gate] {name}: max |G - G_ref| {err:.2e}, G in [{g_ref.min():.3f}, {g_ref.max():.3f}]")
    assert err <= tol
    # the gate is not trivial on these inputs
    assert g_ref.min() < 0.3 and g_ref.max() > 0.7


def test_zero_tokens_launches_nothing():
    cfg = SMALL["bf16_softmax_ragged"]
    layer = Layer(cfg)
    c0 = cfg.with_(num_tokens=0)
    out = torch.full((1, cfg.d_model), 7.0, dtype=api.out_dtype(cfg), device="cuda")
    api.moe_forward(c0, layer.inp["x"], layer.w, out, layer.ws)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_identity_like_experts_reproduce_input():
    # f = d; x[:, 0] = 1; gate columns 32 e_0; up = I/32; down = I; shared down = 0 -> out = x
    # (bf16 output: its rounding is what the bound below allows for)
    cfg = BF.with_(name="identity", num_tokens=96, d_model=128, num_experts=8, top_k=3,
                   d_ff=128, num_shared=1, d_ff_shared=128, score=SQRT_SOFTPLUS,
                   routed_scale=2.5, out_f32=0)
    d, E = 128, 8
    inp = synth.inputs(cfg, "cuda")
    x = inp["x"].clone()
    x[:, 0] = 1.0
    gate = torch.zeros(E, d, d, device="cuda")
    gate[:, 0, :] = 32.0
    up = (torch.eye(d, device="cuda") / 32).expand(E, d, d)
    down = torch.eye(d, device="cuda").expand(E, d, d)
    routed = {"gate": gate.bfloat16().contiguous(), "up": up.bfloat16().contiguous(),
              "down": down.bfloat16().contiguous()}
    shared = {"gate": routed["gate"][:1].contiguous(), "up": routed["up"][:1].contiguous(),
              "down": torch.zeros(1, d, d, dtype=torch.bfloat16, device="cuda")}
    pw = api.pack(cfg, inp["w_router"], routed, shared)
    ws = api.workspace(cfg)
    out = torch.empty(x.shape, dtype=api.out_dtype(cfg), device="cuda")
    api.moe_forward(cfg, x, pw.struct(), out, ws)
    torch.cuda.synchronize()
    # the output is the bf16 rounding of sum_j w_j x with sum_j w_j = 2.5 up to fp32 rounding:
    # within half a bf16 ulp of 2.5 x, i.e. 2^(floor(log2|v|) - 8), plus that fp32 slack
    want = 2.5 * x.double().cpu().numpy()
    got = out.double().cpu().numpy()
    half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 8)
    assert np.all(np.abs(got - want) <= half_ulp + 2e-6 * np.abs(want))
    assert np.all(got[:, 0] == 2.5)


# ---------------------------------------------------------------- full-size workloads

# decode shapes check every token; the prefill shapes a seeded sample of 256 tokens (0.4-6% of
# their rows), which the oracle computes in seconds on the host's cores
@pytest.mark.parametrize("name,sample", [("decode_bf16", 64), ("softmax_bf16", 256),
                                         ("softplus_bf16", 256), ("fp8_block", 256),
                                         ("qwen_gated_bf16", 64), ("mxfp4_decode", 64),
                                         ("mxfp4_block", 64)])
def test_full_size_workloads(name, sample):
    cfg = PRESETS[name]
    layer = Layer(cfg)
    res, _, _ = check_layer(layer, sample=sample, seed=1, max_experts=48)
    del layer
    torch.cuda.empty_cache()


def test_fp16_y_overflow_is_non_finite():
    # bf16 experts keep y_perm as IEEE fp16: an expert output value of magnitude 65520 or more
    # overflows.  Expert 3's down projection scaled by 2^20 (exact in bf16) puts nearly all of its
    # output values past that; every token routed to it must come out non-finite (never a
    # wrong finite row), and every other token must still match the oracle.
    cfg = BF.with_(name="fp16_overflow", num_tokens=96, d_model=256, num_experts=8, top_k=2,
                   d_ff=256, num_shared=1, d_ff_shared=256, seed=31)
    inp = synth.inputs(cfg, "cuda")
    inp["routed"]["down"][3].mul_(2.0 ** 20)
    pw = api.pack(cfg, inp["w_router"], inp["routed"], inp["shared"], inp["logit_bias"],
                  inp["select_bias"], shared_gate=inp["shared_gate"])
    ws = api.workspace(cfg)
    T, k, A = cfg.num_tokens, cfg.top_k, cfg.assignments
    dbg = {"logits": torch.empty(T, cfg.num_experts, dtype=torch.float32, device="cuda"),
           "topk_ids": torch.empty(T, k, dtype=torch.int32, device="cuda"),
           "topk_w": torch.empty(T, k, dtype=torch.float32, device="cuda")}
    out = torch.empty(T, cfg.d_model, dtype=api.out_dtype(cfg), device="cuda")
    api.moe_forward(cfg, inp["x"], pw.struct(), out, ws, dbg)
    torch.cuda.synchronize()
    hit = (dbg["topk_ids"] == 3).any(dim=1).cpu().numpy()
    assert 0 < hit.sum() < T
    finite = torch.isfinite(out).cpu().numpy()
    assert not finite[hit].all(axis=1).any()           # every hit token has non-finite values
    assert (~finite[hit]).mean() > 0.9                  # and nearly all of its values are
    ids, w, _ = oracle_route_on(cfg, dbg["logits"], inp["select_bias"])
    tok = np.nonzero(~hit)[0]
    ref = oracle_block(cfg, inp, tok, ids[tok], w[tok])
    got = out[torch.as_tensor(tok, device="cuda")].double().cpu().numpy()
    assert np.isfinite(got).all()
    assert rel_err(got, ref) <= 2e-2
