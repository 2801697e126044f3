"""Pins of the oracle's expert path: SwiGLU experts, weighted routed sum, shared experts.

Passages (archdiff.com): "Qwen3.5-397B-A17B vs Gemma 4 31B", component table, routed-experts
row (SwiGLU experts) and shared-expert row (shared output added to the routed sum); blueprint
shared-expert box "1-2, always active".  Shared experts are ungated by default (the DeepSeek-style
reading of that row); the Qwen3.5 cell's per-token sigmoid gate sigma(w . x) on the shared output
is pinned by its closed forms (w = 0 halves the shared part, saturation gives the ungated or the
routed-only output) and a per-token numpy check, for bf16 and block-scaled FP8 inputs.  Pins: a hand-computed one-token example, E = k = 1 reducing to a plain
SwiGLU MLP (numpy matmul), a dense brute force (every expert on every token, then mask), the
identity-like experts invariant, zero routed down-projections, and shared-expert
concatenation; for block-scaled FP8, the same dense brute force with torch's float8 cast.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_ffn_softplus_amd import PRESETS, synth
from tests._common import exact64, np_storage

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def silu(z):
    return z / (1.0 + np.exp(-z))


def _set(gate, up, down, **scales):
    n = len(gate)
    return oracle.ExpertSet(n, list(gate), list(up), list(down), **scales)


def _hand_example():
    with open(os.path.join(GOLDEN, "one_token_softmax.json")) as fh:
        ex = json.load(fh)
    f32 = lambda a: np.array(a, np.float32)  # noqa: E731
    routed = _set([f32(e["gate"]) for e in ex["experts"]], [f32(e["up"]) for e in ex["experts"]],
                  [f32(e["down"]) for e in ex["experts"]])
    sh = ex["shared"]
    shared = _set([f32(sh["gate"])], [f32(sh["up"])], [f32(sh["down"])])
    return ex, routed, shared


@pytest.mark.parametrize("k", [1, 2, 3])
def test_hand_example_softmax(k):
    ex, routed, shared = _hand_example()
    x = np.array([ex["x"]], np.float64)
    l = oracle.router_logits(x, np.array(ex["w_router"], np.float32))
    assert l.tolist() == [[1.0, 0.0, 1.0]]
    ids, w, _ = oracle.route(l, k)
    out = oracle.moe_tokens(x, ids, w, routed, shared, d=2, f=1, f_shared=1)
    s1, s2, s3 = 1 / (1 + math.exp(-1)), 2 / (1 + math.exp(-2)), 3 / (1 + math.exp(-3))
    y0, y1, y2 = np.array([2 * s1, 0.0]), np.array([0.0, s2]), np.array([-s3, -s3])
    ys = np.array([s2, s2])
    e = math.e
    want = {1: ys + y0,
            2: ys + 0.5 * y0 + 0.5 * y2,
            3: ys + (e * y0 + e * y2 + y1) / (2 * e + 1)}[k]
    assert np.max(np.abs(out[0] - want)) < 1e-12
    printed = {1: [3.22371131, 1.76159416], 2: [1.06379154, 0.33273297],
               3: [1.17220384, 0.82840978]}[k]
    assert np.max(np.abs(out[0] - printed)) < 2e-8
    # the same values frozen by tests/golden/make_golden.py from the oracle
    assert np.max(np.abs(out[0] - np.array(ex["oracle_out"][str(k)]))) < 1e-15


def test_E_equals_k_equals_1_is_a_plain_swiglu_mlp():
    rng = np.random.default_rng(1)
    T, d, f, fs = 7, 24, 16, 8
    x = rng.standard_normal((T, d))
    g, u, dn = (rng.standard_normal(s).astype(np.float32) for s in ((d, f), (d, f), (f, d)))
    sg, su, sd = (rng.standard_normal(s).astype(np.float32) for s in ((d, fs), (d, fs), (fs, d)))
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1))
    out = oracle.moe_tokens(x, ids, w, _set([g], [u], [dn]), _set([sg], [su], [sd]), d, f, fs)
    G, U, D = (a.astype(np.float64) for a in (g, u, dn))
    SG, SU, SD = (a.astype(np.float64) for a in (sg, su, sd))
    ref = (silu(x @ G) * (x @ U)) @ D + (silu(x @ SG) * (x @ SU)) @ SD
    assert np.max(np.abs(out - ref)) < 1e-12


def _dense_reference(x, ids, w, routed, shared):
    """Every routed expert on every token, masked by the routing and weighted; plus shared."""
    T = x.shape[0]
    E = routed["gate"].shape[0]
    ys = np.zeros_like(x)
    for s in range(shared["gate"].shape[0]):
        ys += (silu(x @ shared["gate"][s]) * (x @ shared["up"][s])) @ shared["down"][s]
    mask = np.zeros((T, E))
    for t in range(T):
        for j in range(ids.shape[1]):
            mask[t, ids[t, j]] += w[t, j]
    out = ys.copy()
    for e in range(E):
        ye = (silu(x @ routed["gate"][e]) * (x @ routed["up"][e])) @ routed["down"][e]
        out += mask[:, e:e + 1] * ye
    return out


def _oracle_sets(inp):
    r, s = inp["routed"], inp["shared"]
    E = r["gate"].shape[0]
    routed = _set([np_storage(r["gate"][e]) for e in range(E)],
                  [np_storage(r["up"][e]) for e in range(E)],
                  [np_storage(r["down"][e]) for e in range(E)])
    S = s["gate"].shape[0]
    shared = _set([np_storage(s["gate"][i]) for i in range(S)],
                  [np_storage(s["up"][i]) for i in range(S)],
                  [np_storage(s["down"][i]) for i in range(S)])
    return routed, shared


@pytest.mark.parametrize("name,score", [("tiny_fp32", oracle.SOFTMAX),
                                        ("tiny_fp32", oracle.SQRT_SOFTPLUS),
                                        ("tiny_fp32", oracle.SIGMOID)])
def test_dense_brute_force_tiny(name, score):
    cfg = PRESETS[name].with_(score=score, routed_scale=2.5 if score else 1.0,
                              select_bias_range=0.1 if score else 0.0, num_shared=2)
    inp = synth.inputs(cfg)
    x = exact64(inp["x"])
    l = oracle.router_logits(x, np_storage(inp["w_router"]))
    b = None if inp["select_bias"] is None else inp["select_bias"].numpy()
    ids, w, _ = oracle.route(l, cfg.top_k, score, True, cfg.routed_scale, b)
    routed, shared = _oracle_sets(inp)
    out = oracle.moe_tokens(x, ids, w, routed, shared, cfg.d_model, cfg.d_ff, cfg.d_ff_shared)
    dense = _dense_reference(x, ids, w, {k: exact64(v) for k, v in inp["routed"].items()},
                             {k: exact64(v) for k, v in inp["shared"].items()})
    assert np.max(np.abs(out - dense)) < 1e-12


@pytest.mark.parametrize("score,gamma", [(oracle.SOFTMAX, 1.0), (oracle.SQRT_SOFTPLUS, 2.5)])
def test_identity_like_experts_reproduce_the_input(score, gamma):
    # f = d, x[:, 0] = 1; every gate column is 32 e_0, so g = 32 and SiLU(32) = 32 to within
    # 4e-13; W_up = I/32 gives u = x/32, so h = x; W_down = I; shared down = 0.
    rng = np.random.default_rng(2)
    T, d, E, k = 12, 16, 5, 3
    x = rng.standard_normal((T, d))
    x[:, 0] = 1.0
    gate = np.zeros((d, d), np.float32)
    gate[0, :] = 32.0
    up = (np.eye(d) / 32).astype(np.float32)
    down = np.eye(d, dtype=np.float32)
    routed = _set([gate] * E, [up] * E, [down] * E)
    shared = _set([gate], [up], [np.zeros((d, d), np.float32)])
    ids, w, _ = oracle.route(rng.standard_normal((T, E)), k, score, True, gamma)
    out = oracle.moe_tokens(x, ids, w, routed, shared, d, d, d)
    assert np.max(np.abs(out - gamma * x)) < 1e-11


def test_zero_routed_down_gives_shared_only_and_shared_concat():
    rng = np.random.default_rng(4)
    T, d, f, fs, E, k = 6, 32, 16, 8, 4, 2
    x = rng.standard_normal((T, d))
    mk = lambda *s: rng.standard_normal(s).astype(np.float32)  # noqa: E731
    routed = _set([mk(d, f) for _ in range(E)], [mk(d, f) for _ in range(E)],
                  [np.zeros((f, d), np.float32) for _ in range(E)])
    sg, su, sd = [mk(d, fs) for _ in range(2)], [mk(d, fs) for _ in range(2)], \
        [mk(fs, d) for _ in range(2)]
    ids, w, _ = oracle.route(rng.standard_normal((T, E)), k)
    two = oracle.moe_tokens(x, ids, w, routed, _set(sg, su, sd), d, f, fs)
    # two shared experts == one shared expert of width 2 f_s (concatenated)
    one = _set([np.concatenate(sg, 1)], [np.concatenate(su, 1)], [np.concatenate(sd, 0)])
    cat = oracle.moe_tokens(x, ids, w, routed, one, d, f, 2 * fs)
    assert np.max(np.abs(two - cat)) < 1e-12
    ref = sum((silu(x @ g.astype(float)) * (x @ u.astype(float))) @ dd.astype(float)
              for g, u, dd in zip(sg, su, sd))
    assert np.max(np.abs(two - ref)) < 1e-12


def _torch_qdq_rows(a: np.ndarray, g: int = 128) -> np.ndarray:
    """Block-scaled E4M3 round trip with torch's cast (an independent codec)."""
    t = torch.from_numpy(a)
    R, C = t.shape
    b = t.reshape(R, C // g, g)
    amax = b.abs().amax(-1, keepdim=True)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
    q = (b.to(torch.float32) / s).clamp(-448, 448).to(torch.float8_e4m3fn)
    return (q.to(torch.float64) * s.to(torch.float64)).reshape(R, C).numpy()


def test_fp8_dense_brute_force():
    cfg = PRESETS["fp8_block"].with_(num_tokens=6, d_model=256, num_experts=3, top_k=2,
                                     d_ff=128, num_shared=1, d_ff_shared=256)
    inp = synth.inputs(cfg)
    x = exact64(inp["x"])
    rng = np.random.default_rng(9)
    ids = np.stack([rng.permutation(3)[:2] for _ in range(6)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, (6, 2))
    r, s = inp["routed"], inp["shared"]
    routed = oracle.ExpertSet(
        3, [np_storage(r["gate"][e]) for e in range(3)], [np_storage(r["up"][e]) for e in range(3)],
        [np_storage(r["down"][e]) for e in range(3)],
        gate_scales=[r["gate_scales"][e].numpy() for e in range(3)],
        up_scales=[r["up_scales"][e].numpy() for e in range(3)],
        down_scales=[r["down_scales"][e].numpy() for e in range(3)])
    shared = oracle.ExpertSet(
        1, [np_storage(s["gate"][0])], [np_storage(s["up"][0])], [np_storage(s["down"][0])],
        gate_scales=[s["gate_scales"][0].numpy()], up_scales=[s["up_scales"][0].numpy()],
        down_scales=[s["down_scales"][0].numpy()])
    out = oracle.moe_tokens(x, ids, w, routed, shared, 256, 128, 256, quant=True)

    def deq(codes, scales):
        c = exact64(codes)
        sc = scales.to(torch.float64).numpy()
        return c * np.kron(sc, np.ones((128, 128)))

    xq = _torch_qdq_rows(x)

    def expert(gq, gs, uq, us, dq, ds):
        h = silu(xq @ deq(gq, gs)) * (xq @ deq(uq, us))
        return _torch_qdq_rows(h) @ deq(dq, ds)

    ref = expert(s["gate"][0], s["gate_scales"][0], s["up"][0], s["up_scales"][0],
                 s["down"][0], s["down_scales"][0])
    for e in range(3):
        ye = expert(r["gate"][e], r["gate_scales"][e], r["up"][e], r["up_scales"][e],
                    r["down"][e], r["down_scales"][e])
        m = np.array([w[t][list(ids[t]).index(e)] if e in ids[t] else 0.0 for t in range(6)])
        ref = ref + m[:, None] * ye
    assert np.max(np.abs(out - ref)) < 1e-10 * np.max(np.abs(ref))


def _gate_case(quant):
    rng = np.random.default_rng(21 if quant else 20)
    T, d, f, fs, E, k = 9, 256, 128, 128, 5, 2
    x = rng.standard_normal((T, d))
    mk = lambda *s: (rng.standard_normal(s) / math.sqrt(s[0])).astype(np.float32)  # noqa: E731
    routed = _set([mk(d, f) for _ in range(E)], [mk(d, f) for _ in range(E)],
                  [mk(f, d) for _ in range(E)])
    shared = _set([mk(d, fs)], [mk(d, fs)], [mk(fs, d)])
    ids, w, _ = oracle.route(rng.standard_normal((T, E)), k)
    run = lambda w_, gate=None: oracle.moe_tokens(  # noqa: E731
        x, ids, w_, routed, shared, d, f, fs, quant=quant, shared_gate=gate)
    ungated = run(w)
    S = run(np.zeros_like(w))          # the shared experts alone
    return x, rng, run, w, ungated, S, ungated - S


@pytest.mark.parametrize("quant", [False, True])
def test_gated_shared_expert_closed_forms(quant):
    x, rng, run, w, ungated, S, R = _gate_case(quant)
    d = x.shape[1]
    # w_g = 0: sigma(0) = 1/2 exactly
    assert np.max(np.abs(run(w, np.zeros(d)) - (0.5 * S + R))) < 1e-12
    # a gate vector along one token's (quantised) input: sigma(+-40) saturates the gate to
    # within 5e-18 of 1 (the ungated block) or of 0 (the routed sum alone)
    xt = _torch_qdq_rows(x) if quant else x
    for sign, want in ((1.0, ungated), (-1.0, R)):
        g = sign * 40.0 * xt[0] / np.dot(xt[0], xt[0])
        assert np.max(np.abs(run(w, g)[0] - want[0])) < 1e-12 * np.max(np.abs(want[0]))


@pytest.mark.parametrize("quant", [False, True])
def test_gated_shared_expert_per_token(quant):
    x, rng, run, w, ungated, S, R = _gate_case(quant)
    g = rng.standard_normal(x.shape[1]) / math.sqrt(x.shape[1])
    xt = _torch_qdq_rows(x) if quant else x      # the gate reads what the experts read
    G = 1.0 / (1.0 + np.exp(-(xt @ g)))
    assert np.max(np.abs(run(w, g) - (G[:, None] * S + R))) < 1e-12


def test_missing_expert_is_an_error():
    d, f = 4, 2
    z = np.zeros((d, f), np.float32)
    routed = oracle.ExpertSet(2, [z, None], [z, None], [np.zeros((f, d), np.float32), None])
    with pytest.raises(ValueError):
        oracle.moe_tokens(np.zeros((1, d)), np.array([[1]], np.int32), np.ones((1, 1)), routed,
                          None, d, f, 1)


# ------------------------------------------------------------------ MXFP4 experts

def _mxfp4_dense(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Logical [K, N] fp64 values of an N-major MXFP4 matrix (codes [N, K/2], two per byte with
    the lower K index in the low nibble; E8M0 scales [N, K/32]), decoded with the OCP E2M1
    table and torch's E8M0 type."""
    table = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    table = np.concatenate([table, -table])
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1)   # [N, K]
    sc = torch.from_numpy(scales).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    return (table[nib] * np.repeat(sc, 32, axis=1)).T


def _rand_mxfp4(rng, n, k):
    codes = rng.integers(0, 256, (n, k // 2)).astype(np.uint8)
    scales = rng.integers(118, 126, (n, k // 32)).astype(np.uint8)
    return codes, scales


def test_mxfp4_one_hot_fixes_layout_and_nibble_order():
    # one nonzero weight: W_gate[k=5, n=3] = 1.5 * 2^1 (odd k: the high nibble of byte 2 of
    # row 3); W_up = 1 everywhere; W_down row 3 = e_7 (scale 2^0)
    d, f = 256, 128
    g = np.zeros((f, d // 2), np.uint8)
    g[3, 2] = 3 << 4
    gs = np.full((f, d // 32), 127, np.uint8)
    gs[3, 0] = 128
    u = np.full((f, d // 2), 0x22, np.uint8)
    us = np.full((f, d // 32), 127, np.uint8)
    dn = np.zeros((d, f // 2), np.uint8)
    dn[7, 1] = 2 << 4                                  # W_down[k=3, n=7] = 1.0
    ds = np.full((d, f // 32), 127, np.uint8)
    x = np.zeros((1, d))
    x[0, 5] = 1.0
    routed = oracle.ExpertSet(1, [g], [u], [dn], gate_scales=[gs], up_scales=[us],
                              down_scales=[ds], fmt="mxfp4")
    out = oracle.moe_tokens(x, np.zeros((1, 1), np.int32), np.ones((1, 1)), routed, None, d, f,
                            128, quant=False)
    want = np.zeros(d)
    want[7] = silu(3.0) * 1.0     # g[3] = x[5] * 3, u[3] = sum(x) = 1, h[3] -> y[7]
    assert np.max(np.abs(out[0] - want)) < 1e-15


def test_mxfp4_expert_equals_dense_swiglu_with_fp8_activations():
    # E = k = 1 reduces to a plain SwiGLU MLP on the dequantised weights; activations (x and
    # h) block-scaled FP8 as for E4M3 experts, checked with torch's float8 cast
    rng = np.random.default_rng(4)
    d, f, n = 256, 256, 5
    gq, gs = _rand_mxfp4(rng, f, d)
    uq, us = _rand_mxfp4(rng, f, d)
    dq, ds = _rand_mxfp4(rng, d, f)
    routed = oracle.ExpertSet(1, [gq], [uq], [dq], gate_scales=[gs], up_scales=[us],
                              down_scales=[ds], fmt="mxfp4")
    x = rng.standard_normal((n, d))
    out = oracle.moe_tokens(x, np.zeros((n, 1), np.int32), np.ones((n, 1)), routed, None, d, f,
                            128, quant=True)
    xq = _torch_qdq_rows(x)
    h = silu(xq @ _mxfp4_dense(gq, gs)) * (xq @ _mxfp4_dense(uq, us))
    ref = _torch_qdq_rows(h) @ _mxfp4_dense(dq, ds)
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))
