"""GPU-test helpers: build a layer on the device, run the block through the C ABI, and compute
the oracle's answers for the same inputs (routing taken on the GPU's fp32 logits)."""
import numpy as np
import torch

import oracle
from mixture_experts_ffn_softplus_amd import api, synth
from mixture_experts_ffn_softplus_amd.configs import F32, FP8_E4M3, MXFP4, MoEConfig
from tests._common import exact64, np_storage, rel_err

# max-abs error / RMS(ref) by expert dtype; MXFP4 experts have the block-scaled E4M3 activations
# of FP8 experts (their weights are exact inputs), so the FP8 bar
TOL = {F32: 1e-5, 1: 2e-2, FP8_E4M3: 6e-2, MXFP4: 6e-2}


class Layer:
    def __init__(self, cfg: MoEConfig, device="cuda", keep_logical=True):
        self.cfg = cfg
        print(f"[layer] {cfg.describe()}", flush=True)
        self.inp = synth.inputs(cfg, device)
        self.pw = api.pack(cfg, self.inp["w_router"], self.inp["routed"], self.inp["shared"],
                           self.inp["logit_bias"], self.inp["select_bias"],
                           shared_gate=self.inp["shared_gate"])
        torch.cuda.synchronize()
        if not keep_logical:
            self.inp["routed"] = None
        self.w = self.pw.struct()
        self.ws = api.workspace(cfg, device)

    def debug_buffers(self):
        c = self.cfg
        T, E, k, A = c.num_tokens, c.num_experts, c.top_k, c.assignments
        dev = self.ws.device
        return {
            "logits": torch.empty(T, E, dtype=torch.float32, device=dev),
            "topk_ids": torch.empty(T, k, dtype=torch.int32, device=dev),
            "topk_w": torch.empty(T, k, dtype=torch.float32, device=dev),
            "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "perm_token": torch.empty(A, dtype=torch.int32, device=dev),
            "inv_perm": torch.empty(A, dtype=torch.int32, device=dev),
            "y_perm": torch.empty(A, c.d_model, dtype=api.y_dtype(c), device=dev),
        }

    def forward(self, dbg=None):
        c = self.cfg
        out = torch.empty(c.num_tokens, c.d_model, dtype=api.out_dtype(c), device=self.ws.device)
        api.moe_forward(c, self.inp["x"], self.w, out, self.ws, dbg)
        return out


def oracle_route_on(cfg: MoEConfig, logits_gpu: torch.Tensor, select_bias):
    sb = None if select_bias is None else select_bias.detach().cpu().numpy()
    return oracle.route(logits_gpu.detach().cpu().double().numpy(), cfg.top_k, cfg.score,
                        bool(cfg.renormalize), cfg.routed_scale, sb)


def _expert_host(stack: dict, e: int) -> dict:
    out = {}
    for key, v in stack.items():
        out[key] = v[e].detach().cpu().numpy() if key.endswith("scales") else np_storage(v[e])
    return out


def _expert_set(parts: list, n: int, index: list, fmt=None) -> oracle.ExpertSet:
    slots = [None] * n
    for e, p in zip(index, parts):
        slots[e] = p

    def col(key):
        return [None if s is None else s.get(key) for s in slots]
    return oracle.ExpertSet(n, col("gate"), col("up"), col("down"), gate_scales=col("gate_scales"),
                            up_scales=col("up_scales"), down_scales=col("down_scales"), fmt=fmt)


def oracle_block(cfg: MoEConfig, inp: dict, tokens, ids, w, max_experts=64):
    """Oracle output rows for `tokens` with the given ids / weights, fetching from the device
    only the experts those tokens use, in batches of at most `max_experts` experts."""
    tokens = np.asarray(tokens)
    x = exact64(inp["x"][torch.as_tensor(tokens, device=inp["x"].device)])
    sh = inp["shared"]
    fmt = "mxfp4" if cfg.expert_dtype == MXFP4 else None
    shared = None
    if sh is not None:
        S = sh["gate"].shape[0]
        shared = _expert_set([_expert_host(sh, s) for s in range(S)], S, list(range(S)), fmt)
    gate = None if inp.get("shared_gate") is None else exact64(inp["shared_gate"])
    out = np.empty((len(tokens), cfg.d_model))
    i = 0
    while i < len(tokens):
        used, j = set(), i
        while j < len(tokens) and len(used | set(ids[j].tolist())) <= max_experts:
            used |= set(ids[j].tolist())
            j += 1
        j = max(j, i + 1)
        used = sorted(used | set(ids[i].tolist()))
        parts = [_expert_host(inp["routed"], e) for e in used]
        routed = _expert_set(parts, cfg.num_experts, used, fmt)
        out[i:j] = oracle.moe_tokens(x[i:j], ids[i:j], w[i:j], routed, shared, cfg.d_model,
                                     cfg.d_ff, cfg.d_ff_shared,
                                     quant=cfg.expert_dtype in (FP8_E4M3, MXFP4),
                                     block=cfg.quant_block,
                                     shared_gate=gate)
        i = j
    return out


def check_layer(layer: Layer, sample=None, seed=0, max_experts=64):
    """Run moe_forward with every debug output and check each step against the oracle.
    Returns a dict of measured errors."""
    cfg, inp = layer.cfg, layer.inp
    dbg = layer.debug_buffers()
    out = layer.forward(dbg)
    torch.cuda.synchronize()
    T = cfg.num_tokens
    rng = np.random.default_rng(seed)
    if sample is None or sample >= T:
        tok = np.arange(T)
    else:
        tok = np.unique(np.concatenate([[0, T - 1], rng.choice(T, sample - 2, replace=False)]))
    res = {}
    # router logits on the sampled tokens, oracle in fp64
    lz = inp["logit_bias"]
    l_ref = oracle.router_logits(exact64(inp["x"][torch.as_tensor(tok, device=inp["x"].device)]),
                                 np_storage(inp["w_router"]),
                                 None if lz is None else lz.cpu().numpy())
    l_gpu = dbg["logits"].cpu().double().numpy()
    rms = float(np.sqrt(np.mean(l_ref ** 2)))
    res["logit_err"] = float(np.max(np.abs(l_gpu[tok] - l_ref))) / rms
    assert res["logit_err"] <= 1e-4, res
    # ids bit-exact and weights to 1e-6 when routed on the GPU's logits (all tokens)
    ids_ref, w_ref, _ = oracle_route_on(cfg, dbg["logits"], inp["select_bias"])
    ids_gpu = dbg["topk_ids"].cpu().numpy()
    res["id_mismatch_tokens"] = int(np.sum(np.any(ids_gpu != ids_ref, axis=1)))
    assert res["id_mismatch_tokens"] == 0, res
    w_gpu = dbg["topk_w"].cpu().double().numpy()
    res["w_err"] = float(np.max(np.abs(w_gpu - w_ref))) / max(cfg.routed_scale, 1.0)
    assert res["w_err"] <= 1e-6, res
    # how often the oracle's own fp64 logits would route differently (reported, not graded)
    ids_own, _, _ = oracle.route(l_ref, cfg.top_k, cfg.score, bool(cfg.renormalize),
                                 cfg.routed_scale,
                                 None if inp["select_bias"] is None
                                 else inp["select_bias"].cpu().numpy())
    res["own_route_diff_tokens"] = int(np.sum(np.any(ids_own != ids_ref[tok], axis=1)))
    # permutation bit-exact
    off, perm, inv = oracle.permute(ids_gpu, cfg.num_experts)
    assert np.array_equal(dbg["expert_offsets"].cpu().numpy(), off)
    assert np.array_equal(dbg["perm_token"].cpu().numpy(), perm)
    assert np.array_equal(dbg["inv_perm"].cpu().numpy(), inv)
    res["touched_experts"] = int(np.sum(np.diff(off) > 0))
    # block output on the sampled tokens
    ref = oracle_block(cfg, inp, tok, ids_ref[tok], w_ref[tok], max_experts)
    got = out[torch.as_tensor(tok, device=out.device)].float().cpu().double().numpy()
    res["out_err"] = rel_err(got, ref)
    res["tokens_checked"] = len(tok)
    print(f"[check] {cfg.name}: {res}", flush=True)
    assert res["out_err"] <= TOL[cfg.expert_dtype], res
    return res, out, dbg
