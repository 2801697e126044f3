"""Seeded synthetic inputs of the mixture-of-experts FFN block.

This module only draws and stores input tensors; it holds none of the block's
arithmetic, and both the GPU path's tests and the oracle consume what it
produces.  Every tensor comes from its own torch generator, seeded from
(workload seed, tensor tag, expert index), so any one expert's weights can be
regenerated alone -- the oracle's token sample needs only the experts those
tokens use, and a 34 GB weight set never has to exist on the host.

Recipe (all logical layouts row-major):

* x [T, d] ~ N(0, 1), stored fp32 or bf16 (round to nearest even).
* W_r [d, E] ~ N(0, 1/d) (standard deviation 1/sqrt(fan_in), fan_in = d).
* W_gate, W_up [E, d, f] ~ N(0, 1/d); W_down [E, f, d] ~ N(0, 1/f); the shared
  experts likewise with f_s, stacked [S, ...].
* FP8 weights: each 128 x 128 block of the fp32 draw gets scale amax/448 (1 if
  the block is zero) and codes = the draw over the scale, cast to E4M3FN by
  torch.  The quantised weights are the inputs; how they were made is not part
  of the block.
* MXFP4 weights: the fp32 draw stored N-major; each 32 consecutive values
  along K get the E8M0 scale 2^(floor(log2 amax) - 2) (2 = the largest E2M1
  exponent; amax = 0 gives 2^-127), and each value over its scale is rounded
  to the nearest E2M1 value (ties to the smaller magnitude, saturating at 6).
* Selection-only bias b_e ~ U(-r, r) (fp32) when the workload asks for one.
* Shared-expert gate vector w_sg [d] ~ N(0, 1/d), stored in the router's dtype,
  when the workload gates its shared experts.
* Load skew: logit bias z_e = ln p_e - mean(ln p), p_e proportional to
  (e + 1)^-s, expert 0 hottest (fp32).
* Hash routing (experts fixed by the token id): a table [vocab, k] of k distinct expert ids
  per token id (the first k of a seeded random permutation of the experts for
  each row), vocab 131072 (the low end of the pages' 128K-262K tokenizers), and
  token ids drawn with Zipf frequencies p(rank r) proportional to 1/r, as word
  frequencies in text fall off, the id of rank r being a seeded random id.

Generators on a CUDA device and on the CPU produce different streams for the
same seed; a test always hands the very same tensors to both sides.
"""
import math

import torch

from .configs import BF16, F32, FP8_E4M3, MXFP4, MoEConfig

TAG_X, TAG_ROUTER, TAG_SELECT_BIAS = 1, 2, 3
TAG_GATE, TAG_UP, TAG_DOWN = 4, 5, 6
TAG_SGATE, TAG_SUP, TAG_SDOWN = 7, 8, 9
TAG_SHARED_GATE_VEC = 10
TAG_HASH_TABLE, TAG_TOKEN_IDS = 11, 12

_MASK64 = (1 << 64) - 1


def _mix(*vals) -> int:
    """A 63-bit seed from a tuple of small integers (splitmix64 finaliser chain)."""
    h = 0x9E3779B97F4A7C15
    for v in vals:
        h = (h ^ (int(v) & _MASK64)) & _MASK64
        h = (h * 0xBF58476D1CE4E5B9) & _MASK64
        h ^= h >> 31
        h = (h * 0x94D049BB133111EB) & _MASK64
        h ^= h >> 29
    return h & ((1 << 63) - 1)


def _gen(device, *vals) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_mix(*vals))
    return g


def _normal(shape, std, device, *seed_vals) -> torch.Tensor:
    g = _gen(device, *seed_vals)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def _store(t: torch.Tensor, dtype: int) -> torch.Tensor:
    if dtype == F32:
        return t.contiguous()
    if dtype == BF16:
        return t.to(torch.bfloat16).contiguous()
    raise ValueError("use _store_fp8 for FP8 weights")


def _store_fp8(t: torch.Tensor, block: int):
    """fp32 [..., R, C] -> (E4M3FN codes [..., R, C], fp32 scales [..., R/block, C/block])."""
    *lead, R, C = t.shape
    assert R % block == 0 and C % block == 0
    b = t.reshape(*lead, R // block, block, C // block, block)
    amax = b.abs().amax(dim=(-3, -1))                       # [..., R/b, C/b]
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
    q = (b / scale[..., :, None, :, None]).to(torch.float8_e4m3fn)
    return q.reshape(*lead, R, C).contiguous(), scale.contiguous()


_E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _store_mxfp4(t: torch.Tensor):
    """fp32 [K, N] -> (codes uint8 [N, K/2], two E2M1 codes a byte with the lower K index in
    the low nibble; E8M0 scales uint8 [N, K/32])."""
    w = t.t().contiguous()                                   # [N, K]
    N, K = w.shape
    b = w.reshape(N, K // 32, 32)
    amax = b.abs().amax(-1)
    e = torch.where(amax > 0, torch.floor(torch.log2(amax.clamp_min(1e-38))) - 2,
                    torch.full_like(amax, -127.0)).clamp(-127, 127)
    v = b / torch.exp2(e)[..., None]
    grid = torch.tensor(_E2M1, device=t.device)
    mag = (v.abs()[..., None] - grid).abs().argmin(-1)       # nearest, lower index on ties
    codes = (mag | torch.where(v < 0, 8, 0)).to(torch.uint8).reshape(N, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).contiguous()
    return packed, (e + 127).to(torch.uint8).contiguous()


def tokens(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    x = _normal((cfg.num_tokens, cfg.d_model), 1.0, device, cfg.seed, TAG_X)
    return _store(x, F32 if cfg.act_dtype == F32 else BF16)


def router(cfg: MoEConfig, device="cpu"):
    """(W_r [d,E], logit bias z [E] or None, selection bias b [E] or None)."""
    d, E = cfg.d_model, cfg.num_experts
    wr = _store(_normal((d, E), 1.0 / math.sqrt(d), device, cfg.seed, TAG_ROUTER),
                cfg.router_dtype)
    z = None
    if cfg.zipf_s > 0:
        lnp = [-cfg.zipf_s * math.log(e + 1) for e in range(E)]
        mean = sum(lnp) / E
        z = torch.tensor([v - mean for v in lnp], dtype=torch.float64).to(torch.float32)
        z = z.to(device)
    b = None
    if cfg.select_bias_range > 0:
        g = _gen(device, cfg.seed, TAG_SELECT_BIAS)
        r = cfg.select_bias_range
        b = (torch.rand((E,), generator=g, device=device, dtype=torch.float32) * (2 * r) - r)
    return wr, z, b


def _expert(cfg: MoEConfig, shared: bool, e: int, device):
    d = cfg.d_model
    f = cfg.d_ff_shared if shared else cfg.d_ff
    tg, tu, td = (TAG_SGATE, TAG_SUP, TAG_SDOWN) if shared else (TAG_GATE, TAG_UP, TAG_DOWN)
    g = _normal((d, f), 1.0 / math.sqrt(d), device, cfg.seed, tg, e)
    u = _normal((d, f), 1.0 / math.sqrt(d), device, cfg.seed, tu, e)
    dn = _normal((f, d), 1.0 / math.sqrt(f), device, cfg.seed, td, e)
    if cfg.expert_dtype == MXFP4:
        (gq, gs), (uq, us), (dq, ds) = (_store_mxfp4(t) for t in (g, u, dn))
        return {"gate": gq, "up": uq, "down": dq, "gate_scales": gs, "up_scales": us,
                "down_scales": ds}
    if cfg.expert_dtype == FP8_E4M3:
        (gq, gs), (uq, us), (dq, ds) = (_store_fp8(t, cfg.quant_block) for t in (g, u, dn))
        return {"gate": gq, "up": uq, "down": dq, "gate_scales": gs, "up_scales": us,
                "down_scales": ds}
    return {"gate": _store(g, cfg.expert_dtype), "up": _store(u, cfg.expert_dtype),
            "down": _store(dn, cfg.expert_dtype)}


def routed_expert(cfg: MoEConfig, e: int, device="cpu"):
    """Weights of routed expert e: gate/up [d,f], down [f,d] (+ FP8 block scales); MXFP4:
    gate/up [f, d/2] and down [d, f/2] codes with E8M0 scales [f, d/32] / [d, f/32]."""
    return _expert(cfg, False, e, device)


def shared_expert(cfg: MoEConfig, s: int, device="cpu"):
    return _expert(cfg, True, s, device)


def _stack(cfg, shared: bool, n: int, device):
    parts = [_expert(cfg, shared, e, device) for e in range(n)]
    if n == 0:
        return None
    return {key: torch.stack([p[key] for p in parts]) for key in parts[0]}


def routed_experts(cfg: MoEConfig, device="cpu"):
    """All routed experts stacked: gate/up [E,d,f], down [E,f,d] (+ scales)."""
    out = {}
    keys = None
    for e in range(cfg.num_experts):
        p = _expert(cfg, False, e, device)
        if keys is None:
            keys = list(p)
            for key in keys:
                out[key] = torch.empty((cfg.num_experts,) + tuple(p[key].shape),
                                       dtype=p[key].dtype, device=device)
        for key in keys:
            out[key][e].copy_(p[key])
        del p
    return out


def shared_experts(cfg: MoEConfig, device="cpu"):
    """All shared experts stacked: gate/up [S,d,f_s], down [S,f_s,d] (+ scales), or None."""
    return _stack(cfg, True, cfg.num_shared, device)


def shared_gate_vector(cfg: MoEConfig, device="cpu"):
    """w_sg [d] in the router's dtype, or None when the shared experts are ungated."""
    if not cfg.shared_gate or cfg.num_shared == 0:
        return None
    d = cfg.d_model
    return _store(_normal((d,), 1.0 / math.sqrt(d), device, cfg.seed, TAG_SHARED_GATE_VEC),
                  cfg.router_dtype)


def inputs(cfg: MoEConfig, device="cpu"):
    """Every input of the block, logical layouts."""
    wr, z, b = router(cfg, device)
    return {"x": tokens(cfg, device), "w_router": wr, "logit_bias": z, "select_bias": b,
            "routed": routed_experts(cfg, device), "shared": shared_experts(cfg, device),
            "shared_gate": shared_gate_vector(cfg, device)}


HASH_VOCAB = 131072


def hash_routing(cfg: MoEConfig, device="cpu", vocab: int = HASH_VOCAB, zipf_s: float = 1.0):
    """(token_ids int32 [T], table int32 [vocab, k]) for hash routing (experts fixed by the token id)."""
    g = _gen(device, cfg.seed, TAG_HASH_TABLE)
    keys = torch.rand((vocab, cfg.num_experts), generator=g, device=device)
    table = keys.argsort(dim=1)[:, :cfg.top_k].to(torch.int32).contiguous()
    del keys
    g = _gen(device, cfg.seed, TAG_TOKEN_IDS)
    p = torch.arange(1, vocab + 1, dtype=torch.float64, device=device) ** -zipf_s
    rank = torch.multinomial(p / p.sum(), cfg.num_tokens, replacement=True, generator=g)
    ids_of_rank = torch.randperm(vocab, generator=g, device=device)
    token_ids = ids_of_rank[rank].to(torch.int32).contiguous()
    return token_ids, table
