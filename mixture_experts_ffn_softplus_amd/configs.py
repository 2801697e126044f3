"""Named workloads of the mixture-of-experts FFN block (shapes and routing recipe only).

Sources for the shapes (archdiff.com comparison pages):

* ``softmax_bf16`` -- Qwen3.5's layer: "Qwen3.5-397B-A17B vs Gemma 4 31B",
  component table, routed-experts row (512 SwiGLU experts, intermediate
  1,024, width 4,096, 10 active) and shared-expert row (one shared expert,
  intermediate 1,024); router row of "Qwen3.5-397B-A17B vs DeepSeek-V4-Pro"
  (softmax, top 10, renormalise).
* ``softplus_bf16`` -- DeepSeek-V4-Pro's router: same router row, V4-Pro cell
  (sqrt-softplus over 384 experts, selection-only bias, top 6, x2.5); width
  7,168 from that page's residual-stream row.  Expert and shared widths, the
  shared count of 2 and the Zipf load skew are workload choices.
* ``decode_bf16`` -- 256 experts, the low end of the blueprint's routed-experts
  box (6 to 22 of 256 to 896 experts); 64 tokens, so the step streams expert weights.
* ``fp8_block`` -- 896 experts, top 22, the high end of that box; the
  blueprint's training box (FP8 with block scales) for the number format.
* ``tiny_fp32`` -- a small fp32 layer that the oracle finishes in well under a
  second, used for parity at every step.
* ``mxfp4_decode`` / ``mxfp4_block`` -- ``decode_bf16`` / ``fp8_block`` with the
  experts' weights in MXFP4 (E2M1 with an E8M0 scale per 32 values along K), the
  other format the blueprint's training box names; activations stay block-scaled
  E4M3.
* ``qwen_gated_bf16`` -- ``softmax_bf16`` with the Qwen3.5 shared expert as the
  shared-expert row of "Qwen3.5-397B-A17B vs Gemma 4 31B" states it: its output
  scaled by a per-token sigmoid gate of a learned d-vector before the routed sum
  is added.

The bf16-expert workloads store the block output as fp32 (``out_f32``): their
arithmetic is bf16 (x, the weights and h, fp32 accumulation), and a bf16 output
would add one more rounding of up to 2^-8 |out|, which alone approaches a 2e-2
max-abs/RMS bound wherever |out| reaches five times its RMS.  The E4M3 and
MXFP4 workloads keep the bf16 output.
"""
from dataclasses import dataclass, replace

F32, BF16, FP8_E4M3, MXFP4 = 0, 1, 2, 3
SOFTMAX, SIGMOID, SQRT_SOFTPLUS = 0, 1, 2

_DT_NAMES = {F32: "f32", BF16: "bf16", FP8_E4M3: "fp8_e4m3", MXFP4: "mxfp4"}


@dataclass(frozen=True)
class MoEConfig:
    name: str
    num_tokens: int
    d_model: int
    num_experts: int
    top_k: int
    d_ff: int
    num_shared: int
    d_ff_shared: int
    score: int = SOFTMAX
    renormalize: int = 1
    routed_scale: float = 1.0
    act_dtype: int = BF16      # storage of x (and of the block output unless out_f32)
    expert_dtype: int = BF16   # expert weights (FP8 / MXFP4: x and h quantised to E4M3)
    router_dtype: int = BF16   # storage of W_r
    quant_block: int = 128
    seed: int = 0
    select_bias_range: float = 0.0   # b_e ~ U(-r, r) when r > 0 (selection-only bias)
    zipf_s: float = 0.0              # per-expert logit bias skewing load when > 0
    shared_gate: int = 0             # 1: sigmoid(x . w_sg) scales the shared output (Qwen3.5)
    out_f32: int = 0                 # 1: the block output is stored as fp32 (else act_dtype)

    @property
    def assignments(self) -> int:
        return self.num_tokens * self.top_k

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)

    def describe(self) -> str:
        sc = {SOFTMAX: "softmax", SIGMOID: "sigmoid", SQRT_SOFTPLUS: "sqrt_softplus"}[self.score]
        return (f"{self.name}: T={self.num_tokens} d={self.d_model} E={self.num_experts} "
                f"top-{self.top_k} d_ff={self.d_ff} shared={self.num_shared}x{self.d_ff_shared} "
                f"{sc} experts={_DT_NAMES[self.expert_dtype]}"
                + (" gated-shared" if self.shared_gate else "")
                + (" fp32-out" if self.out_f32 and self.act_dtype != F32 else ""))


PRESETS = {
    "tiny_fp32": MoEConfig(
        name="tiny_fp32", num_tokens=64, d_model=256, num_experts=16, top_k=2, d_ff=128,
        num_shared=1, d_ff_shared=256, score=SOFTMAX, renormalize=1, routed_scale=1.0,
        act_dtype=F32, expert_dtype=F32, router_dtype=F32, seed=0),
    "softmax_bf16": MoEConfig(
        name="softmax_bf16", num_tokens=4096, d_model=4096, num_experts=512, top_k=10,
        d_ff=1024, num_shared=1, d_ff_shared=1024, score=SOFTMAX, renormalize=1,
        routed_scale=1.0, seed=1, out_f32=1),
    "softplus_bf16": MoEConfig(
        name="softplus_bf16", num_tokens=4096, d_model=7168, num_experts=384, top_k=6,
        d_ff=2048, num_shared=2, d_ff_shared=2048, score=SQRT_SOFTPLUS, renormalize=1,
        routed_scale=2.5, seed=2, select_bias_range=0.1, zipf_s=1.1, out_f32=1),
    "decode_bf16": MoEConfig(
        name="decode_bf16", num_tokens=64, d_model=4096, num_experts=256, top_k=8, d_ff=1536,
        num_shared=1, d_ff_shared=1536, score=SOFTMAX, renormalize=1, routed_scale=1.0, seed=3,
        out_f32=1),
    "fp8_block": MoEConfig(
        name="fp8_block", num_tokens=16384, d_model=4096, num_experts=896, top_k=22, d_ff=512,
        num_shared=1, d_ff_shared=2048, score=SOFTMAX, renormalize=1, routed_scale=1.0,
        act_dtype=BF16, expert_dtype=FP8_E4M3, router_dtype=F32, seed=4),
}
PRESETS["qwen_gated_bf16"] = PRESETS["softmax_bf16"].with_(name="qwen_gated_bf16", shared_gate=1)
PRESETS["mxfp4_decode"] = PRESETS["decode_bf16"].with_(name="mxfp4_decode", expert_dtype=MXFP4,
                                                         out_f32=0)
PRESETS["mxfp4_block"] = PRESETS["fp8_block"].with_(name="mxfp4_block", expert_dtype=MXFP4)

