/*
 * moe.h -- C ABI of the MI355X (gfx950) mixture-of-experts FFN block.
 *
 * The block, as the archdiff.com architecture-comparison pages state it:
 *   x[T,d] -> router logits -> top-k expert ids and weights -> per-expert SwiGLU
 *   -> weighted sum of the routed experts plus the always-active shared expert(s).
 * Passages: "Qwen3.5-397B-A17B vs DeepSeek-V4-Pro", component table, router row
 * (softmax top-k renormalised; sqrt-softplus with a selection-only bias, scaled
 * by 2.5) and blueprint diagram, Mixture-of-experts group (a sigma or
 * sqrt-softplus router balanced by a bias; 6 to 22 of 256 to 896 SwiGLU
 * experts per token; one or two shared experts that every token uses; FP8
 * with block scales in the training box);
 * "Qwen3.5-397B-A17B vs Gemma 4 31B", component table, routed-experts row
 * (SwiGLU experts) and shared-expert row (shared output added to the routed sum).
 *
 * Conventions for every entry point:
 *  - Every pointer argument is a device pointer on the current HIP device
 *    unless stated otherwise; `cfg` and the weight-table structs themselves are
 *    host memory.  The caller owns all memory; the library never allocates,
 *    frees or synchronises, and keeps no state between calls.
 *  - Work is enqueued on `stream` (0 = the null stream).  Arguments are checked
 *    on the host before anything is enqueued: an error status means nothing
 *    was launched.  A kernel fault surfaces at the caller's next synchronisation.
 *  - Inputs are read-only.  Outputs are fully overwritten, never accumulated.
 *  - Layouts are row-major.  Logical weights: W_r [d,E]; per expert W_gate,
 *    W_up [d,f] and W_down [f,d]; stacked over experts.  Kernels read weights
 *    only in the packed layout written by moe_pack_weights.
 *  - A call with num_tokens == 0 is valid and launches nothing.
 *  - Supported type combinations (act / experts / router):
 *      F32 / F32 / F32, BF16 / BF16 / BF16, BF16 / FP8_E4M3 / F32 or BF16.
 *    d_model, d_ff and d_ff_shared must be multiples of 128 and at most 2^24
 *    (d_ff_shared only when num_shared > 0),
 *    num_experts <= 1024, top_k <= 64 and T*k < 2^30; otherwise
 *    MOE_ERR_UNSUPPORTED.  The kernels address each operand through a 32-bit
 *    buffer resource, so a config is also UNSUPPORTED (and moe_workspace_size
 *    returns 0) when any one operand reaches 4 GiB: x, the E4M3 activations or
 *    their scales, h = [T*k, d_ff] or the shared experts' h = [T, S*d_ff_shared]
 *    in the expert dtype (or their scales), the permutation, one routed
 *    expert's packed gate/up or down weights (or their scales), the shared
 *    experts' packed weights, or the packed router.
 *  - No function throws; all are safe to call from several host threads.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifndef MOE_API
#define MOE_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* a bad size, enum value or a NULL required pointer */
  MOE_ERR_UNSUPPORTED = 2,        /* valid, but outside what the kernels implement */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                 /* a HIP launch error */
} moe_status_t;

/* Number formats (moe_config_t.*_dtype).  MOE_MXFP4 is for expert weights only:
 * OCP MX E2M1 elements with one E8M0 (power-of-two) scale per 32 values along
 * the reduction axis (the blueprint's training box names MXFP4); the
 * activations x and h are then block-scaled E4M3 as with MOE_FP8_E4M3. */
enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2, MOE_MXFP4 = 3 };

/* Router score (moe_config_t.score). */
enum {
  MOE_SCORE_SOFTMAX = 0,       /* key = logit; weights = softmax (renormalised over the top k) */
  MOE_SCORE_SIGMOID = 1,       /* s = 1/(1+e^-l) */
  MOE_SCORE_SQRT_SOFTPLUS = 2  /* s = sqrt(log(1+e^l)) */
};

typedef struct {
  int32_t num_tokens;    /* T >= 0 */
  int32_t d_model;       /* d */
  int32_t num_experts;   /* E: routed experts */
  int32_t top_k;         /* k: 1 <= k <= E */
  int32_t d_ff;          /* f: routed-expert intermediate size */
  int32_t num_shared;    /* S >= 0 shared experts */
  int32_t d_ff_shared;   /* f_s: shared-expert intermediate size */
  int32_t score;         /* MOE_SCORE_* */
  int32_t renormalize;   /* 1: normalise the weights over the selected experts */
  float routed_scale;    /* gamma: routed weights are multiplied by it (2.5 / 1) */
  int32_t act_dtype;     /* storage of x (and of the output unless out_f32): MOE_F32 or
                            MOE_BF16 */
  int32_t expert_dtype;  /* expert weights (routed and shared); MOE_FP8_E4M3 and
                            MOE_MXFP4 also quantise x and h to block-scaled E4M3 */
  int32_t router_dtype;  /* storage of W_r: MOE_F32 or MOE_BF16 */
  int32_t quant_block;   /* FP8 block edge; must be 128 */
  int32_t shared_gate;   /* 1: the shared experts' output is multiplied per token by
                            sigmoid(x~ . w_sg), a learned gate, before it joins the routed
                            sum (shared-expert row, Qwen3.5 cell of "Qwen3.5-397B-A17B vs
                            Gemma 4 31B"); x~ is what the shared experts read (the
                            block-scaled x for FP8 experts).  0: ungated (the DeepSeek-style
                            shared expert). */
  int32_t out_f32;       /* 1: the block output is stored as fp32 whatever act_dtype, so the
                            combine's fp32 sum is not rounded again; 0: it is stored in
                            act_dtype (round to nearest even from that same fp32 sum). */
} moe_config_t;

/* Weights in the caller's logical layout, for moe_pack_weights (device pointers).
 * FP8 weights are E4M3FN codes with one fp32 scale per 128 x 128 block, the
 * scale grid laid out [rows/128, cols/128] per expert.  MXFP4 weights are
 * stored N-major, the MX blocks running along the reduction axis: gate and up
 * [E, f, d/2] bytes and down [E, d, f/2] (two E2M1 codes a byte, the lower K
 * index in the low nibble), each with E8M0 scale bytes [E, f, d/32] /
 * [E, d, f/32] (the shared experts likewise with S and f_s).  Scales are NULL
 * for fp32 / bf16 weights.  Shared pointers may be NULL when num_shared == 0. */
typedef struct {
  const void* w_router;          /* [d, E] router_dtype */
  const void* w_gate;            /* [E, d, f] */
  const void* w_up;              /* [E, d, f] */
  const void* w_down;            /* [E, f, d] */
  const void* w_gate_scales;     /* FP8 fp32 [E, d/128, f/128]; MXFP4 E8M0 [E, f, d/32] */
  const void* w_up_scales;       /* as w_gate_scales */
  const void* w_down_scales;     /* FP8 fp32 [E, f/128, d/128]; MXFP4 E8M0 [E, d, f/32] */
  const void* ws_gate;           /* [S, d, f_s] */
  const void* ws_up;             /* [S, d, f_s] */
  const void* ws_down;           /* [S, f_s, d] */
  const void* ws_gate_scales;    /* as w_gate_scales with S and f_s */
  const void* ws_up_scales;      /* as w_up_scales with S and f_s */
  const void* ws_down_scales;    /* as w_down_scales with S and f_s */
} moe_logical_weights_t;

/* Packed buffers, indexes for moe_packed_size / moe_pack_weights. */
enum {
  MOE_PACK_ROUTER = 0,
  MOE_PACK_GATE_UP = 1,
  MOE_PACK_GATE_UP_SCALES = 2,
  MOE_PACK_DOWN = 3,
  MOE_PACK_DOWN_SCALES = 4,
  MOE_PACK_SHARED_GATE_UP = 5,
  MOE_PACK_SHARED_GATE_UP_SCALES = 6,
  MOE_PACK_SHARED_DOWN = 7,
  MOE_PACK_SHARED_DOWN_SCALES = 8,
  MOE_PACK_COUNT = 9
};

/* The weights every compute call reads (device pointers).  The packed
 * pointers come from moe_pack_weights; logit_bias and select_bias are fp32
 * [E] or NULL.  logit_bias z is added to every logit before scoring;
 * select_bias b is added to the sigma / sqrt-softplus score only to choose
 * the experts (router row, DeepSeek-V4-Pro cell: one bias per expert that
 * takes part in the selection only) and never enters the weights. */
typedef struct {
  const void* w_router;
  const float* logit_bias;
  const float* select_bias;
  const void* w_gate_up;
  const void* w_gate_up_scales;  /* FP8: fp32; MXFP4: E8M0 bytes; NULL otherwise */
  const void* w_down;
  const void* w_down_scales;
  const void* ws_gate_up;
  const void* ws_gate_up_scales;
  const void* ws_down;
  const void* ws_down_scales;
  const void* ws_gate_vec;       /* [d] router_dtype gate vector w_sg; required when
                                    shared_gate = 1 and num_shared > 0, else ignored */
} moe_weights_t;

/* Stage boundaries of moe_forward, for moe_debug_t.stage_events. */
enum {
  MOE_STAGE_BEGIN = 0,           /* before the router */
  MOE_STAGE_ROUTED = 1,          /* after router GEMM + top-k (+ FP8 activation quantisation) */
  MOE_STAGE_PERMUTED = 2,        /* after the permutation */
  MOE_STAGE_TILED = 3,           /* after the device tile list of the routed GEMMs */
  MOE_STAGE_GATE_UP = 4,         /* after the routed gate/up GEMM with SiLU*up */
  MOE_STAGE_DOWN = 5,            /* after the routed down GEMM */
  MOE_STAGE_SHARED_GATE_UP = 6,  /* after the shared experts' gate/up GEMM */
  MOE_STAGE_COMBINE = 7,         /* after the shared down GEMM with the weighted combine */
  MOE_NUM_STAGE_EVENTS = 8
};

/* Optional device outputs of moe_forward.  A non-NULL member receives that
 * intermediate; NULL members live in the workspace.  stage_events, if non-NULL,
 * points to MOE_NUM_STAGE_EVENTS caller-created HIP events that are recorded on
 * `stream` at the stage boundaries above (per-kernel timing inside a run). */
typedef struct {
  float* logits;             /* [T, E] fp32 router logits (bias z included) */
  int32_t* topk_ids;         /* [T, k] */
  float* topk_w;             /* [T, k] */
  int32_t* expert_offsets;   /* [E + 1] */
  int32_t* perm_token;       /* [T*k] */
  int32_t* inv_perm;         /* [T*k] */
  void* y_perm;              /* [T*k, d], element type as for moe_expert_ffn */
  hipEvent_t* stage_events;  /* host array of MOE_NUM_STAGE_EVENTS events, or NULL */
} moe_debug_t;

/* Human-readable name of a status code (static string). */
MOE_API const char* moe_status_string(moe_status_t status);

/* Bytes of workspace any compute call of this config needs (0 on a bad cfg).
 * One buffer of this size serves every entry point; the split calls expect
 * the same buffer to be passed to each of them. */
MOE_API size_t moe_workspace_size(const moe_config_t* cfg);

/* Bytes of packed buffer `which` (MOE_PACK_*); 0 if the config does not use it. */
MOE_API size_t moe_packed_size(const moe_config_t* cfg, int which);

/* Rewrite logical weights into the kernels' packed layout (run once, outside
 * any timed region).  packed[i] must point to moe_packed_size(cfg, i) bytes for
 * every i with a nonzero size.  Pure data movement: router transposed to
 * [E, d] (an fp32 router with bf16 activations is split into bf16 hi + lo
 * parts), gate/up interleaved into one K-contiguous [2f, d] matrix per expert,
 * down transposed to [d, f]; shared experts concatenated into one of width
 * S*f_s.  Errors: INVALID_ARGUMENT for a NULL required pointer. */
MOE_API moe_status_t moe_pack_weights(const moe_config_t* cfg, const moe_logical_weights_t* logical,
                              void* const* packed, hipStream_t stream);

/* Router: l = x W_r + z, scores, top-k ids and weights (router row, Qwen3.5
 * cell: linear logits over 512 experts, softmax, the 10 largest kept and
 * renormalised; the sqrt-softplus / sigma variant of the DeepSeek-V4-Pro cell).
 * x [T,d] act_dtype.  logits [T,E] fp32 or NULL.  topk_ids/topk_w [T,k]: slot j
 * holds the j-th largest key (softmax: the logit; sigma / sqrt-softplus: the
 * score rounded to fp32 plus select_bias in fp32), equal keys ordered by the
 * lower expert index.  Weights: softmax renormalised over the selected (or the
 * full softmax probability when renormalize == 0); sigma / sqrt-softplus: the
 * selected scores over their sum (or the score when renormalize == 0); times
 * routed_scale.  FP8 experts: xq [T,d] E4M3 codes and xq_scales [T,d/128]
 * (block-scaled activations, one fp32 scale = group max / 448 per 128 values)
 * are written when both are non-NULL.  ws / ws_bytes: the workspace (the
 * padded fp32 logits live there); WORKSPACE_TOO_SMALL if it is short. */
MOE_API moe_status_t moe_route(const moe_config_t* cfg, const void* x, const moe_weights_t* weights,
                       float* logits, int32_t* topk_ids, float* topk_w, void* xq,
                       float* xq_scales, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_route for the layers whose experts a hash of the token id fixes
 * (router row, DeepSeek-V4-Pro cell: the first three MoE layers).  The hash is
 * a caller-owned table [vocab, k] of expert ids: topk_ids[t] =
 * hash_table[token_ids[t]] in the table's slot order, and topk_w[t] are the
 * router's weights for those experts, computed from this call's logits as in
 * moe_route (softmax renormalised over the table's experts, or the full softmax
 * probability; sigma / sqrt-softplus: the experts' unbiased scores over their
 * sum, or the scores; times routed_scale).  select_bias plays no part.
 * token_ids [T] and hash_table are device int32; each token id must lie in
 * [0, vocab) and each table row hold k distinct ids in [0, E): values outside
 * those ranges are clamped into them (no out-of-bounds access, result
 * unspecified).  Everything else (logits, xq, xq_scales, ws) as in moe_route.
 * The ids then feed moe_permute, moe_expert_ffn and moe_combine unchanged. */
MOE_API moe_status_t moe_route_hashed(const moe_config_t* cfg, const void* x,
                                      const moe_weights_t* weights, const int32_t* token_ids,
                                      const int32_t* hash_table, int32_t vocab, float* logits,
                                      int32_t* topk_ids, float* topk_w, void* xq,
                                      float* xq_scales, void* ws, size_t ws_bytes,
                                      hipStream_t stream);

/* One auxiliary-loss-free balancing step of the selection bias (router row,
 * DeepSeek-V4-Pro cell: bias balancing with speed 0.001; the update is the
 * published sign rule of that method).  With load_e = expert_offsets[e+1] -
 * expert_offsets[e] (moe_permute's output for the batch) and A =
 * expert_offsets[E] = T*k:
 *   select_bias[e] += speed * sign(A - E * load_e)
 * i.e. an expert above the mean load T*k/E moves down by speed, one below it
 * moves up, one exactly at it keeps its bias bit for bit.  The comparison is
 * exact in integers and the step is one fp32 add.  select_bias [E] fp32, updated in
 * place on `stream`.  speed must be finite and >= 0 (0.001 on the pages). */
MOE_API moe_status_t moe_update_bias(const moe_config_t* cfg, const int32_t* expert_offsets,
                                     float speed, float* select_bias, hipStream_t stream);

/* The scoring and top-k step of moe_route on caller-supplied fp32 logits
 * [T,E] (bias z already included); same keys, order and weights. */
MOE_API moe_status_t moe_route_from_logits(const moe_config_t* cfg, const float* logits,
                                   const float* select_bias, int32_t* topk_ids, float* topk_w,
                                   hipStream_t stream);

/* Permutation of the T*k (token, slot) assignments into expert-contiguous
 * order (router row of "Qwen3.5-397B-A17B vs DeepSeek-V4-Pro": each token
 * picks its top k of the routed experts, so each expert's SwiGLU, routed-
 * experts row of "Qwen3.5-397B-A17B vs Gemma 4 31B", runs over the rows that
 * picked it), stable in token order: expert_offsets [E+1] (exclusive prefix sum of
 * the per-expert counts, last = T*k), perm_token [T*k] (token of each row),
 * inv_perm [T*k] (row of assignment t*k + j).  Ids may come from any source
 * (router replay, hash routing); ids outside [0, E) are a precondition
 * violation.  Deterministic: no atomics decide the order. */
MOE_API moe_status_t moe_permute(const moe_config_t* cfg, const int32_t* topk_ids,
                         int32_t* expert_offsets, int32_t* perm_token, int32_t* inv_perm,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* Routed SwiGLU experts (routed-experts row, Qwen3.5 cell):
 * for every row r of expert e, h = SiLU(x~ W_gate[e]) * (x~ W_up[e]) and
 * y_perm[r] = h W_down[e], with x~ = x[perm_token[r]] (FP8: the block-scaled
 * xq / xq_scales from moe_route, and h re-quantised per 128 values).
 * y_perm [T*k, d]: fp32 for MOE_F32 experts; IEEE fp16 for MOE_BF16 experts
 * (round to nearest even: 8x finer than bf16 at half the bytes of fp32; an
 * expert output value of magnitude 65520 or more overflows, and the block
 * output of that token then holds a non-finite value in that column, never a
 * wrong finite one); bf16 for MOE_FP8_E4M3 and MOE_MXFP4 experts. */
MOE_API moe_status_t moe_expert_ffn(const moe_config_t* cfg, const void* x_or_xq, const float* xq_scales,
                            const int32_t* expert_offsets, const int32_t* perm_token,
                            const moe_weights_t* weights, void* y_perm, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* Shared experts and weighted combine (shared-expert row: the shared experts
 * see every token and their output joins the routed sum; blueprint: always
 * active):
 * out[t] = G[t] * sum_s SwiGLU_s(x~[t]) + sum_j topk_w[t,j] * y_perm[inv_perm[t*k+j]],
 * G[t] = sigmoid(x~[t] . ws_gate_vec) when cfg->shared_gate (else 1).
 * out [T,d]: fp32 when cfg->out_f32, else act_dtype.  The residual add outside the
 * block is not included. */
MOE_API moe_status_t moe_combine(const moe_config_t* cfg, const void* x_or_xq, const float* xq_scales,
                         const void* y_perm, const int32_t* inv_perm, const float* topk_w,
                         const moe_weights_t* weights, void* out, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/* The whole block: moe_route -> moe_permute -> moe_expert_ffn -> moe_combine on
 * one stream with no host synchronisation.  out as for moe_combine (fp32 when
 * cfg->out_f32, else act_dtype).  dbg may be NULL (host struct). */
MOE_API moe_status_t moe_forward(const moe_config_t* cfg, const void* x, const moe_weights_t* weights,
                         void* out, const moe_debug_t* dbg, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/* Bytes of the library's own device workspace used by moe_forward_noalloc (per GPU). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* moe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight decode-serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and results as moe_forward, without ws / ws_bytes:
 * the workspace is a static array of MOE_NOALLOC_SCRATCH_BYTES (64 MiB) that
 * the library's code object places on each GPU it runs on, held until the
 * process ends.  Nothing is allocated or freed.  Configs whose
 * moe_workspace_size exceeds that limit return MOE_ERR_WORKSPACE_TOO_SMALL
 * before anything is launched (decode shapes fit: e.g. 64 tokens at d 4096, 256
 * experts, top 8, d_ff 1536 need 11 MB).  All calls on one GPU share its array:
 * calls that may run concurrently on one GPU (other host threads, other
 * streams) race and must be serialised by the caller.  Nothing in the array has
 * to start at zero; each call fully writes what it reads.  The first call on a
 * device looks the array's address up (hipGetSymbolAddress) with that device
 * current; MOE_ERR_HIP if that fails. */
MOE_API moe_status_t moe_forward_noalloc(const moe_config_t* cfg, const void* x,
                                         const moe_weights_t* weights, void* out,
                                         const moe_debug_t* dbg, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
