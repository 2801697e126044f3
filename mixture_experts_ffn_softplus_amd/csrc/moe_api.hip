// moe_api.hip -- the C ABI of include/moe.h: argument checks, workspace layout, packing and
// the launch sequence of the block (route -> permute -> expert FFN -> combine) on one stream.
#include <math.h>
#include <string.h>

#include <mutex>

#include "moe_common.h"
#include "moe_internal.h"

// Workspace of moe_forward_noalloc, for callers that cannot allocate: a file-scope device array
// that each GPU the library runs on holds until the process ends.  In host code `scratch` only
// names the symbol; its device address on the current device comes from hipGetSymbolAddress
// (static_scratch), and only that address is ever handed to kernels.  Every call on one GPU
// shares that GPU's copy: calls that overlap on one GPU race.  No kernel of the block relies on
// the workspace's previous contents (each buffer in it is fully written before it is read), so
// nothing has to be cleared between calls.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace moe {
namespace {

constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void* g_scratch_ptr[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];

// Device address of `scratch` on the current device, looked up once per device (on the first
// call that runs there, with that device current).
hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = g_scratch_ptr[dev];
  return g_scratch_err[dev] != hipSuccess ? g_scratch_err[dev]
         : *ptr == nullptr                ? hipErrorInvalidSymbol
                                          : hipSuccess;
}


constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// E4M3 activations (x and h block-scaled per 128 values): FP8 and MXFP4 experts
bool is_fp8(const moe_config_t* c) {
  return c->expert_dtype == MOE_FP8_E4M3 || c->expert_dtype == MOE_MXFP4;
}
bool is_mx(const moe_config_t* c) { return c->expert_dtype == MOE_MXFP4; }

// Bytes of one h element (the expert activations), of x / out, and of y_perm.
int h_bytes(const moe_config_t* c) {
  return c->expert_dtype == MOE_F32 ? 4 : c->expert_dtype == MOE_BF16 ? 2 : 1;
}
// Bytes of one packed weight row of K elements (E2M1: two a byte).
int64_t wrow(const moe_config_t* c, int64_t K) { return is_mx(c) ? K / 2 : K * h_bytes(c); }
int act_bytes(const moe_config_t* c) { return c->act_dtype == MOE_F32 ? 4 : 2; }
// bytes per element of the block output
int out_bytes(const moe_config_t* c) { return c->out_f32 ? 4 : act_bytes(c); }
// y_perm (RowKind): fp32 for fp32 experts, fp16 for bf16 experts, bf16 for E4M3 activations.
// bf16 experts: a bf16 y_perm would add a third bf16 rounding (after h and the output) to a
// budget the output rounding alone half fills (measured on 62 seeded random bf16 layers: worst
// max-abs/RMS 0.0153 with fp32 rows, 0.0249 with bf16 rows); fp16 rows round 8x finer and halve
// the fp32 rows' HBM traffic.  fp16 overflows where one expert's output reaches 65520 in
// magnitude: the token's block output is then non-finite in that column (inf, or NaN where the
// combine's zero-weight padding rows meet it), never a wrong finite value.
int y_kind(const moe_config_t* c) {
  return is_fp8(c) ? kRowBF16 : c->expert_dtype == MOE_F32 ? kRowF32 : kRowF16;
}
int row_bytes(int kind) { return kind == kRowF32 ? 4 : 2; }
int y_bytes(const moe_config_t* c) { return row_bytes(y_kind(c)); }
// The shared experts' output [T, d], which the combine adds once per token: fp32, or bf16 for
// E4M3 activations, whose block output is bf16 (at fp8_block, 2 T d B = 268 MB less written and
// read than an fp32 copy).
int so_kind(const moe_config_t* c) { return is_fp8(c) ? kRowBF16 : kRowF32; }
int so_bytes(const moe_config_t* c) { return row_bytes(so_kind(c)); }

// Router columns padded to the GEMM's N tiles: 128 for small E, else 256 (the wide 8-wave tile).
int e_pad(const moe_config_t* c) {
  return c->num_experts <= 128 ? 128 : (c->num_experts + 255) / 256 * 256;
}
int64_t assignments(const moe_config_t* c) {
  return static_cast<int64_t>(c->num_tokens) * c->top_k;
}
int64_t shared_width(const moe_config_t* c) {
  return static_cast<int64_t>(c->num_shared) * c->d_ff_shared;
}

int router_kind(const moe_config_t* c) {
  if (c->router_dtype == MOE_F32 && c->act_dtype == MOE_F32) return kRouterF32;
  if (c->router_dtype == MOE_BF16) return kRouterBF16;
  return kRouterBF16HiLo;
}

// Row tile of the router GEMM: the wide 128 x 256 tile when it still gives every CU one, else
// the largest 128-column tile that does.
int router_bm(const moe_config_t* c) {
  const int64_t T = c->num_tokens;
  if (e_pad(c) % 256 == 0 && (T + 127) / 128 * (e_pad(c) / 256) >= 256) return 128;
  const int64_t nt = e_pad(c) / 128;
  for (int bm : {64, 32})
    if ((T + bm - 1) / bm * nt >= 256) return bm;
  return 16;
}

// K split of the router GEMM.  When its tiles fill the GPU at most once (up to two workgroups
// a CU), each tile walks K alone, one latency-bound step after another; split into up to 8
// ranges of at least 8 K-steps, the ranges run side by side, each into its own fp32 plane of
// partial logits, which the top-k waves add in a fixed order (so the logits stay run-to-run
// identical).  Measured on MI355X: decode_bf16 route 0.032 -> 0.022 ms, softmax_bf16 and
// softplus_bf16 -3 to -4 us.
int router_splits(const moe_config_t* c) {
  const int kind = router_kind(c);
  const int64_t T = c->num_tokens, Ep = e_pad(c);
  const int bm = kind == kRouterF32 ? 32 : router_bm(c);  // the fp32 GEMM's tile is 32 x 128
  const int bn = kind != kRouterF32 && bm == 128 && Ep % 256 == 0 ? 256 : 128;
  const int64_t tiles = (T + bm - 1) / bm * (Ep / bn);
  const int64_t K = kind == kRouterBF16HiLo ? 2 * c->d_model : c->d_model;
  const int64_t steps = K * (kind == kRouterF32 ? 4 : 2) / kBlockK;
  int s = 1;
  while (s < 8 && tiles * 2 * s <= 512 && steps % (2 * s) == 0 && steps / (2 * s) >= 8) s *= 2;
  return s;
}

int routed_bm(const moe_config_t* c) {
  int64_t avg = c->num_experts > 0 ? assignments(c) / c->num_experts : 0;
  return gemm_bm(c->expert_dtype, kEpiSwiglu, static_cast<int>(avg < 1 << 20 ? avg : 1 << 20));
}
// The shared experts see every token: their rows per tile follow T.
int shared_bm(const moe_config_t* c) {
  if (c->expert_dtype == MOE_F32) return gemm_bm(MOE_F32, kEpiSwiglu, 0);
  return gemm_bm(c->expert_dtype, kEpiSwiglu, c->num_tokens);
}
// The shared experts run as one extra group of the routed grouped GEMMs for decode-sized
// batches (T <= 256, routed tiles of at most 32 rows, bf16 or E4M3 activations) when together
// they are exactly as wide as a routed expert (S * f_s = f): their few rows then stream their
// weights beside the routed experts' instead of in two launches of their own.  (Measured on
// MI355X: decode_bf16 1.477 -> 1.423 ms, mxfp4_decode 0.538 -> 0.500 ms; at T = 4096 the shared
// tiles are MFMA-bound and lengthened the routed gate/up by as much as their own launches took,
// so larger batches keep them separate.)
bool merge_shared(const moe_config_t* c) {
  return c->num_shared > 0 && shared_width(c) == c->d_ff && c->num_tokens <= 256 &&
         c->expert_dtype != MOE_F32 && routed_bm(c) <= 32;
}
int64_t routed_max_tiles(const moe_config_t* c) {
  int bm = routed_bm(c);
  return (assignments(c) + bm - 1) / bm + c->num_experts +
         (merge_shared(c) ? (c->num_tokens + bm - 1) / bm : 0);
}

// The GEMMs read every operand through a buffer resource whose size and per-lane offsets are
// 32-bit: one operand (x, the FP8 activations and their scales, h and h_s and their scales, the
// permutation, one group's packed weights or weight scales) must stay below 4 GiB, or loads
// past the wrap would read zeros.  Outputs are addressed per tile from a 64-bit base.  Sizes
// are taken in 64-bit arithmetic after check_config has bounded each factor.
bool addressable(const moe_config_t* c) {
  const int64_t lim = 1LL << 32;
  const int64_t T = c->num_tokens, d = c->d_model, f = c->d_ff, A = assignments(c);
  const int64_t F = shared_width(c), hb = h_bytes(c);
  const bool q = is_fp8(c);
  // bytes of one group's weight scales: FP8 fp32 per 16 packed rows and 128 K; MXFP4 a byte
  // per row and 32 K
  auto scales = [&](int64_t N, int64_t K) -> int64_t {
    return !q ? 0 : is_mx(c) ? N * (K / 32) : (N / 16) * (K / 128) * 4;
  };
  const int64_t rk = router_kind(c);
  const int64_t router = e_pad(c) * (rk == kRouterBF16HiLo ? 2 * d : d) * (rk == kRouterF32 ? 4 : 2);
  const int64_t sizes[] = {
      T * d * act_bytes(c),                   // x (router; bf16 / fp32 experts)
      q ? T * d : 0, q ? T * (d / 128) * 4 : 0,  // E4M3 x and its scales
      A * f * hb, q ? A * (f / 128) * 4 : 0,  // h and its scales
      T * F * hb, q ? T * (F / 128) * 4 : 0,  // h_s and its scales
      A * 4,                                  // perm_token
      2 * f * wrow(c, d), d * wrow(c, f),     // one routed expert's gate/up and down
      2 * F * wrow(c, d), d * wrow(c, F),     // the shared experts' gate/up and down
      scales(2 * f, d), scales(d, f), scales(2 * F, d), scales(d, F),
      router};
  for (int64_t v : sizes)
    if (v >= lim) return false;
  return true;
}

moe_status_t check_config(const moe_config_t* c) {
  if (!c) return MOE_ERR_INVALID_ARGUMENT;
  if (c->num_tokens < 0 || c->d_model <= 0 || c->num_experts <= 0 || c->top_k < 1 ||
      c->top_k > c->num_experts || c->d_ff <= 0 || c->num_shared < 0 ||
      (c->num_shared > 0 && c->d_ff_shared <= 0))
    return MOE_ERR_INVALID_ARGUMENT;
  if (c->score < MOE_SCORE_SOFTMAX || c->score > MOE_SCORE_SQRT_SOFTPLUS)
    return MOE_ERR_INVALID_ARGUMENT;
  if (c->renormalize != 0 && c->renormalize != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (c->shared_gate != 0 && c->shared_gate != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (c->out_f32 != 0 && c->out_f32 != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (!isfinite(c->routed_scale)) return MOE_ERR_INVALID_ARGUMENT;
  const int dts[3] = {c->act_dtype, c->expert_dtype, c->router_dtype};
  for (int v : dts)
    if (v < MOE_F32 || v > MOE_MXFP4) return MOE_ERR_INVALID_ARGUMENT;
  const bool ok_types =
      (c->act_dtype == MOE_F32 && c->expert_dtype == MOE_F32 && c->router_dtype == MOE_F32) ||
      (c->act_dtype == MOE_BF16 && c->expert_dtype == MOE_BF16 && c->router_dtype == MOE_BF16) ||
      (c->act_dtype == MOE_BF16 && is_fp8(c) &&
       (c->router_dtype == MOE_F32 || c->router_dtype == MOE_BF16));
  if (!ok_types) return MOE_ERR_UNSUPPORTED;
  if (is_fp8(c) && c->quant_block != 128) return MOE_ERR_UNSUPPORTED;
  if (c->d_model % 128 || c->d_ff % 128 || (c->num_shared > 0 && c->d_ff_shared % 128))
    return MOE_ERR_UNSUPPORTED;
  if (c->num_experts > 1024 || c->top_k > 64) return MOE_ERR_UNSUPPORTED;
  // (bounds every factor of the operand sizes below, so their 64-bit products cannot overflow)
  if (c->d_model > (1 << 24) || c->d_ff > (1 << 24) ||
      (c->num_shared > 0 && c->d_ff_shared > (1 << 24)))
    return MOE_ERR_UNSUPPORTED;
  if (assignments(c) >= (1LL << 30) || shared_width(c) > (1 << 20)) return MOE_ERR_UNSUPPORTED;
  if (!addressable(c)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

struct WsLayout {
  size_t logits, ids, w, offsets, perm, inv, hist, tiles, tiles_count, xq, xq_scales, h,
      h_scales, hs, hs_scales, so, y, total;
};

WsLayout ws_layout(const moe_config_t* c) {
  WsLayout L{};
  const int64_t A = assignments(c), T = c->num_tokens, d = c->d_model, f = c->d_ff;
  const int64_t fs = shared_width(c);
  const int hb = h_bytes(c);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += align_up(bytes);
    return at;
  };
  L.logits = take(router_splits(c) * T * e_pad(c) * 4);  // one fp32 plane per K range
  L.ids = take(A * 4);
  L.w = take(A * 4);
  L.offsets = take((c->num_experts + 1) * 4);
  L.perm = take(A * 4);
  L.inv = take(A * 4);
  L.hist = take((static_cast<size_t>(permute_num_chunks(c->num_tokens, c->top_k)) + 1) *
                c->num_experts * 4);
  L.tiles = take(routed_max_tiles(c) * 16);
  L.tiles_count = take(4);
  L.xq = take(is_fp8(c) ? T * d : 0);
  L.xq_scales = take(is_fp8(c) ? T * (d / 128) * 4 : 0);
  L.h = take(A * f * hb);
  L.h_scales = take(is_fp8(c) ? A * (f / 128) * 4 : 0);
  L.hs = take(T * fs * hb);
  L.hs_scales = take(is_fp8(c) ? T * (fs / 128) * 4 : 0);
  L.so = take(c->num_shared > 0 ? T * d * so_bytes(c) : 0);  // shared experts' output
  L.y = take(A * d * y_bytes(c));
  L.total = o;
  return L;
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

moe_status_t check_ws(const moe_config_t* c, const void* ws, size_t ws_bytes) {
  if (!ws) return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < ws_layout(c).total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return MOE_OK;
}

moe_status_t check_weights(const moe_config_t* c, const moe_weights_t* w, bool router,
                           bool routed, bool shared) {
  if (!w) return MOE_ERR_INVALID_ARGUMENT;
  if (router && !w->w_router) return MOE_ERR_INVALID_ARGUMENT;
  if (routed && (!w->w_gate_up || !w->w_down)) return MOE_ERR_INVALID_ARGUMENT;
  if (routed && is_fp8(c) && (!w->w_gate_up_scales || !w->w_down_scales))  // both formats
    return MOE_ERR_INVALID_ARGUMENT;
  if (shared && c->num_shared > 0) {
    if (!w->ws_gate_up || !w->ws_down) return MOE_ERR_INVALID_ARGUMENT;
    if (c->shared_gate && !w->ws_gate_vec) return MOE_ERR_INVALID_ARGUMENT;
    if (is_fp8(c) && (!w->ws_gate_up_scales || !w->ws_down_scales))
      return MOE_ERR_INVALID_ARGUMENT;
  }
  return MOE_OK;
}

// ---------------------------------------------------------------- launch sequences

RouteArgs route_args(const moe_config_t* c, const float* select_bias, int32_t* ids, float* tw) {
  RouteArgs a{};
  a.select_bias = select_bias;
  a.ids = ids;
  a.weights = tw;
  a.T = c->num_tokens;
  a.E = c->num_experts;
  a.k = c->top_k;
  a.score = c->score;
  a.renorm = c->renormalize;
  a.gamma = c->routed_scale;
  return a;
}

// Router logits on the MFMA GEMM (fp32 out) into the workspace, then one kernel for the logit
// bias, scoring, top-k and weights -- and for FP8 experts the block-scaled activations of each
// token, written by the wave that routes it.
hipError_t do_route(const moe_config_t* c, const void* x, const moe_weights_t* w, float* logits,
                    int32_t* ids, float* tw, void* xq, float* xq_scales, void* ws,
                    hipStream_t s, const int32_t* token_ids = nullptr,
                    const int32_t* table = nullptr, int vocab = 0) {
  const WsLayout L = ws_layout(c);
  const int kind = router_kind(c);
  const int64_t d = c->d_model, Ep = e_pad(c);
  float* lg = at<float>(ws, L.logits);
  GemmArgs g{};
  g.A = x;
  g.lda = d * act_bytes(c);
  g.a_bytes = c->num_tokens * g.lda;
  g.B = w->w_router;
  g.K = static_cast<int>(kind == kRouterBF16HiLo ? 2 * d : d);
  g.ldb = static_cast<int64_t>(g.K) * (kind == kRouterF32 ? 4 : 2);
  g.a_steps = kind == kRouterBF16HiLo ? static_cast<int>(d * 2 / kBlockK) : 0;
  g.N = static_cast<int>(Ep);
  g.M = c->num_tokens;
  g.out = lg;
  g.ldo = Ep * 4;
  g.out_kind = kRowF32;
  const int splits = router_splits(c);
  g.k_splits = splits;
  g.split_plane = c->num_tokens * Ep * 4;
  const int bm = router_bm(c);
  hipError_t e = launch_grouped_gemm(kind == kRouterF32 ? MOE_F32 : MOE_BF16, kEpiStore, bm, g,
                                     (c->num_tokens + bm - 1) / bm, s);
  if (e != hipSuccess) return e;
  RouteArgs ra = route_args(c, w->select_bias, ids, tw);
  ra.logit_bias = w->logit_bias;
  ra.splits = splits;
  ra.plane = c->num_tokens * Ep;
  ra.token_ids = token_ids;
  ra.table = table;
  ra.vocab = vocab;
  if (is_fp8(c) && xq && xq_scales) {  // the same waves quantise their token's activations
    ra.x = static_cast<const uint16_t*>(x);
    ra.xq = static_cast<uint8_t*>(xq);
    ra.xq_scales = xq_scales;
    ra.d = c->d_model;
  }
  return launch_topk(ra, lg, static_cast<int>(Ep), logits, s);
}

// Records stage event i when the caller asked for stage timing.
hipError_t mark(hipEvent_t* ev, int i, hipStream_t s) {
  return ev ? hipEventRecord(ev[i], s) : hipSuccess;
}

// The weight scales of one packed operand [N, K] per group: FP8 one fp32 per 16 packed rows
// and 128 K values; MXFP4 one E8M0 byte per row and 32 K values.
void set_weight_scales(const moe_config_t* c, GemmArgs& g, const void* scales, int64_t N,
                       int64_t K) {
  if (is_mx(c)) {
    g.b_e8m0 = static_cast<const uint8_t*>(scales);
    g.be_group_stride = N * (K / 32);
  } else {
    g.b_scales = static_cast<const float*>(scales);
    g.bs_group_stride = (N / 16) * (K / 128);
  }
}

// The extra group's weights and their scales (the shared experts, packed like one routed expert).
void set_group2_weights(const moe_config_t* c, GemmArgs& g, const void* wts, const void* scales) {
  g.B2 = wts;
  if (is_mx(c))
    g.b2_e8m0 = static_cast<const uint8_t*>(scales);
  else
    g.b2_scales = static_cast<const float*>(scales);
}

// Routed experts; with_shared (and merge_shared) also the shared experts, as one extra group
// whose h goes to the workspace's h_s and whose output rows to the fp32 shared output.
hipError_t do_expert_ffn(const moe_config_t* c, const void* xa, const float* xs,
                         const int32_t* offsets, const int32_t* perm, const moe_weights_t* w,
                         void* y, void* ws, hipStream_t s, hipEvent_t* ev = nullptr,
                         bool with_shared = false, bool tiles_ready = false) {
  const WsLayout L = ws_layout(c);
  const int64_t A = assignments(c), d = c->d_model, f = c->d_ff, T = c->num_tokens;
  const int hb = h_bytes(c);
  const int bm = routed_bm(c);
  const bool ms = with_shared && merge_shared(c);
  int4* tiles = at<int4>(ws, L.tiles);
  int32_t* tcount = at<int32_t>(ws, L.tiles_count);
  // (tiles_ready: the one-workgroup permutation of a small batch has written the tile list)
  hipError_t e = tiles_ready ? hipSuccess
                             : launch_tile_list(offsets, c->num_experts, bm,
                                                ms ? static_cast<int>(T) : 0, tiles, tcount, s);
  if (e == hipSuccess) e = mark(ev, MOE_STAGE_TILED, s);
  if (e != hipSuccess) return e;
  const int max_tiles = static_cast<int>(routed_max_tiles(c));

  GemmArgs g{};
  g.A = xa;
  g.lda = d * (is_fp8(c) ? 1 : act_bytes(c));
  g.a_bytes = c->num_tokens * g.lda;
  g.a_map = perm;
  g.a_scales = xs;
  g.B = w->w_gate_up;
  g.ldb = wrow(c, d);
  g.b_group_stride = 2 * f * g.ldb;
  set_weight_scales(c, g, w->w_gate_up_scales, 2 * f, d);
  g.K = static_cast<int>(d);
  g.N = static_cast<int>(2 * f);
  g.tiles = tiles;
  g.tiles_count = tcount;
  g.M = static_cast<int>(A);
  g.out = at<uint8_t>(ws, L.h);
  g.ldo = f * hb;
  g.out_scales = is_fp8(c) ? at<float>(ws, L.h_scales) : nullptr;
  // an expert whose rows fit one tile streams its weights past the caches
  g.b_stream = 1;
  if (ms) {  // the shared experts: every token, in order, from the same activations
    g.has_group2 = 1;
    g.group2 = c->num_experts;
    g.m2 = static_cast<int>(A);
    g.A2 = xa;
    g.a2_bytes = g.a_bytes;
    g.a2_scales = xs;
    set_group2_weights(c, g, w->ws_gate_up, w->ws_gate_up_scales);
    g.out2 = at<uint8_t>(ws, L.hs);
    g.ldo2 = f * hb;
    g.out2_scales = is_fp8(c) ? at<float>(ws, L.hs_scales) : nullptr;
  }
  e = launch_grouped_gemm(c->expert_dtype, kEpiSwiglu, bm, g, max_tiles, s);
  if (e == hipSuccess) e = mark(ev, MOE_STAGE_GATE_UP, s);
  if (e != hipSuccess) return e;

  GemmArgs h{};
  h.A = at<uint8_t>(ws, L.h);
  h.lda = f * hb;
  h.a_bytes = A * h.lda;
  h.a_map = nullptr;
  h.a_scales = is_fp8(c) ? at<float>(ws, L.h_scales) : nullptr;
  h.B = w->w_down;
  h.ldb = wrow(c, f);
  h.b_group_stride = d * h.ldb;
  set_weight_scales(c, h, w->w_down_scales, d, f);
  h.K = static_cast<int>(f);
  h.N = static_cast<int>(d);
  h.tiles = tiles;
  h.tiles_count = tcount;
  h.M = static_cast<int>(A);
  h.out = y;
  h.ldo = d * y_bytes(c);
  h.out_kind = y_kind(c);
  h.b_stream = g.b_stream;
  if (ms) {
    h.has_group2 = 1;
    h.group2 = c->num_experts;
    h.m2 = static_cast<int>(A);
    h.A2 = at<uint8_t>(ws, L.hs);
    h.a2_bytes = T * f * hb;
    h.a2_scales = is_fp8(c) ? at<float>(ws, L.hs_scales) : nullptr;
    set_group2_weights(c, h, w->ws_down, w->ws_down_scales);
    h.out2 = at<uint8_t>(ws, L.so);
    h.ldo2 = d * so_bytes(c);
    h.out2_kind = so_kind(c);
  }
  e = launch_grouped_gemm(c->expert_dtype, kEpiStore, bm, h, max_tiles, s);
  if (e == hipSuccess) e = mark(ev, MOE_STAGE_DOWN, s);
  return e;
}

// MXFP4 experts, logical N-major rows (see moe_logical_weights_t): gate/up rows [f, d/2] and
// scale rows [f, d/32] interleaved 16 at a time; down rows [d, f/2] and [d, f/32], the shared
// experts' rows concatenated along K.
hipError_t pack_mx(const moe_config_t* c, const moe_logical_weights_t* lw, void* const* packed,
                   hipStream_t s) {
  const int d = c->d_model, f = c->d_ff, E = c->num_experts;
  // E2M1 weights (64 bytes a step) and their E8M0 scales (4 bytes a step) by column tile and
  // K-step: one contiguous block per step of a tile, the GEMMs' tile widths
  const int tn_gu = e4m3_tile_n(kEpiSwiglu, 2 * f), tn_dn = e4m3_tile_n(kEpiStore, d);
  hipError_t e = launch_pack_rows_gate_up(lw->w_gate, lw->w_up, packed[MOE_PACK_GATE_UP], f, 1,
                                          E, d / 2, tn_gu, 64, s);
  if (e == hipSuccess)
    e = launch_pack_rows_gate_up(lw->w_gate_scales, lw->w_up_scales,
                                 packed[MOE_PACK_GATE_UP_SCALES], f, 1, E, d / 32, tn_gu, 4, s);
  if (e == hipSuccess)
    e = launch_pack_rows_concat(lw->w_down, packed[MOE_PACK_DOWN], d, 1, E, f / 2, tn_dn, 64, s);
  if (e == hipSuccess)
    e = launch_pack_rows_concat(lw->w_down_scales, packed[MOE_PACK_DOWN_SCALES], d, 1, E,
                                f / 32, tn_dn, 4, s);
  if (e != hipSuccess || c->num_shared == 0) return e;
  const int S = c->num_shared, fs = c->d_ff_shared;
  const int tn_sgu = e4m3_tile_n(kEpiSwiglu, 2 * S * fs);
  e = launch_pack_rows_gate_up(lw->ws_gate, lw->ws_up, packed[MOE_PACK_SHARED_GATE_UP], fs, S, 1,
                               d / 2, tn_sgu, 64, s);
  if (e == hipSuccess)
    e = launch_pack_rows_gate_up(lw->ws_gate_scales, lw->ws_up_scales,
                                 packed[MOE_PACK_SHARED_GATE_UP_SCALES], fs, S, 1, d / 32, tn_sgu, 4,
                                 s);
  if (e == hipSuccess)
    e = launch_pack_rows_concat(lw->ws_down, packed[MOE_PACK_SHARED_DOWN], d, S, 1, fs / 2,
                                tn_dn, 64, s);
  if (e == hipSuccess)
    e = launch_pack_rows_concat(lw->ws_down_scales, packed[MOE_PACK_SHARED_DOWN_SCALES], d, S, 1,
                                fs / 32, tn_dn, 4, s);
  return e;
}

// shared_done: the shared experts' output is already in the workspace (they ran as the
// extra group of the routed GEMMs), so only the combine runs.
hipError_t do_combine(const moe_config_t* c, const void* xa, const float* xs, const void* y,
                      const int32_t* inv, const float* tw, const moe_weights_t* w, void* out,
                      void* ws, hipStream_t s, hipEvent_t* ev = nullptr,
                      bool shared_done = false) {
  const WsLayout L = ws_layout(c);
  const int64_t T = c->num_tokens, d = c->d_model, F = shared_width(c);
  const int hb = h_bytes(c);
  const int bm = shared_bm(c);
  const int max_tiles = static_cast<int>((T + bm - 1) / bm);
  hipError_t e = hipSuccess;
  uint8_t* shared_out = nullptr;
  if (c->num_shared > 0 && shared_done) {
    shared_out = at<uint8_t>(ws, L.so);
    e = mark(ev, MOE_STAGE_SHARED_GATE_UP, s);
  } else if (c->num_shared > 0) {
    GemmArgs g{};
    g.A = xa;
    g.lda = d * (is_fp8(c) ? 1 : act_bytes(c));
    g.a_bytes = T * g.lda;
    g.a_scales = xs;
    g.B = w->ws_gate_up;
    g.ldb = wrow(c, d);
    set_weight_scales(c, g, w->ws_gate_up_scales, 2 * F, d);
    g.K = static_cast<int>(d);
    g.N = static_cast<int>(2 * F);
    g.M = static_cast<int>(T);
    g.out = at<uint8_t>(ws, L.hs);
    g.ldo = F * hb;
    g.out_scales = is_fp8(c) ? at<float>(ws, L.hs_scales) : nullptr;
    e = launch_grouped_gemm(c->expert_dtype, kEpiSwiglu, bm, g, max_tiles, s);
    if (e == hipSuccess) e = mark(ev, MOE_STAGE_SHARED_GATE_UP, s);
    if (e != hipSuccess) return e;
    shared_out = at<uint8_t>(ws, L.so);
    GemmArgs h{};
    h.A = at<uint8_t>(ws, L.hs);
    h.lda = F * hb;
    h.a_bytes = T * h.lda;
    h.a_scales = is_fp8(c) ? at<float>(ws, L.hs_scales) : nullptr;
    h.B = w->ws_down;
    h.ldb = wrow(c, F);
    set_weight_scales(c, h, w->ws_down_scales, d, F);
    h.K = static_cast<int>(F);
    h.N = static_cast<int>(d);
    h.M = static_cast<int>(T);
    h.out = shared_out;
    h.ldo = d * so_bytes(c);
    h.out_kind = so_kind(c);
    e = launch_grouped_gemm(c->expert_dtype, kEpiStore, bm, h, max_tiles, s);
  } else {
    e = mark(ev, MOE_STAGE_SHARED_GATE_UP, s);
  }
  if (e == hipSuccess) {
    CombineArgs ca{};
    ca.y = y;
    ca.y_kind = y_kind(c);
    ca.base_kind = so_kind(c);
    ca.inv = inv;
    ca.w = tw;
    ca.k = c->top_k;
    ca.base = shared_out;
    if (shared_out && c->shared_gate) {
      // the gate reads what the shared experts read: x, or the block-scaled FP8 x~
      ca.gate_vec = w->ws_gate_vec;
      ca.gate_f32 = c->router_dtype == MOE_F32;
      ca.x = xa;
      ca.x_kind = is_fp8(c) ? 2 : act_bytes(c) == 4 ? 0 : 1;
      ca.x_scales = xs;
    }
    ca.out = out;
    ca.out_f32 = out_bytes(c) == 4;
    ca.T = static_cast<int>(T);
    ca.d = static_cast<int>(d);
    e = launch_combine(ca, s);
  }
  if (e == hipSuccess) e = mark(ev, MOE_STAGE_COMBINE, s);
  return e;
}

// The launch sequence of moe_forward on a workspace laid out by ws_layout (arguments checked).
hipError_t forward(const moe_config_t* c, const void* x, const moe_weights_t* w, void* out,
                   const moe_debug_t* dbg, void* ws, hipStream_t s) {
  const WsLayout L = ws_layout(c);
  moe_debug_t d{};
  if (dbg) d = *dbg;
  int32_t* ids = d.topk_ids ? d.topk_ids : at<int32_t>(ws, L.ids);
  float* tw = d.topk_w ? d.topk_w : at<float>(ws, L.w);
  int32_t* offsets = d.expert_offsets ? d.expert_offsets : at<int32_t>(ws, L.offsets);
  int32_t* perm = d.perm_token ? d.perm_token : at<int32_t>(ws, L.perm);
  int32_t* inv = d.inv_perm ? d.inv_perm : at<int32_t>(ws, L.inv);
  void* y = d.y_perm ? d.y_perm : at<void>(ws, L.y);
  void* xq = is_fp8(c) ? at<void>(ws, L.xq) : nullptr;
  float* xs = is_fp8(c) ? at<float>(ws, L.xq_scales) : nullptr;
  const void* xa = is_fp8(c) ? static_cast<const void*>(xq) : x;
  hipEvent_t* ev = d.stage_events;
  hipError_t e = mark(ev, MOE_STAGE_BEGIN, s);
  if (e == hipSuccess) e = do_route(c, x, w, d.logits, ids, tw, xq, xs, ws, s);
  if (e == hipSuccess) e = mark(ev, MOE_STAGE_ROUTED, s);
  // the shared experts join the routed GEMMs as one extra group when they fit (merge_shared)
  const bool ms = merge_shared(c);
  // a small batch is permuted, and its tile list built, by one workgroup
  const bool small = permute_small_ok(assignments(c), c->num_experts);
  if (e == hipSuccess && small)
    e = launch_permute_small(ids, c->num_tokens, c->top_k, c->num_experts, offsets, perm, inv,
                             routed_bm(c), ms ? c->num_tokens : 0, at<int4>(ws, L.tiles),
                             at<int32_t>(ws, L.tiles_count), s);
  else if (e == hipSuccess)
    e = launch_permute(ids, c->num_tokens, c->top_k, c->num_experts, offsets, perm, inv,
                       at<int32_t>(ws, L.hist), s);
  if (e == hipSuccess) e = mark(ev, MOE_STAGE_PERMUTED, s);
  if (e == hipSuccess) e = do_expert_ffn(c, xa, xs, offsets, perm, w, y, ws, s, ev, ms, small);
  if (e == hipSuccess) e = do_combine(c, xa, xs, y, inv, tw, w, out, ws, s, ev, ms);
  return e;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(moe_status_t st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

size_t moe_workspace_size(const moe_config_t* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  return ws_layout(cfg).total;
}

size_t moe_packed_size(const moe_config_t* c, int which) {
  if (check_config(c) != MOE_OK) return 0;
  const size_t d = c->d_model, f = c->d_ff, E = c->num_experts, F = shared_width(c);
  const bool q = c->expert_dtype == MOE_FP8_E4M3, mx = is_mx(c);
  // FP8: fp32 per 16 packed rows and 128 K; MXFP4: an E8M0 byte per row and 32 K
  auto sc = [&](size_t N, size_t K) -> size_t {
    return q ? (N / 16) * (K / 128) * 4 : mx ? N * (K / 32) : 0;
  };
  switch (which) {
    case MOE_PACK_ROUTER: {
      int k = router_kind(c);
      size_t eb = k == kRouterF32 ? 4 : k == kRouterBF16 ? 2 : 4;  // hi/lo: two bf16 planes
      return static_cast<size_t>(e_pad(c)) * d * eb;
    }
    case MOE_PACK_GATE_UP: return E * 2 * f * wrow(c, d);
    case MOE_PACK_GATE_UP_SCALES: return E * sc(2 * f, d);
    case MOE_PACK_DOWN: return E * d * wrow(c, f);
    case MOE_PACK_DOWN_SCALES: return E * sc(d, f);
    case MOE_PACK_SHARED_GATE_UP: return 2 * F * wrow(c, d);
    case MOE_PACK_SHARED_GATE_UP_SCALES: return sc(2 * F, d);
    case MOE_PACK_SHARED_DOWN: return d * wrow(c, F);
    case MOE_PACK_SHARED_DOWN_SCALES: return sc(d, F);
    default: return 0;
  }
}

moe_status_t moe_pack_weights(const moe_config_t* c, const moe_logical_weights_t* lw,
                              void* const* packed, hipStream_t s) {
  moe_status_t st = check_config(c);
  if (st != MOE_OK) return st;
  if (!lw || !packed) return MOE_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < MOE_PACK_COUNT; ++i)
    if (moe_packed_size(c, i) > 0 && !packed[i]) return MOE_ERR_INVALID_ARGUMENT;
  if (!lw->w_router || !lw->w_gate || !lw->w_up || !lw->w_down) return MOE_ERR_INVALID_ARGUMENT;
  const bool q = is_fp8(c);  // FP8 and MXFP4 weights both carry scales
  if (q && (!lw->w_gate_scales || !lw->w_up_scales || !lw->w_down_scales))
    return MOE_ERR_INVALID_ARGUMENT;
  if (c->num_shared > 0) {
    if (!lw->ws_gate || !lw->ws_up || !lw->ws_down) return MOE_ERR_INVALID_ARGUMENT;
    if (q && (!lw->ws_gate_scales || !lw->ws_up_scales || !lw->ws_down_scales))
      return MOE_ERR_INVALID_ARGUMENT;
  }
  const int d = c->d_model, f = c->d_ff, E = c->num_experts, wb = h_bytes(c);
  hipError_t e;
  const int rk = router_kind(c);
  e = launch_pack_router(lw->w_router, c->router_dtype == MOE_F32 ? 4 : 2,
                         rk == kRouterBF16HiLo, packed[MOE_PACK_ROUTER], d, E, e_pad(c), s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (is_mx(c)) return hip_status(pack_mx(c, lw, packed, s));
  e = launch_pack_gate_up(lw->w_gate, lw->w_up, packed[MOE_PACK_GATE_UP], d, f, 1, E, wb, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = launch_pack_down(lw->w_down, packed[MOE_PACK_DOWN], d, f, 1, E, wb, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (q) {
    e = launch_pack_scales_gate_up(static_cast<const float*>(lw->w_gate_scales),
                                   static_cast<const float*>(lw->w_up_scales),
                                   static_cast<float*>(packed[MOE_PACK_GATE_UP_SCALES]), d, f, 1,
                                   E, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    e = launch_pack_scales_down(static_cast<const float*>(lw->w_down_scales),
                                static_cast<float*>(packed[MOE_PACK_DOWN_SCALES]), d, f, 1, E, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  if (c->num_shared > 0) {
    const int S = c->num_shared, fs = c->d_ff_shared;
    e = launch_pack_gate_up(lw->ws_gate, lw->ws_up, packed[MOE_PACK_SHARED_GATE_UP], d, fs, S, 1,
                            wb, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    e = launch_pack_down(lw->ws_down, packed[MOE_PACK_SHARED_DOWN], d, fs, S, 1, wb, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (q) {
      e = launch_pack_scales_gate_up(static_cast<const float*>(lw->ws_gate_scales),
                                     static_cast<const float*>(lw->ws_up_scales),
                                     static_cast<float*>(packed[MOE_PACK_SHARED_GATE_UP_SCALES]),
                                     d, fs, S, 1, s);
      if (e != hipSuccess) return MOE_ERR_HIP;
      e = launch_pack_scales_down(static_cast<const float*>(lw->ws_down_scales),
                                  static_cast<float*>(packed[MOE_PACK_SHARED_DOWN_SCALES]), d, fs,
                                  S, 1, s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
  }
  return MOE_OK;
}

moe_status_t moe_route(const moe_config_t* c, const void* x, const moe_weights_t* w,
                       float* logits, int32_t* ids, float* tw, void* xq, float* xq_scales,
                       void* ws, size_t ws_bytes, hipStream_t s) {
  moe_status_t st = check_config(c);
  if (st != MOE_OK) return st;
  if (!x || !ids || !tw) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = check_weights(c, w, true, false, false)) != MOE_OK) return st;
  if ((st = check_ws(c, ws, ws_bytes)) != MOE_OK) return st;
  if (c->num_tokens == 0) return MOE_OK;
  return hip_status(do_route(c, x, w, logits, ids, tw, xq, xq_scales, ws, s));
}

moe_status_t moe_route_hashed(const moe_config_t* c, const void* x, const moe_weights_t* w,
                              const int32_t* token_ids, const int32_t* table, int32_t vocab,
                              float* logits, int32_t* ids, float* tw, void* xq, float* xq_scales,
                              void* ws, size_t ws_bytes, hipStream_t s) {
  moe_status_t st = check_config(c);
  if (st != MOE_OK) return st;
  if (!x || !ids || !tw || !token_ids || !table || vocab < 1) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = check_weights(c, w, true, false, false)) != MOE_OK) return st;
  if ((st = check_ws(c, ws, ws_bytes)) != MOE_OK) return st;
  if (c->num_tokens == 0) return MOE_OK;
  return hip_status(
      do_route(c, x, w, logits, ids, tw, xq, xq_scales, ws, s, token_ids, table, vocab));
}

moe_status_t moe_update_bias(const moe_config_t* c, const int32_t* offsets, float speed,
                             float* select_bias, hipStream_t s) {
  moe_status_t st = check_config(c);
  if (st != MOE_OK) return st;
  if (!offsets || !select_bias || !isfinite(speed) || speed < 0.0f)
    return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(launch_bias_update(offsets, c->num_experts, speed, select_bias, s));
}

moe_status_t moe_route_from_logits(const moe_config_t* c, const float* logits,
                                   const float* select_bias, int32_t* ids, float* tw,
                                   hipStream_t s) {
  moe_status_t st = check_config(c);
  if (st != MOE_OK) return st;
  if (!logits || !ids || !tw) return MOE_ERR_INVALID_ARGUMENT;
  if (c->num_tokens == 0) return MOE_OK;
  return hip_status(launch_topk(route_args(c, select_bias, ids, tw), logits, c->num_experts,
                                nullptr, s));
}

moe_status_t moe_permute(const moe_config_t* c, const int32_t* ids, int32_t* offsets,
                         int32_t* perm, int32_t* inv, void* ws, size_t ws_bytes, hipStream_t s) {
  moe_status_t st = check_config(c);
  if (st != MOE_OK) return st;
  if (!ids || !offsets || !perm || !inv) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = check_ws(c, ws, ws_bytes)) != MOE_OK) return st;
  if (c->num_tokens == 0) return MOE_OK;
  const WsLayout L = ws_layout(c);
  if (permute_small_ok(assignments(c), c->num_experts))
    return hip_status(launch_permute_small(ids, c->num_tokens, c->top_k, c->num_experts, offsets,
                                           perm, inv, 0, 0, nullptr, nullptr, s));
  return hip_status(launch_permute(ids, c->num_tokens, c->top_k, c->num_experts, offsets, perm,
                                   inv, at<int32_t>(ws, L.hist), s));
}

moe_status_t moe_expert_ffn(const moe_config_t* c, const void* xa, const float* xs,
                            const int32_t* offsets, const int32_t* perm, const moe_weights_t* w,
                            void* y, void* ws, size_t ws_bytes, hipStream_t s) {
  moe_status_t st = check_config(c);
  if (st != MOE_OK) return st;
  if (!xa || !offsets || !perm || !y || (is_fp8(c) && !xs)) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = check_weights(c, w, false, true, false)) != MOE_OK) return st;
  if ((st = check_ws(c, ws, ws_bytes)) != MOE_OK) return st;
  if (c->num_tokens == 0) return MOE_OK;
  return hip_status(do_expert_ffn(c, xa, xs, offsets, perm, w, y, ws, s));
}

moe_status_t moe_combine(const moe_config_t* c, const void* xa, const float* xs, const void* y,
                         const int32_t* inv, const float* tw, const moe_weights_t* w, void* out,
                         void* ws, size_t ws_bytes, hipStream_t s) {
  moe_status_t st = check_config(c);
  if (st != MOE_OK) return st;
  if (!y || !inv || !tw || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (c->num_shared > 0 && (!xa || (is_fp8(c) && !xs))) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = check_weights(c, w, false, false, true)) != MOE_OK) return st;
  if ((st = check_ws(c, ws, ws_bytes)) != MOE_OK) return st;
  if (c->num_tokens == 0) return MOE_OK;
  return hip_status(do_combine(c, xa, xs, y, inv, tw, w, out, ws, s));
}

moe_status_t moe_forward(const moe_config_t* c, const void* x, const moe_weights_t* w, void* out,
                         const moe_debug_t* dbg, void* ws, size_t ws_bytes, hipStream_t s) {
  moe_status_t st = check_config(c);
  if (st != MOE_OK) return st;
  if (!x || !out) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = check_weights(c, w, true, true, true)) != MOE_OK) return st;
  if ((st = check_ws(c, ws, ws_bytes)) != MOE_OK) return st;
  if (c->num_tokens == 0) return MOE_OK;
  return hip_status(forward(c, x, w, out, dbg, ws, s));
}

moe_status_t moe_forward_noalloc(const moe_config_t* c, const void* x, const moe_weights_t* w,
                                 void* out, const moe_debug_t* dbg, hipStream_t s) {
  moe_status_t st = check_config(c);
  if (st != MOE_OK) return st;
  if (!x || !out) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = check_weights(c, w, true, true, true)) != MOE_OK) return st;
  if (ws_layout(c).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (c->num_tokens == 0) return MOE_OK;
  void* ws = nullptr;
  if (static_scratch(&ws) != hipSuccess) return MOE_ERR_HIP;
  return hip_status(forward(c, x, w, out, dbg, ws, s));
}

}  // extern "C"
