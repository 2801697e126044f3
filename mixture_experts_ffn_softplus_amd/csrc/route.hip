// route.hip -- router scoring and top-k, and the FP8 activation quantiser.
//
// The router of the archdiff.com pages ("Qwen3.5-397B-A17B vs DeepSeek-V4-Pro", component
// table, router row): a linear map of the token to one logit per expert; then either a
// softmax over the experts with the top k kept and renormalised (Qwen3.5 cell), or
// sqrt-softplus (or sigma, blueprint router box) scores with a per-expert bias added only for
// choosing the top k, the chosen unbiased scores normalised and scaled by 2.5 (DeepSeek-V4-Pro
// cell).  Ties at equal keys go to the lower expert index.
//
// The logits come from the grouped MFMA GEMM (one group, fp32 out); the logit bias is added
// here as each logit is read.  One wave owns one token: each lane scores E/64 experts held in
// registers, then k rounds of a 64-lane argmax pick the experts in key order.  In the layers
// that choose by a fixed token-id hash (same row, DeepSeek-V4-Pro cell) a table gives the k
// experts instead, and only the combine weights are computed.
#include <math.h>

#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

constexpr int kMaxPerLane = 16;       // experts per lane in top-k: E <= 1024

// Score of the sigma family, evaluated in fp64 and rounded once to fp32, so the
// selection key is one fixed fp32 number.
__device__ __forceinline__ float sigma_family_score(int score, float l) {
  double s;
  if (score == MOE_SCORE_SIGMOID) {
    s = 1.0 / (1.0 + exp(-static_cast<double>(l)));
  } else {
    double ld = static_cast<double>(l);
    s = sqrt(fmax(ld, 0.0) + log1p(exp(-fabs(ld))));
  }
  return static_cast<float>(s);
}

// Order-preserving 64-bit selection key of one expert: the fp32 key's bits mapped so that
// unsigned order is numeric order (-0 folded into +0 first, so equal keys stay equal), above
// the bitwise complement of the expert id, so that the unsigned maximum is the largest key
// and, among equal keys, the lower expert id.  0 marks "not a candidate".
__device__ __forceinline__ uint64_t select_key(float key, int e) {
  const uint32_t b = __float_as_uint(key + 0.0f);
  const uint32_t u = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<uint64_t>(u) << 32) | static_cast<uint32_t>(~e);
}

// max(v, v moved by one DPP lane pattern) over the 64-bit key; lanes outside ROW_MASK, or
// whose source lane is out of range, see 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint64_t dpp_max(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(v), CTRL, ROW_MASK,
                                                  0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(v >> 32), CTRL,
                                                  ROW_MASK, 0xF, false);
  const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
  return o > v ? o : v;
}

// The wave's largest key, wave-uniform: within each row of 16 lanes by quad swaps and the
// half-row and row mirrors, across rows by the row broadcasts into lane 63.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
  v = dpp_max<0xB1>(v);         // quad_perm [1,0,3,2]
  v = dpp_max<0x4E>(v);         // quad_perm [2,3,0,1]
  v = dpp_max<0x141>(v);        // row_half_mirror
  v = dpp_max<0x140>(v);        // row_mirror
  v = dpp_max<0x142, 0xA>(v);   // row_bcast15 into rows 1 and 3
  v = dpp_max<0x143, 0xC>(v);   // row_bcast31 into rows 2 and 3
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), 63);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Top-k of one token over `row[0..E)` (LDS or global), executed by one full wave.
__device__ void topk_row(const float* row, int t, const RouteArgs& a) {
  const int l = lane_id();
  uint64_t key[kMaxPerLane];
  float val[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    int e = l + kWave * i;
    key[i] = 0;
    val[i] = 0.0f;
    if (e < a.E) {
      const float lg = a.logit_bias ? __fadd_rn(row[e], a.logit_bias[e]) : row[e];
      if (a.score == MOE_SCORE_SOFTMAX) {
        key[i] = select_key(lg, e);
        val[i] = lg;
      } else {
        float s = sigma_family_score(a.score, lg);
        float b = a.select_bias ? a.select_bias[e] : 0.0f;
        val[i] = s;
        key[i] = select_key(__fadd_rn(s, b), e);
      }
    }
  }
  int my_id = 0;
  float my_val = 0.0f;
  if (a.table) {
    // fixed token-id table: lane j < k takes slot j's expert and its unbiased score.  Values
    // outside their ranges (a precondition violation) are clamped, so nothing reads out of
    // bounds.
    if (l < a.k) {
      const int tok = min(max(a.token_ids[t], 0), a.vocab - 1);
      const int e = min(max(a.table[static_cast<size_t>(tok) * a.k + l], 0), a.E - 1);
      const float lg = a.logit_bias ? __fadd_rn(row[e], a.logit_bias[e]) : row[e];
      my_id = e;
      my_val = a.score == MOE_SCORE_SOFTMAX ? lg : sigma_family_score(a.score, lg);
    }
  }
  // k rounds: each lane's largest remaining key, the wave's largest of those; its owner lane
  // drops it and lane j keeps the winner of round j
  for (int j = 0; j < (a.table ? 0 : a.k); ++j) {
    uint64_t best = 0;
    float bv = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const bool gt = key[i] > best;
      best = gt ? key[i] : best;
      bv = gt ? val[i] : bv;
    }
    const uint64_t win = wave_max_key(best);
    const int we = static_cast<int>(~static_cast<uint32_t>(win));
    const int owner = we & (kWave - 1);
    const float wv = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(bv), owner));
    if (l == owner) {
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i)
        if (i == (we >> 6)) key[i] = 0;
    }
    if (l == j) {
      my_id = we;
      my_val = wv;
    }
  }
  float w;
  if (a.score == MOE_SCORE_SOFTMAX) {
    float m, denom;
    if (a.renorm) {
      // the largest selected logit: slot 0's for the top-k choice
      m = a.table ? wave_max(l < a.k ? my_val : -INFINITY) : __shfl(my_val, 0, kWave);
      denom = wave_sum(l < a.k ? expf(my_val - m) : 0.0f);
    } else {
      float mm = -INFINITY;
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i)
        if (l + kWave * i < a.E) mm = fmaxf(mm, val[i]);
      m = wave_max(mm);
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i)
        if (l + kWave * i < a.E) part += expf(val[i] - m);
      denom = wave_sum(part);
    }
    w = a.gamma * expf(my_val - m) / denom;
  } else {
    float denom = a.renorm ? wave_sum(l < a.k ? my_val : 0.0f) : 1.0f;
    w = a.gamma * my_val / denom;
  }
  if (l < a.k) {
    a.ids[static_cast<size_t>(t) * a.k + l] = my_id;
    a.weights[static_cast<size_t>(t) * a.k + l] = w;
  }
}

// One wave per token.  `logits` rows are `ld` floats apart; a.logit_bias (if any) is added to
// each (one fp32 add, the last step of the logits); when `copy` is non-null the E finished
// logits of each row are also written there as [T, E].
__global__ __launch_bounds__(256) void topk_kernel(RouteArgs a, const float* __restrict__ logits,
                                                   int ld, float* __restrict__ copy) {
  int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= a.T) return;  // whole waves leave together
  const float* row = logits + static_cast<size_t>(t) * ld;
  if (copy)
    for (int e = lane_id(); e < a.E; e += kWave)
      copy[static_cast<size_t>(t) * a.E + e] =
          a.logit_bias ? __fadd_rn(row[e], a.logit_bias[e]) : row[e];
  topk_row(row, t, a);
}

// Block-scaled FP8 activations: one fp32 scale = max|x| / 448 (1 for an all-zero group)
// per 128 consecutive values of a row, codes = E4M3(x / scale), both divisions correctly
// rounded fp32.  16 lanes own one group, 8 values each.
__global__ __launch_bounds__(256) void quant_x_fp8_kernel(const uint16_t* __restrict__ x,
                                                          uint8_t* __restrict__ xq,
                                                          float* __restrict__ scales, int T,
                                                          int d) {
  const int groups_per_row = d / 128;
  const int64_t total = static_cast<int64_t>(T) * groups_per_row;
  const int64_t gid = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / 16;
  const int sub = threadIdx.x & 15;
  const bool valid = gid < total;
  const int64_t g = valid ? gid : 0;
  const int64_t row = g / groups_per_row, grp = g - row * groups_per_row;
  const size_t base = static_cast<size_t>(row) * d + grp * 128 + sub * 8;
  i32x4 raw = *reinterpret_cast<const i32x4*>(x + base);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(static_cast<uint32_t>(raw[i]) << 16);
    v[2 * i + 1] = __uint_as_float(static_cast<uint32_t>(raw[i]) & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  const uint32_t lo = e4m3x4(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
  const uint32_t hi = e4m3x4(v[4] / s, v[5] / s, v[6] / s, v[7] / s);
  if (valid) {
    uint2 packed{lo, hi};
    *reinterpret_cast<uint2*>(xq + base) = packed;
    if (sub == 0) scales[g] = s;
  }
}

hipError_t launch_topk(const RouteArgs& a, const float* logits, int ld, float* copy,
                       hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a, logits, ld, copy);
  return hipGetLastError();
}

// Auxiliary-loss-free balancing step (router row, DeepSeek-V4-Pro cell: bias balancing with
// speed 0.001): the selection bias of an expert that took more than the mean load T*k/E moves
// down by `speed`, of one that took less moves up, of one exactly at it stays as it is.  The
// comparison is exact in integers; the step is one fp32 add.  One thread per expert.
__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ offsets,
                                                          int E, float speed,
                                                          float* __restrict__ bias) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int64_t A = offsets[E];
  const int64_t diff = A - static_cast<int64_t>(E) * (offsets[e + 1] - offsets[e]);
  if (diff != 0) bias[e] = __fadd_rn(bias[e], diff > 0 ? speed : -speed);  // at the mean: kept
}

hipError_t launch_bias_update(const int32_t* offsets, int E, float speed, float* bias,
                              hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3((E + 255) / 256), dim3(256), 0, s, offsets, E,
                     speed, bias);
  return hipGetLastError();
}

hipError_t launch_quant_x_fp8(const uint16_t* x, uint8_t* xq, float* scales, int T, int d,
                              hipStream_t s) {
  if (T == 0) return hipSuccess;
  int64_t groups = static_cast<int64_t>(T) * (d / 128);
  int64_t blocks = (groups * 16 + 255) / 256;
  hipLaunchKernelGGL(quant_x_fp8_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     x, xq, scales, T, d);
  return hipGetLastError();
}

}  // namespace moe
