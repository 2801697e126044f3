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
// registers and sorts their keys, then k rounds of a 64-lane maximum over the lanes' largest
// remaining keys pick the experts in key order.  In the layers
// that choose by a fixed token-id hash (same row, DeepSeek-V4-Pro cell) a table gives the k
// experts instead, and only the combine weights are computed.
#include <math.h>

#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

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

// max(v, v moved by one DPP lane pattern) over 32-bit unsigned values; lanes outside ROW_MASK,
// or whose source lane is out of range, see 0.  The wave's maximum, wave-uniform: within each
// row of 16 lanes by quad swaps and the half-row and row mirrors, across rows by the row
// broadcasts into lane 63; the minimum as the maximum of complements.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_max32(uint32_t v) {
  const uint32_t o = __builtin_amdgcn_update_dpp(0u, v, CTRL, ROW_MASK, 0xF, false);
  return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max32<0xB1>(v);        // quad_perm [1,0,3,2]
  v = dpp_max32<0x4E>(v);        // quad_perm [2,3,0,1]
  v = dpp_max32<0x141>(v);       // row_half_mirror
  v = dpp_max32<0x140>(v);       // row_mirror
  v = dpp_max32<0x142, 0xA>(v);  // row_bcast15 into rows 1 and 3
  v = dpp_max32<0x143, 0xC>(v);  // row_bcast31 into rows 2 and 3
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return ~wave_max_u32(~v); }

// The lane's N keys sorted into descending order in registers (a bitonic network: the indices
// are compile-time constants once unrolled, so nothing leaves the registers).
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t* k) {
#pragma unroll
  for (int size = 2; size <= N; size <<= 1)
#pragma unroll
    for (int stride = size / 2; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          // blocks of `size` alternate direction; the last merge (size = N) is descending
          const bool desc = (i & size) == 0;
          const uint64_t a = k[i], b = k[j];
          const bool sw = desc ? a < b : a > b;
          k[i] = sw ? b : a;
          k[j] = sw ? a : b;
        }
      }
}

// Logit of expert e with the logit bias, and its unbiased score (softmax: the logit).
__device__ __forceinline__ float expert_value(const float* row, int e, const RouteArgs& a) {
  const float lg = a.logit_bias ? __fadd_rn(row[e], a.logit_bias[e]) : row[e];
  return a.score == MOE_SCORE_SOFTMAX ? lg : sigma_family_score(a.score, lg);
}

// Top-k of one token over `row[0..E)`, executed by one full wave; lane l holds experts
// l + 64 i, i < SLOTS (E <= 64 * SLOTS).  Each lane sorts its keys once; a round is then the
// wave's largest lane head (the winner) and one shift of the winner's lane, instead of a scan of
// every slot of every lane.  The winners' scores are evaluated again from their ids, by the same
// function that made the keys.
template <int SLOTS>
__device__ void topk_row(const float* row, int t, const RouteArgs& a) {
  const int l = lane_id();
  uint64_t key[SLOTS];
  float val[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    int e = l + kWave * i;
    key[i] = 0;
    val[i] = 0.0f;
    if (e < a.E) {
      const float s = expert_value(row, e, a);
      val[i] = s;
      if (a.score == MOE_SCORE_SOFTMAX) {
        key[i] = select_key(s, e);
      } else {
        const float b = a.select_bias ? a.select_bias[e] : 0.0f;
        key[i] = select_key(__fadd_rn(s, b), e);
      }
    }
  }
  int my_id = 0;
  if (a.table) {
    // fixed token-id table: lane j < k takes slot j's expert.  Values outside their ranges (a
    // precondition violation) are clamped, so nothing reads out of bounds.
    if (l < a.k) {
      const int tok = min(max(a.token_ids[t], 0), a.vocab - 1);
      my_id = min(max(a.table[static_cast<size_t>(tok) * a.k + l], 0), a.E - 1);
    }
  } else {
    sort_desc<SLOTS>(key);
    // The sorted keys split into their upper halves (the ordered fp32 keys; 0: no candidate)
    // and, 4 bits a position, the slots i of the experts l + 64 i they belong to.  Within a
    // lane equal keys are already in ascending expert order.
    uint32_t hi[SLOTS];
    uint64_t order = 0;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      hi[i] = static_cast<uint32_t>(key[i] >> 32);
      order |= static_cast<uint64_t>((~static_cast<uint32_t>(key[i]) >> 6) & 15u) << (4 * i);
    }
    // k rounds: the largest head wins (among equal heads the lowest expert id), its lane drops
    // it; lane j keeps the winner of round j
    for (int j = 0; j < a.k; ++j) {
      const uint32_t m = wave_max_u32(hi[0]);
      const uint64_t tied = __ballot(hi[0] == m);
      int we;
      if (__popcll(tied) == 1) {
        const int wl = __ffsll(static_cast<unsigned long long>(tied)) - 1;
        we = wl + kWave * static_cast<int>(
                          __builtin_amdgcn_readlane(static_cast<uint32_t>(order), wl) & 15u);
      } else {
        const uint32_t id = static_cast<uint32_t>(l + kWave * static_cast<int>(order & 15u));
        we = static_cast<int>(wave_min_u32(hi[0] == m ? id : 0xFFFFFFFFu));
      }
      const bool mine = l == (we & (kWave - 1));
#pragma unroll
      for (int i = 0; i + 1 < SLOTS; ++i) hi[i] = mine ? hi[i + 1] : hi[i];
      hi[SLOTS - 1] = mine ? 0u : hi[SLOTS - 1];
      order = mine ? order >> 4 : order;
      if (l == j) my_id = we;
    }
  }
  const float my_val = l < a.k ? expert_value(row, my_id, a) : 0.0f;
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
      for (int i = 0; i < SLOTS; ++i)
        if (l + kWave * i < a.E) mm = fmaxf(mm, val[i]);
      m = wave_max(mm);
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < SLOTS; ++i)
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

// Block-scaled FP8 activations of token t, by the wave that routed it: one fp32 scale =
// max|x| / 448 (1 for an all-zero group) per 128 consecutive values of the row, codes =
// E4M3(x / scale), both divisions correctly rounded fp32 (blueprint training box: FP8 with
// block scales).  16 lanes own one group, 8 values each; the wave covers four groups at a time.
__device__ void quant_row_fp8(const RouteArgs& a, int t) {
  const int l = lane_id(), sub = l & 15, groups = a.d / 128;
  const uint16_t* xr = a.x + static_cast<size_t>(t) * a.d;
  uint8_t* qr = a.xq + static_cast<size_t>(t) * a.d;
  // (unrolled so that several iterations' loads are in flight: a decode batch has only a few
  // dozen such waves on the whole GPU)
#pragma unroll 4
  for (int g0 = 0; g0 < groups; g0 += 4) {
    const int grp = g0 + (l >> 4);
    const bool valid = grp < groups;  // whole 16-lane groups
    const int at = (valid ? grp : 0) * 128 + sub * 8;
    const i32x4 raw = *reinterpret_cast<const i32x4*>(xr + at);
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
    const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
    // v / sc correctly rounded to fp32 as RN32(v * RN64(1/sc)): the fp64 product is within
    // 2^-52 (relative) of the quotient, and a quotient of two fp32 numbers is never within
    // about 2^-49 of an fp32 rounding midpoint, so both round alike
    const double rs = 1.0 / static_cast<double>(sc);
    auto quo = [rs](float x) { return static_cast<float>(static_cast<double>(x) * rs); };
    const uint32_t lo = e4m3x4(quo(v[0]), quo(v[1]), quo(v[2]), quo(v[3]));
    const uint32_t hi = e4m3x4(quo(v[4]), quo(v[5]), quo(v[6]), quo(v[7]));
    if (valid) {
      *reinterpret_cast<uint2*>(qr + at) = uint2{lo, hi};
      if (sub == 0) a.xq_scales[static_cast<size_t>(t) * groups + grp] = sc;
    }
  }
}

// One wave per token.  `logits` rows are `ld` floats apart; a.logit_bias (if any) is added to
// each (one fp32 add, the last step of the logits); when `copy` is non-null the E finished
// logits of each row are also written there as [T, E].
template <int SLOTS>
__global__ __launch_bounds__(256) void topk_kernel(RouteArgs a, const float* logits, int ld,
                                                   float* __restrict__ copy) {
  // partial logits of a K-split router GEMM, added in plane order into a row of this wave's
  // own in LDS (the row the choice then reads; a wave's LDS accesses complete in order)
  __shared__ float s_sum[4][1024];
  int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= a.T) return;  // whole waves leave together
  const float* row = logits + static_cast<size_t>(t) * ld;
  if (a.splits > 1) {
    float* sum = s_sum[threadIdx.x / kWave];
    for (int e = lane_id(); e < a.E; e += kWave) {
      float v = row[e];
      for (int p = 1; p < a.splits; ++p) v += row[p * a.plane + e];
      sum[e] = v;
    }
    row = sum;
  }
  if (copy)
    for (int e = lane_id(); e < a.E; e += kWave)
      copy[static_cast<size_t>(t) * a.E + e] =
          a.logit_bias ? __fadd_rn(row[e], a.logit_bias[e]) : row[e];
  topk_row<SLOTS>(row, t, a);
  if (a.xq) quant_row_fp8(a, t);
}

hipError_t launch_topk(const RouteArgs& a, const float* logits, int ld, float* copy,
                       hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  // experts per lane: E <= 64 * SLOTS (E <= 1024, checked by the caller)
  const dim3 grid((a.T + 3) / 4), block(256);
  if (a.E <= 256)
    hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, a, logits, ld, copy);
  else if (a.E <= 512)
    hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, s, a, logits, ld, copy);
  else
    hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, s, a, logits, ld, copy);
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

}  // namespace moe
