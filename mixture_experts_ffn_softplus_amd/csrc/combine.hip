// combine.hip -- un-permute and weighted sum of the routed expert rows, plus the shared experts.
//
// out[t] = shared[t] + sum_j w[t, j] * y_perm[inv_perm[t * k + j]]: the routed experts' outputs
// weighted by the router and added to the always-active shared experts' output (routed-experts
// and shared-expert rows of "Qwen3.5-397B-A17B vs Gemma 4 31B"; the block's equation of the
// DeepSeek-V4 blueprint).  Pure streaming: one workgroup per token.  The token's k row indices
// and weights are staged in LDS once (padded to a multiple of eight with zero-weight copies of a
// real row), so each thread, owning one 8-column chunk, issues its y loads eight at a time with
// no dependent index load in between.
//
// Gated shared expert (shared-expert row, Qwen3.5 cell): the shared output is first scaled by
// the token's sigmoid(x~ . w_sg), one dot product of length d per token reduced across the
// workgroup before the streaming loop; x~ is the activation row the shared experts read.
#include <type_traits>

#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

constexpr int kCombineMaxThreads = 1024;
constexpr int kCombineBatch = 8;  // y rows loaded together
constexpr int kCombineMaxK = 64;  // top_k limit of the library

struct CombineGate {
  const uint8_t* vec;  // [d] fp32 or bf16, null: no gate
  const uint8_t* x;    // [T, d] activations (fp32 / bf16 / E4M3 codes)
  const float* xs;     // E4M3: [T, d/128] scales
  int vec_f32, x_kind;
};

// Eight consecutive values of a row of bf16 or fp16 (16 B) or fp32 (32 B) elements (RowKind);
// NT: non-temporal loads.  The expert rows are read once; measured on MI355X, non-temporal
// loads speed up the 2-byte rows (bf16 rows of FP8 experts: 2.95 GB, 668 -> 585 us; fp16 rows
// of softmax_bf16: 0.34 GB, 145 -> 139 us) but slow down the fp32 rows (0.67 GB, 183 -> 216
// us), so only the former use them.
template <int KIND, bool NT = false>
__device__ __forceinline__ void load8(const uint8_t* p, float* v) {
  if constexpr (KIND == kRowF32) {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    const f32x4 a = NT ? __builtin_nontemporal_load(q) : q[0];
    const f32x4 b = NT ? __builtin_nontemporal_load(q + 1) : q[1];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = a[q];
      v[4 + q] = b[q];
    }
  } else {
    const i32x4* q = reinterpret_cast<const i32x4*>(p);
    const i32x4 r = NT ? __builtin_nontemporal_load(q) : q[0];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t bits = static_cast<uint32_t>(r[q]);
      if constexpr (KIND == kRowBF16) {
        v[2 * q] = __uint_as_float(bits << 16);
        v[2 * q + 1] = __uint_as_float(bits & 0xFFFF0000u);
      } else {
        v[2 * q] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
        v[2 * q + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits >> 16)));
      }
    }
  }
}

// sigmoid(x~[t] . vec), reduced over the whole workgroup (every thread gets the value).
__device__ float shared_gate(const CombineGate& g, int t, int d) {
  __shared__ float part[kCombineMaxThreads / kWave];
  float z = 0.0f;
  for (int c = threadIdx.x; c < d / 8; c += blockDim.x) {
    float xv[8], gv[8];
    const int64_t i = static_cast<int64_t>(t) * d + c * 8;
    if (g.x_kind == 0) {
      load8<kRowF32>(g.x + i * 4, xv);
    } else if (g.x_kind == 1) {
      load8<kRowBF16>(g.x + i * 2, xv);
    } else {
      const uint2 codes = *reinterpret_cast<const uint2*>(g.x + i);
      const float sc = g.xs[static_cast<int64_t>(t) * (d / 128) + (c * 8) / 128];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xv[q] = e4m3_to_f32((codes.x >> (8 * q)) & 0xFFu) * sc;
        xv[4 + q] = e4m3_to_f32((codes.y >> (8 * q)) & 0xFFu) * sc;
      }
    }
    if (g.vec_f32)
      load8<kRowF32>(g.vec + c * 32, gv);
    else
      load8<kRowBF16>(g.vec + c * 16, gv);
#pragma unroll
    for (int q = 0; q < 8; ++q) z = fmaf(xv[q], gv[q], z);
  }
  z = wave_sum(z);
  if (lane_id() == 0) part[threadIdx.x / kWave] = z;
  __syncthreads();
  z = 0.0f;
  for (int q = 0; q < static_cast<int>(blockDim.x) / kWave; ++q) z += part[q];
  return 1.0f / (1.0f + expf(-z));
}

// YK: y's RowKind; the shared output is fp32 under fp32 or fp16 rows, bf16 under bf16 rows.
template <int YK, bool OUT_F32>
__global__ __launch_bounds__(kCombineMaxThreads) void combine_kernel(
    const uint8_t* __restrict__ y, const int32_t* __restrict__ inv, const float* __restrict__ w,
    int k, const uint8_t* __restrict__ base, CombineGate gate, uint8_t* __restrict__ out, int d) {
  constexpr int BK = YK == kRowBF16 ? kRowBF16 : kRowF32;
  constexpr int ysz = YK == kRowF32 ? 4 : 2, bsz = BK == kRowF32 ? 4 : 2, osz = OUT_F32 ? 4 : 2;
  constexpr bool kNtY = YK != kRowF32;       // non-temporal y loads (see load8)
  constexpr bool kNtS = BK == kRowBF16;      // and shared-output loads
  __shared__ int32_t s_row[kCombineMaxK];
  __shared__ float s_w[kCombineMaxK];
  const int t = blockIdx.x;
  const int kp = (k + kCombineBatch - 1) / kCombineBatch * kCombineBatch;
  if (static_cast<int>(threadIdx.x) < kp) {
    const int j = threadIdx.x;
    const int64_t at = static_cast<int64_t>(t) * k + (j < k ? j : k - 1);
    s_row[j] = inv[at];
    s_w[j] = j < k ? w[at] : 0.0f;
  }
  const float G = gate.vec ? shared_gate(gate, t, d) : 1.0f;  // uniform branch
  __syncthreads();
  const int64_t ldy = static_cast<int64_t>(d) * ysz;
  for (int c = threadIdx.x; c < d / 8; c += blockDim.x) {
    float v[8];
    if (base) {
      // the shared output, read once as well: non-temporal when it is bf16 (FP8 experts), as
      // measured above
      load8<BK, kNtS>(base + (static_cast<int64_t>(t) * d + c * 8) * bsz, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] *= G;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = 0.0f;
    }
    const uint8_t* yc = y + c * 8 * ysz;
    for (int j0 = 0; j0 < kp; j0 += kCombineBatch) {
      float yv[kCombineBatch][8];
#pragma unroll
      for (int u = 0; u < kCombineBatch; ++u)
        load8<YK, kNtY>(yc + s_row[j0 + u] * ldy, yv[u]);
#pragma unroll
      for (int u = 0; u < kCombineBatch; ++u) {
        const float wj = s_w[j0 + u];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = fmaf(wj, yv[u][q], v[q]);
      }
    }
    uint8_t* dst = out + (static_cast<int64_t>(t) * d + c * 8) * osz;
    if constexpr (OUT_F32) {
      reinterpret_cast<f32x4*>(dst)[0] = f32x4{v[0], v[1], v[2], v[3]};
      reinterpret_cast<f32x4*>(dst)[1] = f32x4{v[4], v[5], v[6], v[7]};
    } else {
      i32x4 pk;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        pk[q] = static_cast<int>(f32_to_bf16(v[2 * q]) |
                                 (static_cast<uint32_t>(f32_to_bf16(v[2 * q + 1])) << 16));
      *reinterpret_cast<i32x4*>(dst) = pk;
    }
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const uint8_t* yb = static_cast<const uint8_t*>(a.y);
  uint8_t* ob = static_cast<uint8_t*>(a.out);
  const uint8_t* bb = static_cast<const uint8_t*>(a.base);
  CombineGate g{};
  if (a.gate_vec && a.base) {
    if (!a.x || a.x_kind < 0 || a.x_kind > 2 || (a.x_kind == 2 && !a.x_scales))
      return hipErrorInvalidValue;
    g.vec = static_cast<const uint8_t*>(a.gate_vec);
    g.x = static_cast<const uint8_t*>(a.x);
    g.xs = a.x_scales;
    g.vec_f32 = a.gate_f32;
    g.x_kind = a.x_kind;
  }
  if (a.k < 1 || a.k > kCombineMaxK || a.d % 8) return hipErrorInvalidValue;
  // one thread per 8-column chunk (whole waves), at most kCombineMaxThreads
  const int chunks = (a.d / 8 + kWave - 1) / kWave * kWave;
  const dim3 grid(a.T), block(chunks < kCombineMaxThreads ? chunks : kCombineMaxThreads);
  // the shared output's element type follows y's (see combine_kernel)
  const int bk = a.y_kind == kRowBF16 ? kRowBF16 : kRowF32;
  if (a.y_kind < kRowBF16 || a.y_kind > kRowF16 || (a.base && a.base_kind != bk))
    return hipErrorInvalidValue;
  auto go = [&](auto yk, auto of) {
    hipLaunchKernelGGL((combine_kernel<decltype(yk)::value, decltype(of)::value>), grid, block,
                       0, s, yb, a.inv, a.w, a.k, bb, g, ob, a.d);
  };
  using F32 = std::integral_constant<int, kRowF32>;
  using F16 = std::integral_constant<int, kRowF16>;
  using BF16 = std::integral_constant<int, kRowBF16>;
  using Yes = std::true_type;
  using No = std::false_type;
  switch (a.y_kind) {
    case kRowF32: a.out_f32 ? go(F32{}, Yes{}) : go(F32{}, No{}); break;
    case kRowF16: a.out_f32 ? go(F16{}, Yes{}) : go(F16{}, No{}); break;
    default: a.out_f32 ? go(BF16{}, Yes{}) : go(BF16{}, No{}); break;
  }
  return hipGetLastError();
}

}  // namespace moe
