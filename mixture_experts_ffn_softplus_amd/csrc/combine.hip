// combine.hip -- un-permute and weighted sum of the routed expert rows, plus the shared experts.
//
// out[t] = shared[t] + sum_j w[t, j] * y_perm[inv_perm[t * k + j]]: the routed experts' outputs
// weighted by the router and added to the always-active shared experts' output (routed-experts
// and shared-expert rows of "Qwen3.5-397B-A17B vs Gemma 4 31B"; the block's equation of the
// DeepSeek-V4 blueprint).  Pure streaming: one workgroup per token, each thread owning
// 8-column chunks and keeping up to eight row loads of y in flight.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

constexpr int kCombineThreads = 256;
constexpr int kCombineBatch = 8;  // y rows loaded together

template <bool Y_F32, bool OUT_F32>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const uint8_t* __restrict__ y, const int32_t* __restrict__ inv, const float* __restrict__ w,
    int k, const float* __restrict__ base, uint8_t* __restrict__ out, int d) {
  constexpr int ysz = Y_F32 ? 4 : 2, osz = OUT_F32 ? 4 : 2;
  const int t = blockIdx.x;
  const int64_t ldy = static_cast<int64_t>(d) * ysz;
  const int32_t* rows = inv + static_cast<int64_t>(t) * k;
  const float* wt = w + static_cast<int64_t>(t) * k;
  for (int c = threadIdx.x; c < d / 8; c += kCombineThreads) {
    float v[8];
    if (base) {
      const f32x4* b = reinterpret_cast<const f32x4*>(base + static_cast<int64_t>(t) * d + c * 8);
      const f32x4 b0 = b[0], b1 = b[1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = b0[q];
        v[4 + q] = b1[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = 0.0f;
    }
    for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
      i32x4 raw[kCombineBatch][Y_F32 ? 2 : 1];
      float wj[kCombineBatch];
#pragma unroll
      for (int u = 0; u < kCombineBatch; ++u) {
        wj[u] = 0.0f;
        raw[u][0] = i32x4{0, 0, 0, 0};
        if constexpr (Y_F32) raw[u][Y_F32 ? 1 : 0] = i32x4{0, 0, 0, 0};
        if (j0 + u < k) {  // uniform: k is the same for the whole grid
          wj[u] = wt[j0 + u];
          const i32x4* src = reinterpret_cast<const i32x4*>(y + rows[j0 + u] * ldy + c * 8 * ysz);
          raw[u][0] = src[0];
          if constexpr (Y_F32) raw[u][Y_F32 ? 1 : 0] = src[1];
        }
      }
#pragma unroll
      for (int u = 0; u < kCombineBatch; ++u) {
        if constexpr (Y_F32) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[q] = fmaf(wj[u], __int_as_float(raw[u][0][q]), v[q]);
            v[4 + q] = fmaf(wj[u], __int_as_float(raw[u][Y_F32 ? 1 : 0][q]), v[4 + q]);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t bits = static_cast<uint32_t>(raw[u][0][q]);
            v[2 * q] = fmaf(wj[u], __uint_as_float(bits << 16), v[2 * q]);
            v[2 * q + 1] = fmaf(wj[u], __uint_as_float(bits & 0xFFFF0000u), v[2 * q + 1]);
          }
        }
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

hipError_t launch_combine(const void* y, bool y_f32, const int32_t* inv, const float* w, int k,
                          const float* base, void* out, bool out_f32, int T, int d,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  const uint8_t* yb = static_cast<const uint8_t*>(y);
  uint8_t* ob = static_cast<uint8_t*>(out);
  const dim3 grid(T), block(kCombineThreads);
  if (y_f32 && out_f32)
    hipLaunchKernelGGL((combine_kernel<true, true>), grid, block, 0, s, yb, inv, w, k, base, ob, d);
  else if (y_f32)
    hipLaunchKernelGGL((combine_kernel<true, false>), grid, block, 0, s, yb, inv, w, k, base, ob, d);
  else if (out_f32)
    hipLaunchKernelGGL((combine_kernel<false, true>), grid, block, 0, s, yb, inv, w, k, base, ob, d);
  else
    hipLaunchKernelGGL((combine_kernel<false, false>), grid, block, 0, s, yb, inv, w, k, base, ob, d);
  return hipGetLastError();
}

}  // namespace moe
