// pack.hip -- one-time rewrite of logical weights into the layouts the kernels stream.
//
// Pure data movement, run outside any timed region.  Expert matrices become K-contiguous
// ([N, K], the reduction axis innermost) so that every MFMA operand fetch is a 16-byte
// row segment; gate and up are interleaved in blocks of 16 rows so one output tile holds
// matching gate and up columns.  Tiles of 64 x 64 elements go through LDS so that both
// the reads and the writes run along contiguous rows.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

template <typename T>
__global__ __launch_bounds__(256) void pack_gate_up_kernel(const T* __restrict__ gate,
                                                           const T* __restrict__ up,
                                                           T* __restrict__ dst, int K, int C,
                                                           int sub) {
  __shared__ T tile[64][65];
  const int F = sub * C;
  const int k0 = blockIdx.x * 64, p0 = blockIdx.y * 64, g = blockIdx.z;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  {
    const int p = p0 + tx;
    const int blk = p >> 4, j = p & 15;
    const int col = (blk >> 1) * 16 + j;  // column of the concatenated [K, F] matrix
    const int sidx = col / C, c = col - sidx * C;
    const T* src = ((blk & 1) ? up : gate) + (static_cast<size_t>(g) * sub + sidx) * K * C;
    for (int kk = ty; kk < 64; kk += 4) tile[kk][tx] = src[static_cast<size_t>(k0 + kk) * C + c];
  }
  __syncthreads();
  T* d = dst + static_cast<size_t>(g) * 2 * F * K;
  for (int pp = ty; pp < 64; pp += 4) d[static_cast<size_t>(p0 + pp) * K + k0 + tx] = tile[tx][pp];
}

template <typename T>
__global__ __launch_bounds__(256) void pack_down_kernel(const T* __restrict__ down,
                                                        T* __restrict__ dst, int N, int C,
                                                        int sub) {
  __shared__ T tile[64][65];
  const int F = sub * C;
  const int f0 = blockIdx.x * 64, n0 = blockIdx.y * 64, g = blockIdx.z;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int ff = ty; ff < 64; ff += 4) {
    const int f = f0 + ff;
    const int sidx = f / C, c = f - sidx * C;
    const T* src = down + (static_cast<size_t>(g) * sub + sidx) * C * N;
    tile[ff][tx] = src[static_cast<size_t>(c) * N + n0 + tx];
  }
  __syncthreads();
  T* d = dst + static_cast<size_t>(g) * N * F;
  for (int nn = ty; nn < 64; nn += 4) d[static_cast<size_t>(n0 + nn) * F + f0 + tx] = tile[tx][nn];
}

// Router [d, E] -> [E_pad, d] K-contiguous, rows >= E zero.  HILO: an fp32 router is split
// into bf16 hi = bf16(w) and lo = bf16(w - hi), stored side by side as one [E_pad, 2d] bf16
// matrix that the GEMM multiplies by [x, x].
template <typename T, bool HILO>
__global__ __launch_bounds__(256) void pack_router_kernel(const T* __restrict__ wr,
                                                          uint8_t* __restrict__ dst, int d,
                                                          int E, int E_pad) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(E_pad) * d) return;
  const int e = static_cast<int>(i / d), k = static_cast<int>(i - static_cast<int64_t>(e) * d);
  T v = e < E ? wr[static_cast<size_t>(k) * E + e] : T(0);
  if constexpr (HILO) {
    float w = static_cast<float>(v);
    uint16_t hi = f32_to_bf16(w);
    uint16_t lo = f32_to_bf16(w - bf16_to_f32(hi));
    uint16_t* row = reinterpret_cast<uint16_t*>(dst) + static_cast<int64_t>(e) * 2 * d;
    row[k] = hi;
    row[d + k] = lo;
  } else {
    reinterpret_cast<T*>(dst)[i] = v;
  }
}

__global__ void pack_scales_gate_up_kernel(const float* __restrict__ gs,
                                           const float* __restrict__ us, float* __restrict__ dst,
                                           int K, int C, int sub, int groups) {
  const int KB = K / 128, CB = C / 128, F = sub * C;
  const int64_t total = static_cast<int64_t>(groups) * (2 * F / 16) * KB;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int kb = static_cast<int>(i % KB);
  const int64_t r = i / KB;
  const int blk = static_cast<int>(r % (2 * F / 16));
  const int g = static_cast<int>(r / (2 * F / 16));
  const int col = (blk >> 1) * 16;
  const int sidx = col / C, cb = (col - sidx * C) / 128;
  const float* src = ((blk & 1) ? us : gs) + (static_cast<size_t>(g) * sub + sidx) * KB * CB;
  dst[i] = src[kb * CB + cb];
}

__global__ void pack_scales_down_kernel(const float* __restrict__ ds, float* __restrict__ dst,
                                        int N, int C, int sub, int groups) {
  const int F = sub * C, KB = F / 128, NB = N / 128, CB = C / 128;
  const int64_t total = static_cast<int64_t>(groups) * (N / 16) * KB;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int kb = static_cast<int>(i % KB);
  const int64_t r = i / KB;
  const int n16 = static_cast<int>(r % (N / 16));
  const int g = static_cast<int>(r / (N / 16));
  const int f = kb * 128;
  const int sidx = f / C, cb = (f - sidx * C) / 128;
  const float* src = ds + (static_cast<size_t>(g) * sub + sidx) * CB * NB;
  dst[i] = src[cb * NB + (n16 * 16) / 128];
}

// Row-wise packing of N-major (MXFP4) operands, one dword per thread; rows are R bytes.
// Dword w of packed row n within a group of rows of W dwords: row-major (tile_rows 0), or by
// column tile and K-step of P dwords (16 for the E2M1 weights, 1 for the E8M0 scales) so that
// one step of a tile is contiguous.
__device__ __forceinline__ int64_t packed_dword(int64_t n, int64_t w, int64_t W, int tile_rows,
                                                int P) {
  if (tile_rows == 0) return n * W + w;
  return ((n / tile_rows) * (W / P) + w / P) * (tile_rows * P) + (n % tile_rows) * P + w % P;
}

// gate/up: packed row p of a group (2F rows, F = sub * C) is gate row n = 16 (p / 32) + p % 16
// when p % 32 < 16, else up row n, where row n of the group is row n % C of its source expert
// n / C.
__global__ __launch_bounds__(256) void pack_rows_gate_up_kernel(
    const uint32_t* __restrict__ gate, const uint32_t* __restrict__ up,
    uint32_t* __restrict__ dst, int C, int sub, int groups, int R4, int tile_rows, int P) {
  const int64_t F = static_cast<int64_t>(sub) * C;
  const int64_t total = static_cast<int64_t>(groups) * 2 * F * R4;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t w = i % R4, row = i / R4;
  const int64_t g = row / (2 * F), p = row % (2 * F);
  const int64_t n = 16 * (p / 32) + p % 16;
  const uint32_t* src = (p % 32) < 16 ? gate : up;
  dst[g * 2 * F * R4 + packed_dword(p, w, R4, tile_rows, P)] =
      src[((g * sub + n / C) * C + n % C) * R4 + w];
}

// down: packed row n of a group holds, for each source expert s, that expert's row n (R bytes)
// at byte s * R: the sources concatenate along K.
__global__ __launch_bounds__(256) void pack_rows_concat_kernel(const uint32_t* __restrict__ src,
                                                               uint32_t* __restrict__ dst, int N,
                                                               int sub, int groups, int R4,
                                                               int tile_rows, int P) {
  const int64_t total = static_cast<int64_t>(groups) * N * sub * R4;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t w = i % R4, rest = i / R4;
  const int64_t sidx = rest % sub, rest2 = rest / sub;
  const int64_t n = rest2 % N, g = rest2 / N;
  const int64_t W = static_cast<int64_t>(sub) * R4;
  dst[g * N * W + packed_dword(n, sidx * R4 + w, W, tile_rows, P)] =
      src[((g * sub + sidx) * N + n) * R4 + w];
}

hipError_t launch_pack_rows_gate_up(const void* gate, const void* up, void* dst, int C, int sub,
                                    int groups, int row_bytes, int tile_rows, int step_bytes,
                                    hipStream_t s) {
  if (row_bytes % 4 || step_bytes < 4 || step_bytes % 4) return hipErrorInvalidValue;
  if (tile_rows > 0 && ((2 * sub * C) % tile_rows || row_bytes % step_bytes))
    return hipErrorInvalidValue;
  const int64_t n = static_cast<int64_t>(groups) * 2 * sub * C * (row_bytes / 4);
  hipLaunchKernelGGL(pack_rows_gate_up_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                     dim3(256), 0, s, static_cast<const uint32_t*>(gate),
                     static_cast<const uint32_t*>(up), static_cast<uint32_t*>(dst), C, sub,
                     groups, row_bytes / 4, tile_rows, step_bytes / 4);
  return hipGetLastError();
}

hipError_t launch_pack_rows_concat(const void* src, void* dst, int N, int sub, int groups,
                                   int row_bytes, int tile_rows, int step_bytes, hipStream_t s) {
  if (row_bytes % 4 || step_bytes < 4 || step_bytes % 4) return hipErrorInvalidValue;
  if (tile_rows > 0 && (N % tile_rows || (sub * row_bytes) % step_bytes))
    return hipErrorInvalidValue;
  const int64_t n = static_cast<int64_t>(groups) * N * sub * (row_bytes / 4);
  hipLaunchKernelGGL(pack_rows_concat_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                     dim3(256), 0, s, static_cast<const uint32_t*>(src),
                     static_cast<uint32_t*>(dst), N, sub, groups, row_bytes / 4, tile_rows,
                     step_bytes / 4);
  return hipGetLastError();
}

hipError_t launch_pack_gate_up(const void* gate, const void* up, void* dst, int K, int C,
                               int sub, int groups, int esize, hipStream_t s) {
  dim3 grid(K / 64, (2 * sub * C) / 64, groups);
  if (esize == 4)
    hipLaunchKernelGGL(pack_gate_up_kernel<uint32_t>, grid, dim3(256), 0, s,
                       static_cast<const uint32_t*>(gate), static_cast<const uint32_t*>(up),
                       static_cast<uint32_t*>(dst), K, C, sub);
  else if (esize == 2)
    hipLaunchKernelGGL(pack_gate_up_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(gate), static_cast<const uint16_t*>(up),
                       static_cast<uint16_t*>(dst), K, C, sub);
  else
    hipLaunchKernelGGL(pack_gate_up_kernel<uint8_t>, grid, dim3(256), 0, s,
                       static_cast<const uint8_t*>(gate), static_cast<const uint8_t*>(up),
                       static_cast<uint8_t*>(dst), K, C, sub);
  return hipGetLastError();
}

hipError_t launch_pack_down(const void* down, void* dst, int N, int C, int sub, int groups,
                            int esize, hipStream_t s) {
  dim3 grid((sub * C) / 64, N / 64, groups);
  if (esize == 4)
    hipLaunchKernelGGL(pack_down_kernel<uint32_t>, grid, dim3(256), 0, s,
                       static_cast<const uint32_t*>(down), static_cast<uint32_t*>(dst), N, C, sub);
  else if (esize == 2)
    hipLaunchKernelGGL(pack_down_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(down), static_cast<uint16_t*>(dst), N, C, sub);
  else
    hipLaunchKernelGGL(pack_down_kernel<uint8_t>, grid, dim3(256), 0, s,
                       static_cast<const uint8_t*>(down), static_cast<uint8_t*>(dst), N, C, sub);
  return hipGetLastError();
}

hipError_t launch_pack_router(const void* wr, int esize, int hilo, void* dst, int d, int E,
                              int E_pad, hipStream_t s) {
  int64_t n = static_cast<int64_t>(E_pad) * d;
  dim3 grid(static_cast<unsigned>((n + 255) / 256));
  if (hilo)
    hipLaunchKernelGGL((pack_router_kernel<float, true>), grid, dim3(256), 0, s,
                       static_cast<const float*>(wr), static_cast<uint8_t*>(dst), d, E, E_pad);
  else if (esize == 4)
    hipLaunchKernelGGL((pack_router_kernel<float, false>), grid, dim3(256), 0, s,
                       static_cast<const float*>(wr), static_cast<uint8_t*>(dst), d, E, E_pad);
  else
    hipLaunchKernelGGL((pack_router_kernel<uint16_t, false>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(wr), static_cast<uint8_t*>(dst), d, E, E_pad);
  return hipGetLastError();
}

hipError_t launch_pack_scales_gate_up(const float* gs, const float* us, float* dst, int K, int C,
                                      int sub, int groups, hipStream_t s) {
  int64_t n = static_cast<int64_t>(groups) * (2 * sub * C / 16) * (K / 128);
  hipLaunchKernelGGL(pack_scales_gate_up_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                     dim3(256), 0, s, gs, us, dst, K, C, sub, groups);
  return hipGetLastError();
}

hipError_t launch_pack_scales_down(const float* ds, float* dst, int N, int C, int sub,
                                   int groups, hipStream_t s) {
  int64_t n = static_cast<int64_t>(groups) * (N / 16) * (sub * C / 128);
  hipLaunchKernelGGL(pack_scales_down_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                     dim3(256), 0, s, ds, dst, N, C, sub, groups);
  return hipGetLastError();
}

}  // namespace moe
