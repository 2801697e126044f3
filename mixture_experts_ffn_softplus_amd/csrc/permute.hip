// permute.hip -- (token, slot) assignments into expert-contiguous order, stable in token order.
//
// The pages select routed experts per token ("keep the top 10", router row of
// "Qwen3.5-397B-A17B vs DeepSeek-V4-Pro"), which the grouped expert GEMMs need as contiguous
// per-expert row ranges.  A counting sort, deterministic by construction:
//   1. per-chunk expert histograms (LDS atomics only count; they decide no order),
//   2. one workgroup scans each expert's counts over the chunks, then over the experts
//      (expert_offsets), leaving every chunk's base row per expert,
//   3. one wave per chunk walks its assignments in order, 64 at a time, ranking equal
//      experts among lower lanes with ballots, and scatters token ids to their rows.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

constexpr int kMaxChunks = 512;

static int chunk_size(int64_t A) {
  int64_t chunks = (A + 255) / 256;
  if (chunks > kMaxChunks) chunks = kMaxChunks;
  if (chunks < 1) chunks = 1;
  int64_t cs = (A + chunks - 1) / chunks;
  cs = (cs + 63) / 64 * 64;
  return static_cast<int>(cs < 64 ? 64 : cs);
}

int permute_num_chunks(int T, int k) {
  int64_t A = static_cast<int64_t>(T) * k;
  int cs = chunk_size(A);
  return static_cast<int>((A + cs - 1) / cs);
}

// Exclusive scan of one value per thread over a block of up to 1024 threads.
__device__ int block_exclusive_scan(int v, int* s_tot, int* total) {
  const int l = lane_id(), w = threadIdx.x / kWave, nw = (blockDim.x + kWave - 1) / kWave;
  int inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int u = __shfl_up(inc, o, kWave);
    if (l >= o) inc += u;
  }
  if (l == kWave - 1) s_tot[w] = inc;
  __syncthreads();
  if (w == 0) {
    int t = l < nw ? s_tot[l] : 0;
    int ti = t;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      int u = __shfl_up(ti, o, kWave);
      if (l >= o) ti += u;
    }
    if (l < nw) s_tot[l] = ti - t;  // exclusive wave bases
    if (l == nw - 1) s_tot[kWave] = ti;
  }
  __syncthreads();
  int r = s_tot[w] + inc - v;
  *total = s_tot[kWave];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ ids, int64_t A,
                                                   int cs, int E, int32_t* __restrict__ hist) {
  extern __shared__ int s_hist[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_hist[e] = 0;
  __syncthreads();
  const int64_t a0 = static_cast<int64_t>(blockIdx.x) * cs;
  const int64_t a1 = min(a0 + cs, A);
  for (int64_t a = a0 + threadIdx.x; a < a1; a += blockDim.x) atomicAdd(&s_hist[ids[a]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    hist[static_cast<size_t>(blockIdx.x) * E + e] = s_hist[e];
}

// hist[c][e] (counts) -> hist[c][e] = first row of chunk c's assignments to expert e.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ hist, int chunks,
                                                    int E, int64_t A,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int s_tot[kWave + 1];
  const int e = threadIdx.x;
  int count = 0;
  if (e < E) {
    for (int c = 0; c < chunks; ++c) {
      int v = hist[static_cast<size_t>(c) * E + e];
      hist[static_cast<size_t>(c) * E + e] = count;
      count += v;
    }
  }
  int total;
  int off = block_exclusive_scan(e < E ? count : 0, s_tot, &total);
  if (e < E) {
    offsets[e] = off;
    for (int c = 0; c < chunks; ++c) hist[static_cast<size_t>(c) * E + e] += off;
  }
  if (e == 0) offsets[E] = static_cast<int32_t>(A);
}

__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ ids, int64_t A,
                                                     int cs, int k, int E,
                                                     const int32_t* __restrict__ base,
                                                     int32_t* __restrict__ perm_token,
                                                     int32_t* __restrict__ inv_perm) {
  extern __shared__ int s_base[];
  for (int e = threadIdx.x; e < E; e += kWave)
    s_base[e] = base[static_cast<size_t>(blockIdx.x) * E + e];
  __syncthreads();
  const int l = lane_id();
  const uint64_t lt_mask = (l == 0) ? 0ull : (~0ull >> (kWave - l));
  const int64_t a0 = static_cast<int64_t>(blockIdx.x) * cs;
  const int64_t a1 = min(a0 + cs, A);
  for (int64_t s = a0; s < a1; s += kWave) {
    const int64_t a = s + l;
    const bool valid = a < a1;
    const int e = valid ? ids[a] : -1;
    uint64_t remaining = __ballot(valid);
    uint64_t peers = 0;
    while (remaining) {
      int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
      int le = __shfl(e, leader, kWave);
      uint64_t m = __ballot(valid && e == le);
      if (valid && e == le) peers = m;
      remaining &= ~m;
    }
    if (valid) {
      int rank = __popcll(peers & lt_mask);
      int cnt = __popcll(peers);
      int pos = s_base[e] + rank;
      perm_token[pos] = static_cast<int32_t>(a / k);
      inv_perm[a] = pos;
      if (rank == cnt - 1) s_base[e] += cnt;
    }
    __syncthreads();
  }
}

// Device tile list of a grouped GEMM with row tile `bm`: tiles[i] = {group, first row, rows},
// groups in order, tiles of a group in row order; tiles_count[0] = number of tiles.  The
// GEMM grid is sized for the worst case (ceil(T*k/bm) + E tiles) and reads the real count,
// so per-expert counts never travel to the host.
__global__ __launch_bounds__(1024) void tile_list_kernel(const int32_t* __restrict__ offsets,
                                                         int E, int bm, int4* __restrict__ tiles,
                                                         int32_t* __restrict__ tiles_count) {
  __shared__ int s_tot[kWave + 1];
  int total = 0;
  int carry = 0;
  for (int e0 = 0; e0 < E; e0 += blockDim.x) {
    const int e = e0 + threadIdx.x;
    int r0 = 0, n = 0;
    if (e < E) {
      r0 = offsets[e];
      n = offsets[e + 1] - r0;
    }
    const int nt = (n + bm - 1) / bm;
    int chunk_total;
    const int first = carry + block_exclusive_scan(nt, s_tot, &chunk_total);
    for (int i = 0; i < nt; ++i) {
      int m0 = r0 + i * bm;
      tiles[first + i] = int4{e, m0, min(bm, r0 + n - m0), 0};
    }
    carry += chunk_total;
  }
  total = carry;
  if (threadIdx.x == 0) tiles_count[0] = total;
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                          int32_t* perm_token, int32_t* inv_perm, int32_t* hist,
                          hipStream_t s) {
  const int64_t A = static_cast<int64_t>(T) * k;
  if (A == 0) {  // no assignments: every offset is 0
    hipLaunchKernelGGL(fill_i32_kernel, dim3((E + 1 + 255) / 256), dim3(256), 0, s, offsets,
                       E + 1, 0);
    return hipGetLastError();
  }
  const int cs = chunk_size(A);
  const int chunks = static_cast<int>((A + cs - 1) / cs);
  hipLaunchKernelGGL(hist_kernel, dim3(chunks), dim3(256), sizeof(int) * E, s, ids, A, cs, E,
                     hist);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, hist, chunks, E, A, offsets);
  hipLaunchKernelGGL(scatter_kernel, dim3(chunks), dim3(64), sizeof(int) * E, s, ids, A, cs, k,
                     E, hist, perm_token, inv_perm);
  return hipGetLastError();
}

hipError_t launch_tile_list(const int32_t* offsets, int E, int bm, int4* tiles,
                            int32_t* tiles_count, hipStream_t s) {
  hipLaunchKernelGGL(tile_list_kernel, dim3(1), dim3(1024), 0, s, offsets, E, bm, tiles,
                     tiles_count);
  return hipGetLastError();
}

}  // namespace moe
