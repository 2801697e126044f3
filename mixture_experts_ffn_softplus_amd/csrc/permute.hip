// permute.hip -- (token, slot) assignments into expert-contiguous order, stable in token order.
//
// The pages select routed experts per token (the k largest, router row of
// "Qwen3.5-397B-A17B vs DeepSeek-V4-Pro"), which the grouped expert GEMMs need as contiguous
// per-expert row ranges.  A counting sort, deterministic by construction, over chunks of 256
// consecutive assignments:
//   1. per-chunk expert histograms, stored expert-major (LDS atomics only count; they decide
//      no order),
//   2. one workgroup per expert scans its counts over the chunks (each chunk's first row
//      within the expert), then one workgroup scans the expert totals (expert_offsets),
//   3. per chunk, each of 4 waves ranks its 64 assignments among equal experts in lower lanes
//      with ballots; the waves' per-expert counts, summed in lane order through LDS, place
//      every assignment, and token ids are scattered to their rows.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

constexpr int kChunk = 256;  // assignments per chunk = 4 waves x 64 lanes

int permute_num_chunks(int T, int k) {
  int64_t A = static_cast<int64_t>(T) * k;
  return static_cast<int>((A + kChunk - 1) / kChunk);
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

// hist[e][c]: assignments of chunk c routed to expert e.
__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ ids, int64_t A,
                                                   int chunks, int E, int32_t* __restrict__ hist) {
  extern __shared__ int s_hist[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_hist[e] = 0;
  __syncthreads();
  const int64_t a = static_cast<int64_t>(blockIdx.x) * kChunk + threadIdx.x;
  if (a < A) atomicAdd(&s_hist[ids[a]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    hist[static_cast<size_t>(e) * chunks + blockIdx.x] = s_hist[e];
}

// One workgroup per expert: hist[e][c] -> first row of chunk c within expert e's rows;
// counts[e] = expert e's total.
__global__ __launch_bounds__(256) void scan_chunks_kernel(int32_t* __restrict__ hist, int chunks,
                                                          int32_t* __restrict__ counts) {
  __shared__ int s_tot[kWave + 1];
  int32_t* h = hist + static_cast<size_t>(blockIdx.x) * chunks;
  const int per = (chunks + blockDim.x - 1) / blockDim.x;
  const int c0 = threadIdx.x * per, c1 = min(c0 + per, chunks);
  int sum = 0;
  for (int c = c0; c < c1; ++c) sum += h[c];
  int total;
  int run = block_exclusive_scan(sum, s_tot, &total);
  for (int c = c0; c < c1; ++c) {
    int v = h[c];
    h[c] = run;
    run += v;
  }
  if (threadIdx.x == 0) counts[blockIdx.x] = total;
}

__global__ __launch_bounds__(1024) void offsets_kernel(const int32_t* __restrict__ counts, int E,
                                                       int64_t A, int32_t* __restrict__ offsets) {
  __shared__ int s_tot[kWave + 1];
  const int e = threadIdx.x;
  int total;
  int off = block_exclusive_scan(e < E ? counts[e] : 0, s_tot, &total);
  if (e < E) offsets[e] = off;
  if (e == 0) offsets[E] = static_cast<int32_t>(A);
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ ids, int64_t A,
                                                      int k, int E, int chunks,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ hist,
                                                      int32_t* __restrict__ perm_token,
                                                      int32_t* __restrict__ inv_perm) {
  extern __shared__ int sm[];
  int* s_base = sm;          // [E] first row of this chunk's assignments to each expert
  int* s_cnt = sm + E;       // [4][E] per-wave counts
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    s_base[e] = offsets[e] + hist[static_cast<size_t>(e) * chunks + c];
#pragma unroll
    for (int w = 0; w < 4; ++w) s_cnt[w * E + e] = 0;
  }
  __syncthreads();
  const int l = lane_id(), wv = threadIdx.x / kWave;
  const uint64_t lt_mask = (l == 0) ? 0ull : (~0ull >> (kWave - l));
  const int64_t a = static_cast<int64_t>(c) * kChunk + threadIdx.x;
  const bool valid = a < A;
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
  const int rank = __popcll(peers & lt_mask);
  const int cnt = __popcll(peers);
  if (valid && rank == cnt - 1) s_cnt[wv * E + e] = cnt;
  __syncthreads();
  if (valid) {
    int pos = s_base[e] + rank;
    for (int w = 0; w < wv; ++w) pos += s_cnt[w * E + e];
    perm_token[pos] = static_cast<int32_t>(a / k);
    inv_perm[a] = pos;
  }
}

// Device tile list of a grouped GEMM with row tile `bm`: tiles[i] = {group, first row,
// rows | (index of the tile within its group << 8), row tiles of that group},
// groups in order, tiles of a group in row order; tiles_count[0] = number of tiles.  The
// GEMM grid is sized for the worst case (ceil(T*k/bm) + E tiles, plus the extra group's) and
// reads the real count, so per-expert counts never travel to the host.  extra_rows > 0 adds
// group E over rows [offsets[E], offsets[E] + extra_rows).  Run by one whole workgroup;
// `offsets` [E+1] may live in global memory or in LDS.
__device__ void build_tile_list(const int32_t* offsets, int E, int bm, int extra_rows,
                                int4* __restrict__ tiles, int32_t* __restrict__ tiles_count) {
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
      // z: rows | index of the tile within its expert << 8;  w: tiles of expert e
      tiles[first + i] = int4{e, m0, min(bm, r0 + n - m0) | (i << 8), nt};
    }
    carry += chunk_total;
  }
  total = carry;
  const int nt2 = (extra_rows + bm - 1) / bm;
  const int r2 = offsets[E];
  for (int i = threadIdx.x; i < nt2; i += blockDim.x) {
    const int m0 = r2 + i * bm;
    tiles[total + i] = int4{E, m0, min(bm, r2 + extra_rows - m0) | (i << 8), nt2};
  }
  if (threadIdx.x == 0) tiles_count[0] = total + nt2;
}

__global__ __launch_bounds__(1024) void tile_list_kernel(const int32_t* __restrict__ offsets,
                                                         int E, int bm, int extra_rows,
                                                         int4* __restrict__ tiles,
                                                         int32_t* __restrict__ tiles_count) {
  build_tile_list(offsets, E, bm, extra_rows, tiles, tiles_count);
}

// The whole permutation in one workgroup for small batches (A <= kSmallA assignments,
// E <= kSmallE experts; decode shapes), and the tile list with it: the same stable counting
// sort as the multi-kernel path, one round of 1024 assignments at a time -- each wave ranks its
// 64 assignments among equal experts in lower lanes with ballots, the waves' per-expert counts
// (summed in wave order through LDS) and the experts' counts of the earlier rounds place every
// assignment.  No atomics decide any order.
constexpr int kSmallThreads = 1024, kSmallWaves = kSmallThreads / kWave;
constexpr int kSmallRounds = 4, kSmallA = kSmallThreads * kSmallRounds, kSmallE = 768;
__global__ __launch_bounds__(kSmallThreads) void permute_small_kernel(
    const int32_t* __restrict__ ids, int A, int k, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm_token, int32_t* __restrict__ inv_perm, int bm, int extra_rows,
    int4* __restrict__ tiles, int32_t* __restrict__ tiles_count) {
  extern __shared__ int sm[];
  int* s_run = sm;                       // [E] assignments to each expert so far
  int* s_off = sm + E;                   // [E + 1] expert offsets
  int* s_wave = sm + 2 * E + 1;          // [kSmallWaves][E] this round's per-wave counts
  __shared__ int s_tot[kWave + 1];
  const int tid = threadIdx.x, l = lane_id(), wv = tid / kWave;
  const uint64_t lt_mask = (l == 0) ? 0ull : (~0ull >> (kWave - l));
  for (int e = tid; e < E; e += kSmallThreads) s_run[e] = 0;
  int my_e[kSmallRounds], my_rank[kSmallRounds];
#pragma unroll
  for (int r = 0; r < kSmallRounds; ++r) {
    my_e[r] = -1;
    my_rank[r] = 0;
    if (r * kSmallThreads >= A) continue;  // uniform
    for (int i = tid; i < kSmallWaves * E; i += kSmallThreads) s_wave[i] = 0;
    __syncthreads();
    const int a = r * kSmallThreads + tid;
    const bool valid = a < A;
    const int e = valid ? ids[a] : -1;
    uint64_t remaining = __ballot(valid);
    uint64_t peers = 0;
    while (remaining) {
      const int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
      const int le = __shfl(e, leader, kWave);
      const uint64_t m = __ballot(valid && e == le);
      if (valid && e == le) peers = m;
      remaining &= ~m;
    }
    const int rank = __popcll(peers & lt_mask), cnt = __popcll(peers);
    if (valid && rank == cnt - 1) s_wave[wv * E + e] = cnt;
    __syncthreads();
    if (valid) {
      int pos = s_run[e] + rank;
      for (int w = 0; w < wv; ++w) pos += s_wave[w * E + e];
      my_e[r] = e;
      my_rank[r] = pos;
    }
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += kSmallThreads) {
      int sum = 0;
      for (int w = 0; w < kSmallWaves; ++w) sum += s_wave[w * E + e2];
      s_run[e2] += sum;
    }
    __syncthreads();
  }
  // expert offsets: exclusive scan of the counts (E <= kSmallThreads: one pass)
  int total;
  const int off = block_exclusive_scan(tid < E ? s_run[tid] : 0, s_tot, &total);
  if (tid < E) {
    offsets[tid] = off;
    s_off[tid] = off;
  }
  if (tid == 0) {
    offsets[E] = A;
    s_off[E] = A;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kSmallRounds; ++r) {
    if (my_e[r] >= 0) {
      const int a = r * kSmallThreads + tid;
      const int pos = s_off[my_e[r]] + my_rank[r];
      perm_token[pos] = a / k;
      inv_perm[a] = pos;
    }
  }
  if (tiles) build_tile_list(s_off, E, bm, extra_rows, tiles, tiles_count);
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// hist: workspace of (chunks + 1) * E ints (histograms, then the per-expert totals).
hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                          int32_t* perm_token, int32_t* inv_perm, int32_t* hist,
                          hipStream_t s) {
  const int64_t A = static_cast<int64_t>(T) * k;
  if (A == 0) {  // no assignments: every offset is 0
    hipLaunchKernelGGL(fill_i32_kernel, dim3((E + 1 + 255) / 256), dim3(256), 0, s, offsets,
                       E + 1, 0);
    return hipGetLastError();
  }
  const int chunks = static_cast<int>((A + kChunk - 1) / kChunk);
  int32_t* counts = hist + static_cast<size_t>(chunks) * E;
  hipLaunchKernelGGL(hist_kernel, dim3(chunks), dim3(kChunk), sizeof(int) * E, s, ids, A, chunks,
                     E, hist);
  hipLaunchKernelGGL(scan_chunks_kernel, dim3(E), dim3(256), 0, s, hist, chunks, counts);
  hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(1024), 0, s, counts, E, A, offsets);
  hipLaunchKernelGGL(scatter_kernel, dim3(chunks), dim3(kChunk), sizeof(int) * 5 * E, s, ids, A,
                     k, E, chunks, offsets, hist, perm_token, inv_perm);
  return hipGetLastError();
}

bool permute_small_ok(int64_t A, int E) { return A >= 1 && A <= kSmallA && E <= kSmallE; }

hipError_t launch_permute_small(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                                int32_t* perm_token, int32_t* inv_perm, int bm, int extra_rows,
                                int4* tiles, int32_t* tiles_count, hipStream_t s) {
  const int64_t A = static_cast<int64_t>(T) * k;
  if (!permute_small_ok(A, E)) return hipErrorInvalidValue;
  const size_t lds = sizeof(int) * (2 * E + 1 + kSmallWaves * E);
  hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kSmallThreads), lds, s, ids,
                     static_cast<int>(A), k, E, offsets, perm_token, inv_perm, bm, extra_rows,
                     tiles, tiles_count);
  return hipGetLastError();
}

hipError_t launch_tile_list(const int32_t* offsets, int E, int bm, int extra_rows, int4* tiles,
                            int32_t* tiles_count, hipStream_t s) {
  hipLaunchKernelGGL(tile_list_kernel, dim3(1), dim3(1024), 0, s, offsets, E, bm, extra_rows,
                     tiles, tiles_count);
  return hipGetLastError();
}

}  // namespace moe
