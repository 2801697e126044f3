// gemm.hip -- grouped expert GEMMs on gfx950 MFMA with fused epilogues.
//
// Computes, for every tile of rows of every group (expert), OUT = A_rows x B_group^T with B
// stored [N, K] K-contiguous (the packed weight layout), followed by one of:
//   kEpiSwiglu  -- h = SiLU(gate) * up: B interleaves gate and up columns in blocks of 16
//                  packed rows, so each wave's accumulators hold matching gate/up columns and
//                  h is formed in registers ("SwiGLU experts", routed-experts row of
//                  "Qwen3.5-397B-A17B vs Gemma 4 31B"); FP8 re-quantises h per 128 values;
//   kEpiStore   -- the down projection, rows stored as they are (y_perm);
//   kEpiCombine -- the shared experts' down projection plus the un-permute and weighted sum
//                  of the routed rows: out[t] = acc[t] + sum_j w[t,j] y[inv_perm[t*k+j]]
//                  (shared-expert row of the same page: the shared output is added to the
//                  routed sum).
//
// Structure.  4 or 8 waves per workgroup (each wave a 64 x 64 or smaller sub-tile), a BM x BN
// output tile, K consumed 128 bytes per step (64 bf16, 32 fp32 or 128 E4M3 values -- exactly
// one FP8 scale block).  Each step's A rows (gathered through a_map: no permuted copy of x is
// ever written) and B rows go straight from global memory into a three-slot LDS ring with
// buffer loads that write LDS directly, issued three steps ahead; their 16-byte chunks land
// XOR-swizzled by row so that the fragment reads of 16 consecutive rows hit distinct banks.
// Fragments of step s+1 are read from LDS while the MFMAs of step s run, one barrier per step.
// Weights of an expert whose rows fit one tile are loaded non-temporally (read once); others
// keep the default policy so the expert's other row tiles find them in L2.  Workgroups map to
// tiles through an XCD-aware remap so that neighbouring tiles (the N-tiles of one expert, which
// share its A rows) run in the same XCD's L2.  Grids are sized for the worst case and read the
// device tile count, so no per-expert count travels to the host.
#include <math.h>

#include <type_traits>

#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

template <int DT>
struct DT_ {};
template <>
struct DT_<MOE_F32> { static constexpr int esize = 4; };
template <>
struct DT_<MOE_BF16> { static constexpr int esize = 2; };
template <>
struct DT_<MOE_FP8_E4M3> { static constexpr int esize = 1; };

__device__ __forceinline__ int swz(int row, int ch) { return row * kBlockK + ((ch ^ (row & 7)) << 4); }

// NW waves per workgroup: 8 for the wide bf16 tiles (BN = 256, each wave still 64 x 64), else 4.
template <int DT, int BN>
constexpr int gemm_waves() { return (DT != MOE_F32 && BN >= 256) ? 8 : 4; }

template <int DT, int BM, int BN, int EPI>
struct GemmShape {
  static constexpr int NW = gemm_waves<DT, BN>();
  static constexpr int NT = NW * kWave;
  static constexpr int WM = BM >= 32 ? 2 : 1;
  static constexpr int WN = NW / WM;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 16, FN = TN / 16;
  static constexpr bool kFp8 = DT == MOE_FP8_E4M3;
  static constexpr int A_CHUNKS = BM * 8, B_CHUNKS = BN * 8;  // 16-byte chunks per step
  static constexpr int A_PER = (A_CHUNKS + NT - 1) / NT, B_PER = (B_CHUNKS + NT - 1) / NT;
  // LDS ring: step s multiplies out of slot s % 3 while steps s+1 and s+2 land in the others
  static constexpr int NSLOT = 3;
  static constexpr int STAGE = (BM + BN) * kBlockK;
  // FP8 scales per slot: BM row scales, 64 weight-block scales, 64 floats for idle waves
  static constexpr int SCALES = kFp8 ? (BM + 128) * 4 : 0;
  static constexpr int SLOT = STAGE + SCALES;
  static constexpr int DUMMY = NW * 1024;  // destination of the loads a wave issues for nothing
  static constexpr int MAIN = NSLOT * SLOT + DUMMY;
  // direct-to-LDS loads each wave issues per step (the same count in every wave)
  static constexpr int LPS = A_PER + B_PER + (kFp8 ? 1 : 0);
  static constexpr int EPI_BYTES =
      EPI == kEpiSwiglu ? BM * (BN / 2 + 4) * 4 : BM * (BN + 4) * 4;
  static constexpr int SMEM = MAIN > EPI_BYTES ? MAIN : EPI_BYTES;
  static_assert(FM >= 1 && FN >= 1, "tile too small for 4 waves");
  static_assert(!kFp8 || NW >= BM / 64 + 1, "FP8 scale loads need BM / 64 + 1 waves");
  static_assert(2 * LPS < 64, "vmcnt holds at most 63");
  static_assert(!kFp8 || (TN <= 128 && 128 % TN == 0), "FP8: two weight scales per wave");
  static_assert(EPI != kEpiSwiglu || FN % 2 == 0, "gate/up pairs must stay within one wave");
  static_assert(!(kFp8 && EPI == kEpiSwiglu) || BN == 256, "FP8 h groups need 128 h columns");
};

// Register fragments of one pipeline step: two 16x16x32 (bf16) or 16x16x4-by-4 (fp32) K-halves,
// or one 16x16x128 E4M3 block with its row scales and the wave's two weight-block scales.
template <int DT, int FM, int FN>
struct Frags {
  using V = typename std::conditional<DT == MOE_BF16, bf16x8, f32x4>::type;
  V a[2][FM], b[2][FN];
};
template <int FM, int FN>
struct Frags<MOE_FP8_E4M3, FM, FN> {
  i32x8 a[1][FM], b[1][FN];
  f32x4 sa[FM];
  float sb[2];
};

// Waves per SIMD the register allocation aims for: what the LDS footprint lets run (160 KiB
// per CU), capped at 2.
template <int DT, int BM, int BN, int EPI>
constexpr int gemm_occupancy() {
  using S = GemmShape<DT, BM, BN, EPI>;
  const int per_cu = (160 * 1024) / S::SMEM * S::NW / 4;
  return per_cu < 1 ? 1 : per_cu > 2 ? 2 : per_cu;
}

// GROUPED: rows come from the device tile list of an expert-grouped problem (the routed
// experts); otherwise one group of a.M rows (router, shared experts, combine).
template <int DT, int BM, int BN, int EPI, bool GROUPED>
__global__ __launch_bounds__((gemm_waves<DT, BN>() * kWave), (gemm_occupancy<DT, BM, BN, EPI>()))
void grouped_gemm_kernel(GemmArgs a) {
  using S = GemmShape<DT, BM, BN, EPI>;
  constexpr int esize = DT_<DT>::esize;
  constexpr int STAGE_BYTES = S::STAGE;
  __shared__ __attribute__((aligned(16))) uint8_t smem[S::SMEM];

  // ---------------------------------------------------------------- which tile
  const int NT = a.N / BN;
  const int ntiles = GROUPED ? a.tiles_count[0] : (a.M + BM - 1) / BM;
  const int nblocks = ntiles * NT;
  if (static_cast<int>(blockIdx.x) >= nblocks) return;
  const int L = xcd_remap(blockIdx.x, nblocks);
  const int tile = L / NT, nt = L - tile * NT;
  int group = 0, m0, rows;
  bool stream_b = false;
  if constexpr (GROUPED) {
    int4 ti = a.tiles[tile];
    group = ti.x;
    m0 = ti.y;
    rows = ti.z;
    stream_b = a.b_stream && ti.w == 1;  // no other row tile of this group reads these weights
  } else {
    m0 = tile * BM;
    rows = min(BM, a.M - m0);
  }
  const int n0 = nt * BN;

  const int tid = threadIdx.x, l = lane_id(), wv = uniform(tid / kWave);
  const int wm = wv / S::WN, wn = wv % S::WN;
  const int lr = l & 15, kq = l >> 4;
  const int KB = a.K * esize / kBlockK;  // pipeline steps
  const int64_t ldb = a.ldb;

  f32x4 acc[S::FM][S::FN];
#pragma unroll
  for (int i = 0; i < S::FM; ++i)
#pragma unroll
    for (int j = 0; j < S::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (KB > 0) {
    // ------------------------------------------------------------ direct-to-LDS loads
    // Every load writes 16 bytes per lane straight into LDS at (wave base + 16 * lane): the
    // lane-to-chunk map is chosen on the global side so that the tile lands in the swizzled
    // layout the fragment reads expect (row r's logical chunk c at slot r*8 + (c ^ (r & 7))).
    // No staging registers, no LDS store instructions.
    const i32x4 a_rs = rsrc_words(a.A, static_cast<uint32_t>(a.a_bytes));
    const uint8_t* bg = static_cast<const uint8_t*>(a.B) + group * a.b_group_stride;
    const i32x4 b_rs = rsrc_words(bg, static_cast<uint32_t>(static_cast<int64_t>(a.N) * ldb));
    constexpr uint32_t kOob = 0x80000000u;  // beyond every buffer: reads zeros
    // A rows repeat every a_steps steps when a_steps > 0 (the router's hi + lo weight planes
    // are one [E, 2d] matrix multiplied by [x, x])
    const int a_steps = a.a_steps > 0 ? a.a_steps : KB;
    uint32_t a_off[S::A_PER], b_off[S::B_PER];
    int a_dst[S::A_PER], b_dst[S::B_PER];  // LDS byte offsets within a slot (-1: dummy)
#pragma unroll
    for (int i = 0; i < S::A_PER; ++i) {
      const int c = tid + S::NT * i, r = c >> 3;
      const int wc = wv * kWave + S::NT * i;  // this wave's first chunk: 1 KiB destination
      a_dst[i] = wc < S::A_CHUNKS ? wc * 16 : -1;
      a_off[i] = kOob;
      // rows past the tile's end read zeros (their outputs are never stored)
      if (c < S::A_CHUNKS && r < rows) {
        const int arow = a.a_map ? a.a_map[m0 + r] : m0 + r;
        a_off[i] = static_cast<uint32_t>(static_cast<int64_t>(arow) * a.lda +
                                         (((c & 7) ^ (r & 7)) << 4));
      }
    }
#pragma unroll
    for (int i = 0; i < S::B_PER; ++i) {
      const int c = tid + S::NT * i, r = c >> 3;
      const int wc = wv * kWave + S::NT * i;
      b_dst[i] = wc < S::B_CHUNKS ? BM * kBlockK + wc * 16 : -1;
      b_off[i] = c < S::B_CHUNKS ? static_cast<uint32_t>(static_cast<int64_t>(n0 + r) * ldb +
                                                         (((c & 7) ^ (r & 7)) << 4))
                                 : kOob;
    }
    // FP8: wave w < BM/64 loads the row scales of rows [64w, 64w+64), wave BM/64 the weight
    // block scales, any other wave a dummy slice
    i32x4 s_rs = rsrc_words(a.A, 0);  // replaced below for FP8
    uint32_t s_off = kOob;
    int s_dst = 0;
    if constexpr (S::kFp8) {
      const int kb_bytes = KB * 4;
      if (wv < BM / 64) {
        const uint32_t a_rows = static_cast<uint32_t>(a.a_bytes / a.lda);
        s_rs = rsrc_words(a.a_scales, a_rows * kb_bytes);
        const int r = wv * 64 + l;
        if (r < rows) {
          const int arow = a.a_map ? a.a_map[m0 + r] : m0 + r;
          s_off = static_cast<uint32_t>(arow) * kb_bytes;
        }
        s_dst = STAGE_BYTES + wv * 256;
      } else if (wv == BM / 64) {
        s_rs = rsrc_words(a.b_scales + group * a.bs_group_stride,
                          static_cast<uint32_t>((a.N / 16) * kb_bytes));
        if (l < BN / 16) s_off = static_cast<uint32_t>(n0 / 16 + l) * kb_bytes;
        s_dst = STAGE_BYTES + BM * 4;
      } else {
        s_rs = rsrc_words(a.b_scales, 4);
        s_dst = STAGE_BYTES + BM * 4 + 256;
      }
    }
    const uint32_t smem_base = lds_addr(smem);
    auto lds_ptr = [&](int slot, int dst) {
      const int o = dst >= 0 ? slot * S::SLOT + dst : S::NSLOT * S::SLOT + wv * 1024;
      return smem_base + static_cast<uint32_t>(o);
    };
    auto issue = [&](int step) {
      const int slot = step % S::NSLOT;
      const uint32_t as =
          static_cast<uint32_t>(step < a_steps ? step : step - a_steps) * kBlockK;
      const uint32_t bs = static_cast<uint32_t>(step) * kBlockK;
#pragma unroll
      for (int i = 0; i < S::A_PER; ++i) lds_dma<16, false>(a_rs, lds_ptr(slot, a_dst[i]), a_off[i], as);
      if (stream_b) {  // weights read by one tile only: do not keep them in the caches
#pragma unroll
        for (int i = 0; i < S::B_PER; ++i) lds_dma<16, true>(b_rs, lds_ptr(slot, b_dst[i]), b_off[i], bs);
      } else {
#pragma unroll
        for (int i = 0; i < S::B_PER; ++i) lds_dma<16, false>(b_rs, lds_ptr(slot, b_dst[i]), b_off[i], bs);
      }
      if constexpr (S::kFp8)
        lds_dma<4, false>(s_rs, lds_ptr(slot, s_dst), s_off, static_cast<uint32_t>(step) * 4);
    };
    // Operand fragments of one step, read from its LDS slot into registers one step ahead of
    // the MFMAs that use them.
    using F = Frags<DT, S::FM, S::FN>;
    auto load = [&](F& f, int slot) {
      const uint8_t* sa = smem + slot * S::SLOT;
      const uint8_t* sb = sa + BM * kBlockK;
      if constexpr (DT == MOE_FP8_E4M3) {
        const float* ss = reinterpret_cast<const float*>(sa + STAGE_BYTES);
#pragma unroll
        for (int i = 0; i < S::FM; ++i) {
          const int r = wm * S::TM + i * 16 + lr;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(sa + swz(r, 2 * kq));
          const i32x4 hi = *reinterpret_cast<const i32x4*>(sa + swz(r, 2 * kq + 1));
          f.a[0][i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          f.sa[i] = *reinterpret_cast<const f32x4*>(ss + wm * S::TM + i * 16 + 4 * kq);
        }
#pragma unroll
        for (int j = 0; j < S::FN; ++j) {
          const int r = wn * S::TN + j * 16 + lr;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(sb + swz(r, 2 * kq));
          const i32x4 hi = *reinterpret_cast<const i32x4*>(sb + swz(r, 2 * kq + 1));
          f.b[0][j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        // a wave's columns lie in one 128-wide weight block per gate/up half (even/odd
        // 16-row blocks of the packed rows), so two weight scales cover all its fragments
        f.sb[0] = ss[BM + wn * S::TN / 16];
        f.sb[1] = ss[BM + wn * S::TN / 16 + 1];
      } else {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int ch = 4 * s + kq;
#pragma unroll
          for (int i = 0; i < S::FM; ++i)
            f.a[s][i] = *reinterpret_cast<const typename F::V*>(sa + swz(wm * S::TM + i * 16 + lr, ch));
#pragma unroll
          for (int j = 0; j < S::FN; ++j)
            f.b[s][j] = *reinterpret_cast<const typename F::V*>(sb + swz(wn * S::TN + j * 16 + lr, ch));
        }
      }
    };
    auto mma = [&](const F& f) {
      if constexpr (DT == MOE_BF16) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int i = 0; i < S::FM; ++i)
#pragma unroll
            for (int j = 0; j < S::FN; ++j) acc[i][j] = mfma_bf16(f.a[s][i], f.b[s][j], acc[i][j]);
      } else if constexpr (DT == MOE_F32) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < S::FM; ++i)
#pragma unroll
              for (int j = 0; j < S::FN; ++j)
                acc[i][j] = mfma_f32(f.a[s][i][e], f.b[s][j][e], acc[i][j]);
      }  // FP8: mma_refill_fp8
    };
    // FP8 step: one E4M3 MFMA covers exactly one 128-deep scale block; its fp32 partial is
    // promoted with the row's activation scale times the block's weight scale.  Written in
    // issue order (sched_barrier pins it): MFMA n runs while partial n-1 is promoted, so only
    // two partials are live, and f is refilled from slot `next` as soon as each fragment's last
    // MFMA has issued (A row block i after its row of MFMAs, the B columns after the last row).
    auto mma_refill_fp8 = [&](F& f, int next) {
      if constexpr (S::kFp8) {
        const uint8_t* sa = smem + next * S::SLOT;
        const uint8_t* sb = sa + BM * kBlockK;
        const float* ss = reinterpret_cast<const float*>(sa + STAGE_BYTES);
        f32x4 prev = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 q[2], qp[2];
#pragma unroll
        for (int i = 0; i < S::FM; ++i) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) q[h][e] = f.sa[i][e] * f.sb[h];
#pragma unroll
          for (int j = 0; j < S::FN; ++j) {
            const f32x4 cur = mfma_fp8(f.a[0][i], f.b[0][j], f32x4{0.f, 0.f, 0.f, 0.f});
            if (i + j > 0) {
              const int pi = j > 0 ? i : i - 1, pj = j > 0 ? j - 1 : S::FN - 1;
              const f32x4& qq = j > 0 ? q[pj & 1] : qp[pj & 1];
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[pi][pj][e] = fmaf(prev[e], qq[e], acc[pi][pj][e]);
            }
            prev = cur;
            __builtin_amdgcn_sched_barrier(0);
          }
          qp[0] = q[0];
          qp[1] = q[1];
          // row block i is done with its A fragment and row scales
          const int r = wm * S::TM + i * 16 + lr;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(sa + swz(r, 2 * kq));
          const i32x4 hi = *reinterpret_cast<const i32x4*>(sa + swz(r, 2 * kq + 1));
          f.a[0][i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          f.sa[i] = *reinterpret_cast<const f32x4*>(ss + wm * S::TM + i * 16 + 4 * kq);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[S::FM - 1][S::FN - 1][e] = fmaf(prev[e], qp[(S::FN - 1) & 1][e], acc[S::FM - 1][S::FN - 1][e]);
#pragma unroll
        for (int j = 0; j < S::FN; ++j) {
          const int r = wn * S::TN + j * 16 + lr;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(sb + swz(r, 2 * kq));
          const i32x4 hi = *reinterpret_cast<const i32x4*>(sb + swz(r, 2 * kq + 1));
          f.b[0][j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        f.sb[0] = ss[BM + wn * S::TN / 16];
        f.sb[1] = ss[BM + wn * S::TN / 16 + 1];
      }
    };

    // FP8 keeps one fragment set (two do not fit beside the accumulators at two waves per
    // SIMD) and refills it in place once the MFMAs reading it are issued.
    constexpr bool kTwoSets = !S::kFp8;
    F f0, f1;
    issue(0);
    issue(1);
    issue(2);
    lds_dma_wait<2 * S::LPS>();
    __syncthreads();
    load(f0, 0);
    // The refill after the last step reads a slot no one wrote for it: harmless, and it keeps
    // the loop body one basic block for the scheduler.
    auto iter = [&](int step, F& cur, F& nxt) {
      lds_dma_wait<S::LPS>();
      __syncthreads();
      issue(step + 3);
      const int next = (step + 1) % S::NSLOT;
      if constexpr (kTwoSets) {
        // one fragment read, then its share of the MFMAs, repeated: the reads of step s+1
        // spread over the MFMAs of step s instead of bunching at either end
        constexpr int NR = 2 * (S::FM + S::FN);
        constexpr int NM = 2 * S::FM * S::FN * (DT == MOE_F32 ? 4 : 1);
        constexpr int PER = NM / NR;
        __builtin_amdgcn_sched_barrier(0);
        load(nxt, next);
        mma(cur);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
          __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // MFMA
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NM - PER * NR, 0);
      } else {
        mma_refill_fp8(cur, next);
      }
    };
    int step = 0;
    if constexpr (kTwoSets) {
      for (; step + 1 < KB; step += 2) {
        iter(step, f0, f1);
        iter(step + 1, f1, f0);
      }
      if (step < KB) iter(step, f0, f1);
    } else {
      for (; step < KB; ++step) iter(step, f0, f0);
    }
    lds_dma_wait<0>();  // the epilogue reuses the ring
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogues
  if constexpr (EPI == kEpiSwiglu) {
    constexpr int HC = BN / 2, HS = HC + 4;
    float* sH = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < S::FM; ++i)
#pragma unroll
      for (int p = 0; p < S::FN / 2; ++p) {
        const int hc = (wn * (S::FN / 2) + p) * 16 + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = wm * S::TM + i * 16 + 4 * kq + e;
          sH[r * HS + hc] = silu(acc[i][2 * p][e]) * acc[i][2 * p + 1][e];
        }
      }
    __syncthreads();
    uint8_t* out = static_cast<uint8_t*>(a.out);
    if constexpr (DT == MOE_FP8_E4M3) {
      // one 128-value group per row: scale = max|h| / 448, codes = E4M3(h / scale)
      const int groups = (a.N / 2) / 128;
      for (int r = wv; r < rows; r += S::NW) {
        float v0 = sH[r * HS + 2 * l], v1 = sH[r * HS + 2 * l + 1];
        float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
        float s = amax > 0.0f ? amax / 448.0f : 1.0f;
        uint32_t c = f32_to_e4m3(v0 / s) | (f32_to_e4m3(v1 / s) << 8);
        *reinterpret_cast<uint16_t*>(out + static_cast<int64_t>(m0 + r) * a.ldo + nt * HC + 2 * l) =
            static_cast<uint16_t>(c);
        if (l == 0) a.out_scales[static_cast<int64_t>(m0 + r) * groups + nt] = s;
      }
    } else {
      constexpr int CPR = HC / 8;  // 8-value chunks per row
      for (int c = tid; c < BM * CPR; c += S::NT) {
        const int r = c / CPR, cc = (c - r * CPR) * 8;
        if (r >= rows) continue;
        const float* v = sH + r * HS + cc;
        uint8_t* dst = out + static_cast<int64_t>(m0 + r) * a.ldo + static_cast<int64_t>(nt * HC + cc) * esize;
        if constexpr (DT == MOE_F32) {
          *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
          *reinterpret_cast<f32x4*>(dst + 16) = f32x4{v[4], v[5], v[6], v[7]};
        } else {
          i32x4 pk;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            pk[q] = static_cast<int>(f32_to_bf16(v[2 * q]) | (static_cast<uint32_t>(f32_to_bf16(v[2 * q + 1])) << 16));
          *reinterpret_cast<i32x4*>(dst) = pk;
        }
      }
    }
  } else {
    constexpr int OS = BN + 4;
    float* sO = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < S::FM; ++i)
#pragma unroll
      for (int j = 0; j < S::FN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sO[(wm * S::TM + i * 16 + 4 * kq + e) * OS + wn * S::TN + j * 16 + lr] = acc[i][j][e];
    __syncthreads();
    // y_perm rows are fp32 except for FP8 experts (bf16); the block output is fp32 only
    // for fp32 activations
    constexpr bool y_f32 = DT != MOE_FP8_E4M3;
    constexpr bool out_f32 = EPI == kEpiStore ? y_f32 : DT == MOE_F32;
    constexpr int osz = out_f32 ? 4 : 2;
    constexpr int ysz = y_f32 ? 4 : 2;
    constexpr int CPR = BN / 8;
    uint8_t* out = static_cast<uint8_t*>(a.out);
    for (int c = tid; c < BM * CPR; c += S::NT) {
      const int r = c / CPR, cc = (c - r * CPR) * 8;
      if (r >= rows) continue;
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = sO[r * OS + cc + q];
      if constexpr (EPI == kEpiStore) {
        if (a.col_bias) {
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] += n0 + cc + q < a.bias_cols ? a.col_bias[n0 + cc + q] : 0.0f;
        }
      }
      if constexpr (EPI == kEpiCombine) {
        // the token's k rows of y_perm, weighted; four rows' loads are issued together
        const int t = m0 + r;
        const uint8_t* y = static_cast<const uint8_t*>(a.y);
        const int64_t base = static_cast<int64_t>(t) * a.top_k;
        for (int j0 = 0; j0 < a.top_k; j0 += 4) {
          const int nj = min(4, a.top_k - j0);
          float wj[4];
          const uint8_t* yr[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int64_t idx = base + j0 + (u < nj ? u : 0);
            wj[u] = u < nj ? a.topk_w[idx] : 0.0f;
            yr[u] = y + static_cast<int64_t>(a.inv_perm[idx]) * a.ldy +
                    static_cast<int64_t>(n0 + cc) * ysz;
          }
          if constexpr (y_f32) {
            f32x4 y0[4], y1[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              y0[u] = *reinterpret_cast<const f32x4*>(yr[u]);
              y1[u] = *reinterpret_cast<const f32x4*>(yr[u] + 16);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                v[q] = fmaf(wj[u], y0[u][q], v[q]);
                v[4 + q] = fmaf(wj[u], y1[u][q], v[4 + q]);
              }
          } else {
            i32x4 yv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) yv[u] = *reinterpret_cast<const i32x4*>(yr[u]);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                uint32_t bits = static_cast<uint32_t>(yv[u][q]);
                v[2 * q] = fmaf(wj[u], __uint_as_float(bits << 16), v[2 * q]);
                v[2 * q + 1] = fmaf(wj[u], __uint_as_float(bits & 0xFFFF0000u), v[2 * q + 1]);
              }
          }
        }
      }
      uint8_t* dst = out + static_cast<int64_t>(m0 + r) * a.ldo + static_cast<int64_t>(n0 + cc) * osz;
      if constexpr (out_f32) {
        *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(dst + 16) = f32x4{v[4], v[5], v[6], v[7]};
      } else {
        i32x4 pk;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          pk[q] = static_cast<int>(f32_to_bf16(v[2 * q]) | (static_cast<uint32_t>(f32_to_bf16(v[2 * q + 1])) << 16));
        *reinterpret_cast<i32x4*>(dst) = pk;
      }
    }
  }
}

// ------------------------------------------------------------------ host side

int gemm_bm(int dtype, int epi, int avg_rows) {
  if (dtype == MOE_F32) return 32;
  if (dtype == MOE_FP8_E4M3) return 128;
  if (avg_rows <= 16) return 16;
  if (avg_rows <= 32) return 32;
  if (avg_rows <= 48) return 64;
  return 128;
}


template <int DT, int BM, int BN, int EPI, bool G>
static hipError_t launch_one(const GemmArgs& a, int max_tiles, hipStream_t s) {
  // grouped: worst-case tile count from the caller; one group: exact, for this BM
  if (!G) max_tiles = (a.M + BM - 1) / BM;
  int nb = max_tiles * (a.N / BN);
  if (nb <= 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_kernel<DT, BM, BN, EPI, G>), dim3(nb),
                     dim3(gemm_waves<DT, BN>() * kWave), 0, s, a);
  return hipGetLastError();
}

template <int DT, int EPI, bool G>
static hipError_t launch_dt(int bm, const GemmArgs& a, int max_tiles, hipStream_t s) {
  if constexpr (DT == MOE_F32) {
    return launch_one<DT, 32, 128, EPI, G>(a, max_tiles, s);
  } else if constexpr (DT == MOE_FP8_E4M3) {
    return launch_one<DT, 128, (EPI == kEpiSwiglu ? 256 : 128), EPI, G>(a, max_tiles, s);
  } else {
    switch (bm) {
      case 16: return launch_one<DT, 16, 128, EPI, G>(a, max_tiles, s);
      case 32: return launch_one<DT, 32, 128, EPI, G>(a, max_tiles, s);
      case 64: return launch_one<DT, 64, 128, EPI, G>(a, max_tiles, s);
      default:  // the wide tile halves the activation re-reads per weight byte
        return a.N % 256 == 0 ? launch_one<DT, 128, 256, EPI, G>(a, max_tiles, s)
                              : launch_one<DT, 128, 128, EPI, G>(a, max_tiles, s);
    }
  }
}

template <int DT>
static hipError_t launch_epi(int epi, int bm, const GemmArgs& a, int max_tiles, hipStream_t s) {
  const bool g = a.tiles != nullptr;
  if (epi == kEpiSwiglu)
    return g ? launch_dt<DT, kEpiSwiglu, true>(bm, a, max_tiles, s)
             : launch_dt<DT, kEpiSwiglu, false>(bm, a, max_tiles, s);
  if (epi == kEpiStore)
    return g ? launch_dt<DT, kEpiStore, true>(bm, a, max_tiles, s)
             : launch_dt<DT, kEpiStore, false>(bm, a, max_tiles, s);
  return launch_dt<DT, kEpiCombine, false>(bm, a, max_tiles, s);
}

hipError_t launch_grouped_gemm(int dtype, int epi, int bm, bool /*out_f32*/, const GemmArgs& a,
                               int max_tiles, hipStream_t s) {
  switch (dtype) {
    case MOE_F32: return launch_epi<MOE_F32>(epi, bm, a, max_tiles, s);
    case MOE_BF16: return launch_epi<MOE_BF16>(epi, bm, a, max_tiles, s);
    default: return launch_epi<MOE_FP8_E4M3>(epi, bm, a, max_tiles, s);
  }
}

}  // namespace moe
