// gemm.hip -- grouped expert GEMMs on gfx950 MFMA with fused epilogues.
//
// Computes, for every tile of rows of every group (expert), OUT = A_rows x B_group^T with B
// stored [N, K] K-contiguous (the packed weight layout; E2M1 weights and their E8M0 scales by
// column tile and K-step, one contiguous block per step of a tile), followed by one of:
//   kEpiSwiglu  -- h = SiLU(gate) * up: B interleaves gate and up columns in blocks of 16
//                  packed rows, so each wave's accumulators hold matching gate/up columns and
//                  h is formed in registers (SwiGLU experts, routed-experts row of
//                  "Qwen3.5-397B-A17B vs Gemma 4 31B"); FP8 re-quantises h per 128 values;
//   kEpiStore   -- rows stored as they are (y_perm, the shared experts' output, router logits).
//
// Structure.  Persistent workgroups: each walks a list of output tiles (the tiles of one XCD's
// contiguous share, so neighbouring tiles -- the N-tiles of one expert, which share its A rows,
// and its M-tiles, which share its weights -- run together in that XCD's L2).  4 or 8 waves per
// workgroup, each wave a 64 x 64 or smaller sub-tile of the BM x BN tile.  K is consumed 128
// bytes per step (64 bf16, 32 fp32 or 128 E4M3 values -- exactly one FP8 scale block).  Every
// step's A rows (gathered through a_map: no permuted copy of x is ever written) and B rows go
// straight from global memory into an LDS ring of three slots (up to eight for row-light E4M3
// tiles) with buffer loads that write LDS directly, issued as many steps ahead, across tile
// boundaries: the next tile's operands are already arriving while the current tile's epilogue
// stores its results from registers.  The 16-byte chunks land XOR-swizzled by row so that
// fragment reads of 16 consecutive rows hit distinct banks; fragments of step s+1 are read
// from LDS while the MFMAs of step s run, one barrier per step.  bf16 and fp32 weights of an
// expert whose rows fit one tile are loaded non-temporally (read once); others keep the default
// policy so the expert's other row tiles find them in L2.  (With E4M3 activations, and in
// launches of one group, a step's loads go out between its MFMAs with the default policy:
// measured on MI355X, the non-temporal hint gains nothing with E4M3 activations.)
#include <math.h>

#include <atomic>
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
template <>
struct DT_<MOE_MXFP4> { static constexpr int esize = 1; };  // A: E4M3 activations

__device__ __forceinline__ int swz(int row, int ch) { return row * kBlockK + ((ch ^ (row & 7)) << 4); }
// E2M1 weight rows hold 64 bytes per step (four 16-byte chunks).  Chunk c of row r sits at
// slot c ^ ((r >> 1) & 2).  A 128-bit LDS read is served for lanes 0-7 and 16-23 together (and
// likewise for the other half-groups) -- eight rows read at chunk c and at chunk c+1 -- and this
// puts those 16 accesses on 16 different 16-byte bank groups.
__device__ __forceinline__ int swz4(int row, int ch) { return row * 64 + ((ch ^ ((row >> 1) & 2)) << 4); }

// NW waves per workgroup: 8 for the wide tiles (BN = 256, each wave still 64 x 64), else 4.
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
  // E4M3 activations with one fp32 scale per row and 128 K values (FP8 and MXFP4 experts)
  static constexpr bool kFp8 = DT == MOE_FP8_E4M3 || DT == MOE_MXFP4;
  // E2M1 weights with one E8M0 scale per column and 32 K values, applied inside the MFMA
  static constexpr bool kMx = DT == MOE_MXFP4;
  static constexpr int B_ROW = kMx ? 64 : kBlockK;    // bytes of one B row per step
  // bytes between consecutive steps of one B row: E2M1 weights are packed by column tile and
  // step (a tile's step is one contiguous BN x 64-byte block), the others row-major
  static constexpr int B_STEP = kMx ? BN * 64 : kBlockK;
  static constexpr int A_CHUNKS = BM * 8, B_CHUNKS = BN * (B_ROW / 16);  // 16-byte chunks
  static constexpr int A_PER = (A_CHUNKS + NT - 1) / NT, B_PER = (B_CHUNKS + NT - 1) / NT;
  static constexpr int STAGE = BM * kBlockK + BN * B_ROW;
  // Scale loads of a step, one 4-byte load per lane of a wave (256 bytes of LDS each): ASW
  // waves the activation row scales (64 rows a wave), BSW waves the weight scales (FP8: one
  // wave, a float per 16 packed rows; MXFP4: a dword of four E8M0 scales per column, 64
  // columns a wave); any other wave loads into a spare 256 bytes
  static constexpr int ASW = kFp8 ? (BM + 63) / 64 : 0;
  static constexpr int BSW = kMx ? BN / 64 : kFp8 ? 1 : 0;
  static constexpr int SCALES = kFp8 ? (ASW + BSW + 1) * 256 : 0;
  static constexpr int SLOT = STAGE + SCALES;
  // destination of the A/B loads a wave issues for nothing (when the chunks do not divide evenly
  // over the waves)
  static constexpr int DUMMY = (A_CHUNKS % NT || B_CHUNKS % NT) ? NW * 1024 : 0;
  // FP8 h quantisation: per-row maxima of each wave column, exchanged between waves
  static constexpr int AMAX = (kFp8 && EPI == kEpiSwiglu) ? BM * WN * 4 : 0;
  // LDS ring: step s multiplies out of slot s % NSLOT while the next NSLOT - 1 steps land in
  // the others.  Three slots; E4M3 and bf16 tiles of at most 32 rows (decode shapes, which do
  // little but stream weights) take as many as 160 KiB of LDS hold, up to 8, for more bytes in
  // flight per CU (measured on MI355X: three slots instead make the MXFP4 decode gate/up ~4% and
  // the bf16 decode gate/up ~1.5% slower).
  static constexpr int DEEP = (160 * 1024 - DUMMY - AMAX) / SLOT;
  static constexpr int NSLOT =
      ((kFp8 || DT == MOE_BF16) && BM <= 32) ? (DEEP > 8 ? 8 : DEEP < 3 ? 3 : DEEP) : 3;
  static constexpr int MAIN = NSLOT * SLOT + DUMMY;
  static constexpr int SMEM = MAIN + AMAX;
  // direct-to-LDS loads each wave issues per step (the same count in every wave)
  static constexpr int LPS = A_PER + B_PER + (kFp8 ? 1 : 0);
  // stores every wave issues in a tile's epilogue (at least; FP8 h scales come on top)
  static constexpr int EPI_STORES = EPI == kEpiStore ? FM * FN : FM * (FN / 2);
  static_assert(FM >= 1 && FN >= 1, "tile too small for its waves");
  static_assert(!kFp8 || NW >= ASW + BSW, "scale loads need ASW + BSW waves");
  static_assert((NSLOT - 1) * LPS < 64 && (NSLOT - 2) * LPS + EPI_STORES < 64,
                "vmcnt holds at most 63");
  static_assert(SMEM <= 160 * 1024, "LDS of one workgroup");
  static_assert(!kFp8 || kMx || (TN <= 128 && 128 % TN == 0), "FP8: two weight scales per wave");
  static_assert(!kMx || BN % 64 == 0, "MXFP4: whole waves of weight scales");
  static_assert(EPI != kEpiSwiglu || FN % 2 == 0, "gate/up pairs must stay within one wave");
  static_assert(!(kFp8 && EPI == kEpiSwiglu) || BN == 256, "FP8 h groups need 128 h columns");
};

// Register fragments of one pipeline step: two 16x16x32 (bf16) or 16x16x4-by-4 (fp32) K-halves,
// or one 16x16x128 E4M3 block with the activation scale of the lane's own row (sa; see the
// epilogues for the accumulator layout) and the wave's two weight-block scales.
template <int DT, int FM, int FN>
struct Frags {
  using V = typename std::conditional<DT == MOE_BF16, bf16x8, f32x4>::type;
  V a[2][FM], b[2][FN];
};
// E4M3: index [p] is the set of steps of parity p.  Row blocks 0 .. FM-2 of A (and their row
// scales) live in set 0 only and are refilled in place once their row of MFMAs has issued; the
// last row block, the B fragments and the two weight scales alternate between the sets, the
// next step's set read at the start of the step (so no fragment read is left to wait for at
// the step's end).  Elements never touched are dropped by the compiler.
template <int FM, int FN>
struct Frags<MOE_FP8_E4M3, FM, FN> {
  i32x8 a[2][FM], b[2][FN];
  float sa[2][FM];
  float sb[2][2];
};
// E4M3 activations against E2M1 weights: 32 B of activations and 16 B of weights per lane, the
// lane's E8M0 weight scale (its output column, its 32-value block) in the low byte of sbx; sets
// as for E4M3.
template <int FM, int FN>
struct Frags<MOE_MXFP4, FM, FN> {
  i32x8 a[2][FM];
  i32x4 b[2][FN];
  float sa[2][FM];
  int sbx[2][FN];
};

// Waves per SIMD the register allocation aims for: what the LDS footprint lets run (160 KiB
// per CU), capped at 2.
template <int DT, int BM, int BN, int EPI>
constexpr int gemm_occupancy() {
  using S = GemmShape<DT, BM, BN, EPI>;
  const int per_cu = (160 * 1024) / S::SMEM * S::NW / 4;
  return per_cu < 1 ? 1 : per_cu > 2 ? 2 : per_cu;
}

// Row tiles of one expert swept together per N-tile (see geo in the kernel).
constexpr int kGroupM = 8;

// One output tile: its group, first row and row count (of the M space), first column, and
// the number of row tiles its group has.
struct TileGeo {
  int group, m0, rows, n0, count;
};

// GROUPED: rows come from the device tile list of an expert-grouped problem (the routed
// experts); otherwise one group of a.M rows (router, shared experts).  G2 (grouped only): the
// tile list also holds the extra group of GemmArgs (the shared experts of decode-sized
// batches); a separate instantiation, so the other launches carry none of its registers.
template <int DT, int BM, int BN, int EPI, bool GROUPED, bool G2>
__global__ __launch_bounds__((gemm_waves<DT, BN>() * kWave), (gemm_occupancy<DT, BM, BN, EPI>()))
void grouped_gemm_kernel(GemmArgs a) {
  using S = GemmShape<DT, BM, BN, EPI>;
  using F = Frags<DT, S::FM, S::FN>;
  constexpr int esize = DT_<DT>::esize;
  constexpr int STAGE_BYTES = S::STAGE;
  __shared__ __attribute__((aligned(16))) uint8_t smem[S::SMEM];

  // ---------------------------------------------------------------- this workgroup's tiles
  // Hardware workgroup b runs on XCD b % 8.  The tiles are split into 8 contiguous shares, one
  // per XCD; the XCD's workgroups take its tiles round-robin, so at any time they work on
  // consecutive tiles.
  const int NT = a.N / BN;
  // one-group launches may split K: tile index = split * (row tiles) + row tile
  const int splits = GROUPED || a.k_splits < 2 ? 1 : a.k_splits;
  const int mtiles = GROUPED ? 0 : (a.M + BM - 1) / BM;
  const int ntiles = GROUPED ? a.tiles_count[0] : mtiles * splits;
  const int nblocks = ntiles * NT;
  const int xcd = blockIdx.x % kNumXcd, wg = blockIdx.x / kNumXcd;
  const int per_xcd = gridDim.x / kNumXcd;
  const int q = nblocks / kNumXcd, qr = nblocks % kNumXcd;
  const int lo = xcd * q + (xcd < qr ? xcd : qr), span = q + (xcd < qr ? 1 : 0);
  const int n_my = wg < span ? (span - wg + per_xcd - 1) / per_xcd : 0;
  if (n_my == 0) return;
  // Within one expert the workgroups of an XCD sweep each N-tile across a group of up to
  // kGroupM row tiles before the next N-tile: co-running workgroups then share every weight
  // tile kGroupM ways and every activation tile about 32 / kGroupM ways.  An expert occupies
  // the logical range [NT * first, NT * (first + count)) whatever the order inside it.
  auto geo = [&](int t) {
    const int L = lo + wg + t * per_xcd;
    TileGeo g;
    if constexpr (GROUPED) {
      const i32x4 t0 = scalar_load16(a.tiles + L / NT);  // some tile of L's expert
      const int count = t0[3], first = L / NT - (t0[2] >> 8);
      const int local = L - NT * first;
      const int full = count / kGroupM, span_full = full * NT * kGroupM;
      int m, nt;
      if (local < span_full) {
        const int grp = local / (NT * kGroupM), rem = local - grp * (NT * kGroupM);
        nt = rem / kGroupM;
        m = grp * kGroupM + (rem - nt * kGroupM);
      } else {
        const int r = count - full * kGroupM, rem = local - span_full;
        nt = rem / r;
        m = full * kGroupM + (rem - nt * r);
      }
      const i32x4 ti = scalar_load16(a.tiles + first + m);
      g = TileGeo{ti[0], ti[1], ti[2] & 0xFF, nt * BN, count};
    } else {
      // (the group field holds the K range of a split launch)
      const int tile = L / NT, nt = L - tile * NT;
      const int split = tile / mtiles, mt = tile - split * mtiles;
      g = TileGeo{split, mt * BM, min(BM, a.M - mt * BM), nt * BN, 1};
    }
    return g;
  };

  const int tid = threadIdx.x, l = lane_id(), wv = uniform(tid / kWave);
  const int wm = wv / S::WN, wn = wv % S::WN;
  const int lr = l & 15, kq = l >> 4;
  const int KB = a.K * esize / kBlockK / splits;  // pipeline steps per tile (K >= 128 elements)
  const int64_t ldb = a.ldb;
  constexpr uint32_t kOob = 0x80000000u;  // beyond every buffer: reads zeros
  // A rows repeat every a_steps steps when a_steps > 0 (the router's hi + lo weight planes
  // are one [E, 2d] matrix multiplied by [x, x])
  const int a_steps = a.a_steps > 0 ? a.a_steps : KB * splits;

  // ---------------------------------------------------------------- direct-to-LDS loads
  // Every load writes 16 bytes per lane straight into LDS at (wave base + 16 * lane): the
  // lane-to-chunk map is chosen on the global side so that the tile lands in the swizzled
  // layout the fragment reads expect (row r's logical chunk c at slot r*8 + (c ^ (r & 7))).
  // No staging registers, no LDS store instructions.
  // the extra group (the shared experts, rows = the tokens in order) reads its own operands
  constexpr bool has2 = GROUPED && G2;
  const i32x4 a_rs1 = rsrc_words(a.A, static_cast<uint32_t>(a.a_bytes));
  const i32x4 a_rs2 = has2 ? rsrc_words(a.A2, static_cast<uint32_t>(a.a2_bytes)) : a_rs1;
  i32x4 a_rs = a_rs1;
  int a_dst[S::A_PER], b_dst[S::B_PER];  // LDS byte offsets within a slot (-1: dummy)
#pragma unroll
  for (int i = 0; i < S::A_PER; ++i) {
    const int wc = wv * kWave + S::NT * i;  // this wave's first chunk: 1 KiB destination
    a_dst[i] = wc < S::A_CHUNKS ? wc * 16 : -1;
  }
#pragma unroll
  for (int i = 0; i < S::B_PER; ++i) {
    const int wc = wv * kWave + S::NT * i;
    b_dst[i] = wc < S::B_CHUNKS ? BM * kBlockK + wc * 16 : -1;
  }
  // Per-tile state of the issuing side, which runs up to NSLOT steps (and so possibly one or
  // more tiles) ahead of the multiplying side.
  uint32_t a_off[S::A_PER], b_off[S::B_PER];
  i32x4 b_rs, s_rs = rsrc_words(a.A, 0);
  uint32_t s_off = kOob;
  // bytes per step of this wave's scale loads: the E8M0 waves read step-major blocks of BN
  // dwords, the others one dword per step of a row-major row
  const uint32_t s_step = S::kMx && wv >= S::ASW && wv < S::ASW + S::BSW ? BN * 4u : 4u;
  int s_dst = 0;
  bool stream_b = false;
  // The gathered rows of a tile come through the scalar path (see scalar_buffer_load32): a
  // wave's lanes cover 8 consecutive rows per load instruction.
  const bool gather = a.a_map != nullptr;
  const i32x4 map_rs = rsrc_words(a.a_map, static_cast<uint32_t>(a.M) * 4);
  // The geometry of the issuing side's current tile and of the one before it, kept for the
  // epilogues: with at least NSLOT - 1 steps per tile the consuming side is on one of the two.
  TileGeo g_iss{}, g_prev{};
  int g_iss_t = -1;
  int iss_k0 = 0;  // first K-step of the issuing side's tile (a split launch's K range)
  auto setup = [&](int t) {
    const TileGeo g = geo(t);
    g_prev = g_iss;
    g_iss = g;
    g_iss_t = t;
    if constexpr (!GROUPED) iss_k0 = g.group * KB;
    const bool second = has2 && g.group == a.group2;  // (uniform)
    const int row0 = second ? g.m0 - a.m2 : g.m0;     // first A row of an unmapped tile
    a_rs = second ? a_rs2 : a_rs1;
#pragma unroll
    for (int i = 0; i < S::A_PER; ++i) {
      const int c = tid + S::NT * i, r = c >> 3;
      int arow = row0 + r;
      if (gather && !second) {
        const int rb = (wv * kWave + S::NT * i) >> 3;  // this wave's first row of load i
        arow = select8(scalar_buffer_load32(map_rs, static_cast<uint32_t>(g.m0 + rb) * 4), l >> 3);
      }
      // rows past the tile's end read zeros (their outputs are never stored)
      a_off[i] = c < S::A_CHUNKS && r < g.rows
                     ? static_cast<uint32_t>(static_cast<int64_t>(arow) * a.lda +
                                             (((c & 7) ^ (r & 7)) << 4))
                     : kOob;
    }
    const uint8_t* bg = second ? static_cast<const uint8_t*>(a.B2)
                               : static_cast<const uint8_t*>(a.B) + g.group * a.b_group_stride;
    b_rs = rsrc_words(bg, static_cast<uint32_t>(static_cast<int64_t>(a.N) * ldb));
#pragma unroll
    for (int i = 0; i < S::B_PER; ++i) {
      const int c = tid + S::NT * i;
      if constexpr (S::kMx) {  // 64-byte rows, see swz4; the tile's block starts at n0 * ldb
        const int r = c >> 2;
        b_off[i] = c < S::B_CHUNKS
                       ? static_cast<uint32_t>(static_cast<int64_t>(g.n0) * ldb + r * 64 +
                                               (((c & 3) ^ ((r >> 1) & 2)) << 4))
                       : kOob;
      } else {
        const int r = c >> 3;
        b_off[i] = c < S::B_CHUNKS
                       ? static_cast<uint32_t>(static_cast<int64_t>(g.n0 + r) * ldb +
                                               (((c & 7) ^ (r & 7)) << 4))
                       : kOob;
      }
    }
    // an expert with one row tile is the only reader of its weights
    stream_b = GROUPED && a.b_stream && g.count == 1;
    // E4M3 activations: wave w < ASW loads the row scales of rows [64w, 64w+64), the next BSW
    // waves the weight scales, any other wave a dummy word
    if constexpr (S::kFp8) {
      const int kb_bytes = KB * splits * 4;
      s_off = kOob;
      if (wv < S::ASW) {
        const uint32_t a_rows = static_cast<uint32_t>((second ? a.a2_bytes : a.a_bytes) / a.lda);
        s_rs = rsrc_words(second ? a.a2_scales : a.a_scales, a_rows * kb_bytes);
        const int r = wv * 64 + l;
        int arow = row0 + r;
        if (gather && !second) {
#pragma unroll
          for (int qd = 0; qd < 8; ++qd) {
            const i32x8 v = scalar_buffer_load32(map_rs, static_cast<uint32_t>(g.m0 + wv * 64 + 8 * qd) * 4);
            if ((l >> 3) == qd) arow = select8(v, l & 7);
          }
        }
        if (r < g.rows && r < BM) s_off = static_cast<uint32_t>(arow) * kb_bytes;
        s_dst = STAGE_BYTES + wv * 256;
      } else if (wv < S::ASW + S::BSW) {
        const int bw = wv - S::ASW;
        if constexpr (S::kMx) {
          // E8M0 scales [N, K/32] bytes per group, by column tile and step: column n0 + c's
          // four scales of a step are one dword at n0 * K/32 + 4 * c + BN * 4 * step
          const int kb32 = a.K / 32;
          s_rs = rsrc_words(second ? a.b2_e8m0 : a.b_e8m0 + g.group * a.be_group_stride,
                            static_cast<uint32_t>(a.N) * kb32);
          s_off = static_cast<uint32_t>(g.n0) * kb32 + static_cast<uint32_t>(bw * 64 + l) * 4;
        } else {
          s_rs = rsrc_words(second ? a.b2_scales : a.b_scales + g.group * a.bs_group_stride,
                            static_cast<uint32_t>((a.N / 16) * kb_bytes));
          if (l < BN / 16) s_off = static_cast<uint32_t>(g.n0 / 16 + l) * kb_bytes;
        }
        s_dst = STAGE_BYTES + wv * 256;
      } else {
        s_rs = rsrc_words(a.a_scales, 4);
        s_dst = STAGE_BYTES + (S::ASW + S::BSW) * 256;  // the slot's spare 256 bytes
      }
    }
  };
  const uint32_t smem_base = lds_addr(smem);
  auto lds_ptr = [&](int slot, int dst) {
    const int o = dst >= 0 ? slot * S::SLOT + dst : S::NSLOT * S::SLOT + (S::DUMMY ? wv * 1024 : 0);
    return smem_base + static_cast<uint32_t>(o);
  };
  // Issue one step.  Past the last tile the loads repeat the last tile's bytes (or zeros) into
  // slots no one reads, so every wave keeps the same count of loads in flight for the waits.
  // issue_begin advances to the next step (and tile); issue_load(n) issues its n-th of the LPS
  // loads, so that a caller can spread them between MFMAs.
  int iss_t = 0, iss_s = 0, iss_slot = 0;
  int q_slot = 0;
  uint32_t q_as = 0, q_bs = 0, q_ss = 0;
  auto issue_begin = [&]() __attribute__((always_inline)) {
    if (iss_s == KB) {
      iss_s = 0;
      if (++iss_t < n_my) setup(iss_t);
    }
    const int step = iss_k0 + iss_s;
    q_slot = iss_slot;
    iss_slot = iss_slot + 1 == S::NSLOT ? 0 : iss_slot + 1;
    ++iss_s;
    q_as = static_cast<uint32_t>(step < a_steps ? step : step - a_steps) * kBlockK;
    q_bs = static_cast<uint32_t>(step) * S::B_STEP;
    q_ss = static_cast<uint32_t>(step) * s_step;
  };
  // nt: the weights' loads are non-temporal (stream_b of the step being issued)
  auto issue_load = [&](int n, auto nt) __attribute__((always_inline)) {
    if (n < S::A_PER) {
      lds_dma<16, false>(a_rs, lds_ptr(q_slot, a_dst[n]), a_off[n], q_as);
    } else if (n < S::A_PER + S::B_PER) {
      const int i = n - S::A_PER;
      lds_dma<16, decltype(nt)::value>(b_rs, lds_ptr(q_slot, b_dst[i]), b_off[i], q_bs);
    } else if constexpr (S::kFp8) {
      lds_dma<4, false>(s_rs, lds_ptr(q_slot, s_dst), s_off, q_ss);
    }
  };
  // (issue and epilogue are called from both parities of the step: forced inline, so the
  // accumulators and fragments stay in registers)
  constexpr std::true_type kStream{};  // weights read by one tile only: not kept in the caches
  constexpr std::false_type kKeep{};
  auto issue = [&]() __attribute__((always_inline)) {
    issue_begin();
    if (stream_b) {
#pragma unroll
      for (int n = 0; n < S::LPS; ++n) issue_load(n, kStream);
    } else {
#pragma unroll
      for (int n = 0; n < S::LPS; ++n) issue_load(n, kKeep);
    }
  };

  // ---------------------------------------------------------------- fragments and MFMAs
  f32x4 acc[S::FM][S::FN];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < S::FM; ++i)
#pragma unroll
      for (int j = 0; j < S::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  zero_acc();
  // One E4M3 fragment of row r of an LDS tile: chunks kq and 4 + kq, the MFMA's own K order (A
  // and B agree, so any order within the 128-value block would do; this one keeps the lanes kq
  // and kq + 1 that one 128-bit LDS read serves together on different bank groups).
  auto frag_e4m3 = [&](const uint8_t* tile, int r) {
    const i32x4 lo4 = *reinterpret_cast<const i32x4*>(tile + swz(r, kq));
    const i32x4 hi4 = *reinterpret_cast<const i32x4*>(tile + swz(r, 4 + kq));
    return i32x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
  };
  // Operand fragments of one step, read from its LDS slot into registers one step ahead of
  // the MFMAs that use them.
  auto load = [&](F& f, int slot) {
    const uint8_t* sa = smem + slot * S::SLOT;
    const uint8_t* sb = sa + BM * kBlockK;
    if constexpr (S::kMx) {  // set 0 of every fragment
      const float* ss = reinterpret_cast<const float*>(sa + STAGE_BYTES);
      const uint32_t* bsc = reinterpret_cast<const uint32_t*>(sa + STAGE_BYTES + S::ASW * 256);
#pragma unroll
      for (int i = 0; i < S::FM; ++i) {
        // activations in the MFMA's K order for an E2M1 partner: bytes 0-15 of the lane hold
        // K 16*kq.., bytes 16-31 K 64+16*kq.. (the E4M3 fragment layout)
        f.a[0][i] = frag_e4m3(sa, wm * S::TM + i * 16 + lr);
        f.sa[0][i] = ss[wm * S::TM + i * 16 + lr];
      }
#pragma unroll
      for (int j = 0; j < S::FN; ++j) {
        const int r = wn * S::TN + j * 16 + lr;  // E2M1: K 32*kq.. of column r
        f.b[0][j] = *reinterpret_cast<const i32x4*>(sb + swz4(r, kq));
        f.sbx[0][j] = static_cast<int>((bsc[r] >> (8 * kq)) & 0xFFu);
      }
    } else if constexpr (DT == MOE_FP8_E4M3) {  // set 0 of every fragment
      const float* ss = reinterpret_cast<const float*>(sa + STAGE_BYTES);
#pragma unroll
      for (int i = 0; i < S::FM; ++i) {
        f.a[0][i] = frag_e4m3(sa, wm * S::TM + i * 16 + lr);
        f.sa[0][i] = ss[wm * S::TM + i * 16 + lr];
      }
#pragma unroll
      for (int j = 0; j < S::FN; ++j) f.b[0][j] = frag_e4m3(sb, wn * S::TN + j * 16 + lr);
      // a wave's columns lie in one 128-wide weight block per gate/up half (even/odd
      // 16-row blocks of the packed rows), so two weight scales cover all its fragments
      f.sb[0][0] = ss[S::ASW * 64 + wn * S::TN / 16];
      f.sb[0][1] = ss[S::ASW * 64 + wn * S::TN / 16 + 1];
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
          for (int j = 0; j < S::FN; ++j) acc[i][j] = mfma_bf16(f.b[s][j], f.a[s][i], acc[i][j]);
    } else if constexpr (DT == MOE_F32) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int i = 0; i < S::FM; ++i)
#pragma unroll
            for (int j = 0; j < S::FN; ++j)
              acc[i][j] = mfma_f32(f.b[s][j][e], f.a[s][i][e], acc[i][j]);
    }  // FP8: mma_refill_fp8
  };
  // bf16 / fp32 step: the MFMAs of step g from `cur` while step g+1's fragments are read into
  // `nxt`, one fragment read then its share of the MFMAs, repeated (the reads spread over the
  // MFMAs instead of bunching at either end).  spread: load n of step g+NSLOT goes out after
  // fragment read n * NR / LPS (the inline-asm loads keep their place among the LDS reads, both
  // touching memory, which the group barriers interleave with the MFMAs); otherwise the caller
  // has issued them.  Grouped launches issue in one burst: their per-tile cache policy (see
  // stream_b) would need a second copy of the step for each policy, and measured on MI355X,
  // the policy is worth more there than the spread; the spread gains 6-13% on the others.
  auto step_two_sets = [&](F& cur, F& nxt, int next, auto spread) {
    if constexpr (!S::kFp8) {
      constexpr int NR = 2 * (S::FM + S::FN);
      constexpr int NM = 2 * S::FM * S::FN * (DT == MOE_F32 ? 4 : 1);
      constexpr int PER = NM / NR;
      static_assert(S::LPS <= NR, "one load per fragment read at most");
      const uint8_t* sa = smem + next * S::SLOT;
      const uint8_t* sb = sa + BM * kBlockK;
      auto loads_after = [&](int r) {
        if constexpr (decltype(spread)::value) {
#pragma unroll
          for (int n = 0; n < S::LPS; ++n)
            if (n * NR / S::LPS == r) issue_load(n, kKeep);
        }
      };
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ch = 4 * h + kq;
#pragma unroll
        for (int i = 0; i < S::FM; ++i) {
          nxt.a[h][i] = *reinterpret_cast<const typename F::V*>(sa + swz(wm * S::TM + i * 16 + lr, ch));
          loads_after(h * (S::FM + S::FN) + i);
        }
#pragma unroll
        for (int j = 0; j < S::FN; ++j) {
          nxt.b[h][j] = *reinterpret_cast<const typename F::V*>(sb + swz(wn * S::TN + j * 16 + lr, ch));
          loads_after(h * (S::FM + S::FN) + S::FM + j);
        }
      }
      mma(cur);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // MFMA
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NM - PER * NR, 0);
    }
  };

  // FP8 step (steps of parity P use fragment set P, see Frags): one E4M3 MFMA covers exactly one
  // 128-deep scale block; its fp32 partial is promoted with the row's activation scale times the
  // block's weight scale.  Written in issue order: MFMA n is issued before partial n-1 is
  // promoted (sched_barrier fences each MFMA with the promotion of the previous one, and
  // sched_group_barrier puts the MFMA first inside the fence, so the promotion waits on an MFMA
  // that has long finished instead of the one just issued).  The next step's reads from slot
  // `next` ride along: its B fragments (set 1-P) one per MFMA of the first row block, its last
  // row block and weight scales in the second, and row block i-1 in place (set 0) once row
  // block i has started.
  auto mma_refill_fp8 = [&](F& f, int next, auto parity) {
    if constexpr (S::kFp8 && !S::kMx) {
      constexpr int P = decltype(parity)::value, Q = 1 - P, L = S::FM - 1;
      // where the next step's last row block and weight scales are read
      constexpr int XI = S::FM > 1 ? 1 : 0;
      constexpr int XJ_A = S::FM > 1 ? (S::FN > 1 ? 1 : 0) : S::FN - 1;
      constexpr int XJ_S = S::FM > 1 ? (S::FN > 2 ? 2 : S::FN - 1) : S::FN - 1;
      const uint8_t* sa = smem + next * S::SLOT;
      const uint8_t* sb = sa + BM * kBlockK;
      const float* ss = reinterpret_cast<const float*>(sa + STAGE_BYTES);
      f32x4 prev = f32x4{0.f, 0.f, 0.f, 0.f};
      float qs[2], qp[2];
#pragma unroll
      for (int i = 0; i < S::FM; ++i) {
        const int ai = i == L ? P : 0;  // constant after unrolling
#pragma unroll
        for (int h = 0; h < 2; ++h) qs[h] = f.sa[ai][i] * f.sb[P][h];
#pragma unroll
        for (int j = 0; j < S::FN; ++j) {
          const f32x4 cur = mfma_fp8(f.b[P][j], f.a[ai][i], f32x4{0.f, 0.f, 0.f, 0.f});
          if (i + j > 0) {
            const int pi = j > 0 ? i : i - 1, pj = j > 0 ? j - 1 : S::FN - 1;
            const float qq = j > 0 ? qs[pj & 1] : qp[pj & 1];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[pi][pj][e] = fmaf(prev[e], qq, acc[pi][pj][e]);
          }
          prev = cur;
          if (i * S::FN + j < S::LPS) issue_load(i * S::FN + j, kKeep);  // step g+NSLOT's loads
          if (i == 0) f.b[Q][j] = frag_e4m3(sb, wn * S::TN + j * 16 + lr);
          if (i == XI && j == XJ_A) {
            f.a[Q][L] = frag_e4m3(sa, wm * S::TM + L * 16 + lr);
            f.sa[Q][L] = ss[wm * S::TM + L * 16 + lr];
          }
          if (i == XI && j == XJ_S) {
            f.sb[Q][0] = ss[S::ASW * 64 + wn * S::TN / 16];
            f.sb[Q][1] = ss[S::ASW * 64 + wn * S::TN / 16 + 1];
          }
          if (j == 0 && i > 0 && i - 1 < L) {  // row block i-1 is done with its fragment
            f.a[0][i - 1] = frag_e4m3(sa, wm * S::TM + (i - 1) * 16 + lr);
            f.sa[0][i - 1] = ss[wm * S::TM + (i - 1) * 16 + lr];
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // the MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);  // then the VALU work
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // then the LDS reads
          __builtin_amdgcn_sched_barrier(0);
        }
        qp[0] = qs[0];
        qp[1] = qs[1];
      }
#pragma unroll
      for (int n = S::FM * S::FN; n < S::LPS; ++n) issue_load(n, kKeep);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[S::FM - 1][S::FN - 1][e] =
            fmaf(prev[e], qp[(S::FN - 1) & 1], acc[S::FM - 1][S::FN - 1][e]);
    }
  };

  // MXFP4 step: one scaled MFMA per (row block, column block) takes E4M3 activations and E2M1
  // weights with the lane's E8M0 weight scale applied inside; its fp32 partial is promoted
  // with the row's activation scale.  Same issue order, fragment sets and placement of the next
  // step's reads and loads as the E4M3 step.
  auto mma_refill_mx = [&](F& f, int next, auto parity) {
    if constexpr (S::kMx) {
      constexpr int P = decltype(parity)::value, Q = 1 - P, L = S::FM - 1;
      constexpr int XI = S::FM > 1 ? 1 : 0;
      constexpr int XJ_A = S::FM > 1 ? (S::FN > 1 ? 1 : 0) : S::FN - 1;
      const uint8_t* sa = smem + next * S::SLOT;
      const uint8_t* sb = sa + BM * kBlockK;
      const float* ss = reinterpret_cast<const float*>(sa + STAGE_BYTES);
      const uint32_t* bsc = reinterpret_cast<const uint32_t*>(sa + STAGE_BYTES + S::ASW * 256);
      f32x4 prev = f32x4{0.f, 0.f, 0.f, 0.f};
      float qp = 0.0f;
#pragma unroll
      for (int i = 0; i < S::FM; ++i) {
        const int ai = i == L ? P : 0;  // constant after unrolling
        const float qs = f.sa[ai][i];
#pragma unroll
        for (int j = 0; j < S::FN; ++j) {
          const f32x4 cur = mfma_mx(f.b[P][j], f.a[ai][i], f.sbx[P][j]);
          if (i + j > 0) {
            const int pi = j > 0 ? i : i - 1, pj = j > 0 ? j - 1 : S::FN - 1;
            const float qq = j > 0 ? qs : qp;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[pi][pj][e] = fmaf(prev[e], qq, acc[pi][pj][e]);
          }
          prev = cur;
          if (i * S::FN + j < S::LPS) issue_load(i * S::FN + j, kKeep);  // step g+NSLOT's loads
          if (i == 0) {
            const int r = wn * S::TN + j * 16 + lr;
            f.b[Q][j] = *reinterpret_cast<const i32x4*>(sb + swz4(r, kq));
            f.sbx[Q][j] = static_cast<int>((bsc[r] >> (8 * kq)) & 0xFFu);
          }
          if (i == XI && j == XJ_A) {
            f.a[Q][L] = frag_e4m3(sa, wm * S::TM + L * 16 + lr);
            f.sa[Q][L] = ss[wm * S::TM + L * 16 + lr];
          }
          if (j == 0 && i > 0 && i - 1 < L) {  // row block i-1 is done with its fragment
            f.a[0][i - 1] = frag_e4m3(sa, wm * S::TM + (i - 1) * 16 + lr);
            f.sa[0][i - 1] = ss[wm * S::TM + (i - 1) * 16 + lr];
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // the MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);  // then the VALU work
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // then the LDS reads
          __builtin_amdgcn_sched_barrier(0);
        }
        qp = qs;
      }
#pragma unroll
      for (int n = S::FM * S::FN; n < S::LPS; ++n) issue_load(n, kKeep);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[S::FM - 1][S::FN - 1][e] = fmaf(prev[e], qp, acc[S::FM - 1][S::FN - 1][e]);
    }
  };

  // ---------------------------------------------------------------- epilogues
  // Every MFMA takes the weights as its first operand and the activation rows as its second,
  // so accumulator block (i, j) holds, in lane l, output row wm*TM + 16i + l%16 at the four
  // consecutive columns wn*TN + 16j + 4*(l/16) + e.  Before a block is stored, lane 4r + c takes
  // the (already packed) values of lane r + 16c by a cross-lane permute, so that consecutive
  // lanes write consecutive bytes of one row, which the store path merges (stored in the
  // accumulator order, the down GEMMs measured 22% slower on MI355X).  16/8/4-byte buffer stores
  // through a resource ending at the tile's last row: rows past it are dropped.  The LDS ring
  // meanwhile keeps receiving the next tile's operands.
  const int orow = wm * S::TM + lr;  // + 16 i: this lane's accumulator row in the tile
  const int srow = wm * S::TM + (l >> 2), scol = 4 * (l & 3);  // its row and column once permuted
  const int xsrc = ((l >> 2) + 16 * (l & 3)) * 4;                // ds_bpermute byte address
  auto xpose = [&](uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(xsrc, static_cast<int>(v)));
  };
  auto xpose4 = [&](f32x4 v) {
    return f32x4{__uint_as_float(xpose(__float_as_uint(v[0]))), __uint_as_float(xpose(__float_as_uint(v[1]))),
                 __uint_as_float(xpose(__float_as_uint(v[2]))), __uint_as_float(xpose(__float_as_uint(v[3])))};
  };
  auto xpose2 = [&](uint2 v) { return uint2{xpose(v.x), xpose(v.y)}; };
  auto epilogue = [&](int t) __attribute__((always_inline)) {
    // (uniform) the kept geometry, or the tile-list lookup when the issuing side is further on
    const TileGeo g = t == g_iss_t ? g_iss : t + 1 == g_iss_t ? g_prev : geo(t);
    // the extra group stores to its own output, rows counted from its first row
    const bool second = has2 && g.group == a.group2;
    const int64_t ldo = second ? a.ldo2 : a.ldo;
    const int orow0 = second ? g.m0 - a.m2 : g.m0;
    // (a split launch stores K range g.group as its own partial plane)
    const int64_t plane = GROUPED ? 0 : static_cast<int64_t>(g.group) * a.split_plane;
    const __amdgpu_buffer_rsrc_t orsrc =
        buffer_rsrc(static_cast<uint8_t*>(second ? a.out2 : a.out) + plane +
                        static_cast<int64_t>(orow0) * ldo,
                    static_cast<uint32_t>(g.rows * ldo));
    if constexpr (EPI == kEpiStore) {
      const bool f32o = (second ? a.out2_kind : a.out_kind) == kRowF32;
      // Rows of an expert whose rows fit one tile (the y_perm of weight-streaming experts) are
      // stored non-temporally: measured on MI355X, softmax_bf16's combine, which reads them,
      // 0.236 -> 0.216 ms.  Multi-tile experts keep the default policy (all-non-temporal y_perm
      // stores made the fp8_block down GEMM 35% slower), and so do the E4M3-activation kernels,
      // whose registers the extra store path costs (fp8_block down +4%).
      const bool nt_out = !S::kFp8 && GROUPED && g.count == 1;
      // One copy of the store loop per (element type, cache policy), chosen once per tile: with
      // the choice inside the loop every block's permutes had to complete before its own store
      // (one LDS round trip per block); in one straight run they overlap the other blocks'.
      // Rows that are not fp32 are bf16 from the E4M3-activation kernels and fp16 from the
      // bf16 / fp32 kernels (RowKind).
      auto store_tile = [&](auto f32_tag, auto nt_tag) __attribute__((always_inline)) {
        constexpr bool F32 = decltype(f32_tag)::value, NT = decltype(nt_tag)::value;
        // a row block's permutes first, then its stores
#pragma unroll
        for (int i = 0; i < S::FM; ++i) {
          const int row = srow + i * 16;
          if constexpr (F32) {
            f32x4 v[S::FN];
#pragma unroll
            for (int j = 0; j < S::FN; ++j) v[j] = xpose4(acc[i][j]);
#pragma unroll
            for (int j = 0; j < S::FN; ++j) {
              const int col = g.n0 + wn * S::TN + j * 16 + scol;
              const uint32_t off = static_cast<uint32_t>(row * ldo + col * 4);
              if constexpr (NT)
                buffer_store16_nt(orsrc, off, v[j]);
              else
                buffer_store16(orsrc, off, v[j]);
            }
          } else {
            uint2 v[S::FN];
#pragma unroll
            for (int j = 0; j < S::FN; ++j)
              v[j] = xpose2(S::kFp8 ? pack_bf16x4(acc[i][j]) : pack_f16x4(acc[i][j]));
#pragma unroll
            for (int j = 0; j < S::FN; ++j) {
              const int col = g.n0 + wn * S::TN + j * 16 + scol;
              const uint32_t off = static_cast<uint32_t>(row * ldo + col * 2);
              if constexpr (NT)
                buffer_store8_nt(orsrc, off, v[j]);
              else
                buffer_store8(orsrc, off, v[j]);
            }
          }
        }
      };
      constexpr std::true_type kYes{};
      constexpr std::false_type kNo{};
      if constexpr (S::kFp8) {
        if (f32o) store_tile(kYes, kNo); else store_tile(kNo, kNo);
      } else if (f32o) {
        if (nt_out) store_tile(kYes, kYes); else store_tile(kYes, kNo);
      } else {
        if (nt_out) store_tile(kNo, kYes); else store_tile(kNo, kNo);
      }
    } else {
      // h = SiLU(gate) * up: pair p of this wave's fragments is (gate, up) = (2p, 2p+1)
      constexpr int HP = S::FN / 2;
      float hv[S::FM][HP][4];
#pragma unroll
      for (int i = 0; i < S::FM; ++i)
#pragma unroll
        for (int p = 0; p < HP; ++p)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            hv[i][p][e] = silu_fast(acc[i][2 * p][e]) * acc[i][2 * p + 1][e];
      const int hc0 = g.n0 / 2 + wn * HP * 16;  // first h column of this wave
      if constexpr (S::kFp8) {
        // one 128-value group per row and tile: scale = max|h| / 448, codes = E4M3(h / scale).
        // Row maxima: over the lane's own values, then over the four lanes holding the same row
        // (l % 16 alike), then over the WN waves through LDS.
        float* amax = reinterpret_cast<float*>(smem + S::MAIN);
#pragma unroll
        for (int i = 0; i < S::FM; ++i) {
          float m = 0.0f;
#pragma unroll
          for (int p = 0; p < HP; ++p)
#pragma unroll
            for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(hv[i][p][e]));
          m = fmaxf(m, __shfl_xor(m, 16, kWave));
          m = fmaxf(m, __shfl_xor(m, 32, kWave));
          if (kq == 0) amax[(orow + i * 16) * S::WN + wn] = m;
        }
        __syncthreads();
        const int groups = (a.N / 2) / 128;
        const int grp = g.n0 / BN;
#pragma unroll
        for (int i = 0; i < S::FM; ++i) {
          const int row = orow + i * 16;  // this lane's row before the permute
          float m = 0.0f;
#pragma unroll
          for (int w2 = 0; w2 < S::WN; ++w2) m = fmaxf(m, amax[row * S::WN + w2]);
          const float sc = m > 0.0f ? m / 448.0f : 1.0f;
          if (wn == 0 && kq == 0 && row < g.rows)
            (second ? a.out2_scales : a.out_scales)[static_cast<int64_t>(orow0 + row) * groups + grp] = sc;
          // h / sc correctly rounded to fp32 without an fp32 division per value: the fp64
          // product h * RN64(1/sc) lies within 2^-52 (relative) of h / sc, and a quotient of two
          // fp32 numbers is never closer than about 2^-49 to an fp32 rounding midpoint, so
          // rounding that product to fp32 gives the correctly rounded quotient.
          const double rs = 1.0 / static_cast<double>(sc);
          auto quo = [rs](float v) { return static_cast<float>(static_cast<double>(v) * rs); };
#pragma unroll
          for (int p = 0; p < HP; ++p) {
            const float* v = hv[i][p];
            const uint32_t codes = e4m3x4(quo(v[0]), quo(v[1]), quo(v[2]), quo(v[3]));
            buffer_store4(orsrc, static_cast<uint32_t>((srow + i * 16) * ldo + hc0 + p * 16 + scol),
                          xpose(codes));
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < S::FM; ++i)
#pragma unroll
          for (int p = 0; p < HP; ++p) {
            const f32x4 v = f32x4{hv[i][p][0], hv[i][p][1], hv[i][p][2], hv[i][p][3]};
            const int row = srow + i * 16;
            const int col = hc0 + p * 16 + scol;
            // h is read once, by the down GEMM: non-temporal stores (measured on MI355X: the
            // softmax_bf16 gate/up 2-4% faster; no change elsewhere)
            if constexpr (DT == MOE_F32)
              buffer_store16_nt(orsrc, static_cast<uint32_t>(row * ldo + col * 4), xpose4(v));
            else
              buffer_store8_nt(orsrc, static_cast<uint32_t>(row * ldo + col * 2),
                               xpose2(pack_bf16x4(v)));
          }
      }
    }
  };

  // ---------------------------------------------------------------- the pipeline
  // Global step g runs through this workgroup's tiles back to back.  Iteration g: wait for
  // this wave's loads of step g+1 (those of g+2 .. g+NSLOT-1 stay in flight) and for its own
  // fragment reads of step g (lds_dma_wait waits for both); barrier (every wave's step-(g+1)
  // data is in LDS and nobody reads slot g any more); issue step g+NSLOT into slot g; read the
  // fragments of step g+1 while the MFMAs of step g run; after a tile's last step, store it.
  // bf16 and fp32 alternate two whole fragment sets; E4M3 activations (FP8 and MXFP4 experts)
  // alternate part of one (see Frags).  These, and launches of one group, issue the loads of
  // step g+NSLOT between the MFMAs of step g rather than in one burst after the barrier.
  constexpr bool kTwoSets = !S::kFp8;
  constexpr std::integral_constant<int, 0> kEven{};
  constexpr std::integral_constant<int, 1> kOdd{};
  F f0, f1;
  setup(0);
#pragma unroll
  for (int s = 0; s < S::NSLOT; ++s) issue();
  lds_dma_wait<(S::NSLOT - 1) * S::LPS>();
  __syncthreads();
  load(f0, 0);
  int c_slot = 0, c_step = 0, c_tile = 0;
  int after_epi = 0;
  // The refill after the last step reads a slot no one wrote for it: harmless, and it keeps
  // the loop body one basic block for the scheduler.  The vector-memory counter retires loads
  // and stores in issue order, so the wait counts what was issued after the loads it needs:
  // normally the loads of the NSLOT - 2 steps after it; in the NSLOT - 1 iterations after an
  // epilogue also that epilogue's stores, which were issued after the loads of those steps.
  // (Counting fewer than were issued only waits longer.)
  auto iter = [&](F& cur, F& nxt, auto parity) {
    if (after_epi > 0) {
      lds_dma_wait<(S::NSLOT - 2) * S::LPS + S::EPI_STORES>();
      --after_epi;
    } else {
      lds_dma_wait<(S::NSLOT - 2) * S::LPS>();
    }
    __syncthreads();
    constexpr bool kSpread = S::kFp8 || !GROUPED;  // the loads go out between the MFMAs
    if constexpr (kSpread)
      issue_begin();
    else
      issue();
    const int next = c_slot + 1 == S::NSLOT ? 0 : c_slot + 1;
    if constexpr (kTwoSets) {
      step_two_sets(cur, nxt, next, std::integral_constant<bool, kSpread>{});
    } else if constexpr (S::kMx) {
      mma_refill_mx(cur, next, parity);
    } else {
      mma_refill_fp8(cur, next, parity);
    }
    c_slot = next;
    if (++c_step == KB) {
      epilogue(c_tile);
      after_epi = S::NSLOT - 1;
      zero_acc();
      c_step = 0;
      ++c_tile;
    }
  };
  const int total = n_my * KB;
  int gs = 0;
  // steps in pairs, one call site per parity: bf16 and fp32 trade f0 and f1, E4M3 activations
  // alternate the sets inside f0
  for (; gs < total; gs += 2) {
    if constexpr (kTwoSets) iter(f0, f1, kEven); else iter(f0, f0, kEven);
    if (gs + 1 == total) break;
    if constexpr (kTwoSets) iter(f1, f0, kOdd); else iter(f0, f0, kOdd);
  }
  lds_dma_wait<0>();  // no load may still write this workgroup's LDS when it ends
}

// ------------------------------------------------------------------ host side

int gemm_bm(int dtype, int epi, int avg_rows) {
  if (dtype == MOE_F32) return 32;
  if (avg_rows <= 16) return 16;
  if (avg_rows <= 32) return 32;
  if (avg_rows <= 48) return 64;
  return 128;
}

// Persistent grid: as many workgroups as fit on the current device at once (a multiple of the
// XCD count), never more than there are tiles (rounded up to that multiple).  The resident
// count is cached per kernel instantiation and device; concurrent first calls from several
// host threads compute the same value and store it atomically.
constexpr int kMaxDevices = 64;
template <typename Kern>
static int persistent_grid(Kern kernel, int threads, int64_t max_blocks) {
  static std::atomic<int> cache[kMaxDevices];  // 0: not known yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  int resident = dev < kMaxDevices ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (resident == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
      return -1;
    resident = cus * (per_cu > 0 ? per_cu : 1);
    if (dev < kMaxDevices) cache[dev].store(resident, std::memory_order_relaxed);
  }
  int64_t g = max_blocks < resident ? max_blocks : resident;
  g = (g + kNumXcd - 1) / kNumXcd * kNumXcd;
  return static_cast<int>(g < kNumXcd ? kNumXcd : g);
}

template <int DT, int BM, int BN, int EPI, bool G, bool G2 = false>
static hipError_t launch_kernel(const GemmArgs& a, int max_tiles, hipStream_t s) {
  // grouped: worst-case tile count from the caller; one group: exact, for this BM and K split
  if (!G) max_tiles = (a.M + BM - 1) / BM * (a.k_splits > 1 ? a.k_splits : 1);
  const int64_t nb = static_cast<int64_t>(max_tiles) * (a.N / BN);
  if (nb <= 0) return hipSuccess;
  auto kernel = grouped_gemm_kernel<DT, BM, BN, EPI, G, G2>;
  constexpr int threads = gemm_waves<DT, BN>() * kWave;
  const int grid = persistent_grid(kernel, threads, nb);
  if (grid < 0) return hipErrorInvalidDevice;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, s, a);
  return hipGetLastError();
}

// The extra group is instantiated for grouped launches of 16- and 32-row bf16 / E4M3 tiles
// (decode-sized batches, the only ones that merge their shared experts).
template <int DT, int BM, int BN, int EPI, bool G>
static hipError_t launch_one(const GemmArgs& a, int max_tiles, hipStream_t s) {
  if constexpr (G && BM <= 32 && DT != MOE_F32) {
    if (a.has_group2) return launch_kernel<DT, BM, BN, EPI, G, true>(a, max_tiles, s);
  } else {
    if (a.has_group2) return hipErrorInvalidValue;
  }
  return launch_kernel<DT, BM, BN, EPI, G>(a, max_tiles, s);
}

template <int DT, int EPI, bool G>
static hipError_t launch_dt(int bm, const GemmArgs& a, int max_tiles, hipStream_t s) {
  if constexpr (DT == MOE_F32) {
    return launch_one<DT, 32, 128, EPI, G>(a, max_tiles, s);
  } else if constexpr (DT == MOE_FP8_E4M3 || DT == MOE_MXFP4) {
    // E4M3 activations.  The SwiGLU output (N = 2 d_ff, d_ff a multiple of 128) always takes
    // the 256-wide tile so each tile quantises whole 128-value groups of h; 8 waves there, two
    // per SIMD, one wave's promotion and loads overlapping the other's MFMAs.  Rows per tile
    // follow the rows per expert (decode shapes take 16).
    auto wide = [&](auto bm_tag) {
      constexpr int BMv = decltype(bm_tag)::value;
      if constexpr (EPI == kEpiSwiglu) return launch_one<DT, BMv, 256, EPI, G>(a, max_tiles, s);
      else
        return e4m3_tile_n(EPI, a.N) == 256 ? launch_one<DT, BMv, 256, EPI, G>(a, max_tiles, s)
                                            : launch_one<DT, BMv, 128, EPI, G>(a, max_tiles, s);
    };
    switch (bm) {
      case 16: return wide(std::integral_constant<int, 16>{});
      case 32: return wide(std::integral_constant<int, 32>{});
      case 64: return wide(std::integral_constant<int, 64>{});
      default: return wide(std::integral_constant<int, 128>{});
    }
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
  return g ? launch_dt<DT, kEpiStore, true>(bm, a, max_tiles, s)
           : launch_dt<DT, kEpiStore, false>(bm, a, max_tiles, s);
}

hipError_t launch_grouped_gemm(int dtype, int epi, int bm, const GemmArgs& a, int max_tiles,
                               hipStream_t s) {
  if (epi == kEpiStore) {
    // the element types each kernel's store epilogue has (see RowKind)
    const int half = dtype == MOE_FP8_E4M3 || dtype == MOE_MXFP4 ? kRowBF16 : kRowF16;
    if ((a.out_kind != kRowF32 && a.out_kind != half) ||
        (a.has_group2 && a.out2_kind != kRowF32 && a.out2_kind != half))
      return hipErrorInvalidValue;
  }
  switch (dtype) {
    case MOE_F32: return launch_epi<MOE_F32>(epi, bm, a, max_tiles, s);
    case MOE_BF16: return launch_epi<MOE_BF16>(epi, bm, a, max_tiles, s);
    case MOE_MXFP4: return launch_epi<MOE_MXFP4>(epi, bm, a, max_tiles, s);
    default: return launch_epi<MOE_FP8_E4M3>(epi, bm, a, max_tiles, s);
  }
}

}  // namespace moe
