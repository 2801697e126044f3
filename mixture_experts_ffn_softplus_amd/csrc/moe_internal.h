// moe_internal.h -- host-side launchers shared between the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ---- router (route.hip)
struct RouteArgs {
  const float* logit_bias;   // [E] added to the logits, or null
  const float* select_bias;  // [E] or null
  int32_t* ids;              // [T, k]
  float* weights;            // [T, k]
  int T, E, k;
  int score, renorm;
  float gamma;
  // choice by a fixed token-id table instead of the top k: ids[t] = table[token_ids[t]]
  const int32_t* token_ids;  // [T], or null (top-k choice)
  const int32_t* table;      // [vocab, k]
  int vocab;
  // block-scaled FP8 activations of the same tokens, written by the same waves when xq is set:
  // x [T, d] bf16 -> xq [T, d] E4M3 codes and xq_scales [T, d/128]
  const uint16_t* x;
  uint8_t* xq;
  float* xq_scales;
  int d;
  // logits given as `splits` partial planes `plane` floats apart (a K-split router GEMM), added
  // in plane order before the choice (0 or 1: one plane)
  int splits;
  int64_t plane;
};
enum RouterKind { kRouterF32 = 0, kRouterBF16 = 1, kRouterBF16HiLo = 2 };
// Scoring + top-k of fp32 logits rows `ld` apart (plus logit_bias), and the FP8 activations
// when a.xq is set; copy: optional [T, E] copy of the biased logits (with a.splits > 1: of the
// planes' sum).
hipError_t launch_topk(const RouteArgs& a, const float* logits, int ld, float* copy,
                       hipStream_t s);
// Balancing step of the fp32 selection bias from the permutation's expert offsets [E+1]:
// bias[e] += speed * sign(A - E * load_e), A = offsets[E].
hipError_t launch_bias_update(const int32_t* offsets, int E, float speed, float* bias,
                              hipStream_t s);

// ---- permutation (permute.hip)
int permute_num_chunks(int T, int k);
hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                          int32_t* perm_token, int32_t* inv_perm, int32_t* hist,
                          hipStream_t s);
// The permutation and (when tiles is set) the tile list in one workgroup, for small batches:
// permute_small_ok(T * k, E).  Same outputs as launch_permute + launch_tile_list.
bool permute_small_ok(int64_t A, int E);
hipError_t launch_permute_small(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                                int32_t* perm_token, int32_t* inv_perm, int bm, int extra_rows,
                                int4* tiles, int32_t* tiles_count, hipStream_t s);
// extra_rows > 0 appends group E: rows [offsets[E], offsets[E] + extra_rows) (the shared
// experts' tokens, after the routed rows).
hipError_t launch_tile_list(const int32_t* offsets, int E, int bm, int extra_rows, int4* tiles,
                            int32_t* tiles_count, hipStream_t s);

// ---- grouped GEMMs (gemm.hip)
enum Epilogue { kEpiSwiglu = 0, kEpiStore = 1 };
// Element type of the rows the store epilogue writes and the combine reads back (y_perm, the
// shared experts' output, router logits): the bf16 / fp32 GEMMs store fp32 or fp16 rows, the
// E4M3-activation GEMMs fp32 or bf16 rows.
enum RowKind { kRowBF16 = 0, kRowF32 = 1, kRowF16 = 2 };

struct GemmArgs {
  // A: activations, K-contiguous rows
  const void* A;
  int64_t a_bytes;            // bytes of the whole A operand (< 4 GiB)
  int64_t lda;                // bytes per A row
  const int32_t* a_map;       // row of the M space -> A row, or null (identity)
  const float* a_scales;      // FP8: [A rows, K/128]
  // B: packed weights of each group, [N, K] K-contiguous
  const void* B;
  int64_t b_group_stride;     // bytes per group
  int64_t ldb;                // bytes between rows of B
  int b_stream;               // B of a group with one row tile: load it non-temporally
  const float* b_scales;      // FP8: [N/16, K/128] per group (one per 16 packed rows)
  int64_t bs_group_stride;    // floats per group
  const uint8_t* b_e8m0;      // MXFP4: E8M0 scales [N, K/32] per group
  int64_t be_group_stride;    // bytes per group
  int K, N;
  // tiles of rows: a device list {group, first row, rows} (grouped), or one group of M rows
  const int4* tiles;          // null: one group, rows [0, M)
  const int32_t* tiles_count; // device count of `tiles`
  int M;
  // output
  void* out;
  int64_t ldo;                // bytes per output row
  float* out_scales;          // FP8 h: [rows, out_cols/128]
  int out_kind;               // store epilogue: RowKind of the stored rows
  // A rows repeat every a_steps K-steps when > 0 (0: no repeat)
  int a_steps;
  // One group only (tiles null): K split into k_splits equal ranges of whole K-steps (0 or 1:
  // no split), range s stored as its own partial product at out + s * split_plane bytes.
  int k_splits;
  int64_t split_plane;
  // One extra group after the routed experts when has_group2 (group index group2): the shared
  // experts, whose rows are the tokens in order.  Its rows [m2, m2 + rows) of the M space take
  // A row (r - m2) of A2 (no a_map), the weights B2 (+ scales), and store to out2 (+ scales)
  // with row stride ldo2 (rows of RowKind out2_kind, store epilogue).
  int has_group2;
  int group2;
  int m2;
  const void* A2;
  int64_t a2_bytes;
  const float* a2_scales;
  const void* B2;
  const float* b2_scales;
  const uint8_t* b2_e8m0;
  void* out2;
  int64_t ldo2;
  float* out2_scales;
  int out2_kind;
};

// dtype: MOE_F32 / MOE_BF16 / MOE_FP8_E4M3 / MOE_MXFP4 (E4M3 activations, E2M1 weights).
// max_tiles: upper bound of the device
// tile count (grouped) for sizing the persistent grid.
int gemm_bm(int dtype, int epi, int avg_rows);
// Columns per output tile of the E4M3-activation GEMMs (FP8 and MXFP4 experts): 256 for the
// SwiGLU output (each tile quantises whole 128-value groups of h) and wherever N allows, else
// 128.  The MXFP4 weight packing lays its column tiles out by the same rule.
inline int e4m3_tile_n(int epi, int N) { return epi == kEpiSwiglu || N % 256 == 0 ? 256 : 128; }
hipError_t launch_grouped_gemm(int dtype, int epi, int bm, const GemmArgs& a, int max_tiles,
                               hipStream_t s);

// ---- un-permute and weighted combine (combine.hip)
// out[t] = G[t] * base[t] + sum_j w[t*k+j] * y[inv[t*k+j]] over d columns; y rows of RowKind
// y_kind, base [T, d] of RowKind base_kind (fp32 under fp16 or fp32 rows, bf16 under bf16 rows) or
// null, out fp32 (out_f32) or bf16.  G = 1, or with gate_vec
// G[t] = sigmoid(x~[t] . gate_vec): x~ fp32 / bf16 (x_kind 0 / 1) or E4M3 codes times their
// per-128 scales (x_kind 2); gate_vec fp32 or bf16 (gate_f32).
struct CombineArgs {
  const void* y;
  int y_kind;
  int base_kind;
  const int32_t* inv;
  const float* w;
  int k;
  const void* base;
  const void* gate_vec;
  bool gate_f32;
  const void* x;
  int x_kind;
  const float* x_scales;
  void* out;
  bool out_f32;
  int T, d;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

// ---- packing (pack.hip)
// Packed gate/up of one group: [2F, K] K-contiguous, rows in blocks of 16 alternating
// gate / up: packed row p = 32c + j (j < 16) is gate column 16c + j, p = 32c + 16 + j is up
// column 16c + j.  F = sub * C: `sub` source experts of C columns each are concatenated
// (the shared experts).  Sources are logical [K, C] (row-major), `groups` of them in a row
// per operand, each group taking `sub` consecutive sources.
hipError_t launch_pack_gate_up(const void* gate, const void* up, void* dst, int K, int C,
                               int sub, int groups, int esize, hipStream_t s);
// Packed down of one group: [N, F] with F = sub * C; packed[n][s*C + c] = down_s[c][n],
// sources logical [C, N].
hipError_t launch_pack_down(const void* down, void* dst, int N, int C, int sub, int groups,
                            int esize, hipStream_t s);
// MXFP4 (N-major rows of `row_bytes`, a multiple of 4): gate/up rows [C] per source expert
// interleaved 16 at a time into [2F, row] per group (F = sub * C, `sub` sources a group), and
// down rows [N] per source concatenated along K into [N, sub * row] per group.  tile_rows = 0
// keeps each group's rows in row-major order; tile_rows = BN (rows a multiple of BN, packed
// rows a multiple of step_bytes = b) stores them by column tile and K-step: piece s of row n
// lands at ((n / BN) * (row / b) + s) * BN * b + (n % BN) * b, so each step of a tile is one
// contiguous BN * b-byte block (E2M1 weights: b = 64; their E8M0 scales: b = 4).
hipError_t launch_pack_rows_gate_up(const void* gate, const void* up, void* dst, int C, int sub,
                                    int groups, int row_bytes, int tile_rows, int step_bytes,
                                    hipStream_t s);
hipError_t launch_pack_rows_concat(const void* src, void* dst, int N, int sub, int groups,
                                   int row_bytes, int tile_rows, int step_bytes, hipStream_t s);
// Router [d, E] -> [E_pad, d] (rows >= E zero).  hilo: fp32 source split into bf16 hi and
// lo = bf16(w - hi), one [E_pad, 2d] bf16 matrix; otherwise the element type is kept.
hipError_t launch_pack_router(const void* wr, int esize, int hilo, void* dst, int d, int E,
                              int E_pad, hipStream_t s);
// FP8 block scales, one per 16 packed rows and 128 K values:
//   gate/up: dst[g][p16][kb] from gate/up scales [K/128, C/128] of the source expert;
//   down:    dst[g][n16][kb] from down scales [C/128, N/128].
hipError_t launch_pack_scales_gate_up(const float* gs, const float* us, float* dst, int K, int C,
                                      int sub, int groups, hipStream_t s);
hipError_t launch_pack_scales_down(const float* ds, float* dst, int N, int C, int sub,
                                   int groups, hipStream_t s);

}  // namespace moe
