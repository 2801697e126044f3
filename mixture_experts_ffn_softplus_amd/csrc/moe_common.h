// moe_common.h -- device building blocks shared by the gfx950 kernels of the MoE block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kNumXcd = 8;     // MI355X: 8 XCDs, workgroups dispatched round-robin over them
constexpr int kBlockK = 128;   // bytes of K per pipeline step (= one FP8 scale block)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// Four E4M3FN codes (byte i from value i): the nearest code, ties to even, saturating at
// +-448 -- the hardware conversion (round to nearest even) after a clamp to +-448 (NaN inputs
// unsupported).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const float lim = 448.0f;
  a = fminf(fmaxf(a, -lim), lim);
  b = fminf(fmaxf(b, -lim), lim);
  c = fminf(fmaxf(c, -lim), lim);
  d = fminf(fmaxf(d, -lim), lim);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return static_cast<uint32_t>(r);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = e == 0 ? static_cast<float>(m) * 0.001953125f
                     : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// ----------------------------------------------------------------------------- MFMA
// 16x16 output blocks, fp32 accumulate.  Lane l holds output column (l % 16) and
// rows 4*(l / 16) + i, i = 0..3.  Operands: lane l supplies row (A) / column (B)
// (l % 16) and one K-slice chosen by (l / 16); A and B use the same K-slices.

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// E4M3 x E4M3, K = 128 per instruction (format selectors 0 = E4M3, unit scales).
__device__ __forceinline__ f32x4 mfma_fp8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// E2M1 x E4M3 (format selectors 4 and 0), K = 128, from zero.  A: 16 bytes per lane, K
// 32*(l/16)..+31 of row l%16, two codes a byte, the lower K in the low nibble, its 32 values
// scaled by the lane's E8M0 byte `sa`; B: 32 bytes per lane, bytes 0-15 holding K 16*(l/16)..
// and bytes 16-31 K 64+16*(l/16).. of column l%16 (B's scale field is 127 = 2^0).
__device__ __forceinline__ f32x4 mfma_mx(i32x4 a, i32x8 b, int sa) {
  const i32x8 a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, f32x4{0.f, 0.f, 0.f, 0.f}, 4,
                                                          0, 0, sa, 0, 127);
}

// ----------------------------------------------------------------------------- buffer loads
// A buffer resource covers [base, base + bytes); a load past `bytes` returns zeros instead of
// touching memory.  Offsets are 32-bit: a per-lane byte offset plus a wave-uniform one, so a
// pipelined loop advances with one scalar add and no per-lane address arithmetic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
// Cache policy bits of a load: 0 = default, kNonTemporal = streamed once (on MI355X a pure
// streaming read reaches ~7.1 TB/s with it against ~6.2 TB/s without).
constexpr int kNonTemporal = 2;
template <int AUX = 0>
__device__ __forceinline__ i32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff),
                                               AUX);
}

// Stores through a buffer resource: bytes at or past the resource's end are dropped.
__device__ __forceinline__ void buffer_store16(__amdgpu_buffer_rsrc_t r, uint32_t voff, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, static_cast<int>(voff), 0, 0);
}
__device__ __forceinline__ void buffer_store8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint2 v) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(i32x2{static_cast<int>(v.x), static_cast<int>(v.y)}, r,
                                        static_cast<int>(voff), 0, 0);
}
// The same stores marked non-temporal (streamed: written once, read once by a later kernel).
__device__ __forceinline__ void buffer_store16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, static_cast<int>(voff), 0,
                                         kNonTemporal);
}
__device__ __forceinline__ void buffer_store8_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint2 v) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(i32x2{static_cast<int>(v.x), static_cast<int>(v.y)}, r,
                                        static_cast<int>(voff), 0, kNonTemporal);
}
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(static_cast<int>(v), r, static_cast<int>(voff), 0, 0);
}
// Two fp32 values as bf16 (round to nearest even, the first in the low half): one packed
// conversion instruction for the pair.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ uint2 pack_bf16x4(f32x4 v) {
  return uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
// The same as IEEE binary16 (round to nearest even; magnitudes from 65520 up become inf).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}
__device__ __forceinline__ uint2 pack_f16x4(f32x4 v) {
  return uint2{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
}

// ----------------------------------------------------------------------------- LDS DMA
// Buffer loads whose data goes straight to LDS: lane l's BYTES land at (lds + BYTES * l), the
// base taken from M0.  Issued from inline asm on purpose: the compiler cannot tell which LDS
// bytes such a load writes, so for its own bookkeeping it would wait for every one in flight
// before any LDS read, serialising a multi-slot ring.  These loads have no register results;
// their completion is awaited explicitly with lds_dma_wait (vector-memory counts complete in
// issue order), followed by a barrier.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return i32x4{uniform(static_cast<int>(static_cast<uint32_t>(p))),
               uniform(static_cast<int>(static_cast<uint32_t>(p >> 32) & 0xFFFFu)),
               uniform(static_cast<int>(bytes)), 0x00020000};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const uint8_t*)(p)));
}
// M0 is written here and listed nowhere: no compiler-generated code in these kernels keeps a
// value in M0 (LDS instructions ignore it on gfx9 and later, and no register array is indexed
// dynamically).
template <int BYTES, bool NT>
__device__ __forceinline__ void lds_dma(i32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  static_assert(BYTES == 16 || BYTES == 4, "dwordx4 or dword");
  const int l = uniform(static_cast<int>(lds)), so = uniform(static_cast<int>(soff));
  rsrc = i32x4{uniform(rsrc[0]), uniform(rsrc[1]), uniform(rsrc[2]), uniform(rsrc[3])};
  if constexpr (BYTES == 16 && NT)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :: "s"(l), "v"(voff), "s"(rsrc), "s"(so) : "memory");
  else if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(l), "v"(voff), "s"(rsrc), "s"(so) : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(l), "v"(voff), "s"(rsrc), "s"(so) : "memory");
}
// Scalar loads of wave-uniform data, for use inside a loop that keeps direct-to-LDS loads in
// flight: they are counted by lgkmcnt, not vmcnt, so waiting for them never drains the vector
// memory pipeline.  Each waits for its own data inside the asm block.
__device__ __forceinline__ i32x4 scalar_load16(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const int lo = uniform(static_cast<int>(static_cast<uint32_t>(a)));
  const int hi = uniform(static_cast<int>(static_cast<uint32_t>(a >> 32)));
  const uint64_t ua = (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
  i32x4 v;
  asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ua) : "memory");
  return v;
}
// Eight consecutive int32 at byte offset `off` of buffer `rsrc` (zeros past its end).
__device__ __forceinline__ i32x8 scalar_buffer_load32(i32x4 rsrc, uint32_t off) {
  rsrc = i32x4{uniform(rsrc[0]), uniform(rsrc[1]), uniform(rsrc[2]), uniform(rsrc[3])};
  const int so = uniform(static_cast<int>(off));
  i32x8 v;
  asm volatile("s_buffer_load_dwordx8 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(rsrc), "s"(so) : "memory");
  return v;
}
// Element `idx` (0..7, per lane) of eight wave-uniform values.
__device__ __forceinline__ int select8(i32x8 v, int idx) {
  int r = v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) r = idx == i ? v[i] : r;
  return r;
}

// Wait until at most N vector-memory operations of this wave are outstanding and every LDS
// operation of this wave has completed.  The vector counter retires loads and stores in issue
// order, so vmcnt(N) means every operation but the N most recently issued is complete.
// Before the barrier that precedes refilling an LDS slot both halves are needed: the loads of
// the slot about to be read must have landed, and this wave's own reads of the slot about to
// be refilled must have executed.  s_barrier waits on no counter, and the compiler adds no LDS
// wait at a workgroup barrier (LDS instructions of all waves execute in one order), but a
// direct-to-LDS load writes LDS outside that order: a refill that returns early (zeros past a
// tile's last row, an L2 hit) could otherwise overwrite a slot that another wave's fragment
// read, issued before the barrier, has not yet reached.
template <int N>
__device__ __forceinline__ void lds_dma_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"(N) : "memory");
}

// ----------------------------------------------------------------------------- wave utilities

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Logical block id with the blocks of one XCD made contiguous: hardware block b
// runs on XCD b % 8, so consecutive logical ids (neighbouring tiles that share
// operands) land in the same XCD's L2.  Bijective on [0, n).
__device__ __forceinline__ int xcd_remap(int b, int n) {
  int q = n / kNumXcd, r = n % kNumXcd;
  int xcd = b % kNumXcd, local = b / kNumXcd;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// SiLU from the hardware exp2 and reciprocal (a few ulp of fp32; its result is rounded to bf16
// or E4M3 next, or kept in fp32 well inside the fp32 tolerance).
__device__ __forceinline__ float silu_fast(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace moe
