// Device-side helpers shared by the gfx950 kernels of the sparse MLA library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace smla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int kWave = 64;
constexpr int kDLatent = 512;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: within each 16-lane group, output lane j gets element
// (j % 4) of the 8-byte words addressed by source lanes 4*i + j/4, i = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr16(const lds_char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)p);
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
// Two 4 x 16-bit transposed reads -> one 8-element bf16 MFMA operand (whole-
// vector bit casts; element-wise casts of the short4 results were lowered
// with elements 2 and 3 replaced by copies of 0 and 1).
__device__ __forceinline__ bf16x8 concat_bf16x4(s16x4 lo, s16x4 hi) {
  const bf16x4 a = __builtin_bit_cast(bf16x4, lo);
  const bf16x4 b = __builtin_bit_cast(bf16x4, hi);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float wave_xor32_max(float v) {
  // exchange with lane ^ 32 (the other half of the wavefront)
  float o = __shfl_xor(v, 32, 64);
  return fmaxf(v, o);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 3-bit swizzle of a tile row: reversal of the bits of (r >> 1) & 7.
__device__ __forceinline__ int swz(int r) {
  const int a = (r >> 1) & 7;
  return ((a & 1) << 2) | (a & 2) | ((a >> 2) & 1);
}

// Staged cache tile layout (32 rows x NC 16-byte chunks, NC = 8 x segments of
// 128 bytes). Block 4s + g (1 KB) holds segment s of rows 8g..8g+7; inside
// it row r's chunk 8s + cc sits at ((r & 7) * 8 + (cc ^ swz(r))) * 16. So a
// 64-lane global->LDS copy fills one block from 8 whole 128-byte lines (lane
// l: row 8g + l/8), a read of one chunk by 16 consecutive rows hits 16
// distinct 16-byte bank groups, and the transposing V reads (4 rows x 2
// chunks per 16 lanes) are conflict-free per 32 lanes.
__device__ __forceinline__ int tile_pos(int r, int c) {
  return (4 * (c >> 3) + (r >> 3)) * 1024 + ((r & 7) * 8 + ((c & 7) ^ swz(r))) * 16;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global loads (the tile DMAs stay in
// flight across it; their completion is waited for with wait_vmcnt).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16-byte global -> LDS copy (global_load_lds_dwordx4): lane i reads 16 bytes
// at gptr + OFF and they land at LDS byte address lds_base + 16*i. The
// instruction's immediate offset is applied to the LDS address too, so M0 is
// set to lds_base - OFF. Issued from asm so the compiler does not order later
// LDS reads behind it; completion is tracked by the caller with wait_vmcnt
// (it counts like any vector load). lds_base must be wave-uniform and >= OFF.
// The s_nop covers the M0-write -> LDS-DMA hazard.
template <int OFF>
__device__ __forceinline__ void dma_16b(const void* gptr, uint32_t lds_base) {
  static_assert(OFF >= 0 && OFF < 4096, "immediate offset range");
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2"
               :
               : "v"(gptr), "s"(lds_base - (uint32_t)OFF), "i"(OFF)
               : "m0", "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace smla
