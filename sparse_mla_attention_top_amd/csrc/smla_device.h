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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) char lds_char;

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int kDLatent = 512;

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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Staged cache tile layout (32 rows x NC 16-byte chunks, NC = 8 x segments of
// 128 bytes). Block 4s + g (1 KB) holds segment s of rows 8g..8g+7; inside
// it row r's chunk 8s + cc sits at ((r & 7) * 8 + (cc ^ swz(r))) * 16. So a
// 64-lane global->LDS copy fills one block from 8 whole 128-byte lines (lane
// l: row 8g + l/8). The swizzle is chosen by measurement (SQ_LDS_BANK_CONFLICT
// of a probe kernel per access pattern, same addressing as the kernel):
// swz(r) = r & 6 leaves both the K reads of QK^T (ds_read_b128, rows 16rh +
// li, chunks 4j + lg) and the transposing V reads of P.V (ds_read_b64_tr_b16)
// free of bank conflicts. The earlier ((r >> 2) & 3) << 1 | ((r >> 1) & 1)
// was conflict-free for K but 2-way for V. For the 8-byte reads the counts
// match a model in which 32 lanes are served per cycle from 256 bytes (64
// four-byte banks); the 16-byte reads follow no simple model, hence the probe.
__device__ __forceinline__ int swz(int r) { return r & 6; }
__device__ __forceinline__ int tile_pos(int r, int c) {
  return (4 * (c >> 3) + (r >> 3)) * 1024 + ((r & 7) * 8 + ((c & 7) ^ swz(r))) * 16;
}

// FP8 tile layout (32 rows x 32 chunks of 16 E4M3 codes, 16 KB): the bf16
// layout at half the bytes, block 4s + g (1 KB) for segment s (chunks
// 8s..8s+7) of rows 8g..8g+7, row r's chunk 8s + cc at ((r & 7) * 8 + (cc ^
// swz8(r))) * 16 inside it. swz8(r) = (((r >> 2) & 3) << 1 | ((r >> 1) & 1)) ^
// (((r >> 4) & 1) << 2), measured free of bank conflicts for the K reads
// (within a wave, rows 16rh..16rh+15: bit 4 is fixed, so the pattern is a
// relabelling of chunks of the bf16-style swizzle whose K reads are
// conflict-free) and for the 8-bit transposing V reads of all 32 rows, where
// bit 4 separates rows r and r + 16. (Taking bit 0 from row bit 4 instead left
// both 2-way conflicted.)
__device__ __forceinline__ int swz8(int r) {
  return ((((r >> 2) & 3) << 1) | ((r >> 1) & 1)) ^ (((r >> 4) & 1) << 2);
}
__device__ __forceinline__ int tile_pos8(int r, int c) {
  return (4 * (c >> 3) + (r >> 3)) * 1024 + ((r & 7) * 8 + ((c & 7) ^ swz8(r))) * 16;
}

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
// Transposing 8-bit LDS read: within each 16-lane group, output lane j gets
// byte (j % 8) of the 8-byte words addressed by source lanes 2*i + j/8,
// i = 0..7, as its byte i (checked with a GPU probe of the instruction).
__device__ __forceinline__ i32x2 lds_read_tr8(const lds_char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 __attribute__((address_space(3)))*)p);
}

// 8 OCP E4M3FN codes (byte e of the two dwords w0, w1 is element e) -> 8 bf16
// values, exact (every E4M3FN value, NaN included, is a bf16 value): one
// v_cvt_scalef32_pk_bf16_fp8 at scale 1.0 per pair (a GPU probe matched the
// format's definition on all 256 codes in both halves of the dword).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const u32x4 o = {
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, true)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, true))};
  return __builtin_bit_cast(bf16x8, o);
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

// 4-byte global -> LDS copy (global_load_lds_dword): lane i reads 4 bytes at
// gptr and they land at LDS byte address lds_base + 4*i. Same rules as dma_16b.
__device__ __forceinline__ void dma_4b(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gptr), "s"(lds_base)
               : "m0", "memory");
}

// x[i] * sa[i] (i < 4) and x[i] * sb[i - 4] (i >= 4), in fp32, rounded to
// nearest-even bf16.
__device__ __forceinline__ bf16x8 scale_bf16x8(bf16x8 x, f32x4 sa, f32x4 sb) {
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  const f32x8 f = __builtin_convertvector(x, f32x8);
  const f32x8 sc = __builtin_shufflevector(sa, sb, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_convertvector(f * sc, bf16x8);
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
