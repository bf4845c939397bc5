// Index conversion and cache write kernels (gfx950).
//
// Conversion: vLLM "Sparse MLA on Hopper" branch, cutlass_fa3_sparse.py
// forward_mqa step 2 and test_cutlass_fa3_sparse_backend.py TEST 2.5/2.9:
// global = block_table[req][l / B] * stride + l % B, -1 stays -1, plus the
// per-row count of valid entries.
// Cache write: the same branch's do_kv_cache_update (concat_and_cache_mla),
// with the FP8 E4M3 per-tensor and per-token x 128-channel-group formats of
// flashinfer_mla_sparse_sm90.py, and the 656-byte packed FP8 rows of the
// FlashMLA sparse backend (layout: the reading of its size given with FMT 3).
#include "smla_device.h"
#include "smla_internal.h"
#include "smla_lookup.h"

namespace smla {

// One workgroup per token row; entries are independent, the count is a
// workgroup reduction (deterministic, no atomics).
__global__ void __launch_bounds__(256)
convert_indices_kernel(const int32_t* __restrict__ req_id, BlockTable bt,
                       const int32_t* __restrict__ topk_local, int64_t loc_stride, int32_t topk,
                       int32_t* __restrict__ global_out, int64_t out_stride,
                       int32_t* __restrict__ valid_counts) {
  const int t = blockIdx.x;
  const int32_t* src = topk_local + (int64_t)t * loc_stride;
  int32_t* dst = global_out + (int64_t)t * out_stride;
  const int r = req_id[t];
  int cnt = 0;
  // 2048 entries per pass, 8 per thread: all local-index loads of a pass are
  // in flight together, then all block-table lookups, then the stores.
  constexpr int PER = 8;
  for (int base = 0; base < topk; base += 256 * PER) {
    int l[PER];
#pragma unroll
    for (int k = 0; k < PER; k++) {
      const int j = base + threadIdx.x + 256 * k;
      l[k] = (j < topk) ? src[j] : -1;
    }
    int64_t g[PER];
#pragma unroll
    for (int k = 0; k < PER; k++) g[k] = local_slot(bt, r, l[k]);
#pragma unroll
    for (int k = 0; k < PER; k++) {
      const int j = base + threadIdx.x + 256 * k;
      if (j < topk) dst[j] = g[k] >= 0 ? (int32_t)g[k] : -1;
      cnt += (g[k] >= 0);
    }
  }
  if (valid_counts) {
    // wave reduction then across the 4 waves
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
    __shared__ int part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) valid_counts[t] = part[0] + part[1] + part[2] + part[3];
  }
}

// Context-parallel shard filter (vLLM FlashMLA sparse backend, forward_mqa:
// triton_filter_and_convert_dcp_index with dcp_size, dcp_rank,
// cp_kv_cache_interleave_size and compact_valid_to_front). Entry p of row t
// is a request token position; runs of `interleave` positions go to ranks 0,
// 1, .., W-1 in turn and each rank stores its runs back to back, so p is on
// rank (p / I) % W at local position (p / (I W)) I + p % I. Positions stored
// on this rank are converted through this rank's block table as in
// convert_indices_kernel, everything else becomes -1. With compact, the valid
// entries of a row are written first in their order, then -1.
// One workgroup per row, 8 consecutive entries per thread; the compaction
// offsets come from a workgroup prefix sum of the per-thread counts.
__global__ void __launch_bounds__(256)
dcp_filter_kernel(const int32_t* __restrict__ req_id, BlockTable bt,
                  const int32_t* __restrict__ topk_tokens, int64_t in_stride, int32_t topk,
                  int32_t dcp_size, int32_t dcp_rank, int32_t interleave, int32_t compact,
                  int32_t* __restrict__ out, int64_t out_stride, int32_t* __restrict__ valid_counts) {
  __shared__ int s_wave[4];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t* src = topk_tokens + (int64_t)t * in_stride;
  int32_t* dst = out + (int64_t)t * out_stride;
  const int r = req_id[t];
  constexpr int PER = 8;
  int running = 0;                                      // valid entries in earlier passes (uniform)
  for (int base = 0; base < topk; base += 256 * PER) {
    int g[PER];
    int c = 0;
#pragma unroll
    for (int k = 0; k < PER; k++) {
      const int j = base + PER * threadIdx.x + k;
      const int pos = (j < topk) ? src[j] : -1;
      int v = -1;
      if (pos >= 0) {
        const int run = pos / interleave;
        if (run % dcp_size == dcp_rank) {
          const int local = (run / dcp_size) * interleave + (pos - run * interleave);
          const int64_t g = local_slot(bt, r, local);
          if (g >= 0) v = (int32_t)g;
        }
      }
      g[k] = v;
      c += (v >= 0);
    }
    if (!compact) {
#pragma unroll
      for (int k = 0; k < PER; k++) {
        const int j = base + PER * threadIdx.x + k;
        if (j < topk) dst[j] = g[k];
      }
    }
    // workgroup prefix sum of the per-thread counts (thread order = entry order)
    int x = c;
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      const int sw = s_wave[w];
      before += (w < wave) ? sw : 0;
      total += sw;
    }
    __syncthreads();                                    // s_wave is rewritten by the next pass
    if (compact) {
      int at = running + before + x - c;                // exclusive offset of this thread's first valid entry
#pragma unroll
      for (int k = 0; k < PER; k++)
        if (g[k] >= 0) dst[at++] = g[k];
    }
    running += total;
  }
  if (compact)
    for (int j = running + threadIdx.x; j < topk; j += 256) dst[j] = -1;
  if (valid_counts && threadIdx.x == 0) valid_counts[t] = running;
}

// E4M3FN code of an fp32 value: round to nearest, ties to even, |y| >= 448
// saturates to 448, NaN -> 0x7F (sign kept). Integer implementation of the
// OCP E4M3 format (bias 7, 3 mantissa bits, min normal 2^-6, step 2^-9 below).
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  uint32_t u = __builtin_bit_cast(uint32_t, y);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t au = u & 0x7fffffffu;
  if (au > 0x7f800000u) return sign | 0x7fu;
  float a = __builtin_bit_cast(float, au);
  if (a >= 448.0f) return sign | 0x7eu;
  int exp = (int)(au >> 23) - 127;
  uint32_t code;
  if (exp < -6) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);  // subnormal steps of 2^-9, RNE
  } else {
    uint32_t mant = au & 0x7fffffu;
    uint32_t m3 = mant >> 20, rem = mant & 0xfffffu;
    uint32_t up = (rem > 0x80000u) || (rem == 0x80000u && (m3 & 1u));
    code = ((uint32_t)(exp + 7) << 3) + m3 + up;
    if (code > 0x7eu) code = 0x7eu;
  }
  return sign | code;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __builtin_bit_cast(float, b << 16); }

// One wave per token. Lane c8 handles channels [8*c8, 8*c8 + 8).
// FMT 3 (packed rows): the latent's codes at bytes 0..511, its 4 group scales
// at 512..527, the rope channels copied as bf16 to 528..655.
template <int FMT>
__global__ void __launch_bounds__(256)
cache_write_kernel(const uint16_t* __restrict__ kv_c, int64_t kv_c_stride,
                   const uint16_t* __restrict__ k_pe, int64_t k_pe_stride,
                   const int64_t* __restrict__ slot_mapping, int32_t num_tokens, int32_t d_rope,
                   float k_scale, uint8_t* __restrict__ cache, int64_t num_slots,
                   int64_t row_stride, float* __restrict__ group_scales, int64_t gs_stride) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= num_tokens) return;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const int D = kDLatent + d_rope;
  const int nchunk = D / 8;            // 8-channel chunks (D is 512 or 576)
  const int G = (D + 127) / 128;
  // lanes 0..63 take chunks 0..63 (latent); lanes 0..7 also take chunks 64..71 (rope)
  for (int pass = 0; pass < 2; pass++) {
    int c8 = lane + pass * 64;
    bool active = c8 < nchunk;
    uint32_t w[4] = {0, 0, 0, 0};
    if (active) {
      const uint16_t* src = c8 < 64 ? kv_c + (int64_t)t * kv_c_stride + c8 * 8
                                    : k_pe + (int64_t)t * k_pe_stride + (c8 - 64) * 8;
      for (int i = 0; i < 4; i++) w[i] = (uint32_t)src[2 * i] | ((uint32_t)src[2 * i + 1] << 16);
    }
    if (FMT == 0 || (FMT == 3 && pass == 1)) {
      if (active) {
        u32x4 v = {w[0], w[1], w[2], w[3]};
        const int at = FMT == 3 ? 528 + (c8 - 64) * 16 : c8 * 16;
        *(u32x4*)(cache + slot * row_stride + at) = v;
      }
      continue;
    }
    float x[8];
    for (int i = 0; i < 8; i++) x[i] = bf16_bits_to_f32((w[i / 2] >> (16 * (i % 2))) & 0xffffu);
    float sc = k_scale;
    if (FMT == 2 || FMT == 3) {
      // group of 128 channels = 16 consecutive chunks = 16 consecutive lanes
      float m = 0.0f;
      for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(x[i]));
      for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      sc = (m == 0.0f) ? 1.0f : m / 448.0f;
      int g = c8 / 16;
      if (FMT == 2 && active && (c8 % 16) == 0 && g < G) group_scales[slot * gs_stride + g] = sc;
      if (FMT == 3 && active && (c8 % 16) == 0) *(float*)(cache + slot * row_stride + 512 + 4 * g) = sc;
    }
    if (active) {
      uint32_t b[8];
      for (int i = 0; i < 8; i++) b[i] = e4m3_encode(x[i] / sc);
      uint32_t lo = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
      uint32_t hi = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
      uint32_t* dst = (uint32_t*)(cache + slot * row_stride + c8 * 8);
      dst[0] = lo;
      dst[1] = hi;
    }
  }
}

// Planned valid counts (FlashInfer sparse SM90 backend, _kv_lens_host and
// _clamp_work_kv_end): row t of request r = req_id[t] sees
// ctx = seq_lens[r] - query_start_loc[r + 1] + t + 1 tokens, and the pooled
// indexer keeps ctx of them up to topk, else topk + ctx % kpool. A request id
// outside [0, num_reqs) or ctx <= 0 gives 0.
__global__ void __launch_bounds__(256)
planned_counts_kernel(const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ query_start_loc,
                      const int32_t* __restrict__ req_id, int32_t num_reqs, int32_t num_tokens, int32_t topk,
                      int32_t kpool, int32_t* __restrict__ out) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= num_tokens) return;
  const int r = req_id[t];
  int64_t ctx = 0;
  if (r >= 0 && r < num_reqs) ctx = (int64_t)seq_lens[r] - query_start_loc[r + 1] + t + 1;
  if (ctx < 0) ctx = 0;
  out[t] = (int32_t)(ctx <= topk ? ctx : topk + ctx % kpool);
}

// Gather and upconvert of packed FP8 rows into a bf16 workspace (the FP8
// prefill path of the FlashMLA sparse backend: cp_gather_and_upconvert of a
// chunk's contexts, then the bf16 kernel over the workspace). Workspace row
// starts[r] + p gets request r's position p: latent channel c is
// bf16_rne(fl32(e4m3 * scale[c / 128])), the rope channels are copied. One wave
// per row: lane c8 converts latent channels 8 c8 .. 8 c8 + 7, lanes 0..7 copy
// the 8 rope chunks.
__global__ void __launch_bounds__(256)
gather_upconvert_kernel(const uint8_t* __restrict__ cache, int64_t num_slots, int64_t row_stride,
                        BlockTable bt, const int32_t* __restrict__ seq_lens,
                        const int32_t* __restrict__ starts, uint16_t* __restrict__ ws, int64_t ws_rows,
                        int64_t ws_stride) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.y;
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n = min((int64_t)seq_lens[r], (int64_t)bt.max_blocks * bt.block_size);
  if (p >= n) return;
  const int64_t w = (int64_t)starts[r] + p;
  if (w < 0 || w >= ws_rows) return;
  const int64_t slot = local_slot(bt, r, p);
  uint16_t* dst = ws + w * ws_stride;
  if (slot < 0 || slot >= num_slots) {
    *(u32x4*)(dst + 8 * lane) = (u32x4){0u, 0u, 0u, 0u};
    if (lane < 8) *(u32x4*)(dst + 512 + 8 * lane) = (u32x4){0u, 0u, 0u, 0u};
    return;
  }
  const uint8_t* row = cache + slot * row_stride;
  const uint2 codes = *(const uint2*)(row + 8 * lane);
  const float sc = *(const float*)(row + 512 + 4 * (lane >> 4));
  u32x4 rope = {};
  if (lane < 8) rope = *(const u32x4*)(row + 528 + 16 * lane);
  // channels 8 lane + 2i, 8 lane + 2i + 1 from bytes 2i, 2i+1 of the 8 codes
  f32x2 v[4] = {__builtin_amdgcn_cvt_pk_f32_fp8((int)codes.x, false), __builtin_amdgcn_cvt_pk_f32_fp8((int)codes.x, true),
                __builtin_amdgcn_cvt_pk_f32_fp8((int)codes.y, false), __builtin_amdgcn_cvt_pk_f32_fp8((int)codes.y, true)};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; i++) o[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v[i] * sc, bf16x2));
  *(u32x4*)(dst + 8 * lane) = (u32x4){o[0], o[1], o[2], o[3]};
  if (lane < 8) *(u32x4*)(dst + 512 + 8 * lane) = rope;
}

hipError_t launch_planned_counts(const PlannedCountsArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  planned_counts_kernel<<<(a.num_tokens + 255) / 256, 256, 0, stream>>>(
      a.seq_lens, a.query_start_loc, a.req_id, a.num_reqs, a.num_tokens, a.topk, a.kpool, a.out);
  return hipGetLastError();
}

hipError_t launch_gather_upconvert(const UpconvertArgs& a, hipStream_t stream) {
  if (a.num_reqs == 0 || a.max_seq_len <= 0) return hipSuccess;
  dim3 grid((a.max_seq_len + 3) / 4, a.num_reqs);
  const BlockTable bt{a.block_table, a.num_reqs, a.max_blocks, a.bt_row_stride, a.block_size,
                      block_shift_of(a.block_size), a.block_stride_rows};
  gather_upconvert_kernel<<<grid, 256, 0, stream>>>(a.cache, a.num_slots, a.row_stride, bt, a.seq_lens,
                                                    a.starts, a.ws, a.ws_rows, a.ws_stride);
  return hipGetLastError();
}

hipError_t launch_convert(const ConvertArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const BlockTable bt{a.block_table, a.num_reqs, a.max_blocks, a.bt_row_stride, a.block_size,
                      block_shift_of(a.block_size), a.block_stride_rows};
  convert_indices_kernel<<<a.num_tokens, 256, 0, stream>>>(a.req_id, bt, a.topk_local, a.topk_local_stride, a.topk,
                                                           a.global_out, a.global_stride, a.valid_counts);
  return hipGetLastError();
}

hipError_t launch_dcp_filter(const DcpFilterArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const BlockTable bt{a.block_table, a.num_reqs, a.max_blocks, a.bt_row_stride, a.block_size,
                      block_shift_of(a.block_size), a.block_stride_rows};
  dcp_filter_kernel<<<a.num_tokens, 256, 0, stream>>>(a.req_id, bt, a.topk_tokens, a.in_stride, a.topk, a.dcp_size,
                                                      a.dcp_rank, a.interleave, a.compact ? 1 : 0, a.out,
                                                      a.out_stride, a.valid_counts);
  return hipGetLastError();
}

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  dim3 grid((a.num_tokens + 3) / 4);
  switch (a.kv_format) {
    case 0:
      cache_write_kernel<0><<<grid, 256, 0, stream>>>(a.kv_c, a.kv_c_stride, a.k_pe, a.k_pe_stride,
                                                      a.slot_mapping, a.num_tokens, a.d_rope, a.k_scale,
                                                      a.cache, a.num_slots, a.row_stride, a.group_scales, a.gs_stride);
      break;
    case 1:
      cache_write_kernel<1><<<grid, 256, 0, stream>>>(a.kv_c, a.kv_c_stride, a.k_pe, a.k_pe_stride,
                                                      a.slot_mapping, a.num_tokens, a.d_rope, a.k_scale,
                                                      a.cache, a.num_slots, a.row_stride, a.group_scales, a.gs_stride);
      break;
    case 2:
      cache_write_kernel<2><<<grid, 256, 0, stream>>>(a.kv_c, a.kv_c_stride, a.k_pe, a.k_pe_stride,
                                                      a.slot_mapping, a.num_tokens, a.d_rope, a.k_scale,
                                                      a.cache, a.num_slots, a.row_stride, a.group_scales, a.gs_stride);
      break;
    case 3:
      cache_write_kernel<3><<<grid, 256, 0, stream>>>(a.kv_c, a.kv_c_stride, a.k_pe, a.k_pe_stride,
                                                      a.slot_mapping, a.num_tokens, a.d_rope, a.k_scale,
                                                      a.cache, a.num_slots, a.row_stride, a.group_scales, a.gs_stride);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace smla
