// Sparse MLA forward kernel for gfx950 (MI355X).
//
// Computes, per query token t and head i, attention over the token's own
// top-k cache slots (vLLM "Sparse MLA on Hopper" branch, cutlass_fa3_sparse.py
// _forward_fa3: score = q_rope . k_rope + q_nope . c_kv, out = softmax(score *
// scale) . c_kv; FlashMLA sparse API docs: heads padded to 64 or 128, LSE per
// (token, head), empty rows give (0, -inf)).
//
// One workgroup = one (token, 64-head block, split), 8 waves in two roles,
// two waves per SIMD (waves w and w+4 share a SIMD):
//   S-waves (0..3): Q^T in registers for the whole kernel. Per tile of 32
//     rows, S^T = K.Q^T on v_mfma_f32_16x16x32_bf16 (wave (hg, rh) scores rows
//     16rh..16rh+15 against heads 32hg..32hg+31, A = K from LDS), then the
//     softmax (base 2, fixed per-head reference, see below) and P (bf16) into
//     a double-buffered LDS block.
//   O-waves (4..7): the tile copies (global_load_lds_dwordx4 straight into
//     LDS), and O += P.V one tile behind the S-waves: wave 4+w owns O for all
//     64 heads x latent channels 128w..128w+127 in accumulator registers,
//     A = P from LDS, B = V read with ds_read_b64_tr_b16 from the same tile
//     (V is the first 512 channels of the gathered row, no second gather).
//   FP8 caches: the tile stays in LDS as E4M3 codes (half the bytes of a
//     bf16 tile) and every MFMA operand is converted to bf16 as it is read:
//     K with ds_read_b128 (16 codes, two k-steps), V with the 8-bit transposing
//     read ds_read_b64_tr_b8 (8 codes, one n-block). The FlashMLA-style design
//     of dequantising into a bf16 tile first costs an LDS round trip per tile.
// So on every SIMD one wave's softmax / conversion work overlaps the other's
// MFMAs, and one barrier per tile orders both roles. Before the loop all
// threads stage the row's indices (converting request-local indices through
// the block table when one is given) and the S-waves load Q.
#include "smla_device.h"
#include "smla_internal.h"
#include "smla_lookup.h"

#include <hip/hip_ext.h>
#include <math.h>

#include <mutex>

namespace smla {

struct KParams {
  const uint16_t* q_nope;
  int64_t qn_st, qn_sh;
  const uint16_t* q_rope;
  int64_t qr_st, qr_sh;
  const uint8_t* kv;
  int64_t kv_row_stride, num_slots;
  const float* group_scales;   // group-scaled FP8: scale g of slot s at [s * gs_stride + g]
  int64_t gs_stride;
  const int32_t* indices;
  int64_t idx_stride;
  int32_t topk;
  const int32_t* topk_length;
  // fused index conversion (bt.table != nullptr: indices are request-local)
  const int32_t* req_id;
  BlockTable bt;
  int32_t num_tokens, num_heads;
  float scale_log2;   // softmax scale * log2(e)
  float out_mult;
  // logit softcap c (softcap_on): base-2 logits t = s * scale_log2 become
  // c1 tanh(t / c1), c1 = c log2(e), as c1 - 2 c1 / (1 + 2^(2t / c));
  // cap_a = 2 scale_log2 / c (applied to s), cap_t = 2 / c (applied to t)
  int32_t softcap_on;
  float cap_a, cap_t, cap_c1;
  const float* sinks;  // [H] extra logits with zero value rows (direct output only), or nullptr
  int32_t splits, longest_first;
  int32_t head_blocks;  // 1 (<= 64 heads) or 2
  int32_t xcd_group;    // 1: all workgroups of token t run on XCD t % 8
  uint16_t* out;
  int64_t out_st, out_sh;
  float* lse;
  int64_t lse_st;
  uint16_t* part_o;     // bf16 [splits][T][H][512]
  float* part_lse;
};

__device__ __forceinline__ bf16x8 lds_ld128(const lds_char* p) {
  return *(const __attribute__((address_space(3))) bf16x8*)p;
}
__device__ __forceinline__ void lds_st64(lds_char* p, uint64_t v) {
  *(__attribute__((address_space(3))) uint64_t*)p = v;
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
// acc + the two bf16 halves of v, in one v_dot2c_f32_bf16 (v . (1, 1) + acc).
__device__ __forceinline__ float sum_bf16x2(uint32_t v, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v), __builtin_bit_cast(bf16x2, 0x3f803f80u), acc,
                                         false);
}

// Reference maximum policy. O and the running sum are accumulated against a
// per-head reference m (base-2 units) fixed at the first tile; p = 2^(t - m)
// stays finite in bf16/fp32 while t - m <= 64. If a row sum of a pass exceeds
// 2^64 (so some later score may exceed m + 64) or is not finite, the workgroup
// restarts with a new reference: m + log2 of the pass's largest per-lane row
// sum (at most 8 above the exact maximum), or, if that sum is not
// finite or zero, the exact maximum from a max-only pass.
constexpr float kRefLimit = 18446744073709551616.0f;    // 2^64
constexpr int kLatKS = kDLatent / 32;                  // k-steps over the 512 latent channels
constexpr int kLatBytes = kTileRows * kDLatent * 2;    // bf16 latent part of a tile (32 KB)
constexpr int kRopeBytes = kTileRows * 64 * 2;         // bf16 rope part of a tile (4 KB)

// Buffers of one workgroup.
//   bf16 cache: a tile is its latent part (chunks 0..63 of every row,
//     tile_pos layout, 32 KB) plus, for D = 576, its rope part (chunks 64..71,
//     4 KB) in a separate ring, since the latent part is read one tile longer
//     (by P.V): 4 latent + 3 rope buffers; tile i+2 is copied during tile i.
//   FP8 cache: a tile stays in LDS as it was copied, and each MFMA operand is
//     converted to bf16 as it is read. One buffer holds the tile's latent
//     codes (tile_pos8 layout, 16 KB), its rope part (D = 576: 64 E4M3 codes
//     per row, 2 KB; packed rows: 64 bf16 channels per row, 4 KB) and, in the
//     group formats, its scales ([group][row] fp32). 5 buffers; tile i+3 is
//     copied during tile i.
// The epilogue stages O (64 heads x 512 channels, bf16) in the first 64 KB of
// the latent ring and the row sums after it.
template <int D, int FMT>
struct Shape {
  static constexpr bool F8 = FMT != 0;
  static constexpr bool ROPE = D > kDLatent;
  static constexpr bool PACKED = FMT == 3;
  static constexpr bool GROUP = FMT == 2 || FMT == 3;
  static constexpr bool ROPE8 = F8 && ROPE && !PACKED; // rope part as E4M3 codes
  static constexpr int QKS = D / 32;                   // k-steps of the QK contraction
  static constexpr int G = PACKED ? 4 : (D + 127) / 128;   // scale groups (packed: the latent's)
  // bf16 ring
  static constexpr int NLAT = F8 ? 0 : 4;
  static constexpr int NROPE = (!F8 && ROPE) ? 3 : 0;
  // FP8 ring: byte offsets inside a tile buffer
  static constexpr int ROPE_AT = 16 * 1024;
  static constexpr int SC_AT = ROPE_AT + (ROPE8 ? 2048 : (PACKED ? 4096 : 0));
  static constexpr int TB = SC_AT + (GROUP ? (G * kTileRows * 4 + 255) / 256 * 256 : 0);
  // tiles copied ahead (FP8: 3; 4 and 5 measured no faster on the decode shapes)
  static constexpr int PD = F8 ? 3 : 2;
  static constexpr int NBUF = PD + 2;
  static constexpr int NSC = GROUP ? (G + 1) / 2 : 0;  // scale copies per tile, by O-waves 0 .. NSC-1
  // copy instructions per O-wave per tile (FP8: besides the scale copy)
  static constexpr int NDMA = F8 ? 4 + (ROPE ? 1 : 0) : D / 64;
  static constexpr int RING = F8 ? NBUF * TB : NLAT * kLatBytes;
  static_assert(D == kDLatent || D == kDLatent + 64, "rope part must be 64 channels");
  static_assert(!PACKED || ROPE, "packed rows carry the rope part");
  static_assert(G * kTileRows * 4 <= 1024, "the scales of a tile fit 1 KB");
  static_assert(RING >= 64 * 1024 + 2048, "the epilogue stages O and the row sums in the ring");
  static_assert(!F8 || NBUF >= PD + 2, "tile i+PD must land in a buffer that no role still reads");
};

// Byte offsets inside a packed row.
constexpr int kPackedScalesAt = 512;
constexpr int kPackedRopeAt = 528;

// FMT: 0 = bf16 cache, 1 = E4M3 with one per-tensor scale, 2 = E4M3 with
// per-row x 128-channel-group scales in a separate array, 3 = packed rows
// (E4M3 latent with its 4 group scales and the bf16 rope part in the row).
template <int D, int FMT>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
smla_attn_kernel(KParams p) {
  using S = Shape<D, FMT>;
  constexpr bool F8 = S::F8;
  constexpr int QKS = S::QKS, NLAT = S::NLAT, NROPE = S::NROPE, PD = S::PD;

  __shared__ __attribute__((aligned(16))) char s_lat[S::RING];
  __shared__ __attribute__((aligned(16))) char s_rope[(NROPE ? NROPE * kRopeBytes : 16)];
  __shared__ __attribute__((aligned(16))) char s_p[2 * 4 * 64 * 16];   // P(i) in block i & 1, [mblock][lane]
  __shared__ int s_idx[kMaxTopk];
  __shared__ int s_flag;
  __shared__ int s_need;    // a flagged pass's own maxima are not usable: a max-only pass is needed
  __shared__ int s_last[8];

  lds_char* lat = (lds_char*)s_lat;
  lds_char* rope = (lds_char*)s_rope;
  lds_char* pbuf = (lds_char*)s_p;
  // per-head maxima exchanged by the S-waves (only while P block 1 is unused)
  float* s_m = (float*)(s_p + 4 * 64 * 16);
  // epilogue: row sums and inverse sums after the staged O block
  float* s_l = (float*)(s_lat + 64 * 1024);
  float* s_inv = s_l + 4 * 32;
  float* s_lb = s_inv + 64;

  const int w = threadIdx.x >> 6;
  const int l = threadIdx.x & 63;
  const int lg = l >> 4, li = l & 15;
  const bool is_s = w < 4;
  const int wr = w & 3;                         // index within the role
  const int hg = wr & 1, rh = wr >> 1;          // S role: 32-head group, 16-row half
  const int T = p.num_tokens, H = p.num_heads;

  // ---- work item. The head blocks and splits of one token run on one XCD
  //      (blocks are dispatched round-robin over the 8 XCDs, so block b runs on
  //      XCD b % 8): its Q and its cache rows are fetched from HBM once and then
  //      hit that XCD's L2. Token t goes to XCD t % 8 (with fewer than 8 tokens
  //      the blocks are dealt in token order instead).
  int t, split, hblk;
  {
    const int b = blockIdx.x;
    const int per_tok = p.head_blocks * p.splits;
    int rem;
    if (p.xcd_group) {
      const int k = b >> 3;
      const int u = k / per_tok;
      rem = k - u * per_tok;
      t = 8 * u + (b & 7);
    } else {
      t = b / per_tok;
      rem = b - t * per_tok;
    }
    if (t >= T) return;
    hblk = rem / p.splits;
    split = rem - hblk * p.splits;
    if (p.longest_first) t = T - 1 - t;
  }
  const int hb = 64 * hblk;

  // ---- the row's index entries -> LDS (-1 marks an entry that does not take
  //      part), loaded without waiting for the row length. A split takes its
  //      share of the entries up to the last valid one, so rows with an
  //      invalid tail (short rows, a context-parallel shard compacted to the
  //      front) spread over the splits too; tiles past the last valid entry
  //      are not visited.
  const int32_t* irow = p.indices + (int64_t)t * p.idx_stride;
  constexpr int kIdxPerThread = kMaxTopk / 512;
  int gi[kIdxPerThread];
  const bool convert = p.bt.table != nullptr;
  const int rq = convert ? p.req_id[t] : 0;                // loaded with the indices
#pragma unroll
  for (int k = 0; k < kIdxPerThread; k++) {
    const int j = threadIdx.x + 512 * k;
    gi[k] = (j < p.topk) ? irow[j] : -1;
  }
  if (convert) {
    // request-local index -> global slot by the rule of smla_convert_indices
    // (anything it maps to -1 stays -1); the table reads of the row are all
    // issued before their results are used
    int64_t g[kIdxPerThread];
#pragma unroll
    for (int k = 0; k < kIdxPerThread; k++) g[k] = local_slot(p.bt, rq, gi[k]);
#pragma unroll
    for (int k = 0; k < kIdxPerThread; k++) gi[k] = (g[k] >= 0 && g[k] < p.num_slots) ? (int)g[k] : -1;
  }
  int len = p.topk;
  if (p.topk_length) len = min(max(p.topk_length[t], 0), p.topk);
  const int nrows = len;
  const int span = (nrows + kTileRows - 1) / kTileRows * kTileRows;
  int last = 0;
#pragma unroll
  for (int k = 0; k < kIdxPerThread; k++) {
    const int j = threadIdx.x + 512 * k;
    if (j < span) {
      int g = (j < nrows) ? gi[k] : -1;
      if (g < 0 || (int64_t)g >= p.num_slots) g = -1;
      s_idx[j] = g;
      if (g >= 0) last = j + 1;
    }
  }
  for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
  if (l == 0) s_last[w] = last;
  if (threadIdx.x == 0) {
    s_flag = 0;
    s_need = 0;
  }
  lds_barrier();
  int nlast = 0;
#pragma unroll
  for (int k = 0; k < 8; k++) nlast = max(nlast, s_last[k]);
  // this split's entries [row0, row1): an equal, tile-aligned share of [0, nlast)
  const int per = ((nlast + p.splits - 1) / p.splits + kTileRows - 1) / kTileRows * kTileRows;
  const int row0 = min(split * per, nlast);
  const int row1 = min(nlast, row0 + per);
  const int ntiles = (row1 - row0 + kTileRows - 1) / kTileRows;
  const int32_t* sidx = s_idx + row0;                      // entries of tile i: sidx[32 i ..]

  // bf16: latent and rope buffers of tile i; FP8: the buffer of tile i
  auto lat_buf = [&](int i) -> lds_char* { return lat + (NLAT ? (i % (NLAT ? NLAT : 1)) * kLatBytes : 0); };
  auto rope_buf = [&](int i) -> lds_char* { return rope + (NROPE ? (i % (NROPE ? NROPE : 1)) * kRopeBytes : 0); };
  auto tile8 = [&](int i) -> lds_char* { return lat + (i % S::NBUF) * S::TB; };

  // ---- tile copies, issued by the O-waves. Lane l copies into row 8w + l/8
  //      of the tile (w: the O-wave's index) the logical chunk (l & 7) ^ swz
  //      of 128-byte segment u, for every u: the same row and column, so one
  //      address per tile serves all copies through the immediate offset 128u.
  const int wu = __builtin_amdgcn_readfirstlane(wr);
  const uint32_t kv_stride = (uint32_t)p.kv_row_stride;
  const uint32_t lat_addr = (uint32_t)(uintptr_t)lat;
  const uint32_t rope_addr = (uint32_t)(uintptr_t)rope;
  const int drow = 8 * wu + (l >> 3);
  const uint32_t dcol = (uint32_t)(16 * ((l & 7) ^ swz(drow)));      // bf16 rows, packed bf16 rope
  const uint32_t dcol8 = (uint32_t)(16 * ((l & 7) ^ swz8(drow)));    // E4M3 latent codes
  // E4M3 rope codes (D = 576): lanes 0..31 copy chunk (l & 3) ^ sr of row
  // 8w + l/4 (sr = 2 for rows 8..15 and 24..31), at ((r & 7) * 4 + chunk) * 16
  // in the wave's 512 bytes
  const int rrow = 8 * wu + ((l >> 2) & 7);
  const uint32_t rcol8 = (uint32_t)(kDLatent + 16 * ((l & 3) ^ (((rrow >> 3) & 1) << 1)));
  // scales: copy c (c < NSC, by O-wave c) carries groups 2c and 2c+1 of all 32
  // rows, lane l: row l & 31, group 2c + l/32, at 4 * (group * 32 + row)
  const int sc_g = 2 * wu + (l >> 5);
  auto slot_of = [&](int e) -> uint64_t { return (uint64_t)(uint32_t)max(sidx[e], 0); };
  // O-wave copies of tile i (bf16: segment u of rows 8w .. 8w+7 into block
  // 4u + w, segment 8 is the rope part)
  auto issue_tile_o = [&](int i) {
    const int base = i * kTileRows;
    if constexpr (!F8) {
      const uint8_t* src = p.kv + slot_of(base + drow) * kv_stride + dcol;
      static_for<S::NDMA>([&](auto u_c) {
        constexpr int u = decltype(u_c)::value;
        if constexpr (u < 8)
          dma_16b<128 * u>(src, __builtin_amdgcn_readfirstlane(lat_addr + (i % (NLAT ? NLAT : 1)) * kLatBytes + (4 * u + wu) * 1024));
        else
          dma_16b<128 * u>(src, __builtin_amdgcn_readfirstlane(rope_addr + (i % (NROPE ? NROPE : 1)) * kRopeBytes + wu * 1024));
      });
    } else {
      const uint32_t tb = lat_addr + (i % S::NBUF) * S::TB;
      const uint8_t* row = p.kv + slot_of(base + drow) * kv_stride;
      const uint8_t* src = row + dcol8;
      static_for<4>([&](auto u_c) {
        constexpr int u = decltype(u_c)::value;
        dma_16b<128 * u>(src, __builtin_amdgcn_readfirstlane(tb + (4 * u + wu) * 1024));
      });
      if constexpr (S::ROPE8) {
        const uint8_t* rsrc = p.kv + slot_of(base + rrow) * kv_stride + rcol8;
        if (l < 32) dma_16b<0>(rsrc, __builtin_amdgcn_readfirstlane(tb + S::ROPE_AT + wu * 512));
      }
      if constexpr (S::PACKED)
        dma_16b<0>(row + kPackedRopeAt + dcol, __builtin_amdgcn_readfirstlane(tb + S::ROPE_AT + wu * 1024));
      if constexpr (S::GROUP) {
        if (wu < S::NSC) {
          const uint64_t slot = slot_of(base + (l & 31));
          const float* ssrc = S::PACKED ? (const float*)(p.kv + slot * kv_stride + kPackedScalesAt) + sc_g
                                        : p.group_scales + (slot * (uint64_t)p.gs_stride + sc_g);
          if (sc_g < S::G) dma_4b(ssrc, __builtin_amdgcn_readfirstlane(tb + S::SC_AT + wu * 256));
        }
      }
    }
  };
  // this wave's copies of tile k have landed (the copies of the tiles after k
  // that are already issued, up to k + PD - 1, may stay in flight)
  auto wait_tile = [&](int k) {
    const int later = min(ntiles - 1, k + PD - 1) - k;
    const bool sc = S::GROUP && wu < S::NSC;              // this wave copies scales too
    static_for<PD>([&](auto n_c) {
      constexpr int n = decltype(n_c)::value;
      if (later == n) {
        if (sc) wait_vmcnt<n * (S::NDMA + 1)>();
        else wait_vmcnt<n * S::NDMA>();
      }
    });
  };

  if (is_s) {
    // ======================================================================
    // S-waves: QK^T, softmax, P
    // ======================================================================
    // Q^T as the B operand of 16x16x32: lane holds head hb + 32hg + 16nbq + li
    // and 8 channels of k-step ks. bf16 cache: channels 32ks + 8lg .. +8.
    // FP8 cache: the K operand of k-steps 2j and 2j+1 comes from one 16-byte
    // read of codes 64j + 16lg .. +16, so lane lg holds channels 64j + 16lg .. +8
    // in k-step 2j and the next 8 in 2j+1 (the contraction sums over the same
    // channels in another order); the packed rows' bf16 rope part keeps the
    // bf16 order. Heads past h are zero.
    bf16x8 q[2][QKS];
    if constexpr (!F8) {
      // bf16 cache: the two row halves need the same Q. Each loads half of
      // the k-steps and the halves are swapped through LDS that tiles 0 and 1
      // leave idle (latent buffers 2, 3; rope buffer 2 and the P block).
      auto qslot = [&](int nbq, int ks) -> lds_char* {
        if (ks < kLatKS) return lat + (2 + hg) * kLatBytes + ((nbq * kLatKS + ks) * 64 + l) * 16;
        lds_char* base = hg ? pbuf : rope + 2 * kRopeBytes;
        return base + ((nbq * 2 + (ks - kLatKS)) * 64 + l) * 16;
      };
      constexpr int H0 = QKS / 2, H1 = QKS - QKS / 2;
      auto load_half = [&](auto off_c, auto cnt_c) {
        constexpr int off = decltype(off_c)::value, cnt = decltype(cnt_c)::value;
#pragma unroll
        for (int nbq = 0; nbq < 2; nbq++) {
          const int head = hb + 32 * hg + 16 * nbq + li;
          const bool valid = head < H;
          const int hq = valid ? head : 0;
          const uint16_t* qn = p.q_nope + t * p.qn_st + hq * p.qn_sh + 8 * lg;
          const uint16_t* qr = p.q_rope + t * p.qr_st + hq * p.qr_sh + 8 * lg;
          static_for<cnt>([&](auto k_c) {
            constexpr int ks = off + decltype(k_c)::value;
            if constexpr (ks < kLatKS) q[nbq][ks] = *(const bf16x8*)(qn + 32 * ks);
            else q[nbq][ks] = *(const bf16x8*)(qr + 32 * (ks - kLatKS));
          });
          wait_vmcnt<0>();
          static_for<cnt>([&](auto k_c) {
            constexpr int ks = off + decltype(k_c)::value;
            if (!valid) q[nbq][ks] = (bf16x8){};
            *(__attribute__((address_space(3))) bf16x8*)qslot(nbq, ks) = q[nbq][ks];
          });
        }
      };
      auto get_half = [&](auto off_c, auto cnt_c) {
        constexpr int off = decltype(off_c)::value, cnt = decltype(cnt_c)::value;
#pragma unroll
        for (int nbq = 0; nbq < 2; nbq++)
          static_for<cnt>([&](auto k_c) {
            constexpr int ks = off + decltype(k_c)::value;
            q[nbq][ks] = *(const __attribute__((address_space(3))) bf16x8*)qslot(nbq, ks);
          });
      };
      if (rh == 0) load_half(std::integral_constant<int, 0>{}, std::integral_constant<int, H0>{});
      else load_half(std::integral_constant<int, H0>{}, std::integral_constant<int, H1>{});
      lds_barrier();                                       // both halves are in LDS (the O-waves match it)
      if (rh == 0) get_half(std::integral_constant<int, H0>{}, std::integral_constant<int, H1>{});
      else get_half(std::integral_constant<int, 0>{}, std::integral_constant<int, H0>{});
    } else {
#pragma unroll
      for (int nbq = 0; nbq < 2; nbq++) {
        const int head = hb + 32 * hg + 16 * nbq + li;
        const bool valid = head < H;
        const int hq = valid ? head : 0;
        const uint16_t* qn = p.q_nope + t * p.qn_st + hq * p.qn_sh + 16 * lg;
        static_for<kLatKS / 2>([&](auto j_c) {
          constexpr int j = decltype(j_c)::value;
          q[nbq][2 * j] = *(const bf16x8*)(qn + 64 * j);
          q[nbq][2 * j + 1] = *(const bf16x8*)(qn + 64 * j + 8);
        });
        if constexpr (S::ROPE8) {
          const uint16_t* qr = p.q_rope + t * p.qr_st + hq * p.qr_sh + 16 * lg;
          q[nbq][kLatKS] = *(const bf16x8*)qr;
          q[nbq][kLatKS + 1] = *(const bf16x8*)(qr + 8);
        }
        if constexpr (S::PACKED) {
          const uint16_t* qr = p.q_rope + t * p.qr_st + hq * p.qr_sh + 8 * lg;
          q[nbq][kLatKS] = *(const bf16x8*)qr;
          q[nbq][kLatKS + 1] = *(const bf16x8*)(qr + 32);
        }
        if (!valid) {
#pragma unroll
          for (int ks = 0; ks < QKS; ks++) q[nbq][ks] = (bf16x8){};
        }
      }
    }
    // complete here, so that the compiler puts no wait on the Q registers inside the loop
    wait_vmcnt<0>();

    // K reads (A operand of 16x16x32): row 16rh + li. bf16: chunk 4ks + lg;
    // k-steps 0..15 in the latent buffer at kbase[ks & 1] + 4096 (ks >> 1),
    // 16..17 in the rope buffer at kbase[ks & 1] + 4096 (ks >> 1) - 32768
    // (packed rows' bf16 rope: kbase[ks - 16] in the tile's rope part).
    // FP8: codes of k-pair j < 8 (chunk 4j + lg) at kb8[j & 1] + 4096 (j >> 1),
    // the E4M3 rope part (chunk lg) at kr8.
    int kbase[2], kb8[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
      kbase[j] = tile_pos(16 * rh + li, 4 * j + lg);
      kb8[j] = tile_pos8(16 * rh + li, 4 * j + lg);
    }
    const int kr = 16 * rh + li;
    const int kr8 = S::ROPE_AT + (kr >> 3) * 512 + ((kr & 7) * 4 + (lg ^ (((kr >> 3) & 1) << 1))) * 16;

    // S^T[16 rows x 32 heads] of the wave for tile i (unscaled sums), bf16
    // cache. Lane holds rows 16rh + 4lg + r (r = 0..3) of heads 32hg + 16nbq + li.
    auto scores = [&](int i, f32x4& r0, f32x4& r1) {
      const lds_char* lb = lat_buf(i);
      const lds_char* rb = rope_buf(i);
      auto kaddr = [&](auto ks_c) -> const lds_char* {
        constexpr int ks = decltype(ks_c)::value;
        if constexpr (ks < kLatKS) return lb + kbase[ks & 1] + 4096 * (ks >> 1);
        else return rb + kbase[ks & 1] + 4096 * (ks >> 1) - kLatBytes;
      };
      // 4 independent accumulator chains (k-step ks into chain ks & 1 of each
      // head block). A dependent 16x16x32 MFMA waits about 7 MFMA slots for its
      // accumulator, so alone one wave reaches ~60% of the matrix core with
      // them, but the O-wave's P.V fills the gaps: 8 chains measured the same.
      f32x4 acc[2][2] = {};
      constexpr int PF = 6;                       // K operand reads kept in flight
      bf16x8 a[PF];
      static_for<PF>([&](auto ks_c) { a[decltype(ks_c)::value] = lds_ld128(kaddr(ks_c)); });
      static_for<QKS>([&](auto ks_c) {
        constexpr int ks = decltype(ks_c)::value;
        const bf16x8 cur = a[ks % PF];
        if constexpr (ks + PF < QKS) a[ks % PF] = lds_ld128(kaddr(std::integral_constant<int, ks + PF>{}));
        __builtin_amdgcn_sched_barrier(0);          // keep the read-ahead ahead of the MFMAs
        acc[ks & 1][0] = mfma16x16x32(cur, q[0][ks], acc[ks & 1][0]);
        acc[ks & 1][1] = mfma16x16x32(cur, q[1][ks], acc[ks & 1][1]);
        __builtin_amdgcn_sched_barrier(0);
      });
      r0 = acc[0][0] + acc[1][0];
      r1 = acc[0][1] + acc[1][1];
    };
    // FP8: per k-pair j one 16-byte read of 16 codes per lane, converted to the
    // A operands of k-steps 2j (codes 0..7) and 2j+1 (codes 8..15).
    //   per-tensor: each pair converted one pair ahead of its MFMAs, into
    //     accumulator sets 0 (k-step 2j) and 1 (k-step 2j+1): 4 chains (8
    //     measured the same: the O-wave's P.V fills the gaps);
    //   group formats: one accumulator pair per scale group, kept to the end
    //     of the contraction and then scaled by the rows' group scales (the
    //     schedule is described at the branch below). Folding each group into
    //     running sums during the contraction made that VALU wait for MFMA
    //     results and cost ~4% of the long-context kernel.
    auto scores8 = [&](int i, f32x4& r0, f32x4& r1) {
      const lds_char* tb = tile8(i);
      auto kaddr = [&](auto j_c) -> const lds_char* {
        constexpr int j = decltype(j_c)::value;
        if constexpr (j < kLatKS / 2) return tb + kb8[j & 1] + 4096 * (j >> 1);
        else return tb + kr8;
      };
      auto ld_codes = [&](auto j_c) -> u32x4 { return *(const __attribute__((address_space(3))) u32x4*)kaddr(j_c); };
      if constexpr (S::GROUP) {
        // One accumulator per scale group and head block, all kept to the end
        // of QK^T, then scaled by the rows' group scales and summed: no VALU
        // waits for MFMA results inside the contraction. The MFMAs go round
        // the groups: the first k-pair of latent groups 0..3 (pair 2g), low
        // then high halves; then their second k-pair (2g + 1) with the E4M3
        // rope part (group 4, one pair) alongside. An accumulator's next MFMA
        // comes 8 to 10 MFMAs after its last one. Packed rows: the bf16 rope
        // part's two k-steps, unscaled, come last.
        constexpr int NG = 4 + (S::ROPE8 ? 1 : 0);       // groups held as codes
        f32x4 acc[NG][2] = {};
        u32x4 c0[4], c1[NG];
        static_for<4>([&](auto g_c) {
          constexpr int g = decltype(g_c)::value;
          c0[g] = ld_codes(std::integral_constant<int, 2 * g>{});
        });
        static_for<4>([&](auto g_c) {
          constexpr int g = decltype(g_c)::value, j = 2 * g;
          const bf16x8 lo = e4m3x8_to_bf16x8(c0[g][0], c0[g][1]);
          acc[g][0] = mfma16x16x32(lo, q[0][2 * j], acc[g][0]);
          acc[g][1] = mfma16x16x32(lo, q[1][2 * j], acc[g][1]);
          __builtin_amdgcn_sched_barrier(0);
        });
        // high halves; the second k-pairs' codes are read as registers free up
        static_for<4>([&](auto g_c) {
          constexpr int g = decltype(g_c)::value, j = 2 * g;
          const bf16x8 hi = e4m3x8_to_bf16x8(c0[g][2], c0[g][3]);
          c1[g] = ld_codes(std::integral_constant<int, j + 1>{});
          if constexpr (g == 3 && NG == 5) c1[4] = ld_codes(std::integral_constant<int, kLatKS / 2>{});
          acc[g][0] = mfma16x16x32(hi, q[0][2 * j + 1], acc[g][0]);
          acc[g][1] = mfma16x16x32(hi, q[1][2 * j + 1], acc[g][1]);
          __builtin_amdgcn_sched_barrier(0);
        });
        auto ks_of = [](int g) { return g < 4 ? 2 * (2 * g + 1) : kLatKS; };   // first k-step of the second pair
        [[maybe_unused]] bf16x8 k0, k1;
        static_for<NG>([&](auto g_c) {
          constexpr int g = decltype(g_c)::value;
          const bf16x8 lo = e4m3x8_to_bf16x8(c1[g][0], c1[g][1]);
          if constexpr (S::PACKED && g == 0) {             // the bf16 rope part's two k-steps
            k0 = lds_ld128(tb + S::ROPE_AT + kbase[0]);
            k1 = lds_ld128(tb + S::ROPE_AT + kbase[1]);
          }
          acc[g][0] = mfma16x16x32(lo, q[0][ks_of(g)], acc[g][0]);
          acc[g][1] = mfma16x16x32(lo, q[1][ks_of(g)], acc[g][1]);
          __builtin_amdgcn_sched_barrier(0);
        });
        static_for<NG>([&](auto g_c) {
          constexpr int g = decltype(g_c)::value;
          const bf16x8 hi = e4m3x8_to_bf16x8(c1[g][2], c1[g][3]);
          acc[g][0] = mfma16x16x32(hi, q[0][ks_of(g) + 1], acc[g][0]);
          acc[g][1] = mfma16x16x32(hi, q[1][ks_of(g) + 1], acc[g][1]);
          __builtin_amdgcn_sched_barrier(0);
        });
        f32x4 t0 = {}, t1 = {};
        if constexpr (S::PACKED) {
          t0 = mfma16x16x32(k0, q[0][kLatKS], t0);
          t1 = mfma16x16x32(k0, q[1][kLatKS], t1);
          t0 = mfma16x16x32(k1, q[0][kLatKS + 1], t0);
          t1 = mfma16x16x32(k1, q[1][kLatKS + 1], t1);
        }
        // scale and sum: rows 16rh + 4lg .. +3 of the [group][row] scale block
        const lds_char* rs = tb + S::SC_AT + 4 * (16 * rh + 4 * lg);
        f32x4 u0 = {}, u1 = {};
        static_for<NG>([&](auto g_c) {
          constexpr int g = decltype(g_c)::value;
          const f32x4 gsc = *(const __attribute__((address_space(3))) f32x4*)(rs + 4 * kTileRows * g);
          u0 += gsc * acc[g][0];
          u1 += gsc * acc[g][1];
        });
        r0 = u0 + t0;
        r1 = u1 + t1;
      } else {
        // per-tensor: pair j+1 is converted during pair j
        constexpr int NP = kLatKS / 2 + (S::ROPE8 ? 1 : 0);  // k-pairs held as codes
        constexpr int PF = 3;                     // code reads kept in flight
        f32x4 acc[2][2] = {};
        u32x4 a[PF];
        static_for<PF>([&](auto j_c) { a[decltype(j_c)::value] = ld_codes(j_c); });
        bf16x8 clo = e4m3x8_to_bf16x8(a[0][0], a[0][1]);
        bf16x8 chi = e4m3x8_to_bf16x8(a[0][2], a[0][3]);
        static_for<NP>([&](auto j_c) {
          constexpr int j = decltype(j_c)::value;
          const bf16x8 lo = clo, hi = chi;
          if constexpr (j + PF < NP) a[j % PF] = ld_codes(std::integral_constant<int, j + PF>{});
          if constexpr (j + 1 < NP) {
            const u32x4 nx = a[(j + 1) % PF];
            clo = e4m3x8_to_bf16x8(nx[0], nx[1]);
            chi = e4m3x8_to_bf16x8(nx[2], nx[3]);
          }
          acc[0][0] = mfma16x16x32(lo, q[0][2 * j], acc[0][0]);
          acc[0][1] = mfma16x16x32(lo, q[1][2 * j], acc[0][1]);
          acc[1][0] = mfma16x16x32(hi, q[0][2 * j + 1], acc[1][0]);
          acc[1][1] = mfma16x16x32(hi, q[1][2 * j + 1], acc[1][1]);
          __builtin_amdgcn_sched_barrier(0);
        });
        r0 = acc[0][0] + acc[1][0];
        r1 = acc[0][1] + acc[1][1];
      }
    };
    // maximum over the workgroup's 32 rows (both row halves), per head; one
    // barrier, which the O-waves match
    auto wg_max = [&](float (&mx)[2]) {
#pragma unroll
      for (int nbq = 0; nbq < 2; nbq++) {
        float m = mx[nbq];
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        mx[nbq] = m;
      }
      if (lg == 0) {
        s_m[wr * 32 + li] = mx[0];
        s_m[wr * 32 + 16 + li] = mx[1];
      }
      lds_barrier();
      mx[0] = fmaxf(mx[0], s_m[(wr ^ 2) * 32 + li]);
      mx[1] = fmaxf(mx[1], s_m[(wr ^ 2) * 32 + 16 + li]);
    };

    float m_ref[2] = {-INFINITY, -INFINITY};
    // Two row sums per head: l_lane of the fp32 p (the LSE and the rerun
    // test), lb_lane of the bf16-rounded p that P.V multiplies (the output's
    // normaliser: the output is then a weighted mean of the V rows with the
    // weights P.V used, so rounding P moves it by sum_j dw_j (v_j - out), not
    // by sum_j dw_j v_j; a row dominated by a few similar values comes out
    // nearly exact). Summing the bf16 p for the LSE as well moved the LSE by
    // up to 2^-9 relative in l, beyond its 1e-3 bar.
    float l_lane[2] = {0.0f, 0.0f}, lb_lane[2] = {0.0f, 0.0f};
    bool have_ref = false;                                 // workgroup-uniform
    // capped value of a base-2 logit (the cap is increasing, so the capped
    // maximum is the cap of the maximum)
    auto cap2 = [&](float t) -> float {
      if (!p.softcap_on || t == -INFINITY) return t;
      const float e = fast_exp2(t * p.cap_t);
      return fmaf(-2.0f * p.cap_c1, __builtin_amdgcn_rcpf(1.0f + e), p.cap_c1);
    };

    // Scores in base-2 units, masked rows at -inf (for the maxima).
    auto scaled = [&](const f32x4& r0, const f32x4& r1, uint32_t vmask, float (&tv)[2][4], float (&mx)[2]) {
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const bool ok = (vmask >> (16 * rh + 4 * lg + r)) & 1;
        tv[0][r] = ok ? r0[r] * p.scale_log2 : -INFINITY;
        tv[1][r] = ok ? r1[r] * p.scale_log2 : -INFINITY;
      }
#pragma unroll
      for (int nbq = 0; nbq < 2; nbq++)
        mx[nbq] = fmaxf(fmaxf(tv[nbq][0], tv[nbq][1]), fmaxf(tv[nbq][2], tv[nbq][3]));
    };

    // one pass over the tiles; full = softmax and P, otherwise only the
    // per-head maximum (into mx_all). Barriers: one per tile, plus the
    // reference exchange in tile 0 of a full pass. A full pass ends by
    // flagging a rerun if a row sum left the range the reference guarantees
    // (some p = 2^(t - m) above 2^64, or not finite), or if tile 0 held no
    // valid entry (no reference) while a later tile did.
    auto s_pass = [&](auto cap_c, const bool full, float (&mx_all)[2]) {
      constexpr bool CAP = decltype(cap_c)::value;          // softcap on (uniform, hoisted out of the loop)
      l_lane[0] = l_lane[1] = 0.0f;
      lb_lane[0] = lb_lane[1] = 0.0f;
      bool seen = false;                                   // a valid entry in some tile (uniform)
      // the index entry of row l & 31 of the next tile is read one tile ahead,
      // so the row mask needs no LDS round trip at the start of a tile
      int idx_next = ntiles > 0 ? sidx[l & 31] : -1;
      lds_barrier();                                       // pass start: tile 0 is in LDS
      for (int i = 0; i <= ntiles; i++) {
        const bool have = i < ntiles;
        const int idx_cur = idx_next;
        if (i + 1 < ntiles) idx_next = sidx[(i + 1) * kTileRows + (l & 31)];
        f32x4 r0 = {}, r1 = {};
        uint32_t vmask = 0;
        float tv[2][4];
        float mx[2] = {-INFINITY, -INFINITY};
        if (have) {
          vmask = (uint32_t)__ballot(l < 32 && idx_cur >= 0);
          seen = seen || vmask != 0;
          if constexpr (F8) scores8(i, r0, r1);
          else scores(i, r0, r1);
          if (!full || i == 0) scaled(r0, r1, vmask, tv, mx);
        }
        if (!full) {
          mx_all[0] = fmaxf(mx_all[0], mx[0]);
          mx_all[1] = fmaxf(mx_all[1], mx[1]);
          lds_barrier();
          continue;
        }
        if (i == 0) {                                      // the reference: tile 0's maximum
          wg_max(mx);                                      // (its barrier always runs: the O-waves match it)
          if (!have_ref) {                                 // a rerun keeps the reference it was given
            m_ref[0] = cap2(mx[0]);
            m_ref[1] = cap2(mx[1]);
            have_ref = true;
          }
        }
        if (have) {
          lds_char* pb = pbuf + (i & 1) * (4 * 64 * 16);
          float pr[2][4];
#pragma unroll
          for (int nbq = 0; nbq < 2; nbq++) {
            const float nm = (m_ref[nbq] == -INFINITY) ? 0.0f : -m_ref[nbq];
            const f32x4& rs = nbq ? r1 : r0;
            if constexpr (CAP) {
              const float base = p.cap_c1 + nm, k2 = -2.0f * p.cap_c1;
#pragma unroll
              for (int r = 0; r < 4; r++) {
                const float e = fast_exp2(rs[r] * p.cap_a);
                pr[nbq][r] = fast_exp2(fmaf(k2, __builtin_amdgcn_rcpf(1.0f + e), base));
              }
            } else {
#pragma unroll
              for (int r = 0; r < 4; r++) pr[nbq][r] = fast_exp2(fmaf(rs[r], p.scale_log2, nm));
            }
          }
          if (vmask != 0xffffffffu) {                      // uniform
#pragma unroll
            for (int r = 0; r < 4; r++)
              if (!((vmask >> (16 * rh + 4 * lg + r)) & 1)) pr[0][r] = pr[1][r] = 0.0f;
          }
#pragma unroll
          for (int nbq = 0; nbq < 2; nbq++) {
            // the row sum adds the fp32 p (the LSE stays exact to fp32
            // rounding; summing the bf16-rounded p instead moved it by up to
            // 2^-9 relative, beyond the 1e-3 LSE bar)
            l_lane[nbq] += (pr[nbq][0] + pr[nbq][1]) + (pr[nbq][2] + pr[nbq][3]);
            const uint32_t p01 = pack_bf16x2(pr[nbq][0], pr[nbq][1]);
            const uint32_t p23 = pack_bf16x2(pr[nbq][2], pr[nbq][3]);
            lb_lane[nbq] = sum_bf16x2(p23, sum_bf16x2(p01, lb_lane[nbq]));
            const uint64_t pk = (uint64_t)p01 | ((uint64_t)p23 << 32);
            // A operand of m-block 2hg + nbq, elements 4rh .. 4rh+3
            lds_st64(pb + ((2 * hg + nbq) * 64 + l) * 16 + 8 * rh, pk);
          }
        } else {
          // end of the pass: 2^64 bounds every p while the reference holds
          if (!(l_lane[0] <= kRefLimit) || !(l_lane[1] <= kRefLimit) || (seen && m_ref[0] == -INFINITY)) s_flag = 1;
        }
        lds_barrier();
      }
    };

    for (int attempt = 0; attempt < 2; attempt++) {
      float unused[2] = {-INFINITY, -INFINITY};
      if (p.softcap_on) s_pass(std::true_type{}, true, unused);
      else s_pass(std::false_type{}, true, unused);
      // uniform (after the pass's last barrier). The rerun's reference is at
      // or above every score, so it is only flagged by a NaN or infinite
      // score: that result stands (NaN propagates to the output and LSE)
      if (!s_flag || attempt == 1) break;
      // a new per-head reference, then the full pass again. The largest
      // per-lane row sum L of the flagged pass lies between its largest p and
      // 256 times it (a lane sums 4 of each tile's 32 entries, of at most
      // 2048), so with m + log2(L) every p of the rerun is at most 1 and the
      // largest is at least 2^-8 (the scores are already capped). Unless some L is 0,
      // infinite or NaN: then a max-only pass finds the exact maximum.
      // Barriers: the exchange and the decision, which the O-waves match.
      float pmx[2] = {l_lane[0], l_lane[1]};
      wg_max(pmx);
      float m_new[2];
      bool usable = true;
#pragma unroll
      for (int nbq = 0; nbq < 2; nbq++) {
        usable = usable && pmx[nbq] > 0.0f && pmx[nbq] <= 3.4028234663852886e38f;
        m_new[nbq] = (m_ref[nbq] == -INFINITY ? 0.0f : m_ref[nbq]) + log2f(pmx[nbq]);
      }
      if (!usable) s_need = 1;
      lds_barrier();
      if (s_need) {                                        // uniform (after the barrier)
        float mx_all[2] = {-INFINITY, -INFINITY};
        s_pass(std::false_type{}, false, mx_all);
        wg_max(mx_all);
        m_ref[0] = cap2(mx_all[0]);
        m_ref[1] = cap2(mx_all[1]);
      } else {
        m_ref[0] = m_new[0];
        m_ref[1] = m_new[1];
      }
      if (threadIdx.x == 0) s_flag = 0;
    }

    // ---- epilogue (S side): row sums per head, LSE, inverse sums
#pragma unroll
    for (int nbq = 0; nbq < 2; nbq++) {
      float v = l_lane[nbq], vb = lb_lane[nbq];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      vb += __shfl_xor(vb, 16, 64);
      vb += __shfl_xor(vb, 32, 64);
      l_lane[nbq] = v;
      lb_lane[nbq] = vb;
    }
    if (lg == 0) {
      s_l[wr * 32 + li] = l_lane[0];
      s_l[wr * 32 + 16 + li] = l_lane[1];
      s_lb[wr * 32 + li] = lb_lane[0];
      s_lb[wr * 32 + 16 + li] = lb_lane[1];
    }
    lds_barrier();                                         // E1
    if (rh == 0 && lg == 0) {
#pragma unroll
      for (int nbq = 0; nbq < 2; nbq++) {
        float lt = s_l[wr * 32 + 16 * nbq + li] + s_l[(wr ^ 2) * 32 + 16 * nbq + li];
        float lbt = s_lb[wr * 32 + 16 * nbq + li] + s_lb[(wr ^ 2) * 32 + 16 * nbq + li];
        const int hl = 32 * hg + 16 * nbq + li;          // head within the block
        const int head = hb + hl;
        float mr = m_ref[nbq], om = p.out_mult;
        if (p.sinks && head < H) {
          // the sink joins the denominator: rescale to M = max(m, sink)
          const float sg = p.sinks[head] * 1.4426950408889634f;
          const float M = fmaxf(mr, sg);
          if (M != -INFINITY) {
            const float a = exp2f(mr - M);                 // 0 for an empty row
            lt = fmaf(lt, a, exp2f(sg - M));
            lbt = fmaf(lbt, a, exp2f(sg - M));
            om *= a;
            mr = M;
          }
        }
        const bool nonempty = !(lt <= 0.0f);              // a NaN sum stays NaN
        s_inv[hl] = nonempty ? om / lbt : 0.0f;
        const float lse_v = nonempty ? (mr + log2f(lt)) * 0.69314718055994531f : -INFINITY;
        if (head < H) {
          if (p.splits == 1) {
            if (p.lse) p.lse[(int64_t)t * p.lse_st + head] = lse_v;
          } else {
            p.part_lse[((int64_t)split * T + t) * H + head] = lse_v;
          }
        }
      }
    }
    lds_barrier();                                         // E2
    lds_barrier();                                         // E3: O staged
  } else {
    // ======================================================================
    // O-waves: tile copies, P.V
    // ======================================================================
    // bf16 V transposing reads (B operand of P.V): in 16-lane group lg, lane
    // li = 4e + q reads row 4lg + e (then 16 + 4lg + e), channels 128w + 16nb +
    // 4q .. +3, at vbase[half][nb & 3] + 4096 (nb >> 2).
    // FP8 V transposing reads: lane li = 2e + q reads row 4lg + e (e < 4) or
    // 12 + 4lg + e (e >= 4), codes 128w + 16nb + 8q .. +7, at vb8[nb]; lane li
    // then holds channel 128w + 16nb + li of the 8 rows, in the P operand's
    // row order.
    int vbase[2][4], vb8[8];
    {
      const int e = li >> 2, q4 = li & 3;
#pragma unroll
      for (int half = 0; half < 2; half++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          vbase[half][j] = tile_pos(16 * half + 4 * lg + e, 16 * wr + 2 * j + (q4 >> 1)) + 8 * (q4 & 1);
      const int e8 = li >> 1, q2 = li & 1;
      const int vr8 = e8 < 4 ? 4 * lg + e8 : 12 + 4 * lg + e8;
#pragma unroll
      for (int nb = 0; nb < 8; nb++) vb8[nb] = tile_pos8(vr8, 8 * wr + nb) + 8 * q2;
    }

    f32x4 O[4][8];
    // O[64 heads x 128 ch] += P(i)[64 x 32] . V(i)[32 x 128]
    auto pv = [&](int i) {
      const lds_char* lb = lat_buf(i);
      const lds_char* pb = pbuf + (i & 1) * (4 * 64 * 16);
      constexpr int VPF = 3;                                // V reads kept in flight (n-blocks)
      s16x4 vr[VPF + 1][2];
#pragma unroll
      for (int nb = 0; nb < VPF; nb++) {
        vr[nb][0] = lds_read_tr16(lb + vbase[0][nb & 3] + 4096 * (nb >> 2));
        vr[nb][1] = lds_read_tr16(lb + vbase[1][nb & 3] + 4096 * (nb >> 2));
      }
      bf16x8 pa[4];
#pragma unroll
      for (int mb = 0; mb < 4; mb++) pa[mb] = lds_ld128(pb + (mb * 64 + l) * 16);
#pragma unroll
      for (int nb = 0; nb < 8; nb++) {
        const s16x4 v0 = vr[nb % (VPF + 1)][0];
        const s16x4 v1 = vr[nb % (VPF + 1)][1];
        if (nb + VPF < 8) {
          const int n2 = nb + VPF;
          vr[n2 % (VPF + 1)][0] = lds_read_tr16(lb + vbase[0][n2 & 3] + 4096 * (n2 >> 2));
          vr[n2 % (VPF + 1)][1] = lds_read_tr16(lb + vbase[1][n2 & 3] + 4096 * (n2 >> 2));
        }
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 bv = concat_bf16x4(v0, v1);
#pragma unroll
        for (int mb = 0; mb < 4; mb++) O[mb][nb] = mfma16x16x32(pa[mb], bv, O[mb][nb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // FP8: 8 codes per lane per n-block, converted one n-block ahead of its MFMAs
    auto pv8 = [&](int i) {
      const lds_char* tb = tile8(i);
      const lds_char* pb = pbuf + (i & 1) * (4 * 64 * 16);
      constexpr int VPF = 3;                                // V reads kept in flight (n-blocks)
      // the scales and P are read before the V read-ahead, so that scaling P
      // waits only for them (LDS reads return in order)
      [[maybe_unused]] f32x4 sa, sb;
      if constexpr (S::GROUP) {
        const lds_char* rw = tb + S::SC_AT + 4 * (wr * kTileRows + 4 * lg);
        sa = *(const __attribute__((address_space(3))) f32x4*)rw;
        sb = *(const __attribute__((address_space(3))) f32x4*)(rw + 64);
      }
      bf16x8 pa[4];
#pragma unroll
      for (int mb = 0; mb < 4; mb++) pa[mb] = lds_ld128(pb + (mb * 64 + l) * 16);
      i32x2 vr[VPF];
#pragma unroll
      for (int nb = 0; nb < VPF; nb++) vr[nb] = lds_read_tr8(tb + vb8[nb]);
      if constexpr (S::GROUP) {
        // wave w's channels are group w: P[h][j] * scale[j][w] (elements 0..3 of
        // the operand are rows 4lg .. 4lg+3, elements 4..7 rows 16+4lg .. 16+4lg+3)
#pragma unroll
        for (int mb = 0; mb < 4; mb++) pa[mb] = scale_bf16x8(pa[mb], sa, sb);
      }
      bf16x8 cv = e4m3x8_to_bf16x8((uint32_t)vr[0][0], (uint32_t)vr[0][1]);
#pragma unroll
      for (int nb = 0; nb < 8; nb++) {
        const bf16x8 bv = cv;
        if (nb + VPF < 8) vr[nb % VPF] = lds_read_tr8(tb + vb8[nb + VPF]);
        if (nb + 1 < 8) cv = e4m3x8_to_bf16x8((uint32_t)vr[(nb + 1) % VPF][0], (uint32_t)vr[(nb + 1) % VPF][1]);
#pragma unroll
        for (int mb = 0; mb < 4; mb++) O[mb][nb] = mfma16x16x32(pa[mb], bv, O[mb][nb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // one pass over the tiles, the same barriers as s_pass. Tiles 0 .. PD-1
    // are copied before the pass (in the prologue for the first pass).
    auto o_pass = [&](const bool full, const bool issued) {
#pragma unroll
      for (int mb = 0; mb < 4; mb++)
#pragma unroll
        for (int nb = 0; nb < 8; nb++) O[mb][nb] = (f32x4){};
      if (!issued) {
        for (int k = 0; k < PD; k++)
          if (k < ntiles) issue_tile_o(k);
      }
      if (ntiles > 0) wait_tile(0);
      lds_barrier();                                       // pass start
      for (int i = 0; i <= ntiles; i++) {
        if (i + PD < ntiles) issue_tile_o(i + PD);
        if (full && i == 0) lds_barrier();                 // matches the S-waves' reference exchange
        if (full && i >= 1) {
          if constexpr (F8) pv8(i - 1);
          else pv(i - 1);
        }
        if (i + 1 < ntiles) wait_tile(i + 1);              // tile i+1 has landed
        lds_barrier();
      }
    };

    for (int k = 0; k < PD; k++)
      if (k < ntiles) issue_tile_o(k);
    if constexpr (!F8) lds_barrier();                      // matches the S-waves' Q exchange
    for (int attempt = 0; attempt < 2; attempt++) {
      o_pass(true, attempt == 0);
      if (!s_flag || attempt == 1) break;                  // uniform (after the pass's last barrier)
      lds_barrier();                                       // matches the S-waves' exchange of the pass's maxima
      lds_barrier();                                       // s_need is written
      if (s_need) {
        o_pass(false, false);
        lds_barrier();                                     // matches the S-waves' final maximum exchange
      }
    }

    // ---- epilogue (O side)
    lds_barrier();                                         // E1: row sums written
    lds_barrier();                                         // E2: inverse sums written
    // Stage the normalised O block [64 heads][512 ch] as bf16 in the first
    // 64 KB of the latent ring (idle now), then all waves write whole 16-byte
    // chunks. O lane layout: m-block mb, n-block nb: head 16mb + 4lg + r,
    // channel 128w + 16nb + li. Two heads of one channel are rounded together
    // (v_cvt_pk_bf16_f32). Staged row h, byte b sits at h*1024 + (b ^ (((h >>
    // 2) & 3) << 5)): the 4 head groups of one store instruction fall in
    // different banks.
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int mb = 0; mb < 4; mb++) {
#pragma unroll
      for (int rp = 0; rp < 2; rp++) {
        const int h0 = 16 * mb + 4 * lg + 2 * rp;
        const float sc0 = s_inv[h0], sc1 = s_inv[h0 + 1];
#pragma unroll
        for (int nb = 0; nb < 8; nb++) {
          const int off = (2 * (128 * wr + 16 * nb + li)) ^ (lg << 5);
          const f32x2 v = {O[mb][nb][2 * rp] * sc0, O[mb][nb][2 * rp + 1] * sc1};
          const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
          *(__attribute__((address_space(3))) uint16_t*)(lat + h0 * 1024 + off) = (uint16_t)pk;
          *(__attribute__((address_space(3))) uint16_t*)(lat + (h0 + 1) * 1024 + off) = (uint16_t)(pk >> 16);
        }
      }
    }
    lds_barrier();                                         // E3
  }

  // ---- all waves: write the staged block
  uint16_t* dst_base;
  int64_t dst_sh;
  if (p.splits == 1) {
    dst_base = p.out + (int64_t)t * p.out_st + (int64_t)hb * p.out_sh;
    dst_sh = p.out_sh;
  } else {
    dst_base = p.part_o + (((int64_t)split * T + t) * H + hb) * kDLatent;
    dst_sh = kDLatent;
  }
  const int hmax = min(64, H - hb);
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const int id = k * 512 + threadIdx.x;
    const int hl = id >> 6, c16 = id & 63;
    if (hl < hmax) {
      const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(lat + hl * 1024 + ((16 * c16) ^ (((hl >> 2) & 3) << 5)));
      *(u32x4*)(dst_base + (int64_t)hl * dst_sh + 8 * c16) = v;
    }
  }
}

// Merge partial results by their LSE: lse = ln sum_s exp(lse_s),
// out = sum_s exp(lse_s - lse) * O_s; (0, -inf) is the identity, and a sink
// enters as one more partial (0, sink). Partials are
// the normalised O_s in bf16 (the decode splits, or the context-parallel
// ranks' outputs: the cross-rank merge of the FlashMLA sparse docs).
__global__ void __launch_bounds__(256)
smla_combine_kernel(const uint16_t* __restrict__ part_o, int64_t po_rank, int64_t po_tok, int64_t po_head,
                    const float* __restrict__ part_lse, int64_t pl_rank, int64_t pl_tok, int splits,
                    int T, int H, uint16_t* __restrict__ out, int64_t out_st, int64_t out_sh,
                    float* __restrict__ lse, int64_t lse_st, const float* __restrict__ sinks) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;   // one thread = 8 channels
  const int64_t total = (int64_t)T * H * (kDLatent / 8);
  if (gid >= total) return;
  const int c8 = (int)(gid % (kDLatent / 8));
  const int64_t th = gid / (kDLatent / 8);
  const int head = (int)(th % H);
  const int t = (int)(th / H);
  const float* pl = part_lse + (int64_t)t * pl_tok + head;
  const uint16_t* po = part_o + (int64_t)t * po_tok + (int64_t)head * po_head + 8 * c8;
  // a sink is one more partial with a zero output and LSE sinks[head]
  const float sg = sinks ? sinks[head] : -INFINITY;
  float m = sg;
  bool nan = false;                                    // a NaN partial makes the result NaN
  for (int s = 0; s < splits; s++) {
    const float ls = pl[s * pl_rank];
    m = fmaxf(m, ls);
    nan = nan || ls != ls;
  }
  if (nan) m = __builtin_nanf("");
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float tot = 0.0f;
  if (m != -INFINITY) {
    if (sg != -INFINITY) tot = expf(sg - m);
    for (int s = 0; s < splits; s++) {
      const float ls = pl[s * pl_rank];
      const float wgt = (ls == -INFINITY) ? 0.0f : expf(ls - m);
      tot += wgt;
      const u32x4 o = *(const u32x4*)(po + s * po_rank);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        acc[2 * i] += wgt * __builtin_bit_cast(float, o[i] << 16);
        acc[2 * i + 1] += wgt * __builtin_bit_cast(float, o[i] & 0xffff0000u);
      }
    }
    const float inv = 1.0f / tot;
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] *= inv;
  }
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; i++) r[i] = f32_to_bf16_rne(acc[2 * i]) | ((uint32_t)f32_to_bf16_rne(acc[2 * i + 1]) << 16);
  *(u32x4*)(out + (int64_t)t * out_st + (int64_t)head * out_sh + 8 * c8) = r;
  if (c8 == 0 && lse) lse[(int64_t)t * lse_st + head] = (m == -INFINITY) ? -INFINITY : m + logf(tot);
}

// With timing events the launch goes through hipExtLaunchKernel, which sets
// the events from the kernel's own start and end timestamps.
template <int D, int FMT>
static hipError_t launch_kernel(const KParams& kp, int grid, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (ev0 || ev1) {
    KParams arg = kp;
    void* args[] = {&arg};
    return hipExtLaunchKernel((const void*)smla_attn_kernel<D, FMT>, dim3(grid), dim3(512), args, 0, stream,
                              ev0, ev1, 0);
  }
  smla_attn_kernel<D, FMT><<<grid, 512, 0, stream>>>(kp);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int32_t splits, void* workspace, bool longest_first,
                            hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  KParams kp;
  kp.q_nope = a.q_nope; kp.qn_st = a.qn_st; kp.qn_sh = a.qn_sh;
  kp.q_rope = a.d_rope ? a.q_rope : a.q_nope; kp.qr_st = a.qr_st; kp.qr_sh = a.qr_sh;
  kp.kv = a.kv; kp.kv_row_stride = a.kv_row_stride; kp.num_slots = a.num_slots;
  kp.group_scales = a.group_scales;
  kp.gs_stride = a.gs_stride;
  kp.indices = a.indices; kp.idx_stride = a.idx_stride; kp.topk = a.topk;
  kp.topk_length = a.topk_length;
  kp.req_id = a.req_id;
  kp.bt = BlockTable{a.block_table, a.num_reqs, a.max_blocks, a.bt_row_stride, a.block_size,
                     block_shift_of(a.block_size), a.block_stride_rows};
  kp.num_tokens = a.num_tokens; kp.num_heads = a.num_heads;
  kp.scale_log2 = a.softmax_scale * 1.4426950408889634f;
  kp.out_mult = 1.0f;
  if (a.kv_format == 1) {
    // value = e4m3 * k_scale: the scale moves out of both contractions
    kp.scale_log2 *= a.k_scale;
    kp.out_mult = a.k_scale;
  }
  kp.softcap_on = a.softcap > 0.0f ? 1 : 0;
  kp.cap_a = kp.softcap_on ? 2.0f * kp.scale_log2 / a.softcap : 0.0f;
  kp.cap_t = kp.softcap_on ? 2.0f / a.softcap : 0.0f;
  kp.cap_c1 = a.softcap * 1.4426950408889634f;
  kp.sinks = splits == 1 ? a.sinks : nullptr;        // with splits the merge adds the sink
  kp.splits = splits;
  kp.longest_first = longest_first ? 1 : 0;
  kp.head_blocks = a.num_heads > 64 ? 2 : 1;
  kp.xcd_group = a.num_tokens >= 8 ? 1 : 0;
  kp.out = a.out; kp.out_st = a.out_st; kp.out_sh = a.out_sh;
  kp.lse = a.lse; kp.lse_st = a.lse_st;
  kp.part_o = nullptr; kp.part_lse = nullptr;
  if (splits > 1) {
    const size_t n = (size_t)splits * a.num_tokens * a.num_heads;
    kp.part_o = (uint16_t*)workspace;
    kp.part_lse = (float*)((char*)workspace + n * kDLatent * sizeof(uint16_t));
  }
  const int per_tok = kp.head_blocks * splits;
  const int grid = kp.xcd_group ? 8 * ((a.num_tokens + 7) / 8) * per_tok : a.num_tokens * per_tok;
  const bool rope = a.d_rope == 64;
  const hipEvent_t e0 = a.ev_start, e1 = a.ev_end;
  hipError_t e;
  switch (a.kv_format) {
    case 0: e = rope ? launch_kernel<576, 0>(kp, grid, stream, e0, e1) : launch_kernel<512, 0>(kp, grid, stream, e0, e1); break;
    case 1: e = rope ? launch_kernel<576, 1>(kp, grid, stream, e0, e1) : launch_kernel<512, 1>(kp, grid, stream, e0, e1); break;
    case 2: e = rope ? launch_kernel<576, 2>(kp, grid, stream, e0, e1) : launch_kernel<512, 2>(kp, grid, stream, e0, e1); break;
    case 3:
      if (!rope) return hipErrorInvalidValue;
      e = launch_kernel<576, 3>(kp, grid, stream, e0, e1);
      break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || splits == 1) return e;
  MergeArgs m;
  m.part_o = kp.part_o;
  m.po_head = kDLatent;
  m.po_tok = (int64_t)a.num_heads * kDLatent;
  m.po_rank = (int64_t)a.num_tokens * m.po_tok;
  m.part_lse = kp.part_lse;
  m.pl_tok = a.num_heads;
  m.pl_rank = (int64_t)a.num_tokens * a.num_heads;
  m.parts = splits;
  m.num_tokens = a.num_tokens;
  m.num_heads = a.num_heads;
  m.out = a.out; m.out_st = a.out_st; m.out_sh = a.out_sh;
  m.lse = a.lse; m.lse_st = a.lse_st;
  m.sinks = a.sinks;
  return launch_merge(m, stream);
}

hipError_t launch_merge(const MergeArgs& m, hipStream_t stream) {
  const int64_t total = (int64_t)m.num_tokens * m.num_heads * (kDLatent / 8);
  if (total == 0) return hipSuccess;
  smla_combine_kernel<<<(int)((total + 255) / 256), 256, 0, stream>>>(
      m.part_o, m.po_rank, m.po_tok, m.po_head, m.part_lse, m.pl_rank, m.pl_tok, m.parts, m.num_tokens,
      m.num_heads, m.out, m.out_st, m.out_sh, m.lse, m.lse_st, m.sinks);
  return hipGetLastError();
}

// Split partials of the allocation-free decode entry point: a file-scope
// device array, one copy per GPU for the life of the process. Host code never
// uses the array's name as an address: the device address of each GPU's copy
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_buffer(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

}  // namespace smla
