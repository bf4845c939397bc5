// Host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

struct ConvertArgs {
  const int32_t* req_id;
  const int32_t* block_table;
  int32_t num_reqs, max_blocks;
  int64_t bt_row_stride;
  const int32_t* topk_local;
  int64_t topk_local_stride;
  int32_t num_tokens, topk, block_size, block_stride_rows;
  int32_t* global_out;
  int64_t global_stride;
  int32_t* valid_counts;
};

struct DcpFilterArgs {
  const int32_t* req_id;
  const int32_t* block_table;
  int32_t num_reqs, max_blocks;
  int64_t bt_row_stride;
  const int32_t* topk_tokens;
  int64_t in_stride;
  int32_t num_tokens, topk, dcp_size, dcp_rank, interleave, block_size, block_stride_rows;
  bool compact;
  int32_t* out;
  int64_t out_stride;
  int32_t* valid_counts;
};

// Partial results to merge by LSE: out_r [T][H][512] bf16 and lse_r [T][H],
// part r at part_o + r * po_rank (elements) and part_lse + r * pl_rank.
struct MergeArgs {
  const uint16_t* part_o;
  int64_t po_rank, po_tok, po_head;
  const float* part_lse;
  int64_t pl_rank, pl_tok;
  int32_t parts, num_tokens, num_heads;
  uint16_t* out;
  int64_t out_st, out_sh;
  float* lse;
  int64_t lse_st;
  const float* sinks;   // [num_heads] extra logits (zero value rows), or nullptr
};

struct PlannedCountsArgs {
  const int32_t* seq_lens;
  const int32_t* query_start_loc;
  const int32_t* req_id;
  int32_t num_reqs, num_tokens, topk, kpool;
  int32_t* out;
};

struct UpconvertArgs {
  const uint8_t* cache;
  int64_t num_slots, row_stride;
  const int32_t* block_table;
  int32_t num_reqs, max_blocks;
  int64_t bt_row_stride;
  int32_t block_size, block_stride_rows;
  const int32_t* seq_lens;
  const int32_t* starts;
  int32_t max_seq_len;
  uint16_t* ws;
  int64_t ws_rows, ws_stride;
};

struct CacheWriteArgs {
  const uint16_t* kv_c;
  int64_t kv_c_stride;
  const uint16_t* k_pe;
  int64_t k_pe_stride;
  const int64_t* slot_mapping;
  int32_t num_tokens, d_rope, kv_format;
  float k_scale;
  uint8_t* cache;
  int64_t num_slots, row_stride;
  float* group_scales;
  int64_t gs_stride;             // floats between consecutive slots' scale rows
};

// Attention launch description (validated by the ABI layer).
struct AttnArgs {
  const uint16_t* q_nope;
  int64_t qn_st, qn_sh;
  const uint16_t* q_rope;
  int64_t qr_st, qr_sh;
  int32_t num_tokens, num_heads, d_rope;
  const uint8_t* kv;
  int64_t num_slots, kv_row_stride;
  int32_t kv_format;
  float k_scale;
  const float* group_scales;
  int64_t gs_stride;             // floats between consecutive slots' scale rows
  const int32_t* indices;
  int64_t idx_stride;
  int32_t topk;
  const int32_t* topk_length;
  float softmax_scale;
  uint16_t* out;
  int64_t out_st, out_sh;
  float* lse;
  int64_t lse_st;
  // fused index conversion (block_table != nullptr: indices are request-local)
  const int32_t* req_id;
  const int32_t* block_table;
  int32_t num_reqs, max_blocks;
  int64_t bt_row_stride;
  int32_t block_size, block_stride_rows;
  float softcap;                 // > 0: logits c tanh(z / c)
  const float* sinks;            // [num_heads] or nullptr
  hipEvent_t ev_start, ev_end;   // optional, recorded around the main kernel
};

constexpr int kTileRows = 32;
constexpr int kMaxTopk = 2048;

// Size of the static device scratch of the allocation-free decode (the split
// partials; the automatic plan needs at most 256 workgroups x 64 heads x
// (1024 + 4) bytes = 16.8 MB).
constexpr size_t kScratchBytes = size_t(32) << 20;
// Device address of the current GPU's copy of that scratch (looked up once per device).
hipError_t scratch_buffer(void** out);

// Split plan from shapes only.
int32_t plan_splits(int32_t num_tokens, int32_t num_heads, int32_t topk, int32_t requested);
size_t workspace_bytes(int32_t num_tokens, int32_t num_heads, int32_t topk, int32_t splits);

hipError_t launch_convert(const ConvertArgs& a, hipStream_t stream);
hipError_t launch_dcp_filter(const DcpFilterArgs& a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream);
hipError_t launch_planned_counts(const PlannedCountsArgs& a, hipStream_t stream);
hipError_t launch_gather_upconvert(const UpconvertArgs& a, hipStream_t stream);
// splits == 1: direct output. splits > 1: partials into workspace + combine.
hipError_t launch_attention(const AttnArgs& a, int32_t splits, void* workspace, bool longest_first,
                            hipStream_t stream);

}  // namespace smla
