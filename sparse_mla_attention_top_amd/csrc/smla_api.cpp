// C ABI of the sparse MLA library: argument checks, error reporting and
// dispatch to the gfx950 kernel launchers. No allocation, no host sync.
#include "../../include/smla.h"
#include "smla_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_ev_start = nullptr, g_ev_end = nullptr;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SMLA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SMLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_attn(const smla_attn_args* a, bool decode) {
  if (!a) return fail(SMLA_ERR_INVALID_ARG, "args is NULL");
  if (a->num_tokens < 0) return fail(SMLA_ERR_INVALID_ARG, "num_tokens < 0");
  if (a->num_heads < 1 || a->num_heads > 128)
    return fail(SMLA_ERR_UNSUPPORTED, "num_heads=%d outside 1..128", a->num_heads);
  if (a->d_rope != 0 && a->d_rope != 64)
    return fail(SMLA_ERR_UNSUPPORTED, "d_rope=%d (only 0 or 64)", a->d_rope);
  if (a->topk < 1 || a->topk > smla::kMaxTopk)
    return fail(SMLA_ERR_UNSUPPORTED, "topk=%d outside 1..%d", a->topk, smla::kMaxTopk);
  if (a->kv_format < SMLA_KV_BF16 || a->kv_format > SMLA_KV_FP8_DS_MLA)
    return fail(SMLA_ERR_INVALID_ARG, "unknown kv_format %d", a->kv_format);
  if (a->kv_format == SMLA_KV_FP8_DS_MLA && a->d_rope != 64)
    return fail(SMLA_ERR_UNSUPPORTED, "the packed FP8 format holds 512 latent + 64 rope channels (d_rope=%d)",
                a->d_rope);
  if (!std::isfinite(a->softmax_scale)) return fail(SMLA_ERR_INVALID_ARG, "softmax_scale not finite");
  if (a->num_tokens == 0) return SMLA_OK;
  if (!a->q_nope || !a->kv_cache || !a->indices || !a->out)
    return fail(SMLA_ERR_INVALID_ARG, "q_nope, kv_cache, indices and out must be non-NULL");
  if (a->d_rope > 0 && !a->q_rope) return fail(SMLA_ERR_INVALID_ARG, "q_rope is NULL with d_rope=64");
  if (a->num_slots < 1 || a->num_slots > INT32_MAX)
    return fail(SMLA_ERR_INVALID_ARG, "num_slots=%lld outside 1..2^31-1", (long long)a->num_slots);
  const int D = 512 + a->d_rope;
  const int64_t row_bytes = a->kv_format == SMLA_KV_BF16 ? 2 * D : a->kv_format == SMLA_KV_FP8_DS_MLA ? 656 : D;
  if (a->kv_row_stride_bytes < row_bytes || a->kv_row_stride_bytes % 16 != 0)
    return fail(SMLA_ERR_INVALID_ARG, "kv_row_stride_bytes=%lld must be >= %lld and a multiple of 16",
                (long long)a->kv_row_stride_bytes, (long long)row_bytes);
  if (a->kv_row_stride_bytes > (int64_t)UINT32_MAX)
    return fail(SMLA_ERR_UNSUPPORTED, "kv_row_stride_bytes must be below 2^32");
  if (!aligned16(a->kv_cache)) return fail(SMLA_ERR_INVALID_ARG, "kv_cache must be 16-byte aligned");
  if (!aligned16(a->q_nope) || (a->d_rope && !aligned16(a->q_rope)))
    return fail(SMLA_ERR_INVALID_ARG, "q_nope/q_rope must be 16-byte aligned");
  if (a->q_nope_stride_tok % 8 || a->q_nope_stride_head % 8 ||
      (a->d_rope && (a->q_rope_stride_tok % 8 || a->q_rope_stride_head % 8)))
    return fail(SMLA_ERR_INVALID_ARG, "query strides must be multiples of 8 elements");
  if (a->indices_stride < a->topk) return fail(SMLA_ERR_INVALID_ARG, "indices_stride < topk");
  if (a->out_stride_head < 512 && a->num_heads > 1)
    return fail(SMLA_ERR_INVALID_ARG, "out_stride_head < 512");
  if (!aligned16(a->out) || a->out_stride_tok % 8 || a->out_stride_head % 8)
    return fail(SMLA_ERR_INVALID_ARG, "out must be 16-byte aligned with strides that are multiples of 8 elements");
  if (a->lse && a->lse_stride_tok < a->num_heads) return fail(SMLA_ERR_INVALID_ARG, "lse_stride_tok < num_heads");
  if (a->block_table) {
    if (!a->req_id) return fail(SMLA_ERR_INVALID_ARG, "req_id is NULL with a block table");
    if (a->num_reqs < 1 || a->max_blocks < 1 || a->bt_row_stride < a->max_blocks)
      return fail(SMLA_ERR_INVALID_ARG, "block table shape invalid (num_reqs=%d max_blocks=%d stride=%lld)",
                  a->num_reqs, a->max_blocks, (long long)a->bt_row_stride);
    if (a->block_size < 1 || a->block_stride_rows < 0)
      return fail(SMLA_ERR_INVALID_ARG, "block_size=%d block_stride_rows=%d", a->block_size, a->block_stride_rows);
  }
  if (a->kv_format == SMLA_KV_FP8_E4M3_GROUP128 && !a->group_scales)
    return fail(SMLA_ERR_INVALID_ARG, "group_scales is NULL for the group-scaled FP8 format");
  if (a->kv_format == SMLA_KV_FP8_E4M3_PER_TENSOR && !(std::isfinite(a->k_scale) && a->k_scale > 0))
    return fail(SMLA_ERR_INVALID_ARG, "k_scale must be finite and > 0");
  if (a->kv_format == SMLA_KV_FP8_E4M3_GROUP128 && ((uintptr_t)a->group_scales & 3))
    return fail(SMLA_ERR_INVALID_ARG, "group_scales must be 4-byte aligned");
  if (a->kv_format == SMLA_KV_FP8_E4M3_GROUP128 && a->group_scales_stride != 0 &&
      a->group_scales_stride < (D + 127) / 128)
    return fail(SMLA_ERR_INVALID_ARG, "group_scales_stride=%lld below the %d groups of a %d-channel row",
                (long long)a->group_scales_stride, (D + 127) / 128, D);
  if (a->group_scales_stride < 0) return fail(SMLA_ERR_INVALID_ARG, "group_scales_stride < 0");
  if (!(std::isfinite(a->softcap) && a->softcap >= 0.0f))
    return fail(SMLA_ERR_INVALID_ARG, "softcap must be finite and >= 0 (0 = off)");
  if ((uintptr_t)a->sinks & 3) return fail(SMLA_ERR_INVALID_ARG, "sinks must be 4-byte aligned");
  if (a->kv_format == SMLA_KV_FP8_DS_MLA && a->group_scales)
    return fail(SMLA_ERR_INVALID_ARG, "group_scales must be NULL for the packed FP8 format (its scales are in the row)");
  if (decode && a->num_splits < 0) return fail(SMLA_ERR_INVALID_ARG, "num_splits < 0");
  return SMLA_OK;
}

smla::AttnArgs to_internal(const smla_attn_args* a) {
  smla::AttnArgs r;
  r.q_nope = (const uint16_t*)a->q_nope;
  r.qn_st = a->q_nope_stride_tok;
  r.qn_sh = a->q_nope_stride_head;
  r.q_rope = (const uint16_t*)a->q_rope;
  r.qr_st = a->q_rope_stride_tok;
  r.qr_sh = a->q_rope_stride_head;
  r.num_tokens = a->num_tokens;
  r.num_heads = a->num_heads;
  r.d_rope = a->d_rope;
  r.kv = (const uint8_t*)a->kv_cache;
  r.num_slots = a->num_slots;
  r.kv_row_stride = a->kv_row_stride_bytes;
  r.kv_format = a->kv_format;
  r.k_scale = a->k_scale;
  r.group_scales = a->group_scales;
  r.gs_stride = a->group_scales_stride ? a->group_scales_stride : (512 + a->d_rope + 127) / 128;
  r.indices = a->indices;
  r.idx_stride = a->indices_stride;
  r.topk = a->topk;
  r.topk_length = a->topk_length;
  r.softmax_scale = a->softmax_scale;
  r.out = (uint16_t*)a->out;
  r.out_st = a->out_stride_tok;
  r.out_sh = a->out_stride_head;
  r.lse = a->lse;
  r.lse_st = a->lse_stride_tok;
  r.req_id = a->req_id;
  r.block_table = a->block_table;
  r.num_reqs = a->num_reqs;
  r.max_blocks = a->max_blocks;
  r.bt_row_stride = a->bt_row_stride;
  r.block_size = a->block_size;
  r.block_stride_rows = a->block_stride_rows == 0 ? a->block_size : a->block_stride_rows;
  r.softcap = a->softcap;
  r.sinks = a->sinks;
  r.ev_start = g_ev_start;
  r.ev_end = g_ev_end;
  return r;
}

}  // namespace

namespace smla {

int32_t plan_splits(int32_t num_tokens, int32_t num_heads, int32_t topk, int32_t requested) {
  // 64-bit throughout: the sizing entry points take any int32 arguments
  const int64_t max_splits = std::max<int64_t>(1, ((int64_t)topk + kTileRows - 1) / kTileRows);
  if (requested > 0) return (int32_t)std::min<int64_t>(requested, max_splits);
  if (num_tokens <= 0) return 1;
  // One workgroup per CU (the LDS use allows one): the most splits that keep
  // tokens x head blocks x splits within one round of 256 workgroups, since a
  // second partial round costs a whole workgroup time.
  const int64_t head_blocks = num_heads > 64 ? 2 : 1;
  const int64_t target_wgs = 256;
  int64_t s = target_wgs / ((int64_t)num_tokens * head_blocks);
  const int64_t min_rows = 256;                // keep >= 8 tiles per split
  s = std::min<int64_t>(s, std::max<int64_t>(1, (int64_t)topk / min_rows));
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>(s, max_splits));
}


// The partials take the same space whatever the top-k width (topk is part of
// the signature so that a later plan may size by it).
size_t workspace_bytes(int32_t num_tokens, int32_t num_heads, [[maybe_unused]] int32_t topk, int32_t splits) {
  if (splits <= 1) return 0;
  const size_t n = (size_t)splits * num_tokens * num_heads;
  return n * 512 * sizeof(uint16_t) + n * sizeof(float);   // bf16 [splits][T][H][512] + fp32 LSE
}

}  // namespace smla

extern "C" {

const char* smla_last_error(void) { return g_err; }

const char* smla_version(void) { return "smla 0.2 gfx950"; }

size_t smla_attn_args_size(void) { return sizeof(smla_attn_args); }

int smla_set_timing_events(void* start, void* end) {
  if ((start == nullptr) != (end == nullptr)) return fail(SMLA_ERR_INVALID_ARG, "set both events or neither");
  g_ev_start = (hipEvent_t)start;
  g_ev_end = (hipEvent_t)end;
  return ok();
}

int smla_convert_indices(const int32_t* req_id, const int32_t* block_table, int32_t num_reqs,
                         int32_t max_blocks, int64_t bt_row_stride, const int32_t* topk_local,
                         int64_t topk_local_stride, int32_t num_tokens, int32_t topk, int32_t block_size,
                         int32_t block_stride_rows, int32_t* global_out, int64_t global_stride,
                         int32_t* valid_counts, void* stream) {
  if (num_tokens < 0 || topk < 0) return fail(SMLA_ERR_INVALID_ARG, "num_tokens/topk < 0");
  if (block_size < 1) return fail(SMLA_ERR_INVALID_ARG, "block_size=%d must be >= 1", block_size);
  if (block_stride_rows < 0) return fail(SMLA_ERR_INVALID_ARG, "block_stride_rows < 0");
  if (num_reqs < 1 || max_blocks < 1 || bt_row_stride < max_blocks)
    return fail(SMLA_ERR_INVALID_ARG, "block table shape invalid (num_reqs=%d max_blocks=%d stride=%lld)",
                num_reqs, max_blocks, (long long)bt_row_stride);
  if (topk_local_stride < topk || global_stride < topk)
    return fail(SMLA_ERR_INVALID_ARG, "row strides must be >= topk");
  if (num_tokens == 0) return ok();
  if (!req_id || !block_table || (topk > 0 && (!topk_local || !global_out)))
    return fail(SMLA_ERR_INVALID_ARG, "NULL pointer argument");
  smla::ConvertArgs a{req_id, block_table, num_reqs, max_blocks, bt_row_stride, topk_local,
                      topk_local_stride, num_tokens, topk, block_size,
                      block_stride_rows == 0 ? block_size : block_stride_rows, global_out, global_stride,
                      valid_counts};
  return hip_status(smla::launch_convert(a, (hipStream_t)stream), "convert_indices launch");
}

int smla_dcp_filter_convert(const int32_t* req_id, const int32_t* block_table, int32_t num_reqs,
                            int32_t max_blocks, int64_t bt_row_stride, const int32_t* topk_tokens,
                            int64_t topk_tokens_stride, int32_t num_tokens, int32_t topk, int32_t dcp_size,
                            int32_t dcp_rank, int32_t interleave, int32_t block_size, int32_t block_stride_rows,
                            int32_t compact_valid_to_front, int32_t* local_out, int64_t local_stride,
                            int32_t* valid_counts, void* stream) {
  if (num_tokens < 0 || topk < 0) return fail(SMLA_ERR_INVALID_ARG, "num_tokens/topk < 0");
  if (dcp_size < 1 || dcp_rank < 0 || dcp_rank >= dcp_size)
    return fail(SMLA_ERR_INVALID_ARG, "dcp_rank=%d outside 0..dcp_size-1 (dcp_size=%d)", dcp_rank, dcp_size);
  if (interleave < 1) return fail(SMLA_ERR_INVALID_ARG, "interleave=%d must be >= 1", interleave);
  if (block_size < 1) return fail(SMLA_ERR_INVALID_ARG, "block_size=%d must be >= 1", block_size);
  if (block_stride_rows < 0) return fail(SMLA_ERR_INVALID_ARG, "block_stride_rows < 0");
  if (num_reqs < 1 || max_blocks < 1 || bt_row_stride < max_blocks)
    return fail(SMLA_ERR_INVALID_ARG, "block table shape invalid (num_reqs=%d max_blocks=%d stride=%lld)",
                num_reqs, max_blocks, (long long)bt_row_stride);
  if (topk_tokens_stride < topk || local_stride < topk) return fail(SMLA_ERR_INVALID_ARG, "row strides must be >= topk");
  if (num_tokens == 0) return ok();
  if (!req_id || !block_table || (topk > 0 && (!topk_tokens || !local_out)))
    return fail(SMLA_ERR_INVALID_ARG, "NULL pointer argument");
  smla::DcpFilterArgs a{req_id, block_table, num_reqs, max_blocks, bt_row_stride, topk_tokens, topk_tokens_stride,
                        num_tokens, topk, dcp_size, dcp_rank, interleave, block_size,
                        block_stride_rows == 0 ? block_size : block_stride_rows, compact_valid_to_front != 0,
                        local_out, local_stride, valid_counts};
  return hip_status(smla::launch_dcp_filter(a, (hipStream_t)stream), "dcp_filter_convert launch");
}

int smla_planned_valid_counts(const int32_t* seq_lens, const int32_t* query_start_loc,
                              const int32_t* req_id_per_token, int32_t num_reqs, int32_t num_tokens, int32_t topk,
                              int32_t kpool, int32_t* valid_counts_out, void* stream) {
  if (num_reqs < 1 || num_tokens < 0) return fail(SMLA_ERR_INVALID_ARG, "num_reqs=%d num_tokens=%d", num_reqs, num_tokens);
  if (topk < 1 || kpool < 1) return fail(SMLA_ERR_INVALID_ARG, "topk=%d kpool=%d must be >= 1", topk, kpool);
  if (num_tokens == 0) return ok();
  if (!seq_lens || !query_start_loc || !req_id_per_token || !valid_counts_out)
    return fail(SMLA_ERR_INVALID_ARG, "NULL pointer argument");
  smla::PlannedCountsArgs a{seq_lens, query_start_loc, req_id_per_token, num_reqs, num_tokens, topk, kpool,
                            valid_counts_out};
  return hip_status(smla::launch_planned_counts(a, (hipStream_t)stream), "planned_valid_counts launch");
}

int smla_gather_upconvert(const void* kv_cache, int64_t num_slots, int64_t kv_row_stride_bytes, int32_t kv_format,
                          const int32_t* block_table, int32_t num_reqs, int32_t max_blocks, int64_t bt_row_stride,
                          int32_t block_size, int32_t block_stride_rows, const int32_t* seq_lens,
                          const int32_t* workspace_starts, int32_t max_seq_len, void* workspace,
                          int64_t workspace_rows, int64_t workspace_row_stride, void* stream) {
  if (kv_format != SMLA_KV_FP8_DS_MLA)
    return fail(SMLA_ERR_UNSUPPORTED, "gather_upconvert reads the packed FP8 format only (kv_format=%d)", kv_format);
  if (num_reqs < 0 || max_seq_len < 0) return fail(SMLA_ERR_INVALID_ARG, "num_reqs=%d max_seq_len=%d", num_reqs, max_seq_len);
  if (num_slots < 1 || num_slots > INT32_MAX)
    return fail(SMLA_ERR_INVALID_ARG, "num_slots=%lld outside 1..2^31-1", (long long)num_slots);
  if (kv_row_stride_bytes < 656 || kv_row_stride_bytes % 16 != 0)
    return fail(SMLA_ERR_INVALID_ARG, "kv_row_stride_bytes=%lld must be >= 656 and a multiple of 16",
                (long long)kv_row_stride_bytes);
  if (max_blocks < 1 || bt_row_stride < max_blocks || block_size < 1 || block_stride_rows < 0)
    return fail(SMLA_ERR_INVALID_ARG, "block table shape invalid (max_blocks=%d stride=%lld block_size=%d)",
                max_blocks, (long long)bt_row_stride, block_size);
  if (workspace_rows < 0 || workspace_row_stride < 576 || workspace_row_stride % 8 != 0)
    return fail(SMLA_ERR_INVALID_ARG, "workspace row stride must be >= 576 and a multiple of 8 elements");
  if (num_reqs > 65535) return fail(SMLA_ERR_UNSUPPORTED, "num_reqs above 65535");
  if (num_reqs == 0 || max_seq_len == 0 || workspace_rows == 0) return ok();
  if (!kv_cache || !block_table || !seq_lens || !workspace_starts || !workspace)
    return fail(SMLA_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned16(kv_cache) || !aligned16(workspace))
    return fail(SMLA_ERR_INVALID_ARG, "kv_cache and workspace must be 16-byte aligned");
  smla::UpconvertArgs a{(const uint8_t*)kv_cache, num_slots, kv_row_stride_bytes, block_table, num_reqs, max_blocks,
                        bt_row_stride, block_size, block_stride_rows == 0 ? block_size : block_stride_rows,
                        seq_lens, workspace_starts, max_seq_len, (uint16_t*)workspace, workspace_rows,
                        workspace_row_stride};
  return hip_status(smla::launch_gather_upconvert(a, (hipStream_t)stream), "gather_upconvert launch");
}

int smla_merge_partials(const void* part_out, int64_t part_out_stride_part, int64_t part_out_stride_tok,
                        int64_t part_out_stride_head, const float* part_lse, int64_t part_lse_stride_part,
                        int64_t part_lse_stride_tok, int32_t num_parts, int32_t num_tokens, int32_t num_heads,
                        void* out, int64_t out_stride_tok, int64_t out_stride_head, float* lse,
                        int64_t lse_stride_tok, void* stream) {
  if (num_parts < 1 || num_tokens < 0 || num_heads < 1)
    return fail(SMLA_ERR_INVALID_ARG, "num_parts=%d num_tokens=%d num_heads=%d", num_parts, num_tokens, num_heads);
  if (num_tokens == 0) return ok();
  if (!part_out || !part_lse || !out) return fail(SMLA_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned16(part_out) || !aligned16(out) || part_out_stride_part % 8 || part_out_stride_tok % 8 ||
      part_out_stride_head % 8 || out_stride_tok % 8 || out_stride_head % 8)
    return fail(SMLA_ERR_INVALID_ARG, "part_out/out must be 16-byte aligned with strides that are multiples of 8 elements");
  if (part_out_stride_head < 512 && num_heads > 1) return fail(SMLA_ERR_INVALID_ARG, "part_out_stride_head < 512");
  if (out_stride_head < 512 && num_heads > 1) return fail(SMLA_ERR_INVALID_ARG, "out_stride_head < 512");
  if (part_lse_stride_tok < num_heads || (lse && lse_stride_tok < num_heads))
    return fail(SMLA_ERR_INVALID_ARG, "LSE token stride < num_heads");
  smla::MergeArgs m;
  m.part_o = (const uint16_t*)part_out;
  m.po_rank = part_out_stride_part;
  m.po_tok = part_out_stride_tok;
  m.po_head = part_out_stride_head;
  m.part_lse = part_lse;
  m.pl_rank = part_lse_stride_part;
  m.pl_tok = part_lse_stride_tok;
  m.parts = num_parts;
  m.num_tokens = num_tokens;
  m.num_heads = num_heads;
  m.out = (uint16_t*)out;
  m.out_st = out_stride_tok;
  m.out_sh = out_stride_head;
  m.lse = lse;
  m.lse_st = lse_stride_tok;
  m.sinks = nullptr;
  return hip_status(smla::launch_merge(m, (hipStream_t)stream), "merge_partials launch");
}

int32_t smla_decode_num_splits(int32_t num_tokens, int32_t num_heads, int32_t topk, int32_t num_splits) {
  return smla::plan_splits(num_tokens, num_heads, topk, num_splits);
}

size_t smla_decode_workspace_size(int32_t num_tokens, int32_t num_heads, int32_t topk, int32_t num_splits) {
  if (num_tokens <= 0 || num_heads <= 0 || topk <= 0) return 0;
  const int32_t s = smla::plan_splits(num_tokens, num_heads, topk, num_splits);
  return smla::workspace_bytes(num_tokens, num_heads, topk, s);
}

int smla_decode_fwd(const smla_attn_args* args, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_attn(args, true);
  if (rc != SMLA_OK) return rc;
  if (args->num_tokens == 0) return ok();
  const int32_t s = smla::plan_splits(args->num_tokens, args->num_heads, args->topk, args->num_splits);
  const size_t need = smla::workspace_bytes(args->num_tokens, args->num_heads, args->topk, s);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(SMLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if (need > 0 && !aligned16(workspace)) return fail(SMLA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return hip_status(smla::launch_attention(to_internal(args), s, workspace, false, (hipStream_t)stream),
                    "decode launch");
}

int smla_decode_fwd_noalloc(const smla_attn_args* args, void* stream) {
  int rc = check_attn(args, true);
  if (rc != SMLA_OK) return rc;
  if (args->num_tokens == 0) return ok();
  const int32_t s = smla::plan_splits(args->num_tokens, args->num_heads, args->topk, args->num_splits);
  const size_t need = smla::workspace_bytes(args->num_tokens, args->num_heads, args->topk, s);
  if (need > smla::kScratchBytes)
    return fail(SMLA_ERR_WORKSPACE_TOO_SMALL,
                "%d splits x %d tokens x %d heads need %zu bytes of split partials, above the %zu-byte static "
                "scratch of the allocation-free decode (use smla_decode_fwd with a workspace, or fewer splits)",
                s, args->num_tokens, args->num_heads, need, smla::kScratchBytes);
  void* scratch = nullptr;
  if (need > 0) {
    const hipError_t e = smla::scratch_buffer(&scratch);
    if (e != hipSuccess) return hip_status(e, "static scratch address");
  }
  return hip_status(smla::launch_attention(to_internal(args), s, scratch, false, (hipStream_t)stream),
                    "decode launch");
}

int smla_prefill_fwd(const smla_attn_args* args, void* stream) {
  int rc = check_attn(args, false);
  if (rc != SMLA_OK) return rc;
  if (args->num_tokens == 0) return ok();
  return hip_status(smla::launch_attention(to_internal(args), 1, nullptr, true, (hipStream_t)stream),
                    "prefill launch");
}

int smla_cache_write(const void* kv_c, int64_t kv_c_stride, const void* k_pe, int64_t k_pe_stride,
                     const int64_t* slot_mapping, int32_t num_tokens, int32_t d_rope, int32_t kv_format,
                     float k_scale, void* kv_cache, int64_t num_slots, int64_t kv_row_stride_bytes,
                     float* group_scales, int64_t group_scales_stride, void* stream) {
  if (num_tokens < 0) return fail(SMLA_ERR_INVALID_ARG, "num_tokens < 0");
  if (d_rope != 0 && d_rope != 64) return fail(SMLA_ERR_UNSUPPORTED, "d_rope=%d (only 0 or 64)", d_rope);
  if (kv_format < SMLA_KV_BF16 || kv_format > SMLA_KV_FP8_DS_MLA)
    return fail(SMLA_ERR_INVALID_ARG, "unknown kv_format %d", kv_format);
  if (kv_format == SMLA_KV_FP8_DS_MLA && d_rope != 64)
    return fail(SMLA_ERR_UNSUPPORTED, "the packed FP8 format holds 512 latent + 64 rope channels (d_rope=%d)", d_rope);
  if (num_tokens == 0) return ok();
  if (!kv_c || !slot_mapping || !kv_cache) return fail(SMLA_ERR_INVALID_ARG, "NULL pointer argument");
  if (d_rope && !k_pe) return fail(SMLA_ERR_INVALID_ARG, "k_pe is NULL with d_rope=64");
  if (kv_c_stride < 512 || (d_rope && k_pe_stride < d_rope))
    return fail(SMLA_ERR_INVALID_ARG, "source row strides too small");
  const int D = 512 + d_rope;
  const int64_t row_bytes = kv_format == SMLA_KV_BF16 ? 2 * D : kv_format == SMLA_KV_FP8_DS_MLA ? 656 : D;
  if (kv_row_stride_bytes < row_bytes || kv_row_stride_bytes % 16 != 0 || !aligned16(kv_cache))
    return fail(SMLA_ERR_INVALID_ARG, "cache row stride must be >= %lld and a multiple of 16, base 16-byte aligned",
                (long long)row_bytes);
  if (num_slots < 1) return fail(SMLA_ERR_INVALID_ARG, "num_slots < 1");
  if (kv_format == SMLA_KV_FP8_E4M3_PER_TENSOR && !(std::isfinite(k_scale) && k_scale > 0))
    return fail(SMLA_ERR_INVALID_ARG, "k_scale must be finite and > 0");
  if (kv_format == SMLA_KV_FP8_E4M3_GROUP128 && !group_scales)
    return fail(SMLA_ERR_INVALID_ARG, "group_scales is NULL for the group-scaled FP8 format");
  const int G = (D + 127) / 128;
  if (group_scales_stride < 0 || (group_scales_stride != 0 && group_scales_stride < G))
    return fail(SMLA_ERR_INVALID_ARG, "group_scales_stride=%lld: 0 or >= %d", (long long)group_scales_stride, G);
  if (kv_format == SMLA_KV_FP8_E4M3_GROUP128 && ((uintptr_t)group_scales & 3))
    return fail(SMLA_ERR_INVALID_ARG, "group_scales must be 4-byte aligned");
  smla::CacheWriteArgs a{(const uint16_t*)kv_c, kv_c_stride, (const uint16_t*)k_pe, k_pe_stride, slot_mapping,
                         num_tokens, d_rope, kv_format, k_scale, (uint8_t*)kv_cache, num_slots,
                         kv_row_stride_bytes, group_scales, group_scales_stride ? group_scales_stride : G};
  return hip_status(smla::launch_cache_write(a, (hipStream_t)stream), "cache_write launch");
}

}  // extern "C"
