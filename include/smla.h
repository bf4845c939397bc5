/*
 * smla.h -- C ABI of the sparse multi-head latent attention (MLA) forward
 * path on AMD Instinct MI355X (gfx950).
 *
 * What the library computes is fixed by the pages it follows:
 *
 *  - vLLM "Sparse MLA on Hopper" branch (compare bz/sleep-metric...
 *    rebase-fa3-mla-sparse): backends/mla/cutlass_fa3_sparse.py
 *    (CutlassFA3MLASparseImpl.forward_mqa, _forward_fa3, do_kv_cache_update)
 *    and tests/v1/attention/test_cutlass_fa3_sparse_backend.py;
 *  - the FA3 kernel test file of the same branch (compare rebase-fa3-mla-
 *    sparse..cutlass_fa3_mla_sparse), test_fa3_mla_correctness_vs_reference;
 *  - vLLM API docs, vllm.v1.attention.backends.mla.flashmla_sparse
 *    (FlashMLASparseImpl: head padding, _forward_fp8_kv_mixed_batch LSE);
 *  - flashinfer_mla_sparse_sm90.py (module docstring: NoPE, FP8 E4M3 cache
 *    with per-tensor or per-token x 128-channel-group scales; forward_mqa).
 *
 * Every query token t has h heads q[t, i, 0:D] (D = 512 latent channels
 * followed by d_rope = 64 rope channels, or d_rope = 0 for NoPE) and one
 * row of top-k global cache slots shared by all of its heads. Over the
 * valid entries j of that row (position j < topk_length[t] when a length
 * array is given, and 0 <= slot < num_slots):
 *     s_j   = softmax_scale * sum_d q[t,i,d] * kv[slot_j, d]      (d < D)
 *     out   = sum_j softmax(s)_j * kv[slot_j, 0:512]               (latent)
 *     lse   = ln sum_j exp(s_j)
 * A row with no valid entry gives out = 0 and lse = -inf.
 *
 * Conventions for every entry point:
 *  - All pointers are DEVICE pointers unless stated otherwise; the caller
 *    owns every buffer. The library allocates nothing per call.
 *  - Calls only enqueue work on `stream` (a hipStream_t, NULL = default
 *    stream); they never synchronise the host, and the launch plan depends
 *    on shapes only, so the calls can be captured in a HIP graph.
 *  - Arguments are checked on the host; a bad argument returns
 *    SMLA_ERR_INVALID_ARG or SMLA_ERR_UNSUPPORTED without launching
 *    anything, and smla_last_error() describes it. A failed launch returns
 *    SMLA_ERR_HIP. No C++ exception crosses this interface.
 *  - bf16 tensors are passed as raw 16-bit storage; strides are in
 *    ELEMENTS of the tensor's own type unless named *_bytes.
 */
#ifndef SMLA_H_
#define SMLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SMLA_OK = 0,
  SMLA_ERR_INVALID_ARG = -1,
  SMLA_ERR_UNSUPPORTED = -2,
  SMLA_ERR_WORKSPACE_TOO_SMALL = -3,
  SMLA_ERR_HIP = -4
} smla_status;

/* Cache row storage formats (flashinfer_mla_sparse_sm90.py docstring;
 * vLLM kv_cache_dtype "auto"/"bfloat16" and "fp8"/"fp8_e4m3"). */
typedef enum {
  /* row = D bf16 values */
  SMLA_KV_BF16 = 0,
  /* row = D OCP E4M3FN bytes; value = e4m3(byte) * k_scale */
  SMLA_KV_FP8_E4M3_PER_TENSOR = 1,
  /* row = D OCP E4M3FN bytes; value = e4m3(byte) * scale g = c/128 of the
   * slot, from a separate fp32 array with one row of ceil(D/128) scales per
   * slot (rows group_scales_stride floats apart) */
  SMLA_KV_FP8_E4M3_GROUP128 = 2,
  /* Packed 656-byte row (the FP8 cache of the FlashMLA sparse backend, whose
   * docs give 656 bytes per token but no layout; this layout is the split of
   * that size by the group-scale rule above): bytes 0..511 the E4M3FN codes
   * of the 512 latent channels, 512..527 four little-endian fp32 scales
   * (latent channel c is e4m3(byte c) * scale[c / 128]), 528..655 the 64
   * rope channels as plain bf16. Requires d_rope = 64 and group_scales =
   * NULL; kv_row_stride_bytes >= 656 (a multiple of 16, e.g. 656). */
  SMLA_KV_FP8_DS_MLA = 3
} smla_kv_format;

/* Arguments of the attention entry points. */
typedef struct {
  /* Query, bf16. q_nope: [T][h][512]; q_rope: [T][h][d_rope], may be NULL
   * iff d_rope == 0. Both may be views of one [T][h][576] tensor. */
  const void* q_nope;
  int64_t q_nope_stride_tok, q_nope_stride_head;
  const void* q_rope;
  int64_t q_rope_stride_tok, q_rope_stride_head;
  int32_t num_tokens;   /* T >= 0 */
  int32_t num_heads;    /* h, 1..128; padded internally to 64 or 128 with zero heads */
  int32_t d_rope;       /* 64, or 0 for NoPE (D = 512 + d_rope) */

  /* Latent cache: num_slots rows, kv_row_stride_bytes apart (a paged
   * [num_blocks][block_size][D] cache is num_blocks*block_size rows). The
   * row stride must be a multiple of 16 bytes and the base 16-byte aligned. */
  const void* kv_cache;
  int64_t num_slots;
  int64_t kv_row_stride_bytes;
  int32_t kv_format;            /* smla_kv_format */
  float k_scale;                /* SMLA_KV_FP8_E4M3_PER_TENSOR */
  const float* group_scales;    /* SMLA_KV_FP8_E4M3_GROUP128: row `slot` holds the scales
                                 * of groups 0..ceil(D/128)-1 at group_scales[slot *
                                 * group_scales_stride + g] (group_scales_stride below) */

  /* Global slot indices [T][topk] int32 (row stride indices_stride), as
   * produced by smla_convert_indices; negative = invalid. (Request-local
   * indices when the fused conversion below is used.) */
  const int32_t* indices;
  int64_t indices_stride;
  int32_t topk;                 /* 1..2048 */
  /* Optional [T] int32: only entries j < topk_length[t] are read. NULL =
   * the whole row. The valid_counts output of smla_convert_indices is a
   * correct length when invalid entries form a tail. */
  const int32_t* topk_length;

  float softmax_scale;

  /* Output bf16 [T][h][512], 16-byte aligned, strides multiples of 8
   * elements; LSE fp32 [T][h] natural log (NULL = not wanted). Only the h
   * true heads are written. */
  void* out;
  int64_t out_stride_tok, out_stride_head;
  float* lse;
  int64_t lse_stride_tok;

  /* Decode only: number of top-k splits, 0 = choose from the shapes. */
  int32_t num_splits;

  /* Optional fused index conversion (the operation of smla_convert_indices,
   * done by the attention kernel while it stages a row's indices). When
   * block_table is not NULL, `indices` holds request-local indices (the
   * topk_local input of smla_convert_indices) and entry l of row t is used
   * as slot block_table[r][l / block_size] * block_stride_rows
   * + l % block_size, r = req_id[t]; an entry that smla_convert_indices would
   * turn into -1 is skipped. block_stride_rows = 0 means block_size. No valid
   * counts are produced (a -1 tail needs none). NULL = `indices` are global. */
  const int32_t* req_id;        /* [T] int32 */
  const int32_t* block_table;   /* [num_reqs][bt_row_stride] int32, first max_blocks used */
  int32_t num_reqs, max_blocks;
  int64_t bt_row_stride;
  int32_t block_size, block_stride_rows;

  /* Optional softmax options of the FA3 API (flash_attn_with_kvcache
   * arguments softcap and sinks; the pages give the names, not the
   * formulas, and these are the plain readings):
   *   softcap > 0: every scaled logit z = softmax_scale * q.k becomes
   *     softcap * tanh(z / softcap) before the softmax; 0 = off.
   *   sinks: fp32 [num_heads] (4-byte aligned) or NULL. sinks[i] is one more
   *     logit of head i (natural-log units, not capped) whose value row is
   *     zero: out = sum_j e^z_j v_j / (sum_j e^z_j + e^sinks[i]) and LSE is
   *     the log of that denominator; a row with no valid entry gives
   *     (0, sinks[i]). A sink enters a result once: with context-parallel
   *     ranks merged by smla_merge_partials, give it to one rank only. */
  float softcap;
  const float* sinks;

  /* SMLA_KV_FP8_E4M3_GROUP128: floats between the scale rows of consecutive
   * slots, >= ceil(D/128); 0 means exactly ceil(D/128). A cache written with
   * d_rope = 64 (5 scales per row) and read by a NoPE call (d_rope = 0, 4
   * groups used) passes 5 here. Ignored by the other formats. */
  int64_t group_scales_stride;
} smla_attn_args;

/*
 * Request-local top-k indices -> global cache slots (vLLM "Sparse MLA on
 * Hopper" branch, cutlass_fa3_sparse.py forward_mqa step 2 and the test
 * file's TEST 2.5 / TEST 2.9): for entry l of row t, with r = req_id[t],
 *     global[t][j] = block_table[r][l / block_size] * block_stride_rows
 *                    + l % block_size
 * if l >= 0, l / block_size < max_blocks and the table entry is >= 0; else
 * -1. valid_counts[t] (optional, may be NULL) = number of entries != -1.
 * Entries keep their positions (a -1 tail stays a -1 tail).
 *   req_id          [T] int32, each in [0, num_reqs)
 *   block_table     [num_reqs][bt_row_stride] int32, first max_blocks used
 *   topk_local      [T][topk] int32 (row stride topk_local_stride)
 *   global_out      [T][topk] int32 (row stride global_stride)
 * block_stride_rows = 0 means block_size.
 */
int smla_convert_indices(const int32_t* req_id, const int32_t* block_table,
                         int32_t num_reqs, int32_t max_blocks, int64_t bt_row_stride,
                         const int32_t* topk_local, int64_t topk_local_stride,
                         int32_t num_tokens, int32_t topk,
                         int32_t block_size, int32_t block_stride_rows,
                         int32_t* global_out, int64_t global_stride,
                         int32_t* valid_counts, void* stream);

/*
 * Context-parallel shard filter: one rank's view of top-k rows of request
 * token positions (vLLM FlashMLA sparse backend, forward_mqa: the
 * triton_filter_and_convert_dcp_index call with dcp_size, dcp_rank,
 * cp_kv_cache_interleave_size and compact_valid_to_front). The pages name the
 * parameters but print no placement; the one used is the plain interleave:
 * runs of `interleave` consecutive positions of a request go to ranks 0, 1,
 * .., dcp_size-1 in turn and each rank stores its runs back to back, so
 * position p is on rank (p / I) % W at local position (p / (I W)) I + p % I.
 * For entry p of row t with r = req_id[t]:
 *     local_out[t][j] = block_table[r][q / block_size] * block_stride_rows
 *                       + q % block_size,   q = the local position of p,
 * if p >= 0, p is on rank dcp_rank and the lookup is valid as for
 * smla_convert_indices (this rank's block table); else -1. With
 * compact_valid_to_front != 0 the valid entries of a row come first in
 * their order, then -1 (otherwise each entry keeps its position).
 * valid_counts[t] (optional) = entries != -1. local_out may alias topk_tokens.
 *   req_id [T] int32; block_table [num_reqs][bt_row_stride] int32 (this
 *   rank's, first max_blocks used); topk_tokens [T][topk] int32 (row stride
 *   topk_tokens_stride); local_out [T][topk] int32 (row stride local_stride).
 * block_stride_rows = 0 means block_size.
 */
int smla_dcp_filter_convert(const int32_t* req_id, const int32_t* block_table, int32_t num_reqs,
                            int32_t max_blocks, int64_t bt_row_stride, const int32_t* topk_tokens,
                            int64_t topk_tokens_stride, int32_t num_tokens, int32_t topk,
                            int32_t dcp_size, int32_t dcp_rank, int32_t interleave,
                            int32_t block_size, int32_t block_stride_rows,
                            int32_t compact_valid_to_front, int32_t* local_out,
                            int64_t local_stride, int32_t* valid_counts, void* stream);

/*
 * Merge of partial attention results over disjoint parts of the same rows by
 * their LSE, the cross-rank merge of the FlashMLA sparse docs
 * (_forward_fp8_kv_mixed_batch; (0, -inf) is the identity):
 *     lse[t][i] = ln sum_r exp(lse_r[t][i]),
 *     out[t][i] = sum_r exp(lse_r[t][i] - lse[t][i]) * out_r[t][i]
 * and (0, -inf) where every part is (0, -inf). The decode splits use the
 * same kernel.
 *   part_out bf16: part r, token t, head i, channel c at
 *     part_out[r*stride_part + t*stride_tok + i*stride_head + c], c < 512;
 *   part_lse fp32 at part_lse[r*lse_stride_part + t*lse_stride_tok + i];
 *   out bf16 [T][h][512] by its strides; lse fp32 [T][h] or NULL.
 * part_out and out 16-byte aligned, their strides multiples of 8 elements.
 */
int smla_merge_partials(const void* part_out, int64_t part_out_stride_part,
                        int64_t part_out_stride_tok, int64_t part_out_stride_head,
                        const float* part_lse, int64_t part_lse_stride_part,
                        int64_t part_lse_stride_tok, int32_t num_parts, int32_t num_tokens,
                        int32_t num_heads, void* out, int64_t out_stride_tok,
                        int64_t out_stride_head, float* lse, int64_t lse_stride_tok,
                        void* stream);

/* Bytes of caller-owned device workspace smla_decode_fwd needs for these
 * shapes (0 when no split is used). num_splits = 0 means automatic. */
size_t smla_decode_workspace_size(int32_t num_tokens, int32_t num_heads, int32_t topk,
                                  int32_t num_splits);

/* Number of splits smla_decode_fwd will use for these shapes. */
int32_t smla_decode_num_splits(int32_t num_tokens, int32_t num_heads, int32_t topk,
                               int32_t num_splits);

/*
 * Decode forward: the sparse attention above, with the top-k row of each
 * token optionally cut into splits processed in parallel and merged by
 * their LSE (FA3's split-KV + combine; the merge rule is the one the
 * FlashMLA sparse page uses across ranks, with (0, -inf) as identity).
 * workspace: device buffer of at least smla_decode_workspace_size() bytes,
 * contents need not be initialised; may be NULL when that size is 0.
 */
int smla_decode_fwd(const smla_attn_args* args, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): smla_decode_fwd with the split partials kept in a static device
 * scratch of the library instead of a caller workspace. The scratch is one
 * file-scope device array of 32 MiB per GPU, held until the process ends; its
 * address is looked up once per device on the first call there (with that
 * device current). No call allocates. Every call on a GPU shares that GPU's
 * scratch: calls that overlap in time on one GPU (two streams, two threads)
 * race and give wrong results; serialise them. The partials are fully written
 * before they are read, so nothing in the scratch needs clearing. A plan
 * whose partials exceed 32 MiB (num_splits x num_tokens x num_heads x 1028
 * bytes; the automatic plan stays below 17 MB) returns
 * SMLA_ERR_WORKSPACE_TOO_SMALL without launching. Arguments and results as
 * for smla_decode_fwd; the stream must belong to the current device.
 */
int smla_decode_fwd_noalloc(const smla_attn_args* args, void* stream);

/* Prefill forward: the same function without splitting (one workgroup per
 * token); args->num_splits is ignored. */
int smla_prefill_fwd(const smla_attn_args* args, void* stream);

/*
 * Planned valid counts (FlashInfer sparse SM90 backend, _kv_lens_host and
 * _clamp_work_kv_end): the valid count of every query row from the batch
 * layout alone, with no device-to-host copy. Row t belongs to request
 * r = req_id_per_token[t]; the rows of request r are query_start_loc[r] ..
 * query_start_loc[r+1]-1, and row t sees
 *   ctx = seq_lens[r] - query_start_loc[r+1] + t + 1
 * tokens. The pooled top-k indexer keeps all of them when ctx <= topk and
 * otherwise topk pool-expanded tokens plus the trailing incomplete pool:
 *   valid_counts_out[t] = ctx <= topk ? ctx : topk + ctx % kpool.
 * A request id outside [0, num_reqs) or ctx <= 0 gives 0. The counts equal the
 * valid entries of the converted rows when the indexer's selection has that
 * shape, and serve as topk_length for the attention.
 *   seq_lens [num_reqs], query_start_loc [num_reqs + 1], req_id_per_token
 *   [num_tokens], valid_counts_out [num_tokens]: int32 device arrays.
 * Errors: num_reqs < 1, topk < 1 or kpool < 1, NULL pointers.
 */
int smla_planned_valid_counts(const int32_t* seq_lens, const int32_t* query_start_loc,
                              const int32_t* req_id_per_token, int32_t num_reqs, int32_t num_tokens,
                              int32_t topk, int32_t kpool, int32_t* valid_counts_out, void* stream);

/*
 * Gather and upconvert (the FP8 prefill path of the FlashMLA sparse backend,
 * forward_mqa: cp_gather_and_upconvert_fp8_kv_cache of a chunk's contexts into
 * a bf16 workspace, then the bf16 kernel over the workspace). For every
 * request r and position p < min(seq_lens[r], max_blocks * block_size),
 * workspace row workspace_starts[r] + p gets the packed FP8 row at slot
 * block_table[r][p / block_size] * block_stride_rows + p % block_size, as bf16:
 * latent channel c = bf16_rne(fl32(e4m3(code c) * scale[c / 128])) (the pages
 * name the operation, not its rounding; this is the plain reading), rope
 * channels copied. A negative table entry or a slot >= num_slots gives a zero
 * row; rows outside [0, workspace_rows) are not written.
 *   kv_cache: packed rows (kv_format must be SMLA_KV_FP8_DS_MLA), stride >= 656.
 *   block_table [num_reqs][bt_row_stride] int32; seq_lens, workspace_starts
 *   [num_reqs] int32; max_seq_len >= every seq_lens[r] (positions past it are
 *   not written); block_stride_rows = 0 means block_size.
 *   workspace: bf16 [workspace_rows][workspace_row_stride] (>= 576 elements, a
 *   multiple of 8), 16-byte aligned.
 * The bf16 attention then reads the workspace with indices
 * workspace_starts[r] + p (or request-local indices through a block table
 * that maps request r's block b to workspace block starts[r] / B + b).
 */
int smla_gather_upconvert(const void* kv_cache, int64_t num_slots, int64_t kv_row_stride_bytes,
                          int32_t kv_format, const int32_t* block_table, int32_t num_reqs, int32_t max_blocks,
                          int64_t bt_row_stride, int32_t block_size, int32_t block_stride_rows,
                          const int32_t* seq_lens, const int32_t* workspace_starts, int32_t max_seq_len,
                          void* workspace, int64_t workspace_rows, int64_t workspace_row_stride,
                          void* stream);

/*
 * Cache write (vLLM concat_and_cache_mla as called by do_kv_cache_update):
 * row slot_mapping[t] of the cache gets [kv_c[t][0:512] | k_pe[t][0:d_rope]].
 * slot_mapping < 0 skips the token. Formats:
 *   SMLA_KV_BF16                 bf16 copy;
 *   SMLA_KV_FP8_E4M3_PER_TENSOR  byte = e4m3_rne(fl32(x / k_scale)), saturated at 448;
 *   SMLA_KV_FP8_E4M3_GROUP128    per row and 128-channel group g (g < ceil(D/128),
 *                                D = 512 + d_rope): scale = fl32(absmax / 448) (1 if the
 *                                group is all zero), written to group_scales[slot *
 *                                group_scales_stride + g] (a stride of 0 means
 *                                ceil(D/128); otherwise it must be >= that); byte as above;
 *   SMLA_KV_FP8_DS_MLA           (d_rope = 64) the 512 latent channels as in the group
 *                                format with the 4 scales written into the row at bytes
 *                                512..527, the rope channels copied as bf16 to 528..655;
 *                                group_scales is not used.
 * Duplicate slots in one call are not allowed (which row lands is unspecified).
 *   kv_c [T][512] bf16 (row stride kv_c_stride), k_pe [T][d_rope] bf16 or NULL.
 */
int smla_cache_write(const void* kv_c, int64_t kv_c_stride, const void* k_pe, int64_t k_pe_stride,
                     const int64_t* slot_mapping, int32_t num_tokens, int32_t d_rope,
                     int32_t kv_format, float k_scale, void* kv_cache, int64_t num_slots,
                     int64_t kv_row_stride_bytes, float* group_scales, int64_t group_scales_stride,
                     void* stream);

/*
 * Profiling hook (not part of the computation). When set for the calling
 * thread, every following smla_decode_fwd / smla_prefill_fwd call records
 * the main attention kernel through hipExtLaunchKernel with `start` and
 * `end` (hipEvent_t, created with timing): the events take that kernel's own
 * start and end timestamps, so hipEventElapsedTime gives its duration (the
 * split combine, a separate kernel, is excluded). Pass
 * NULL, NULL to clear. The events are owned by the caller.
 */
int smla_set_timing_events(void* start, void* end);

/* sizeof(smla_attn_args) as this library was built (for bindings that lay
 * the struct out themselves). */
size_t smla_attn_args_size(void);

/* Thread-local description of the last non-OK return ("" if none). */
const char* smla_last_error(void);

/* Library version string. */
const char* smla_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SMLA_H_ */
