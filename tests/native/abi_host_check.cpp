// The C ABI layer of the library (argument checks, error text, split planning,
// dispatch) driven on the CPU against stub launchers, built with the address
// and undefined-behaviour sanitizers by tests/test_host_sanitized.py. Checks
// the return code of every entry point on valid and invalid arguments, what a
// valid call hands to its launcher, and runs randomised argument structs
// through the attention entry points (any out-of-bounds access or undefined
// arithmetic in the checks aborts the run).
#include "../../include/smla.h"
#include "../../sparse_mla_attention_top_amd/csrc/smla_internal.h"

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>

namespace stub {
extern int launches;
extern smla::ConvertArgs convert;
extern smla::MergeArgs merge;
extern smla::CacheWriteArgs cache_write;
extern smla::AttnArgs attn;
extern int32_t attn_splits;
extern void* attn_workspace;
extern bool attn_longest_first;
extern char scratch_stand_in[64];
}  // namespace stub

static int failures = 0;

#define EXPECT(cond)                                                              \
  do {                                                                            \
    if (!(cond)) {                                                                \
      std::fprintf(stderr, "FAIL %s:%d: %s (last error: %s)\n", __FILE__, __LINE__, #cond, smla_last_error()); \
      failures++;                                                                 \
    }                                                                             \
  } while (0)

// fake device addresses: aligned, never dereferenced by the ABI layer
static void* P(uintptr_t v) { return reinterpret_cast<void*>(v); }
static const int32_t* I(uintptr_t v) { return reinterpret_cast<const int32_t*>(v); }

static smla_attn_args valid_args() {
  smla_attn_args a;
  std::memset(&a, 0, sizeof(a));
  a.q_nope = P(0x10000);
  a.q_nope_stride_tok = 128 * 576;
  a.q_nope_stride_head = 576;
  a.q_rope = P(0x10400);
  a.q_rope_stride_tok = 128 * 576;
  a.q_rope_stride_head = 576;
  a.num_tokens = 32;
  a.num_heads = 128;
  a.d_rope = 64;
  a.kv_cache = P(0x200000);
  a.num_slots = 4096 * 64;
  a.kv_row_stride_bytes = 1152;
  a.kv_format = SMLA_KV_BF16;
  a.k_scale = 1.0f;
  a.indices = I(0x300000);
  a.indices_stride = 2048;
  a.topk = 2048;
  a.softmax_scale = 0.0723f;
  a.out = P(0x400000);
  a.out_stride_tok = 128 * 512;
  a.out_stride_head = 512;
  a.lse = reinterpret_cast<float*>(0x500000);
  a.lse_stride_tok = 128;
  return a;
}

static void check_attention() {
  // a valid decode: the automatic plan, the workspace handed through
  smla_attn_args a = valid_args();
  const size_t ws = smla_decode_workspace_size(32, 128, 2048, 0);
  EXPECT(smla_decode_num_splits(32, 128, 2048, 0) == 4);
  EXPECT(ws == (size_t)4 * 32 * 128 * (1024 + 4));
  int before = stub::launches;
  EXPECT(smla_decode_fwd(&a, P(0x600000), ws, nullptr) == SMLA_OK);
  EXPECT(stub::launches == before + 1 && stub::attn_splits == 4 && stub::attn_workspace == P(0x600000));
  EXPECT(!stub::attn_longest_first && stub::attn.num_heads == 128 && stub::attn.d_rope == 64);
  EXPECT(std::strcmp(smla_last_error(), "") == 0);
  // too small, missing or misaligned workspace
  EXPECT(smla_decode_fwd(&a, P(0x600000), ws - 1, nullptr) == SMLA_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(std::strlen(smla_last_error()) > 0);
  EXPECT(smla_decode_fwd(&a, nullptr, ws, nullptr) == SMLA_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(smla_decode_fwd(&a, P(0x600008), ws, nullptr) == SMLA_ERR_INVALID_ARG);
  // prefill never splits and runs the longest rows first
  EXPECT(smla_prefill_fwd(&a, nullptr) == SMLA_OK && stub::attn_splits == 1 && stub::attn_longest_first);
  // the allocation-free decode: the static scratch, and plans beyond it refused
  EXPECT(smla_decode_fwd_noalloc(&a, nullptr) == SMLA_OK && stub::attn_workspace == stub::scratch_stand_in);
  smla_attn_args big = a;
  big.num_tokens = 256;
  big.num_splits = 64;
  before = stub::launches;
  EXPECT(smla_decode_fwd_noalloc(&big, nullptr) == SMLA_ERR_WORKSPACE_TOO_SMALL && stub::launches == before);
  // defaults filled in for the kernels
  a.kv_format = SMLA_KV_FP8_E4M3_GROUP128;
  a.kv_row_stride_bytes = 576;
  a.group_scales = reinterpret_cast<const float*>(0x700000);
  EXPECT(smla_prefill_fwd(&a, nullptr) == SMLA_OK && stub::attn.gs_stride == 5);
  a.group_scales_stride = 8;
  EXPECT(smla_prefill_fwd(&a, nullptr) == SMLA_OK && stub::attn.gs_stride == 8);
  a.group_scales_stride = 4;                       // below the 5 groups of a 576-channel row
  EXPECT(smla_prefill_fwd(&a, nullptr) == SMLA_ERR_INVALID_ARG);
  a.group_scales_stride = -1;
  EXPECT(smla_prefill_fwd(&a, nullptr) == SMLA_ERR_INVALID_ARG);
  a = valid_args();
  a.block_table = I(0x800000);
  a.req_id = I(0x900000);
  a.num_reqs = 32;
  a.max_blocks = 128;
  a.bt_row_stride = 128;
  a.block_size = 64;
  EXPECT(smla_decode_fwd(&a, P(0x600000), ws, nullptr) == SMLA_OK && stub::attn.block_stride_rows == 64);

  // invalid arguments, one at a time: nothing is launched
  struct Bad {
    const char* what;
    void (*edit)(smla_attn_args&);
    int code;
  };
  const Bad bad[] = {
      {"heads 0", [](smla_attn_args& x) { x.num_heads = 0; }, SMLA_ERR_UNSUPPORTED},
      {"heads 129", [](smla_attn_args& x) { x.num_heads = 129; }, SMLA_ERR_UNSUPPORTED},
      {"d_rope 32", [](smla_attn_args& x) { x.d_rope = 32; }, SMLA_ERR_UNSUPPORTED},
      {"topk 0", [](smla_attn_args& x) { x.topk = 0; }, SMLA_ERR_UNSUPPORTED},
      {"topk 4096", [](smla_attn_args& x) { x.topk = 4096; }, SMLA_ERR_UNSUPPORTED},
      {"tokens -1", [](smla_attn_args& x) { x.num_tokens = -1; }, SMLA_ERR_INVALID_ARG},
      {"format 9", [](smla_attn_args& x) { x.kv_format = 9; }, SMLA_ERR_INVALID_ARG},
      {"scale nan", [](smla_attn_args& x) { x.softmax_scale = __builtin_nanf(""); }, SMLA_ERR_INVALID_ARG},
      {"q null", [](smla_attn_args& x) { x.q_nope = nullptr; }, SMLA_ERR_INVALID_ARG},
      {"rope null", [](smla_attn_args& x) { x.q_rope = nullptr; }, SMLA_ERR_INVALID_ARG},
      {"slots 0", [](smla_attn_args& x) { x.num_slots = 0; }, SMLA_ERR_INVALID_ARG},
      {"slots 2^31", [](smla_attn_args& x) { x.num_slots = (int64_t)1 << 31; }, SMLA_ERR_INVALID_ARG},
      {"row stride short", [](smla_attn_args& x) { x.kv_row_stride_bytes = 1136; }, SMLA_ERR_INVALID_ARG},
      {"row stride odd", [](smla_attn_args& x) { x.kv_row_stride_bytes = 1160; }, SMLA_ERR_INVALID_ARG},
      {"row stride 2^32", [](smla_attn_args& x) { x.kv_row_stride_bytes = (int64_t)1 << 32; }, SMLA_ERR_UNSUPPORTED},
      {"cache misaligned", [](smla_attn_args& x) { x.kv_cache = P(0x200008); }, SMLA_ERR_INVALID_ARG},
      {"q stride", [](smla_attn_args& x) { x.q_nope_stride_head = 577; }, SMLA_ERR_INVALID_ARG},
      {"indices stride", [](smla_attn_args& x) { x.indices_stride = 2047; }, SMLA_ERR_INVALID_ARG},
      {"out stride", [](smla_attn_args& x) { x.out_stride_head = 256; }, SMLA_ERR_INVALID_ARG},
      {"out misaligned", [](smla_attn_args& x) { x.out = P(0x400002); }, SMLA_ERR_INVALID_ARG},
      {"lse stride", [](smla_attn_args& x) { x.lse_stride_tok = 64; }, SMLA_ERR_INVALID_ARG},
      {"table no req", [](smla_attn_args& x) { x.block_table = I(0x800000); x.num_reqs = 1; x.max_blocks = 1;
                                                x.bt_row_stride = 1; x.block_size = 64; }, SMLA_ERR_INVALID_ARG},
      {"table stride", [](smla_attn_args& x) { x.block_table = I(0x800000); x.req_id = I(0x900000); x.num_reqs = 1;
                                                x.max_blocks = 8; x.bt_row_stride = 7; x.block_size = 64; },
       SMLA_ERR_INVALID_ARG},
      {"block size 0", [](smla_attn_args& x) { x.block_table = I(0x800000); x.req_id = I(0x900000); x.num_reqs = 1;
                                                x.max_blocks = 8; x.bt_row_stride = 8; x.block_size = 0; },
       SMLA_ERR_INVALID_ARG},
      {"group no scales", [](smla_attn_args& x) { x.kv_format = SMLA_KV_FP8_E4M3_GROUP128; x.kv_row_stride_bytes = 576; },
       SMLA_ERR_INVALID_ARG},
      {"k_scale 0", [](smla_attn_args& x) { x.kv_format = SMLA_KV_FP8_E4M3_PER_TENSOR; x.kv_row_stride_bytes = 576;
                                             x.k_scale = 0.0f; }, SMLA_ERR_INVALID_ARG},
      {"packed no rope", [](smla_attn_args& x) { x.kv_format = SMLA_KV_FP8_DS_MLA; x.d_rope = 0; x.q_rope = nullptr; },
       SMLA_ERR_UNSUPPORTED},
      {"packed short row", [](smla_attn_args& x) { x.kv_format = SMLA_KV_FP8_DS_MLA; x.kv_row_stride_bytes = 640; },
       SMLA_ERR_INVALID_ARG},
      {"softcap -1", [](smla_attn_args& x) { x.softcap = -1.0f; }, SMLA_ERR_INVALID_ARG},
      {"sinks misaligned", [](smla_attn_args& x) { x.sinks = reinterpret_cast<const float*>(0x900002); },
       SMLA_ERR_INVALID_ARG},
      {"splits -1", [](smla_attn_args& x) { x.num_splits = -1; }, SMLA_ERR_INVALID_ARG},
  };
  for (const Bad& b : bad) {
    smla_attn_args x = valid_args();
    b.edit(x);
    before = stub::launches;
    const int rc = smla_decode_fwd(&x, P(0x600000), (size_t)1 << 40, nullptr);
    if (rc != b.code || stub::launches != before || std::strlen(smla_last_error()) == 0)
      std::fprintf(stderr, "FAIL bad argument '%s': rc %d (want %d), error '%s'\n", b.what, rc, b.code,
                   smla_last_error()), failures++;
  }
  EXPECT(smla_decode_fwd(nullptr, nullptr, 0, nullptr) == SMLA_ERR_INVALID_ARG);
  smla_attn_args empty = valid_args();
  empty.num_tokens = 0;
  before = stub::launches;
  EXPECT(smla_decode_fwd(&empty, nullptr, 0, nullptr) == SMLA_OK && smla_prefill_fwd(&empty, nullptr) == SMLA_OK);
  EXPECT(stub::launches == before);
}

static void check_other_entry_points() {
  int before = stub::launches;
  // index conversion: block_stride_rows 0 means the block size
  EXPECT(smla_convert_indices(I(0x1000), I(0x2000), 4, 8, 8, I(0x3000), 64, 3, 64, 16, 0, (int32_t*)0x4000, 64,
                              nullptr, nullptr) == SMLA_OK);
  EXPECT(stub::launches == before + 1 && stub::convert.block_stride_rows == 16 && stub::convert.topk == 64);
  EXPECT(smla_convert_indices(I(0x1000), I(0x2000), 4, 8, 8, I(0x3000), 64, 3, 64, 0, 0, (int32_t*)0x4000, 64,
                              nullptr, nullptr) == SMLA_ERR_INVALID_ARG);       // block size 0
  EXPECT(smla_convert_indices(I(0x1000), I(0x2000), 4, 8, 7, I(0x3000), 64, 3, 64, 16, 0, (int32_t*)0x4000, 64,
                              nullptr, nullptr) == SMLA_ERR_INVALID_ARG);       // row stride < max_blocks
  EXPECT(smla_convert_indices(nullptr, I(0x2000), 4, 8, 8, I(0x3000), 64, 3, 64, 16, 0, (int32_t*)0x4000, 64,
                              nullptr, nullptr) == SMLA_ERR_INVALID_ARG);
  EXPECT(smla_convert_indices(I(0x1000), I(0x2000), 4, 8, 8, I(0x3000), 63, 3, 64, 16, 0, (int32_t*)0x4000, 64,
                              nullptr, nullptr) == SMLA_ERR_INVALID_ARG);       // input stride < topk
  // context-parallel filter: rank outside the ranks, interleave 0
  EXPECT(smla_dcp_filter_convert(I(0x1000), I(0x2000), 4, 8, 8, I(0x3000), 64, 3, 64, 4, 4, 64, 16, 0, 1,
                                 (int32_t*)0x4000, 64, nullptr, nullptr) == SMLA_ERR_INVALID_ARG);
  EXPECT(smla_dcp_filter_convert(I(0x1000), I(0x2000), 4, 8, 8, I(0x3000), 64, 3, 64, 4, 1, 0, 16, 0, 1,
                                 (int32_t*)0x4000, 64, nullptr, nullptr) == SMLA_ERR_INVALID_ARG);
  EXPECT(smla_dcp_filter_convert(I(0x1000), I(0x2000), 4, 8, 8, I(0x3000), 64, 3, 64, 4, 1, 64, 16, 0, 1,
                                 (int32_t*)0x4000, 64, nullptr, nullptr) == SMLA_OK);
  // merge of partials
  EXPECT(smla_merge_partials(P(0x10000), 7 * 20 * 640, 20 * 640, 640, reinterpret_cast<const float*>(0x20000), 140,
                             20, 5, 7, 20, P(0x30000), 20 * 512, 512, reinterpret_cast<float*>(0x40000), 20,
                             nullptr) == SMLA_OK);
  EXPECT(stub::merge.parts == 5 && stub::merge.po_head == 640 && stub::merge.sinks == nullptr);
  EXPECT(smla_merge_partials(P(0x10000), 7 * 20 * 640, 20 * 640, 641, reinterpret_cast<const float*>(0x20000), 140,
                             20, 5, 7, 20, P(0x30000), 20 * 512, 512, nullptr, 0, nullptr) == SMLA_ERR_INVALID_ARG);
  EXPECT(smla_merge_partials(P(0x10000), 0, 0, 640, reinterpret_cast<const float*>(0x20000), 0, 20, 0, 7, 20,
                             P(0x30000), 20 * 512, 512, nullptr, 0, nullptr) == SMLA_ERR_INVALID_ARG);
  // planned counts and the FP8 prefill gather
  EXPECT(smla_planned_valid_counts(I(0x1000), I(0x2000), I(0x3000), 4, 100, 2048, 1, (int32_t*)0x4000, nullptr) ==
         SMLA_OK);
  EXPECT(smla_planned_valid_counts(I(0x1000), I(0x2000), I(0x3000), 4, 100, 2048, 0, (int32_t*)0x4000, nullptr) ==
         SMLA_ERR_INVALID_ARG);
  EXPECT(smla_gather_upconvert(P(0x10000), 4096, 656, SMLA_KV_FP8_DS_MLA, I(0x2000), 1, 64, 64, 64, 0, I(0x3000),
                               I(0x4000), 4096, P(0x50000), 4096, 576, nullptr) == SMLA_OK);
  EXPECT(smla_gather_upconvert(P(0x10000), 4096, 656, SMLA_KV_FP8_E4M3_GROUP128, I(0x2000), 1, 64, 64, 64, 0,
                               I(0x3000), I(0x4000), 4096, P(0x50000), 4096, 576, nullptr) == SMLA_ERR_UNSUPPORTED);
  EXPECT(smla_gather_upconvert(P(0x10000), 4096, 648, SMLA_KV_FP8_DS_MLA, I(0x2000), 1, 64, 64, 64, 0, I(0x3000),
                               I(0x4000), 4096, P(0x50000), 4096, 576, nullptr) == SMLA_ERR_INVALID_ARG);
  // cache write: group-scale stride default and bounds, formats
  const int64_t* slots = reinterpret_cast<const int64_t*>(0x6000);
  float* gs = reinterpret_cast<float*>(0x7000);
  EXPECT(smla_cache_write(P(0x1000), 512, P(0x2000), 64, slots, 10, 64, SMLA_KV_FP8_E4M3_GROUP128, 1.0f, P(0x3000),
                          100, 576, gs, 0, nullptr) == SMLA_OK);
  EXPECT(stub::cache_write.gs_stride == 5);
  EXPECT(smla_cache_write(P(0x1000), 512, nullptr, 0, slots, 10, 0, SMLA_KV_FP8_E4M3_GROUP128, 1.0f, P(0x3000), 100,
                          576, gs, 5, nullptr) == SMLA_OK);
  EXPECT(stub::cache_write.gs_stride == 5);
  EXPECT(smla_cache_write(P(0x1000), 512, P(0x2000), 64, slots, 10, 64, SMLA_KV_FP8_E4M3_GROUP128, 1.0f, P(0x3000),
                          100, 576, gs, 4, nullptr) == SMLA_ERR_INVALID_ARG);
  EXPECT(smla_cache_write(P(0x1000), 512, P(0x2000), 64, slots, 10, 64, SMLA_KV_FP8_E4M3_PER_TENSOR, 0.0f, P(0x3000),
                          100, 576, nullptr, 0, nullptr) == SMLA_ERR_INVALID_ARG);
  EXPECT(smla_cache_write(P(0x1000), 512, P(0x2000), 64, slots, 10, 64, SMLA_KV_FP8_DS_MLA, 1.0f, P(0x3000), 100,
                          648, nullptr, 0, nullptr) == SMLA_ERR_INVALID_ARG);  // below the 656-byte row
  EXPECT(smla_cache_write(P(0x1000), 512, P(0x2000), 64, slots, 10, 64, SMLA_KV_FP8_DS_MLA, 1.0f, P(0x3000), 100,
                          672, nullptr, 0, nullptr) == SMLA_OK);
  // timing hook: both events or neither
  EXPECT(smla_set_timing_events(P(0x10), nullptr) == SMLA_ERR_INVALID_ARG);
  EXPECT(smla_set_timing_events(nullptr, nullptr) == SMLA_OK);
  EXPECT(smla_attn_args_size() == sizeof(smla_attn_args) && std::strlen(smla_version()) > 0);
}

// Random argument structs (extreme and ordinary values mixed) through the
// attention entry points: the checks must neither read out of bounds nor
// overflow, and whatever they accept must be launchable as described.
static void fuzz_attention(int rounds) {
  std::mt19937_64 rng(12345);
  const int64_t edges64[] = {0, 1, -1, 7, 8, 15, 16, 64, 512, 576, 640, 1152, 2048, INT32_MAX, (int64_t)INT32_MAX + 1,
                             INT64_MAX, INT64_MIN, (int64_t)1 << 32};
  const int32_t edges32[] = {0, 1, -1, 2, 16, 63, 64, 65, 100, 128, 129, 512, 2048, 2049, INT32_MAX, INT32_MIN};
  auto pick64 = [&](int64_t ordinary) { return (rng() % 3) ? ordinary : edges64[rng() % (sizeof(edges64) / 8)]; };
  auto pick32 = [&](int32_t ordinary) { return (rng() % 3) ? ordinary : edges32[rng() % (sizeof(edges32) / 4)]; };
  auto addr = [&](uintptr_t base) -> uintptr_t {
    switch (rng() % 6) {
      case 0: return 0;
      case 1: return base + 2;
      default: return base;
    }
  };
  for (int k = 0; k < rounds; k++) {
    smla_attn_args a = valid_args();
    a.num_tokens = pick32(1 + (int32_t)(rng() % 300));
    a.num_heads = pick32(1 + (int32_t)(rng() % 128));
    a.d_rope = (rng() % 2) ? 64 : pick32(0);
    a.topk = pick32(1 + (int32_t)(rng() % 2048));
    a.indices_stride = pick64(a.topk);
    a.kv_format = (int32_t)(rng() % 5);
    a.num_slots = pick64(1 + (int64_t)(rng() % 100000));
    a.kv_row_stride_bytes = pick64(16 * (1 + (int64_t)(rng() % 80)));
    a.q_nope_stride_tok = pick64(a.q_nope_stride_tok);
    a.q_nope_stride_head = pick64(576);
    a.out_stride_head = pick64(512);
    a.out_stride_tok = pick64(a.out_stride_tok);
    a.lse_stride_tok = pick64(a.num_heads);
    a.q_nope = P(addr(0x10000));
    a.q_rope = P(addr(0x10400));
    a.kv_cache = P(addr(0x200000));
    a.out = P(addr(0x400000));
    a.indices = I(addr(0x300000));
    a.group_scales = reinterpret_cast<const float*>(addr(0x700000));
    a.group_scales_stride = pick64(0);
    a.k_scale = (rng() % 4) ? 0.02f : -1.0f;
    a.num_splits = pick32(0);
    a.softcap = (rng() % 4) ? 0.0f : 30.0f;
    if (rng() % 2) {
      a.block_table = I(addr(0x800000));
      a.req_id = I(addr(0x900000));
      a.num_reqs = pick32(4);
      a.max_blocks = pick32(128);
      a.bt_row_stride = pick64(128);
      a.block_size = pick32(64);
      a.block_stride_rows = pick32(0);
    }
    const int before = stub::launches;
    const size_t need = smla_decode_workspace_size(a.num_tokens, a.num_heads, a.topk, a.num_splits);
    const int rc = (k % 3 == 0)   ? smla_prefill_fwd(&a, nullptr)
                   : (k % 3 == 1) ? smla_decode_fwd(&a, P(0x10000000), need, nullptr)
                                  : smla_decode_fwd_noalloc(&a, nullptr);
    if (rc == SMLA_OK && a.num_tokens > 0) {
      // an accepted call launched once, with the shapes it was given
      EXPECT(stub::launches == before + 1);
      EXPECT(stub::attn.num_heads >= 1 && stub::attn.num_heads <= 128 && stub::attn.topk >= 1 &&
             stub::attn.topk <= 2048 && stub::attn_splits >= 1);
      EXPECT(stub::attn.kv_row_stride % 16 == 0 && stub::attn.num_slots >= 1 && stub::attn.num_slots <= INT32_MAX);
    } else {
      EXPECT(stub::launches == before);
    }
  }
}

int main() {
  check_attention();
  check_other_entry_points();
  fuzz_attention(200000);
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi host checks passed\n");
  return 0;
}
