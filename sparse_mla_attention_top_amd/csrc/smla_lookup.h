// Slot lookup of the index conversion (vLLM "Sparse MLA on Hopper" branch,
// cutlass_fa3_sparse.py forward_mqa step 2; test_cutlass_fa3_sparse_backend.py
// TEST 2.5 / 2.9): request-local position l of request r is cache slot
//     block_table[r][l / block_size] * block_stride_rows + l % block_size,
// and -1 when l < 0, r is not a row of the table, l / block_size is at or past
// max_blocks, or the table entry is negative.
//
// Host and device code: every kernel that reads a block table (the standalone
// conversion, the attention kernel's fused conversion, the context-parallel
// filter, the FP8 prefill gather) goes through block_entry, and a host build
// with SMLA_BOUNDS_CHECK defined checks each table read against the length of
// the table array (the harness that defines it supplies that length and
// bounds_failure).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define SMLA_HD __host__ __device__
#else
#define SMLA_HD
#endif

namespace smla {

#ifdef SMLA_BOUNDS_CHECK
// Reports a table read outside [0, size) and ends the program.
[[noreturn]] void bounds_failure(const char* what, int64_t index, int64_t size);
#endif

struct BlockTable {
  const int32_t* table;        // row r at table + r * row_stride; max_blocks entries used per row
  int32_t num_reqs, max_blocks;
  int64_t row_stride;
  int32_t block_size;
  int32_t block_shift;         // log2(block_size) for a power of two, else -1
  int32_t block_stride_rows;   // rows between consecutive blocks (block_size for a plain paged cache)
#ifdef SMLA_BOUNDS_CHECK
  int64_t table_len;           // entries the table array really holds (set by the host harness)
#endif
};

// log2 of a power of two, else -1.
SMLA_HD inline int32_t block_shift_of(int32_t block_size) {
  if (block_size <= 0 || (block_size & (block_size - 1)) != 0) return -1;
  int32_t s = 0;
  while ((1 << s) != block_size) s++;
  return s;
}

// Entry of block `blk` of request `r`, or -1 when (r, blk) is outside the table.
SMLA_HD inline int32_t block_entry(const BlockTable& bt, int32_t r, int32_t blk) {
  if (r < 0 || r >= bt.num_reqs || blk < 0 || blk >= bt.max_blocks) return -1;
  const int64_t at = (int64_t)r * bt.row_stride + blk;
#ifdef SMLA_BOUNDS_CHECK
  if (at < 0 || at >= bt.table_len) bounds_failure("block table", at, bt.table_len);
#endif
  return bt.table[at];
}

// Cache slot of request-local position l of request r, or -1.
SMLA_HD inline int64_t local_slot(const BlockTable& bt, int32_t r, int32_t l) {
  if (l < 0) return -1;
  int32_t blk, off;
  if (bt.block_shift >= 0) {
    blk = l >> bt.block_shift;
    off = l & (bt.block_size - 1);
  } else {
    blk = l / bt.block_size;
    off = l - blk * bt.block_size;
  }
  const int32_t e = block_entry(bt, r, blk);
  return e < 0 ? -1 : (int64_t)e * bt.block_stride_rows + off;
}

}  // namespace smla
