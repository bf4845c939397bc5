// Host build of the slot lookup the kernels use (csrc/smla_lookup.h), with
// SMLA_BOUNDS_CHECK: every block-table read is checked against the length of
// the table array. Built with the address and undefined-behaviour sanitizers
// by tests/test_host_sanitized.py, which compares its output with the oracle.
//
//   lookup_check IN OUT [DECLARED_LEN]
// IN: int64 header {num_reqs, max_blocks, row_stride, block_size,
//     block_stride_rows, T, K, table_len}, then int32 table[table_len],
//     req_id[T], topk_local[T*K]. OUT: int64 slots[T*K] (-1 = invalid).
// DECLARED_LEN (optional) tells the bounds check that the table is shorter
// than it is, so that a read past it must be reported (a check of the check).
#include "smla_lookup.h"

#include <cstdio>
#include <cstdlib>
#include <vector>

namespace smla {
[[noreturn]] void bounds_failure(const char* what, int64_t index, int64_t size) {
  std::fprintf(stderr, "bounds: %s read at %lld outside [0, %lld)\n", what, (long long)index, (long long)size);
  std::abort();
}
}  // namespace smla

template <typename T>
static std::vector<T> read_n(FILE* f, int64_t n) {
  std::vector<T> v((size_t)n);
  if (n > 0 && std::fread(v.data(), sizeof(T), (size_t)n, f) != (size_t)n) {
    std::fprintf(stderr, "short input\n");
    std::exit(2);
  }
  return v;
}

int main(int argc, char** argv) {
  if (argc < 3) {
    std::fprintf(stderr, "usage: lookup_check IN OUT [DECLARED_LEN]\n");
    return 2;
  }
  FILE* in = std::fopen(argv[1], "rb");
  if (!in) return 2;
  const std::vector<int64_t> h = read_n<int64_t>(in, 8);
  const int64_t R = h[0], MB = h[1], stride = h[2], B = h[3], BS = h[4], T = h[5], K = h[6], len = h[7];
  // exact-length heap copies, so that the sanitizer sees any read past them
  const std::vector<int32_t> table = read_n<int32_t>(in, len);
  const std::vector<int32_t> req = read_n<int32_t>(in, T);
  const std::vector<int32_t> loc = read_n<int32_t>(in, T * K);
  std::fclose(in);
  smla::BlockTable bt{table.data(), (int32_t)R, (int32_t)MB, stride, (int32_t)B,
                      smla::block_shift_of((int32_t)B), (int32_t)BS, argc > 3 ? std::atoll(argv[3]) : len};
  std::vector<int64_t> out((size_t)(T * K));
  for (int64_t t = 0; t < T; t++)
    for (int64_t j = 0; j < K; j++) out[(size_t)(t * K + j)] = smla::local_slot(bt, req[(size_t)t], loc[(size_t)(t * K + j)]);
  FILE* o = std::fopen(argv[2], "wb");
  if (!o) return 2;
  std::fwrite(out.data(), sizeof(int64_t), out.size(), o);
  std::fclose(o);
  return 0;
}
