// Host stand-ins for the kernel launchers of the library (csrc/smla_internal.h),
// so that the C ABI layer (csrc/smla_api.cpp: argument checks, error
// reporting, split planning, dispatch) can be built and run on the CPU under
// the sanitizers. Each launcher records what it was given and launches
// nothing.
#include "../../sparse_mla_attention_top_amd/csrc/smla_internal.h"

namespace stub {
int launches = 0;
smla::ConvertArgs convert;
smla::DcpFilterArgs dcp;
smla::MergeArgs merge;
smla::CacheWriteArgs cache_write;
smla::PlannedCountsArgs planned;
smla::UpconvertArgs upconvert;
smla::AttnArgs attn;
int32_t attn_splits = 0;
void* attn_workspace = nullptr;
bool attn_longest_first = false;
char scratch_stand_in[64];
}  // namespace stub

namespace smla {
hipError_t launch_convert(const ConvertArgs& a, hipStream_t) { stub::convert = a; stub::launches++; return hipSuccess; }
hipError_t launch_dcp_filter(const DcpFilterArgs& a, hipStream_t) { stub::dcp = a; stub::launches++; return hipSuccess; }
hipError_t launch_merge(const MergeArgs& a, hipStream_t) { stub::merge = a; stub::launches++; return hipSuccess; }
hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t) {
  stub::cache_write = a;
  stub::launches++;
  return hipSuccess;
}
hipError_t launch_planned_counts(const PlannedCountsArgs& a, hipStream_t) {
  stub::planned = a;
  stub::launches++;
  return hipSuccess;
}
hipError_t launch_gather_upconvert(const UpconvertArgs& a, hipStream_t) {
  stub::upconvert = a;
  stub::launches++;
  return hipSuccess;
}
hipError_t launch_attention(const AttnArgs& a, int32_t splits, void* workspace, bool longest_first, hipStream_t) {
  stub::attn = a;
  stub::attn_splits = splits;
  stub::attn_workspace = workspace;
  stub::attn_longest_first = longest_first;
  stub::launches++;
  return hipSuccess;
}
hipError_t scratch_buffer(void** out) {
  *out = stub::scratch_stand_in;
  return hipSuccess;
}
}  // namespace smla

extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }
