// Test-only stand-ins for the kernel launches, so the C ABI's host code
// (validation, planning, skip decisions) can be built for the CPU alone -
// with AddressSanitizer - and driven without a GPU.  Every launch is recorded
// instead of enqueued; nothing here touches a device.
#include <cstring>

#include "kernels.h"

namespace {
int g_launches = 0;
attnring::FwdParams g_last{};
int g_last_units = 0;
}  // namespace

namespace attnring {

hipError_t launch_fwd_bf16(const FwdParams& p, const Bf16Geometry&, int n_units, hipStream_t) {
  ++g_launches;
  g_last = p;
  g_last_units = n_units;
  return hipSuccess;
}

hipError_t launch_fwd_f32(const FwdParams& p, int n_units, hipStream_t) {
  ++g_launches;
  g_last = p;
  g_last_units = n_units;
  return hipSuccess;
}

hipError_t launch_merge(int32_t, int32_t, float*, float*, const float*, const float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}

}  // namespace attnring

// Number of launches recorded so far.
extern "C" int attn_test_launches(void) { return g_launches; }

// Work units and merge flag of the last recorded forward launch; `unit_off`
// receives its per-sequence prefix unit counts (nseq + 1 entries, at most 65).
extern "C" int attn_test_last_forward(int* n_units, int* merge, int* nseq, int* unit_off) {
  *n_units = g_last_units;
  *merge = g_last.merge;
  *nseq = g_last.nseq;
  std::memcpy(unit_off, g_last.unit_off, sizeof(int) * (g_last.nseq + 1));
  return g_launches;
}
