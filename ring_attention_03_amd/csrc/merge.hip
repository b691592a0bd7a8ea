// Merge of two partial attention results over disjoint key sets, in place on
// the running state.  This is the step that lets Ring Attention's per-block
// partial results add up to full attention (Moreh, "Optimizing Long-Context
// Prefill on Multiple Older-Generation GPU Nodes", section "Introduction to
// Context Parallelism", Ring Attention bullet): softmax over a union of
// disjoint key sets is the log-sum-exp-weighted sum of the per-set results.
//
//   M = max(La, Lb), L = M + ln(e^(La-M) + e^(Lb-M)),
//   O = e^(La-L) * Oa + e^(Lb-L) * Ob,   (0, -inf) is the identity.
//
// HBM-bound: 16 lanes own one (row, head) pair (64 floats = 16 float4), so a
// wave moves four whole rows with fully coalesced 16-byte accesses, and the
// lane that writes the new LSE belongs to the same wave as the lanes that
// read the old one (no cross-wave race on the in-place update).
#include "kernels.h"
#include "merge_math.h"

namespace attnring {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int LANES_PER_ROW = kHeadDim / 4;
constexpr int THREADS = 256;
constexpr int ROWS_PER_BLOCK = THREADS / LANES_PER_ROW;

__global__ __launch_bounds__(THREADS) void merge_kernel(int32_t total_q, int32_t hq, f32x4* o_acc,
                                                        float* lse_acc, const f32x4* o_part,
                                                        const float* lse_part) {
  const int64_t rh = (int64_t)blockIdx.x * ROWS_PER_BLOCK + threadIdx.x / LANES_PER_ROW;
  const int sub = threadIdx.x % LANES_PER_ROW;
  if (rh >= (int64_t)total_q * hq) return;
  const int64_t q = rh / hq;
  const int h = (int)(rh - q * hq);
  const int64_t li = (int64_t)h * total_q + q;
  float lse, wa, wb;
  lse_merge_weights(lse_acc[li], lse_part[li], &lse, &wa, &wb);
  const int64_t oi = rh * LANES_PER_ROW + sub;
  const f32x4 a = o_acc[oi], b = o_part[oi];
  o_acc[oi] = wa * a + wb * b;
  if (sub == 0) lse_acc[li] = lse;
}

}  // namespace

hipError_t launch_merge(int32_t total_q, int32_t hq, float* o_acc, float* lse_acc,
                        const float* o_part, const float* lse_part, hipStream_t stream) {
  const int64_t rows = (int64_t)total_q * hq;
  const int64_t blocks = (rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(THREADS), 0, stream, total_q, hq,
                     reinterpret_cast<f32x4*>(o_acc), lse_acc,
                     reinterpret_cast<const f32x4*>(o_part), lse_part);
  return hipGetLastError();
}

}  // namespace attnring
