// Log-sum-exp merge weights shared by the merge kernel and the attention
// kernels' merging epilogue (device code only).
//
// Softmax over the union of two disjoint key sets with log-sum-exps La, Lb
// (natural log) and normalised outputs Oa, Ob is
//   L = M + ln(e^(La-M) + e^(Lb-M)),  M = max(La, Lb),
//   O = e^(La-L) Oa + e^(Lb-L) Ob,
// and (O = 0, L = -inf) is the identity (Moreh, "Optimizing Long-Context
// Prefill on Multiple Older-Generation GPU Nodes", section "Introduction to
// Context Parallelism", Ring Attention bullet: per-block partial results that
// add up to full attention).
#pragma once

#include <hip/hip_runtime.h>

namespace attnring {

__device__ __forceinline__ void lse_merge_weights(float la, float lb, float* lse, float* wa, float* wb) {
  const float mx = fmaxf(la, lb);
  if (mx == -INFINITY) {  // both empty: the identity
    *lse = -INFINITY;
    *wa = 0.f;
    *wb = 0.f;
    return;
  }
  *lse = mx + logf(expf(la - mx) + expf(lb - mx));
  *wa = expf(la - *lse);
  *wb = expf(lb - *lse);
}

}  // namespace attnring
