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
  // Branch-free, on the hardware base-2 exponential, logarithm and reciprocal
  // (about 1 ulp each): one of the two exponentials is exactly 1, so s is in
  // [1, 2] unless both sets are empty (then any finite shift gives s = 0).
  constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
  const float mx = fmaxf(la, lb);
  const float m0 = mx == -INFINITY ? 0.f : mx;
  const float ea = __builtin_amdgcn_exp2f((la - m0) * kLog2e);
  const float eb = __builtin_amdgcn_exp2f((lb - m0) * kLog2e);
  const float s = ea + eb;
  const float r = s > 0.f ? __builtin_amdgcn_rcpf(s) : 0.f;
  *lse = s > 0.f ? m0 + __builtin_amdgcn_logf(s) * kLn2 : -INFINITY;
  *wa = ea * r;
  *wb = eb * r;
}

}  // namespace attnring
