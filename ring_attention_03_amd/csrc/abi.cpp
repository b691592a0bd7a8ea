// C ABI of the ring-attention library: host-side validation, work planning and
// launches.  Every check runs before anything touches HIP, so an invalid call
// enqueues nothing (and the checks can run on a host without a GPU).
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <numeric>

#include "attnring.h"
#include "kernels.h"

using namespace attnring;

namespace {

thread_local char g_err[512] = "";

attn_status fail(attn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

attn_status ok() {
  g_err[0] = '\0';
  return ATTN_OK;
}

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

attn_status check_offsets(const int32_t* cu, int32_t nseq, int32_t total, const char* name,
                          int32_t* out) {
  if (!cu) {
    if (nseq != 1) return fail(ATTN_EINVAL, "%s is NULL but num_seqs=%d (NULL needs num_seqs=1)", name, nseq);
    out[0] = 0;
    out[1] = total;
    return ATTN_OK;
  }
  if (cu[0] != 0) return fail(ATTN_EINVAL, "%s[0]=%d, must be 0", name, cu[0]);
  for (int b = 0; b < nseq; ++b)
    if (cu[b + 1] < cu[b]) return fail(ATTN_EINVAL, "%s is not non-decreasing at %d", name, b);
  if (cu[nseq] != total)
    return fail(ATTN_EINVAL, "%s[num_seqs]=%d but the total row count is %d", name, cu[nseq], total);
  std::copy(cu, cu + nseq + 1, out);
  return ATTN_OK;
}

attn_status check_positions(const int32_t* pos, int32_t nseq, const int32_t* len, const char* name,
                            int32_t* out) {
  for (int b = 0; b < nseq; ++b) {
    const int64_t p0 = pos ? pos[b] : 0;
    if (p0 < 0) return fail(ATTN_EINVAL, "%s[%d]=%lld is negative", name, b, (long long)p0);
    if (p0 + len[b] > INT32_MAX)
      return fail(ATTN_EINVAL, "%s[%d] + length overflows int32", name, b);
    out[b] = (int32_t)p0;
  }
  return ATTN_OK;
}

struct Plan {
  FwdParams p;
  int n_units;
  bool any_visible;
};

// Validate a forward problem and fill the kernel parameters.
attn_status plan_forward(const attn_problem* pr, attn_dtype dt, const void* q, const void* k,
                         const void* v, float* o, float* lse, Plan* plan) {
  if (!pr) return fail(ATTN_EINVAL, "problem is NULL");
  if (dt != ATTN_DTYPE_BF16 && dt != ATTN_DTYPE_FP32)
    return fail(ATTN_EINVAL, "unknown dtype %d", (int)dt);
  const int32_t nseq = pr->num_seqs;
  if (nseq < 1 || nseq > ATTN_MAX_SEQS)
    return fail(ATTN_EINVAL, "num_seqs=%d outside [1, %d]", nseq, ATTN_MAX_SEQS);
  if (pr->total_q < 0 || pr->total_k < 0)
    return fail(ATTN_EINVAL, "negative total_q=%d or total_k=%d", pr->total_q, pr->total_k);
  if (pr->num_q_heads < 1 || pr->num_kv_heads < 1)
    return fail(ATTN_EINVAL, "head counts must be >= 1 (Hq=%d, Hkv=%d)", pr->num_q_heads,
                pr->num_kv_heads);
  if (pr->num_q_heads % pr->num_kv_heads != 0)
    return fail(ATTN_EINVAL, "Hq=%d is not a multiple of Hkv=%d", pr->num_q_heads, pr->num_kv_heads);
  if (pr->head_dim < 1) return fail(ATTN_EINVAL, "head_dim=%d", pr->head_dim);
  if (pr->head_dim != kHeadDim)
    return fail(ATTN_EUNSUPPORTED, "head_dim=%d is not supported (only %d)", pr->head_dim, kHeadDim);
  if (!std::isfinite(pr->scale) || pr->scale < 0.f)
    return fail(ATTN_EINVAL, "scale=%g must be finite and >= 0 (0 selects 1/sqrt(d))", (double)pr->scale);
  if (pr->causal != 0 && pr->causal != 1) return fail(ATTN_EINVAL, "causal=%d must be 0 or 1", pr->causal);

  int32_t cq[ATTN_MAX_SEQS + 1], ql[ATTN_MAX_SEQS], kr0[ATTN_MAX_SEQS], kl[ATTN_MAX_SEQS];
  int32_t qp[ATTN_MAX_SEQS], kp[ATTN_MAX_SEQS];
  attn_status st;
  if ((st = check_offsets(pr->cu_q, nseq, pr->total_q, "cu_q", cq)) != ATTN_OK) return st;
  for (int b = 0; b < nseq; ++b) ql[b] = cq[b + 1] - cq[b];
  if (pr->k_row0 || pr->k_len) {  // explicit key ranges: any order, may overlap
    if (!pr->k_row0 || !pr->k_len) return fail(ATTN_EINVAL, "k_row0 and k_len must be given together");
    if (pr->cu_k) return fail(ATTN_EINVAL, "give either cu_k or k_row0/k_len, not both");
    for (int b = 0; b < nseq; ++b) {
      if (pr->k_row0[b] < 0 || pr->k_len[b] < 0)
        return fail(ATTN_EINVAL, "k_row0[%d]=%d / k_len[%d]=%d must be >= 0", b, pr->k_row0[b], b,
                    pr->k_len[b]);
      if ((int64_t)pr->k_row0[b] + pr->k_len[b] > pr->total_k)
        return fail(ATTN_EINVAL, "keys of sequence %d end at row %lld, past total_k=%d", b,
                    (long long)pr->k_row0[b] + pr->k_len[b], pr->total_k);
      kr0[b] = pr->k_row0[b];
      kl[b] = pr->k_len[b];
    }
  } else {
    int32_t ck[ATTN_MAX_SEQS + 1];
    if ((st = check_offsets(pr->cu_k, nseq, pr->total_k, "cu_k", ck)) != ATTN_OK) return st;
    for (int b = 0; b < nseq; ++b) {
      kr0[b] = ck[b];
      kl[b] = ck[b + 1] - ck[b];
    }
  }
  if ((st = check_positions(pr->q_pos0, nseq, ql, "q_pos0", qp)) != ATTN_OK) return st;
  if ((st = check_positions(pr->k_pos0, nseq, kl, "k_pos0", kp)) != ATTN_OK) return st;

  const size_t esz = dt == ATTN_DTYPE_BF16 ? 2 : 4;
  const int64_t d = pr->head_dim;
  // the bf16 kernel addresses one sequence's keys and values with 32-bit byte offsets
  for (int b = 0; b < nseq && dt == ATTN_DTYPE_BF16; ++b)
    if ((int64_t)kl[b] * pr->num_kv_heads * d * 2 >= (int64_t(1) << 31))
      return fail(ATTN_EUNSUPPORTED, "sequence %d: keys and values span 2 GiB or more per tensor", b);
  const size_t q_bytes = (size_t)pr->total_q * pr->num_q_heads * d * esz;
  const size_t kv_bytes = (size_t)pr->total_k * pr->num_kv_heads * d * esz;
  const size_t o_bytes = (size_t)pr->total_q * pr->num_q_heads * d * 4;
  const size_t lse_bytes = (size_t)pr->total_q * pr->num_q_heads * 4;
  if (pr->total_q > 0 && (!q || !o || !lse)) return fail(ATTN_EINVAL, "q, o or lse is NULL");
  if (pr->total_k > 0 && (!k || !v)) return fail(ATTN_EINVAL, "k or v is NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(ATTN_EINVAL, "q, k, v and o must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(ATTN_EINVAL, "lse must be 4-byte aligned");
  if (overlap(o, o_bytes, q, q_bytes) || overlap(o, o_bytes, k, kv_bytes) ||
      overlap(o, o_bytes, v, kv_bytes) || overlap(o, o_bytes, lse, lse_bytes) ||
      overlap(lse, lse_bytes, q, q_bytes) || overlap(lse, lse_bytes, k, kv_bytes) ||
      overlap(lse, lse_bytes, v, kv_bytes))
    return fail(ATTN_EINVAL, "outputs overlap the inputs or each other");

  FwdParams& p = plan->p;
  p = FwdParams{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.total_q = pr->total_q;
  p.hq = pr->num_q_heads;
  p.hkv = pr->num_kv_heads;
  p.causal = pr->causal;
  const float scale = pr->scale == 0.f ? 1.f / std::sqrt((float)d) : pr->scale;
  p.scale_log2 = scale * 1.4426950408889634f;

  int rows_per_tile;
  if (dt == ATTN_DTYPE_BF16) {
    const Bf16Geometry geo = bf16_geometry(p.hq, p.hkv);
    rows_per_tile = geo.rows_per_tile();
    p.n_head_groups = p.hq / geo.heads_per_group;
  } else {
    rows_per_tile = kF32RowsPerTile;
    p.n_head_groups = p.hq;
  }
  p.rows_per_tile = rows_per_tile;

  // Visible-key work of each sequence decides the processing order (heaviest first),
  // so the longest workgroups start first and the tail of the launch is short.
  bool any_visible = false;
  int order[ATTN_MAX_SEQS];
  double work[ATTN_MAX_SEQS];
  for (int b = 0; b < nseq; ++b) {
    const int64_t lq = ql[b], lk = kl[b];
    int64_t kend = lk;
    if (pr->causal) kend = std::min<int64_t>(lk, std::max<int64_t>(0, (int64_t)qp[b] + lq - 1 - kp[b] + 1));
    if (lq > 0 && kend > 0) any_visible = true;
    work[b] = (double)lq * (double)kend;
    order[b] = b;
  }
  std::stable_sort(order, order + nseq, [&](int a, int b) { return work[a] > work[b]; });
  int units = 0;
  p.nseq = nseq;
  for (int i = 0; i < nseq; ++i) {
    const int b = order[i];
    p.q_row0[i] = cq[b];
    p.q_len[i] = cq[b + 1] - cq[b];
    p.k_row0[i] = kr0[b];
    p.k_len[i] = kl[b];
    p.q_pos0[i] = qp[b];
    p.k_pos0[i] = kp[b];
    p.unit_off[i] = units;
    units += (p.q_len[i] + rows_per_tile - 1) / rows_per_tile;
  }
  p.unit_off[nseq] = units;
  if ((int64_t)units * p.n_head_groups > INT32_MAX) return fail(ATTN_EUNSUPPORTED, "problem too large");
  plan->n_units = units;
  plan->any_visible = any_visible;
  return ATTN_OK;
}

attn_status launch_forward(const Plan& plan, attn_dtype dt, hipStream_t stream) {
  if (plan.n_units == 0) return ok();
  hipError_t e;
  if (dt == ATTN_DTYPE_BF16) {
    e = launch_fwd_bf16(plan.p, bf16_geometry(plan.p.hq, plan.p.hkv), plan.n_units, stream);
  } else {
    e = launch_fwd_f32(plan.p, plan.n_units, stream);
  }
  if (e != hipSuccess) return fail(ATTN_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int32_t attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_last_error(void) { return g_err; }

attn_status attn_ring_step(const attn_problem* problem, attn_dtype dtype, const void* q,
                           const void* k, const void* v, float* o_part, float* lse_part,
                           int32_t* launched, hipStream_t stream) {
  if (launched) *launched = 0;
  Plan plan;
  attn_status st = plan_forward(problem, dtype, q, k, v, o_part, lse_part, &plan);
  if (st != ATTN_OK) return st;
  if (plan.n_units == 0) return ok();               // no local rows: nothing to write
  if (!plan.any_visible && launched) return ok();   // fully masked: caller skips the merge
  st = launch_forward(plan, dtype, stream);         // (without `launched`, writes the identity)
  if (st == ATTN_OK && launched) *launched = 1;
  return st;
}

attn_status attn_ring_step_merge(const attn_problem* problem, attn_dtype dtype, const void* q,
                                 const void* k, const void* v, float* o_acc, float* lse_acc,
                                 int32_t* launched, hipStream_t stream) {
  if (launched) *launched = 0;
  Plan plan;
  attn_status st = plan_forward(problem, dtype, q, k, v, o_acc, lse_acc, &plan);
  if (st != ATTN_OK) return st;
  if (plan.n_units == 0 || !plan.any_visible) return ok();  // merging the identity: nothing to do
  plan.p.merge = 1;
  st = launch_forward(plan, dtype, stream);
  if (st == ATTN_OK && launched) *launched = 1;
  return st;
}

attn_status attn_prefill_causal(const attn_problem* problem, attn_dtype dtype, const void* q,
                                const void* k, const void* v, float* o, float* lse,
                                hipStream_t stream) {
  if (!problem) return fail(ATTN_EINVAL, "problem is NULL");
  if (problem->causal != 1) return fail(ATTN_EINVAL, "prefill is causal: causal must be 1");
  if (problem->total_k != problem->total_q)
    return fail(ATTN_EINVAL, "prefill needs total_k == total_q (%d vs %d)", problem->total_k,
                problem->total_q);
  if ((problem->cu_q == nullptr) != (problem->cu_k == nullptr))
    return fail(ATTN_EINVAL, "prefill needs cu_k equal to cu_q");
  if ((problem->q_pos0 == nullptr) != (problem->k_pos0 == nullptr))
    return fail(ATTN_EINVAL, "prefill needs k_pos0 equal to q_pos0");
  if (problem->k_row0 || problem->k_len)
    return fail(ATTN_EINVAL, "prefill takes its keys from cu_k (k_row0/k_len must be NULL)");
  const int32_t nseq = problem->num_seqs;
  if (nseq >= 1 && nseq <= ATTN_MAX_SEQS) {
    if (problem->cu_q)
      for (int b = 0; b <= nseq; ++b)
        if (problem->cu_q[b] != problem->cu_k[b]) return fail(ATTN_EINVAL, "prefill needs cu_k equal to cu_q");
    if (problem->q_pos0)
      for (int b = 0; b < nseq; ++b)
        if (problem->q_pos0[b] != problem->k_pos0[b])
          return fail(ATTN_EINVAL, "prefill needs k_pos0 equal to q_pos0");
  }
  Plan plan;
  attn_status st = plan_forward(problem, dtype, q, k, v, o, lse, &plan);
  if (st != ATTN_OK) return st;
  return launch_forward(plan, dtype, stream);
}

attn_status attn_ring_merge(int32_t total_q, int32_t num_q_heads, int32_t head_dim, float* o_acc,
                            float* lse_acc, const float* o_part, const float* lse_part,
                            hipStream_t stream) {
  if (total_q < 0) return fail(ATTN_EINVAL, "total_q=%d is negative", total_q);
  if (num_q_heads < 1) return fail(ATTN_EINVAL, "num_q_heads=%d", num_q_heads);
  if (head_dim < 1) return fail(ATTN_EINVAL, "head_dim=%d", head_dim);
  if (head_dim != kHeadDim)
    return fail(ATTN_EUNSUPPORTED, "head_dim=%d is not supported (only %d)", head_dim, kHeadDim);
  if (total_q == 0) return ok();
  if (!o_acc || !lse_acc || !o_part || !lse_part) return fail(ATTN_EINVAL, "NULL buffer");
  if (!aligned(o_acc, 16) || !aligned(o_part, 16)) return fail(ATTN_EINVAL, "o buffers must be 16-byte aligned");
  if (!aligned(lse_acc, 4) || !aligned(lse_part, 4)) return fail(ATTN_EINVAL, "lse buffers must be 4-byte aligned");
  const size_t o_bytes = (size_t)total_q * num_q_heads * head_dim * 4;
  const size_t l_bytes = (size_t)total_q * num_q_heads * 4;
  if (overlap(o_acc, o_bytes, o_part, o_bytes) || overlap(lse_acc, l_bytes, lse_part, l_bytes) ||
      overlap(o_acc, o_bytes, lse_acc, l_bytes) || overlap(o_acc, o_bytes, lse_part, l_bytes) ||
      overlap(lse_acc, l_bytes, o_part, o_bytes))
    return fail(ATTN_EINVAL, "merge buffers overlap");
  const hipError_t e = launch_merge(total_q, num_q_heads, o_acc, lse_acc, o_part, lse_part, stream);
  if (e != hipSuccess) return fail(ATTN_EHIP, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
