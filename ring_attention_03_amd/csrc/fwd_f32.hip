// fp32-input variant of the ring-step / prefill attention (same definition as
// the bf16 MFMA kernel: Ring Attention's per-device attention of a partial
// query against one key/value block, Moreh, "Optimizing Long-Context Prefill
// on Multiple Older-Generation GPU Nodes", section "Introduction to Context
// Parallelism").  It serves fp32 callers and small problems, so it favours
// plainness over speed: one thread per (query row, head), key/value tiles
// staged in LDS and read as broadcasts, an online softmax in base 2 with fp32
// throughout.
#include "kernels.h"
#include "merge_math.h"

namespace attnring {
namespace {

constexpr int D = kHeadDim;
constexpr int TK = 32;  // keys per LDS tile
constexpr int ROWS = kF32RowsPerTile;

__global__ __launch_bounds__(ROWS) void fwd_f32_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) float Ks[TK * D];
  __shared__ __attribute__((aligned(16))) float Vs[TK * D];

  const int lane = threadIdx.x;
  const int head = blockIdx.x % p.hq;
  const int unit = blockIdx.x / p.hq;
  int s = 0;
  while (unit >= p.unit_off[s + 1]) ++s;
  const int tile = (p.unit_off[s + 1] - 1) - unit;
  const int Lq = p.q_len[s], Lk = p.k_len[s];
  const int qp0 = p.q_pos0[s], kp0 = p.k_pos0[s];
  const int kvh = head / (p.hq / p.hkv);
  const int row = tile * ROWS + lane;
  const bool valid = row < Lq;
  const int qpos = qp0 + row;

  const int last_row = min((tile + 1) * ROWS, Lq) - 1;
  int kend = Lk;
  if (p.causal) kend = min(Lk, max(0, qp0 + last_row - kp0 + 1));

  const float* qg = reinterpret_cast<const float*>(p.q);
  const float* kg = reinterpret_cast<const float*>(p.k) + ((size_t)p.k_row0[s] * p.hkv + kvh) * D;
  const float* vg = reinterpret_cast<const float*>(p.v) + ((size_t)p.k_row0[s] * p.hkv + kvh) * D;
  const size_t kstride = (size_t)p.hkv * D;

  float qv[D];
  const float* qsrc = qg + ((size_t)(p.q_row0[s] + row) * p.hq + head) * D;
#pragma unroll
  for (int i = 0; i < D; ++i) qv[i] = valid ? qsrc[i] : 0.f;

  float acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) acc[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = p.scale_log2;

  for (int k0 = 0; k0 < kend; k0 += TK) {
    __syncthreads();
    // 64 threads load TK keys: each thread a half row (32 floats) of K and of V
    {
      const int kr = lane >> 1, part = (lane & 1) * (D / 2);
      const int key = k0 + kr;
#pragma unroll
      for (int i = 0; i < D / 2; i += 4) {
        float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
        if (key < Lk) {
          kk = *reinterpret_cast<const float4*>(kg + key * kstride + part + i);
          vv = *reinterpret_cast<const float4*>(vg + key * kstride + part + i);
        }
        *reinterpret_cast<float4*>(&Ks[kr * D + part + i]) = kk;
        *reinterpret_cast<float4*>(&Vs[kr * D + part + i]) = vv;
      }
    }
    __syncthreads();

    float sv[TK];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) dot = fmaf(qv[i], Ks[j * D + i], dot);
      const int key = k0 + j;
      const bool vis = key < Lk && (!p.causal || kp0 + key <= qpos);
      sv[j] = vis ? dot * c2 : -INFINITY;
      mx = fmaxf(mx, sv[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < D; ++i) acc[i] *= alpha;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      const float pj = exp2f(sv[j] - m_use);
      l_run += pj;
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] = fmaf(pj, Vs[j * D + i], acc[i]);
    }
  }

  if (valid) {
    // O = acc / l, LSE = (m + log2 l) * ln 2: written, or merged into the running
    // state (o, lse) by log-sum-exp (rows that saw no key here leave it as it is)
    const size_t grow = (size_t)(p.q_row0[s] + row);
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* dst = p.o + (grow * p.hq + head) * D;
    float* lse_dst = p.lse + (size_t)head * p.total_q + grow;
    const float lse_b = l_run > 0.f ? (m_run + log2f(l_run)) * 0.6931471805599453f : -INFINITY;
    if (!p.merge) {
#pragma unroll
      for (int i = 0; i < D; i += 4)
        *reinterpret_cast<float4*>(dst + i) =
            make_float4(acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv);
      *lse_dst = lse_b;
    } else if (l_run > 0.f) {
      float lse, wa, wb;
      lse_merge_weights(*lse_dst, lse_b, &lse, &wa, &wb);
#pragma unroll
      for (int i = 0; i < D; i += 4) {
        float4* o4 = reinterpret_cast<float4*>(dst + i);
        const float4 a = *o4;
        const float4 b = make_float4(acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv);
        *o4 = make_float4(wa * a.x + wb * b.x, wa * a.y + wb * b.y, wa * a.z + wb * b.z, wa * a.w + wb * b.w);
      }
      *lse_dst = lse;
    }
  }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, int n_units, hipStream_t stream) {
  hipLaunchKernelGGL(fwd_f32_kernel, dim3(n_units * p.hq), dim3(ROWS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attnring
