// Blockwise causal GQA attention of a query block against one key/value block,
// bf16 inputs, MFMA on gfx950, fp32 accumulation, partial (O, LSE) output.
//
// This is the per-device computation of Ring Attention: attention with the
// device's partial query against one partial key/value block (Moreh,
// "Optimizing Long-Context Prefill on Multiple Older-Generation GPU Nodes",
// section "Introduction to Context Parallelism", Ring Attention bullet), with
// an online softmax so the block's result can later be merged by its
// log-sum-exp.  The same kernel run over a whole sequence is full causal
// prefill.
//
// Work decomposition.  A workgroup owns (sequence, row tile, group of query
// heads that share one key/value head).  Each wave owns 64 query rows of one
// head and keeps them in registers; the key/value tile (64 keys) is staged in
// LDS once per workgroup and read by every wave, so a tile is reused by all
// query heads of its GQA group.
//
// Register layouts (v_mfma_f32_32x32x16_bf16: A is 32x16, B is 16x32, lane l
// supplies row/col l%32 and k-slots 8*(l/32)..+7; D lane l holds column l%32,
// rows 8*(e/4) + 4*(l/32) + e%4 for e = 0..15):
//  * scores are computed transposed, S^T = K Q^T (A = K from LDS, B = Q from
//    registers), so a lane holds 16 keys of ONE query: the row max and row sum
//    are lane-local plus one exchange with lane l^32;
//  * the output is computed transposed, O^T = V^T P^T.  The B operand is P^T
//    straight from the score accumulator, which holds keys in the order
//    8*(e/4) + 4*(l/32) + e%4; V^T is stored in LDS with its keys permuted the
//    same way so that each lane's A operand is one 16-byte LDS read.
#include "kernels.h"

namespace attnring {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int D = kHeadDim;  // 64
constexpr int BK = 64;       // keys per LDS tile
constexpr int QB = 2;        // 32-row query blocks per wave (64 rows)
constexpr int KSTR = D + 8;  // K row stride in LDS (bf16 elements): 144 B, conflict-free 16-B reads
constexpr int VSTR = BK + 8; // V^T row stride in LDS

// Position inside a 16-key group where key j is stored in the V^T tile: the
// inverse of the accumulator's key order (see the file comment).
__device__ __forceinline__ int vt_pos(int key) {
  const int j = key & 15;
  return (key & ~15) + ((j >> 2) & 1) * 8 + ((j >> 3) & 1) * 4 + (j & 3);
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

template <int NW, int HPW>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][BK * KSTR];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[2][D * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // ---- which (sequence, row tile, head group) this workgroup owns
  const int hg = blockIdx.x % p.n_head_groups;
  const int unit = blockIdx.x / p.n_head_groups;
  int s = 0;
  while (unit >= p.unit_off[s + 1]) ++s;
  const int tile = (p.unit_off[s + 1] - 1) - unit;  // heaviest (last) row tile first
  const int rows_per_tile = QB * 32 * (NW / HPW);
  const int r0 = tile * rows_per_tile;
  const int Lq = p.q_len[s], Lk = p.k_len[s];
  const int qp0 = p.q_pos0[s], kp0 = p.k_pos0[s];
  const int group = p.hq / p.hkv;
  const int head = hg * HPW + (wave % HPW);
  const int kvh = (hg * HPW) / group;
  const int rw0 = r0 + (wave / HPW) * (QB * 32);  // this wave's first row (within the sequence)

  // keys [0, kend) can be visible to some row of the tile; keys [0, kfull) to all of them
  const int last_row = min(r0 + rows_per_tile, Lq) - 1;
  int kend = Lk, kfull = Lk;
  if (p.causal) {
    kend = min(Lk, max(0, qp0 + last_row - kp0 + 1));
    kfull = min(Lk, max(0, qp0 + r0 - kp0 + 1));
  }
  const int ntiles = (kend + BK - 1) / BK;

  const __bf16* qg = reinterpret_cast<const __bf16*>(p.q);
  const __bf16* kg = reinterpret_cast<const __bf16*>(p.k) +
                     ((size_t)p.k_row0[s] * p.hkv + kvh) * D;
  const __bf16* vg = reinterpret_cast<const __bf16*>(p.v) +
                     ((size_t)p.k_row0[s] * p.hkv + kvh) * D;
  const size_t kstride = (size_t)p.hkv * D;

  // ---- this wave's queries as MFMA B operands: Qr[qb][ks] = q[row][ks*16 + 8*half .. +7]
  bf16x8 Qr[QB][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = rw0 + qb * 32 + l32;
    const __bf16* src = qg + ((size_t)(p.q_row0[s] + row) * p.hq + head) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (row < Lq) {
        Qr[qb][ks] = *reinterpret_cast<const bf16x8*>(src + ks * 16);
      } else {
        Qr[qb][ks] = bf16x8{};
      }
    }
  }

  // ---- cooperative tile loads: BK keys x 8 chunks of 8 bf16, for K and for V
  constexpr int CHUNKS = BK * (D / 8);
  constexpr int PER_THREAD = (CHUNKS + NW * 64 - 1) / (NW * 64);
  u16x8 kreg[PER_THREAD], vreg[PER_THREAD];

  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int c = tid + i * NW * 64;
      const int kr = c >> 3, ch = c & 7;
      const int key = t * BK + kr;
      if (c < CHUNKS && key < Lk) {
        kreg[i] = *reinterpret_cast<const u16x8*>(kg + key * kstride + ch * 8);
        vreg[i] = *reinterpret_cast<const u16x8*>(vg + key * kstride + ch * 8);
      } else {
        kreg[i] = u16x8{};
        vreg[i] = u16x8{};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int c = tid + i * NW * 64;
      if (c < CHUNKS) {
        const int kr = c >> 3, ch = c & 7;
        *reinterpret_cast<u16x8*>(reinterpret_cast<unsigned short*>(&Ks[buf][kr * KSTR + ch * 8])) =
            kreg[i];
        unsigned short* vt = reinterpret_cast<unsigned short*>(&Vt[buf][0]);
        const int pos = vt_pos(kr);
#pragma unroll
        for (int j = 0; j < 8; ++j) vt[(ch * 8 + j) * VSTR + pos] = vreg[i][j];
      }
    }
  };

  // ---- running state: O^T accumulators, row max (log2 units) and lane-partial row sums
  f32x16 acc[2][QB];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) acc[db][qb] = f32x16{};
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }
  const float c2 = p.scale_log2;

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);

    // S^T = K Q^T for 64 keys x 64 queries: sc[kb][qb] holds keys kb*32.., queries qb*32..
    f32x16 sc[2][QB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[kb][qb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(&Ks[buf][(kb * 32 + l32) * KSTR + ks * 16 + half * 8]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, Qr[qb][ks], sc[kb][qb], 0, 0, 0);
      }
    }

    // mask: only tiles that reach past the keys every row can see.  Key
    // kb*32 + 8*(e/4) + 4*half + e%4 of the tile is visible to this lane's
    // query iff it is <= lim; written as selects (no divergent branches).
    const int k0 = t * BK;
    if (k0 + BK > kfull) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qpos = qp0 + rw0 + qb * 32 + l32;
        int last = Lk - 1;                                 // last key index of the sequence
        if (p.causal) last = min(last, qpos - kp0);        // ... and not in the query's future
        const int lim = last - k0 - half * 4;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int off = kb * 32 + (e >> 2) * 8 + (e & 3);
            sc[kb][qb][e] = off <= lim ? sc[kb][qb][e] : -INFINITY;
          }
      }
    }

    // online softmax in base 2
    bf16x8 pb[2][QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[kb][qb][e]);
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run[qb], mx * c2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_use);
      m_run[qb] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(sc[kb][qb][hh * 8 + j], c2, -m_use));
            rs += pv;
            pb[kb][qb][hh][j] = (__bf16)pv;
          }
      l_run[qb] = l_run[qb] * alpha + rs;
#pragma unroll
      for (int db = 0; db < 2; ++db) acc[db][qb] *= alpha;
    }

    // O^T += V^T P^T over 4 steps of 16 keys
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kb = st >> 1, hh = st & 1;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(&Vt[buf][(db * 32 + l32) * VSTR + st * 16 + half * 8]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][qb][hh], acc[db][qb], 0, 0, 0);
      }
    }

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2
  float* og = p.o;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + xor32(l_run[qb]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int row = rw0 + qb * 32 + l32;
    if (row < Lq) {
      const size_t grow = (size_t)(p.q_row0[s] + row);
      float* dst = og + (grow * p.hq + head) * D + half * 4;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 v4;
          v4[0] = acc[db][qb][i * 4 + 0] * inv;
          v4[1] = acc[db][qb][i * 4 + 1] * inv;
          v4[2] = acc[db][qb][i * 4 + 2] * inv;
          v4[3] = acc[db][qb][i * 4 + 3] * inv;
          *reinterpret_cast<f32x4*>(dst + db * 32 + i * 8) = v4;
        }
      if (half == 0) {
        const float lse = l_tot > 0.f ? (m_run[qb] + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
        p.lse[(size_t)head * p.total_q + grow] = lse;
      }
    }
  }
}

}  // namespace

Bf16Geometry bf16_geometry(int hq, int hkv) {
  const int group = hq / hkv;
  Bf16Geometry g;
  g.waves = 8;
  g.rows_per_wave = QB * 32;
  // heads per workgroup: largest of 8, 4, 2, 1 dividing the GQA group size
  g.heads_per_group = (group % 8 == 0) ? 8 : (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1;
  return g;
}

hipError_t launch_fwd_bf16(const FwdParams& p, const Bf16Geometry& geo, int n_units,
                           hipStream_t stream) {
  const dim3 grid(n_units * p.n_head_groups), block(geo.waves * 64);
  switch (geo.heads_per_group) {
    case 8: hipLaunchKernelGGL((fwd_bf16_kernel<8, 8>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((fwd_bf16_kernel<8, 4>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((fwd_bf16_kernel<8, 2>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((fwd_bf16_kernel<8, 1>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace attnring
