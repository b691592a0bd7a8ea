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
// Work decomposition.  A workgroup of 8 waves owns (sequence, row tile, group
// of query heads that share one key/value head); each wave owns 32 query rows
// of one head, kept in registers.  Key/value tiles of 64 keys are copied from
// HBM straight into LDS (global_load_lds, no register staging), double
// buffered, and read by all 8 waves, so a tile is shared by every query head
// of its GQA group.  A wave needs under 128 VGPRs, so two workgroups - four
// waves per SIMD - share a CU, and the hardware overlaps one wave's MFMAs with
// another's softmax arithmetic.  (A single wave cannot issue vector
// instructions fast enough to keep the VALU busy on its own, which is why the
// overlap is left to several resident waves rather than to one wave's
// instruction order.)
//
// Register layouts (v_mfma_f32_32x32x16_bf16: A is 32x16, B is 16x32, lane l
// supplies row/col l%32 and k-slots 8*(l/32)..+7; D lane l holds column l%32,
// rows 8*(e/4) + 4*(l/32) + e%4 for e = 0..15):
//  * scores are computed transposed, S^T = K Q^T (A = K rows from LDS, B = Q
//    from registers), so a lane holds keys of ONE query: the row max and row
//    sum are lane-local plus one v_permlane32_swap;
//  * the output is computed transposed, O^T = V^T P^T.  B is P^T taken
//    straight from the score accumulator; A (V^T) is gathered from row-major
//    V in LDS by ds_read_b64_tr_b16 (within each 16 lanes, lane j receives
//    element j%4 of the 4-element row read by lane 4i + j/4, for i = 0..3),
//    with addresses chosen so the key order matches the accumulator's.
//
// The reference max of each row is updated lazily: the exponentials of a block
// are taken against the current reference unless some score exceeds it by
// more than 2^8 (p <= 256 keeps fp32 exact in range and bf16 at its usual
// relative precision); only then - or on a row's first block - is the
// accumulator rescaled and the reference moved to the row max.  O and LSE are
// normalised with the same reference, so the result does not depend on which
// reference was used.
#include "kernels.h"

namespace attnring {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned short lds_u16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void global_cvoid;

constexpr int D = kHeadDim;       // 64
constexpr int NW = 8;             // waves per workgroup
constexpr int QW = 32;            // query rows per wave
constexpr int BT = 128;           // keys per LDS tile
constexpr int BPT = BT / 32;      // 32-key blocks per tile

constexpr int TILE_ELEMS = BT * D;
constexpr float SUM_LIMIT = 256.0f;  // a block's exponentials are kept when each lane-partial sum is <= 2^8

// LDS tile layout: row-major [key][64], 16-byte chunks XOR-swizzled per row so
// that the MFMA operand reads hit distinct banks (K: 16-byte reads of 8
// consecutive rows; V: transposing reads of 4 consecutive rows x 32 bytes).
__device__ __forceinline__ int k_pos(int key, int chunk) { return chunk ^ (key & 7); }
__device__ __forceinline__ int v_pos(int key, int chunk) { return chunk ^ ((key & 3) << 1); }
__device__ __forceinline__ int k_off(int key, int chunk) { return key * D + (k_pos(key, chunk) << 3); }
__device__ __forceinline__ int v_off(int key, int chunk) { return key * D + (v_pos(key, chunk) << 3); }

template <bool B>
struct MaskTag {
  static constexpr bool value = B;
};
template <int V>
struct Int {
  static constexpr int value = V;
};

__device__ __forceinline__ float max_halves(float x) {
  // max of x over lanes l and l^32 (v_permlane32_swap exchanges the wave halves)
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int HPW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 4)))
void fwd_bf16_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) unsigned short lds_k[2][TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) unsigned short lds_v[2][TILE_ELEMS];

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
  constexpr int ROWS = QW * (NW / HPW);
  const int r0 = tile * ROWS;
  const int Lq = p.q_len[s], Lk = p.k_len[s];
  const int qp0 = p.q_pos0[s], kp0 = p.k_pos0[s];
  const int group = p.hq / p.hkv;
  const int head = hg * HPW + (wave % HPW);
  const int kvh = (hg * HPW) / group;
  const int rw0 = r0 + (wave / HPW) * QW;  // this wave's first row (within the sequence)

  // keys [0, kend) can be visible to some row of the tile; keys [0, kfull) to all of them
  const int last_row = min(r0 + ROWS, Lq) - 1;
  int kend = Lk, kfull = Lk;
  if (p.causal) {
    kend = min(Lk, max(0, qp0 + last_row - kp0 + 1));
    kfull = min(Lk, max(0, qp0 + r0 - kp0 + 1));
  }
  const int nblk = (kend + 31) >> 5;
  const int ntile = (kend + BT - 1) / BT;

  // ---- this wave's queries as MFMA B operands: qr[ks] = q[row][16*ks + 8*half .. +7]
  bf16x8 qr[4];
  {
    const int row = rw0 + l32;
    const __bf16* src = reinterpret_cast<const __bf16*>(p.q) +
                        ((size_t)(p.q_row0[s] + row) * p.hq + head) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qr[ks] = row < Lq ? *reinterpret_cast<const bf16x8*>(src + ks * 16) : bf16x8{};
  }

  // ---- tile copy HBM -> LDS: 16-byte slot i of a tile (lane-linear per wave and
  // instruction) is (key row i/8, position i%8) and holds global chunk
  // position ^ swizzle(row).  A pass of the workgroup fills NW*64 slots (NW*8
  // rows, a multiple of 8, so every pass sees the same swizzle); keys past the
  // end read the last row instead (finite data, masked out of the scores).
  constexpr int ROWS_PER_PASS = NW * 8;
  constexpr int PASSES = BT / ROWS_PER_PASS;
  const int slot_key = tid >> 3, slot_pos = tid & 7;
  const unsigned short* kg = reinterpret_cast<const unsigned short*>(p.k) +
                             ((size_t)p.k_row0[s] * p.hkv + kvh) * D +
                             ((slot_pos ^ (slot_key & 7)) << 3);
  const unsigned short* vg = reinterpret_cast<const unsigned short*>(p.v) +
                             ((size_t)p.k_row0[s] * p.hkv + kvh) * D +
                             ((slot_pos ^ ((slot_key & 3) << 1)) << 3);
  const size_t kstride = (size_t)p.hkv * D;
  auto copy_tile = [&](int t, int buf) {
#pragma unroll
    for (int j = 0; j < PASSES; ++j) {
      const int key = min(t * BT + j * ROWS_PER_PASS + slot_key, Lk - 1);
      const int dst = j * ROWS_PER_PASS * D + wave * 512;  // this wave's 64 slots of the pass
      __builtin_amdgcn_global_load_lds((global_cvoid*)(kg + key * kstride),
                                       (lds_void*)&lds_k[buf][dst], 16, 0, 0);
      __builtin_amdgcn_global_load_lds((global_cvoid*)(vg + key * kstride),
                                       (lds_void*)&lds_v[buf][dst], 16, 0, 0);
    }
  };

  // ---- per-lane parts of the LDS operand addresses (everything else is an immediate)
  // K (A operand of S^T): row l32 (+32 per block, +BT per buffer), chunk 2*ks + half;
  // the swizzle depends on row & 7 = l32 & 7 only.
  int k_lane[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) k_lane[ks] = k_off(l32, 2 * ks + half) * 2;
  // V (A operand of O^T via transposing reads): lane = 16*g + r reads key
  // 16*step + 4*(g/2) + r/4 (+8 for the upper 4 k-slots) at d = 32*dblk +
  // 16*(g%2) + 4*(r%4); the swizzle depends on key & 3 = (r/4) & 3 only.
  int v_lane[2];
  {
    const int g16 = (lane >> 4) & 3, r16 = lane & 15;
    const int v_key = 4 * (g16 >> 1) + (r16 >> 2);
    const int v_chunk = 2 * (g16 & 1) + ((r16 & 3) >> 1);
    const int v_sub = 4 * (r16 & 1);
#pragma unroll
    for (int db = 0; db < 2; ++db) v_lane[db] = (v_off(v_key, 4 * db + v_chunk) + v_sub) * 2;
  }
  const lds_u16* lds_k0 = (const lds_u16*)(const unsigned short*)lds_k;
  const lds_u16* lds_v0 = (const lds_u16*)(const unsigned short*)lds_v;

  f32x16 acc[2];  // O^T, [dblk]
  acc[0] = f32x16{};
  acc[1] = f32x16{};
  float m_run = -INFINITY;  // reference max of this lane's query (log2 units, scaled)
  float l_run = 0.f;        // lane-partial sum of 2^(s*c - m_run)
  const float c2 = p.scale_log2;
  f32x16 S;                 // scores of the current block: keys x this wave's 32 queries
  bf16x8 P[2];              // bf16 probabilities of the current block, per 16-key step

  // exponentials of the block against the current reference max (-> P, lane-partial sum;
  // four partial sums keep the additions independent)
  auto exps = [&](float& rs) {
    // Without a reference yet (-inf), use -3e38: every visible score then
    // overflows to +inf, which sends the block down the exact path, while a
    // fully masked row still contributes exact zeros.
    const float m_use = m_run == -INFINITY ? -3.0e38f : m_run;
    float part[4];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(S[st * 8 + j], c2, -m_use));
        const int k = (st * 8 + j) & 3;
        part[k] = (st == 0 && j < 4) ? pv : part[k] + pv;
        P[st][j] = (__bf16)pv;
      }
    rs = (part[0] + part[1]) + (part[2] + part[3]);
  };

  // S^T = K Q^T for the 32 keys at row offset `row0` of LDS buffer `buf` (compile-time)
  auto scores = [&](auto buf_tag, auto half_tag) {
    constexpr int BASE = (decltype(buf_tag)::value * TILE_ELEMS + decltype(half_tag)::value * 32 * D) * 2;
    S = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 a = *(const __attribute__((address_space(3))) bf16x8*)(
          (const __attribute__((address_space(3))) char*)lds_k0 + k_lane[ks] + BASE);
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr[ks], S, 0, 0, 0);
    }
  };
  auto mask = [&](int b) {
    const int qpos = qp0 + rw0 + l32;
    int last = Lk - 1;
    if (p.causal) last = min(last, qpos - kp0);
    const int lim = last - b * 32 - half * 4;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int off = (e >> 2) * 8 + (e & 3);
      S[e] = off <= lim ? S[e] : -INFINITY;
    }
  };
  // raise the reference max of each row to the row max of S (rescaling acc and l)
  auto settle_reference = [&]() {
    float mx = fmaxf(fmaxf(S[0], S[1]), S[2]);  // chains of 3-input max over the lane's 16 keys
#pragma unroll
    for (int e = 3; e < 15; e += 2) mx = fmaxf(fmaxf(mx, S[e]), S[e + 1]);
    mx = fmaxf(mx, S[15]);
    const float m_new = fmaxf(m_run, max_halves(mx) * c2);
    if (m_new > m_run) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run was -inf
      l_run *= alpha;
      acc[0] *= alpha;
      acc[1] *= alpha;
      m_run = m_new;
    }
  };

  // softmax of the scores of block b (keys 32b.. of the sequence chunk) -> P, l.
  // Fast path: exponentials against the current reference max, kept when every
  // lane-partial row sum is <= 2^8 (then no score exceeded the reference by more
  // than 8 in log2 units, so p <= 256).  Otherwise - the row's first visible
  // block (reference -inf, sums inf), or a score that outgrew the reference -
  // the scores are recomputed (they are not kept live: registers), the
  // reference is raised to the row max with acc and l rescaled, and the
  // exponentials redone.
  auto softmax = [&](auto masked_tag, auto buf_tag, auto half_tag, int b) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    if constexpr (MASKED) mask(b);
    float rs;
    exps(rs);
    if (__builtin_amdgcn_ballot_w64(rs > SUM_LIMIT) != 0) {  // wave-uniform, rare
      scores(buf_tag, half_tag);
      if constexpr (MASKED) mask(b);
      settle_reference();
      exps(rs);
    }
    l_run += rs;
  };
  // O^T += V^T P^T for the block in quarter `half_tag` of LDS buffer `buf_tag`
  auto pv = [&](auto buf_tag, auto half_tag) {
    constexpr int VBASE = (decltype(buf_tag)::value * TILE_ELEMS + decltype(half_tag)::value * 32 * D) * 2;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const __attribute__((address_space(3))) char* vb =
            (const __attribute__((address_space(3))) char*)lds_v0 + v_lane[db] + VBASE + st * 16 * D * 2;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vb);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * D * 2));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[st], acc[db], 0, 0, 0);
      }
    }
  };
  // One block of a tile.  Once the exponentials of block b have consumed the
  // scores, the scores of the tile's next block are issued into the same
  // registers BEFORE O += P V of block b, so the matrix core finishes them
  // first and the next softmax overlaps the P V products.
  auto block = [&](auto masked_tag, auto buf_tag, auto half_tag, int b) {
    softmax(masked_tag, buf_tag, half_tag, b);
    constexpr int H = decltype(half_tag)::value;
    if constexpr (H + 1 < BPT) scores(buf_tag, Int<H + 1>{});
    pv(buf_tag, half_tag);
  };

  // blocks [0, nfull) are visible to every row of the tile; later ones need the mask
  const int nfull = min(nblk, kfull >> 5);
  // one tile: it has landed in buffer BUF (own copies waited for, then the
  // barrier); every wave is done with the other buffer, which takes tile t+1
  auto tile_step = [&](auto buf_tag, int t) {
    constexpr int BUF = decltype(buf_tag)::value;
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
    __syncthreads();
    if (t + 1 < ntile) copy_tile(t + 1, BUF ^ 1);
    const int b0 = t * BPT;
    scores(buf_tag, Int<0>{});
    if (b0 + 3 < nfull) {
      block(MaskTag<false>{}, buf_tag, Int<0>{}, b0);
      block(MaskTag<false>{}, buf_tag, Int<1>{}, b0 + 1);
      block(MaskTag<false>{}, buf_tag, Int<2>{}, b0 + 2);
      block(MaskTag<false>{}, buf_tag, Int<3>{}, b0 + 3);
    } else {
      if (b0 < nfull) block(MaskTag<false>{}, buf_tag, Int<0>{}, b0); else block(MaskTag<true>{}, buf_tag, Int<0>{}, b0);
      if (b0 + 1 < nfull) block(MaskTag<false>{}, buf_tag, Int<1>{}, b0 + 1); else if (b0 + 1 < nblk) block(MaskTag<true>{}, buf_tag, Int<1>{}, b0 + 1);
      if (b0 + 2 < nfull) block(MaskTag<false>{}, buf_tag, Int<2>{}, b0 + 2); else if (b0 + 2 < nblk) block(MaskTag<true>{}, buf_tag, Int<2>{}, b0 + 2);
      if (b0 + 3 < nblk) block(MaskTag<true>{}, buf_tag, Int<3>{}, b0 + 3);
    }
  };
  if (ntile > 0) copy_tile(0, 0);
  for (int t = 0; t < ntile; t += 2) {
    tile_step(Int<0>{}, t);
    if (t + 1 < ntile) tile_step(Int<1>{}, t + 1);
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2
  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int row = rw0 + l32;
  if (row < Lq) {
    const size_t grow = (size_t)(p.q_row0[s] + row);
    float* dst = p.o + (grow * p.hq + head) * D + half * 4;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 v4;
        v4[0] = acc[db][i * 4 + 0] * inv;
        v4[1] = acc[db][i * 4 + 1] * inv;
        v4[2] = acc[db][i * 4 + 2] * inv;
        v4[3] = acc[db][i * 4 + 3] * inv;
        *reinterpret_cast<f32x4*>(dst + db * 32 + i * 8) = v4;
      }
    if (half == 0) {
      const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
      p.lse[(size_t)head * p.total_q + grow] = lse;
    }
  }
}

}  // namespace

Bf16Geometry bf16_geometry(int hq, int hkv) {
  const int group = hq / hkv;
  Bf16Geometry g;
  g.waves = NW;
  g.rows_per_wave = QW;
  // heads per workgroup: largest of 8, 4, 2, 1 dividing the GQA group size
  g.heads_per_group = (group % 8 == 0) ? 8 : (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1;
  return g;
}

hipError_t launch_fwd_bf16(const FwdParams& p, const Bf16Geometry& geo, int n_units,
                           hipStream_t stream) {
  const dim3 grid(n_units * p.n_head_groups), block(geo.waves * 64);
  switch (geo.heads_per_group) {
    case 8: hipLaunchKernelGGL((fwd_bf16_kernel<8>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((fwd_bf16_kernel<4>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((fwd_bf16_kernel<2>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((fwd_bf16_kernel<1>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace attnring
