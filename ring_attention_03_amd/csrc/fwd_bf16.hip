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
// Work decomposition.  A workgroup of 4 waves owns (sequence, row tile, group
// of query heads that share one key/value head); each wave owns 64 query rows
// of one head, kept in registers as two 32-row sub-tiles.  Key/value tiles of
// 128 keys are copied from HBM straight into LDS (global_load_lds, no register
// staging) and read by all 4 waves, so a tile is shared by the query heads of
// the group.  Every key or value operand a wave reads from LDS feeds the
// MFMAs of both sub-tiles: per score, half the LDS bytes of a 32-row wave, and
// two independent dependency chains per wave.  A wave needs up to 256 VGPRs,
// so two workgroups - two waves per SIMD, one of each - share a CU.
//
// Software pipeline.  Each wave walks its key range in 32-key blocks; the
// softmax of block i (vector ALU) is interleaved with O += P V of block i-1
// and S = K Q^T of block i+1 (matrix cores), which do not depend on it: the
// first half of a step exponentiates sub-tile 0 beside O += P V of both
// sub-tiles, the second half sub-tile 1 beside S = K Q^T of both.  Keys of
// block i+1 are read from LDS at the start of the step and values of block i
// at the end of it (held in registers for the next step's
// O += P V), so values live one tile longer than keys: LDS holds two key
// buffers and three value buffers (80 KiB), and one barrier per tile separates
// the copy of tile t+2 from the last reads of the buffers it reuses.
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
// The reference max of each row is updated lazily.  It starts at the row max
// of the first 128-key tile, so that tile's weights are all <= 1 and the
// largest is exactly 1.  A later block's exponentials are taken against the
// current reference and kept unless, in some lane, their sum exceeds the
// lane's accumulated sum (at least 1, at most 2^8); only then is the
// accumulator rescaled and the reference moved to the row max.  So no kept
// block carries more weight than the keys before it: a key that would dominate
// the row moves the reference onto itself and enters with weight exactly 1,
// not with a weight rounded to bf16 (relative error up to 2^-8), which would
// shift O by up to 2^-8 |v|.  O and LSE are normalised with the same
// reference, so the result does not depend on which reference was used.
#include "kernels.h"
#include "merge_math.h"

namespace attnring {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned short lds_u16;

constexpr int D = kHeadDim;       // 64
constexpr int NW = kBf16Waves;    // waves per workgroup (4)
constexpr int QW = kBf16RowsPerWave;  // query rows per wave (64)
constexpr int SUB = QW / 32;      // 32-row sub-tiles per wave (2)
static_assert(SUB == 2, "a step exponentiates one sub-tile in each half");
constexpr int BT = 128;           // keys per LDS tile
constexpr int BPT = BT / 32;      // 32-key blocks per tile

constexpr int NKB = 2;            // key tile buffers in LDS
constexpr int NVB = 3;            // value tile buffers in LDS (values are read one tile later)
constexpr int TILE_ELEMS = BT * D;
constexpr int TILE_BYTES = TILE_ELEMS * 2;
constexpr float SUM_LIMIT = 256.0f;  // no block's exponentials are kept when a lane-partial sum exceeds 2^8

// LDS tile layout: row-major [key][64], 16-byte chunks XOR-swizzled per row so
// that the MFMA operand reads hit distinct banks.  The LDS serves 256 bytes
// (64 banks) per clock, so a 16-byte read is conflict-free when each group of
// 16 lanes covers all of them: the K reads (lane = key row) take 16
// consecutive rows, two rows per 256 bytes, so the K chunk is XORed with
// bits 1-3 of the row; the transposing V reads take 4 consecutive rows x 32
// bytes per 16 lanes, so the V chunk pair is XORed with the row's low 2 bits.
__device__ __forceinline__ int k_pos(int key, int chunk) { return chunk ^ ((key >> 1) & 7); }
__device__ __forceinline__ int v_pos(int key, int chunk) { return chunk ^ ((key & 3) << 1); }
__device__ __forceinline__ int k_off(int key, int chunk) { return key * D + (k_pos(key, chunk) << 3); }
__device__ __forceinline__ int v_off(int key, int chunk) { return key * D + (v_pos(key, chunk) << 3); }

template <int V>
struct Int {
  static constexpr int value = V;
};

// One 16-byte slot per lane from global memory straight into LDS, lane-linear
// from the wave-uniform LDS byte address `lds_addr`.  Written as assembly so
// the compiler does not treat every later LDS read as dependent on it (it would
// wait for the copy to land before the next ds_read, which defeats the double
// buffering); the kernel waits for its copies itself, with vmcnt(0) before the
// barrier that publishes a tile.  M0 carries the LDS address and is restored.
__device__ __forceinline__ void lds_dma16(const void* gbase, unsigned voff, unsigned lds_addr) {
  // gbase and lds_addr are wave-uniform; readfirstlane puts them in scalar registers
  // (readfirstlane returns int: each half goes through unsigned so the low half
  // is not sign-extended into the high one)
  const unsigned long long a = (unsigned long long)gbase;
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)a);
  const void* sbase = (const void*)(((unsigned long long)hi << 32) | (unsigned long long)lo);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
      : "memory");
}

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
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(FwdParams p) {
  // LDS: NKB key tile buffers, then NVB value tile buffers (16 KiB each)
  __shared__ __attribute__((aligned(16))) unsigned short lds[(NKB + NVB) * TILE_ELEMS];

  // (the index builtins directly: the device-library wrappers are compiled with
  // IEEE mode on and would not inline into this kernel)
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int wg = __builtin_amdgcn_workgroup_id_x();
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // ---- which (sequence, row tile, head group) this workgroup owns
  // (the division runs on the vector unit; readfirstlane keeps everything derived
  // from it in scalar registers)
  const int G = p.n_head_groups;
  const int unit = __builtin_amdgcn_readfirstlane(wg / G);
  int hg = wg - unit * G;
  // workgroup w runs on XCD w % 8: when the groups divide evenly, XCD x takes a
  // contiguous range of head groups, so groups that share a key/value head
  // also share that XCD's L2
  if ((G & 7) == 0) hg = (hg & 7) * (G >> 3) + (hg >> 3);
  int s = 0;
  while (unit >= p.unit_off[s + 1]) ++s;
  const int tile = (p.unit_off[s + 1] - 1) - unit;  // heaviest (last) row tile first
  constexpr int ROWS = QW * (NW / HPW);
  const int r0 = tile * ROWS;
  const int Lq = p.q_len[s], Lk = p.k_len[s];
  const int qp0 = p.q_pos0[s], kp0 = p.k_pos0[s];
  const int group = p.hq / p.hkv;
  const int head = hg * HPW + (wave % HPW);
  const int kvh = __builtin_amdgcn_readfirstlane((hg * HPW) / group);
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
  // blocks [0, nfull) are visible to every row of the tile; later ones need the mask
  const int nfull = min(nblk, kfull >> 5);

  // ---- this wave's queries as MFMA B operands, per sub-tile sb (rows rw0 + 32*sb ..):
  // qr[sb][ks] = q[row][16*ks + 8*half .. +7]
  bf16x8 qr[SUB][4];
#pragma unroll
  for (int sb = 0; sb < SUB; ++sb) {
    const int row = rw0 + 32 * sb + l32;
    const __bf16* src = reinterpret_cast<const __bf16*>(p.q) +
                        ((size_t)(p.q_row0[s] + row) * p.hq + head) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qr[sb][ks] = row < Lq ? *reinterpret_cast<const bf16x8*>(src + ks * 16) : bf16x8{};
  }

  // ---- tile copy HBM -> LDS: 16-byte slot i of a tile (lane-linear per wave and
  // instruction) is (key row i/8, position i%8) and holds global chunk
  // position ^ swizzle(row).  A pass of the workgroup fills NW*64 slots (NW*8
  // rows, a multiple of 16, so every pass sees the same swizzle); keys past the
  // end read the last row instead (finite data, masked out of the scores).
  constexpr int ROWS_PER_PASS = NW * 8;
  constexpr int PASSES = BT / ROWS_PER_PASS;
  const int slot_key = tid >> 3, slot_pos = tid & 7;
  const int kstride = p.hkv * D;  // elements between consecutive keys
  const size_t kv_base = ((size_t)p.k_row0[s] * p.hkv + kvh) * D;
  const char* kgb = reinterpret_cast<const char*>(reinterpret_cast<const unsigned short*>(p.k) + kv_base);
  const char* vgb = reinterpret_cast<const char*>(reinterpret_cast<const unsigned short*>(p.v) + kv_base);
  // Per-lane byte offsets stay 32-bit (the host bounds a sequence's K/V to 2 GiB),
  // so the copies use a scalar base plus one vector offset.
  const unsigned k_lane_off = (unsigned)k_pos(slot_key, slot_pos) << 4;  // bytes within a key row
  const unsigned v_lane_off = (unsigned)v_pos(slot_key, slot_pos) << 4;
  // this wave's LDS byte address within a pass, wave-uniform
  const unsigned lds_wave = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(const lds_u16*)(const unsigned short*)lds + wave * 1024);
  // per-lane source offsets of a tile's first pass; a tile or pass adds a
  // wave-uniform amount to the scalar base instead
  const unsigned k_src = (unsigned)(slot_key * kstride) * 2u + k_lane_off;
  const unsigned v_src = (unsigned)(slot_key * kstride) * 2u + v_lane_off;
  const unsigned pass_bytes = (unsigned)(ROWS_PER_PASS * kstride) * 2u;
  auto copy_tile = [&](int t) __attribute__((always_inline)) {
    const unsigned kb = (t % NKB) * TILE_BYTES, vb = (NKB + t % NVB) * TILE_BYTES;
    if (t * BT + BT <= Lk) {  // every key of the tile exists: no clamping
      const size_t tile_off = (size_t)(t * BT) * kstride * 2;
#pragma unroll
      for (int j = 0; j < PASSES; ++j) {
        const unsigned dst = lds_wave + j * ROWS_PER_PASS * D * 2;  // this wave's 64 slots of the pass
        lds_dma16(kgb + tile_off + j * pass_bytes, k_src, dst + kb);
        lds_dma16(vgb + tile_off + j * pass_bytes, v_src, dst + vb);
      }
    } else {
#pragma unroll
      for (int j = 0; j < PASSES; ++j) {
        const int key = min(t * BT + j * ROWS_PER_PASS + slot_key, Lk - 1);
        const unsigned row_off = (unsigned)(key * kstride) * 2u;
        const unsigned dst = lds_wave + j * ROWS_PER_PASS * D * 2;
        lds_dma16(kgb, row_off + k_lane_off, dst + kb);
        lds_dma16(vgb, row_off + v_lane_off, dst + vb);
      }
    }
  };

  // ---- per-lane LDS operand addresses (bytes; the block within a tile is an immediate).
  // K (A operand of S^T): row l32 (+32 per block), chunk 2*ks + half; the
  // swizzle depends on (row >> 1) & 7 = (l32 >> 1) & 7 only.  k_addr points into the buffer of
  // the tile whose keys are read next.
  int k_addr[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) k_addr[ks] = k_off(l32, 2 * ks + half) * 2;
  // V (A operand of O^T via transposing reads): lane = 16*g + r reads key
  // 16*step + 4*(g/2) + r/4 (+8 for the upper 4 k-slots) at d = 32*dblk +
  // 16*(g%2) + 4*(r%4); the swizzle depends on key & 3 = (r/4) & 3 only.
  int v_addr[2];
  {
    const int g16 = (lane >> 4) & 3, r16 = lane & 15;
    const int v_key = 4 * (g16 >> 1) + (r16 >> 2);
    const int v_chunk = 2 * (g16 & 1) + ((r16 & 3) >> 1);
    const int v_sub = 4 * (r16 & 1);
#pragma unroll
    for (int db = 0; db < 2; ++db)
      v_addr[db] = (NKB * TILE_ELEMS + v_off(v_key, 4 * db + v_chunk) + v_sub) * 2;
  }
  const __attribute__((address_space(3))) char* lds_b =
      (const __attribute__((address_space(3))) char*)(const lds_u16*)(const unsigned short*)lds;
  // the values of tile t sit in buffer t % NVB: step v_addr from tile t-1's buffer to tile t's
  // (v_addr starts at tile 0's)
  auto advance_v = [&](int t) __attribute__((always_inline)) {
    const int delta = t == 0 ? 0 : (t % NVB == 0) ? -(NVB - 1) * TILE_BYTES : TILE_BYTES;
    v_addr[0] += delta;
    v_addr[1] += delta;
  };

  // Per sub-tile: O^T accumulators [sb][dblk]; the reference max of this
  // lane's query (log2 units, scaled); the exponent offset; the lane-partial
  // sum of 2^(s*c - m_run).  A row that sees no key keeps no reference: its
  // offset stays +3e38, which still gives exact zeros for its -inf scores (and
  // would overflow any visible score to +inf, sending it down the exact path).
  f32x16 acc[SUB][2];
  float m_run[SUB], neg_m[SUB], l_run[SUB];
#pragma unroll
  for (int sb = 0; sb < SUB; ++sb) {
    acc[sb][0] = f32x16{};
    acc[sb][1] = f32x16{};
    m_run[sb] = -INFINITY;
    neg_m[sb] = 3.0e38f;
    l_run[sb] = 0.f;
  }
  const float c2 = p.scale_log2;
  // Make the scalar load of c2 complete here: otherwise its wait (lgkmcnt,
  // shared with LDS reads) lands inside the loop, where the first use is, and
  // drains every LDS read in flight at the top of each iteration.
  asm volatile("" ::"s"(c2));
  f32x16 S[2][SUB];         // scores of blocks i (S[i&1]) and i+1 per sub-tile: keys x 32 queries
  bf16x8 P[2][SUB][2];      // bf16 probabilities of blocks i and i-1 ([i&1]), per sub-tile and 16-key step
  bf16x8 vnext[4];          // values of the block whose O += P V comes next

  // K operand of 16-key step ks of block `sub` in the current key buffer
  auto kread = [&](int ks, auto sub_tag) __attribute__((always_inline)) {
    constexpr int OFF = decltype(sub_tag)::value * 32 * D * 2;
    return *(const __attribute__((address_space(3))) bf16x8*)(lds_b + k_addr[ks] + OFF);
  };
  // V^T operand of (16-key step st, d block db) of block `sub` in the current value buffer
  auto vread = [&](int st, int db, auto sub_tag) __attribute__((always_inline)) {
    constexpr int OFF = decltype(sub_tag)::value * 32 * D * 2;
    const __attribute__((address_space(3))) char* vb = lds_b + v_addr[db] + OFF + st * 16 * D * 2;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vb);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * D * 2));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // exponentials of the 8 scores of 16-key step ST of sub-tile SB against its
  // current reference (-> Pst; four independent partial sums)
  auto exps_half = [&](const f32x16& Sb, bf16x8& Pst, float* part, auto st_tag, auto sb_tag)
      __attribute__((always_inline)) {
    constexpr int ST = decltype(st_tag)::value;
    constexpr int SB = decltype(sb_tag)::value;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float pv = __builtin_amdgcn_exp2f(fmaf(Sb[ST * 8 + j], c2, neg_m[SB]));
      if (ST == 0 && j < 4) part[j] = pv; else part[j & 3] += pv;
      Pst[j] = (__bf16)pv;
    }
  };
  auto mask = [&](f32x16& Sb, int b, int sb) __attribute__((always_inline)) {
    const int qpos = qp0 + rw0 + 32 * sb + l32;
    int last = Lk - 1;
    if (p.causal) last = min(last, qpos - kp0);
    const int lim = last - b * 32 - half * 4;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int off = (e >> 2) * 8 + (e & 3);
      Sb[e] = off <= lim ? Sb[e] : -INFINITY;
    }
  };
  // max of the lane's 16 scores (chains of 3-input max)
  auto lane_max = [&](const f32x16& Sb) __attribute__((always_inline)) {
    float mx = fmaxf(fmaxf(Sb[0], Sb[1]), Sb[2]);
#pragma unroll
    for (int e = 3; e < 15; e += 2) mx = fmaxf(fmaxf(mx, Sb[e]), Sb[e + 1]);
    return fmaxf(mx, Sb[15]);
  };
  // raise the reference max of each row of sub-tile SB to the row max whose
  // lane maxima are mx (rescaling its acc and l)
  auto raise_reference = [&](float mx, auto sb_tag) __attribute__((always_inline)) {
    constexpr int SB = decltype(sb_tag)::value;
    const float m_new = fmaxf(m_run[SB], max_halves(mx) * c2);
    if (m_new > m_run[SB]) {
      const float alpha = __builtin_amdgcn_exp2f(m_run[SB] - m_new);  // 0 when m_run was -inf
      l_run[SB] *= alpha;
      acc[SB][0] *= alpha;
      acc[SB][1] *= alpha;
      m_run[SB] = m_new;
      neg_m[SB] = -m_new;
    }
  };
  // scores of block b (its keys at `kfetch`) for both sub-tiles, masked if need be
  auto scores2 = [&](f32x16* Sb, int b, auto kfetch) __attribute__((always_inline)) {
    Sb[0] = f32x16{};
    Sb[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 kk = kfetch(ks);
      Sb[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, qr[0][ks], Sb[0], 0, 0, 0);
      Sb[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, qr[1][ks], Sb[1], 0, 0, 0);
    }
    if (b >= nfull) {
      mask(Sb[0], b, 0);
      mask(Sb[1], b, 1);
    }
  };

  // One step of the software pipeline for block i (i % 4 == J, compile-time).
  // The softmax of block i runs on the vector ALU while the matrix core does
  // O += P V for block i-1 (first half, beside sub-tile 0's exponentials) and
  // S = K Q^T for block i+1 (second half, beside sub-tile 1's); both are
  // independent of block i, so one wave keeps both units fed.
  //
  // Exponentials are taken against each row's current reference max and kept
  // when every lane-partial row sum is <= the lane's accumulated sum (clamped
  // to [1, 2^8]), so p <= 256 and the block does not dominate the row.
  // Otherwise - a score outgrew its reference, in either sub-tile - both
  // sub-tiles' scores are recomputed (they are not kept live: registers), each
  // reference is raised to its row max with acc and l rescaled, and the
  // exponentials redone.
  //
  // Buffers: block i+1's keys are read at the start of the step (of the second
  // half at J == 3) and block i's values at the end of the step, after the
  // matrix work is issued,
  // so their latency is covered by the step's tail and they are in registers
  // when step i+1 starts.  At J == 3, between the two halves, all waves meet at
  // the tile barrier: by then every wave has read the keys of this tile and the
  // values of the tile before it, so the next-but-one tile is copied into those
  // buffers.  The only later read of this tile's keys would be a recompute at
  // J == 3, which therefore reads the keys from global memory.
  auto step = [&](auto j_tag, int i) __attribute__((always_inline)) {
    constexpr int J = decltype(j_tag)::value;
    constexpr int CUR = J & 1, NXT = CUR ^ 1;
    const bool masked = i >= nfull;  // workgroup-uniform
    if (masked) {
      mask(S[CUR][0], i, 0);
      mask(S[CUR][1], i, 1);
    }
    if constexpr (J == 0) advance_v(i >> 2);
    float part0[4], part1[4];
    // keys of block i+1, read before the first half (at J == 3 they sit in the
    // next tile, which the barrier between the halves publishes)
    bf16x8 ka[4];
    if constexpr (J != 3) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) ka[ks] = kread(ks, Int<(J + 1) & 3>{});
    }
    // ---- first half: exponentials of sub-tile 0 with O += V^T P^T of block i-1
    {
      exps_half(S[CUR][0], P[CUR][0][0], part0, Int<0>{}, Int<0>{});
      exps_half(S[CUR][0], P[CUR][0][1], part0, Int<1>{}, Int<0>{});
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int sb = 0; sb < SUB; ++sb)
            acc[sb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vnext[2 * st + db], P[NXT][sb][st],
                                                                  acc[sb][db], 0, 0, 0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x402, 7, 0);  // exp / fma / add / convert
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      }
    }
    if constexpr (J == 3) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's share of the next tile landed
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) k_addr[ks] ^= TILE_BYTES;
      if ((i >> 2) + 2 < ntile) copy_tile((i >> 2) + 2);
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- second half: exponentials of sub-tile 1 with S = K Q^T of block i+1
    {
      if constexpr (J == 3) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) ka[ks] = kread(ks, Int<(J + 1) & 3>{});
      }
      exps_half(S[CUR][1], P[CUR][1][0], part1, Int<0>{}, Int<1>{});
      exps_half(S[CUR][1], P[CUR][1][1], part1, Int<1>{}, Int<1>{});
      S[NXT][0] = f32x16{};
      S[NXT][1] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb)
          S[NXT][sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qr[sb][ks], S[NXT][sb], 0, 0, 0);
      if constexpr (J == 3) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // key reads
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x402, 7, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // values of this block for the next step's O += P V (its tile was published
    // at the previous tile's barrier and is overwritten two barriers later)
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int db = 0; db < 2; ++db) vnext[2 * st + db] = vread(st, db, Int<J>{});
    // convert the probabilities here, before the check, so the conversions sit
    // among this step's instructions instead of trailing it
    asm volatile("" ::"v"(P[CUR][0][0]), "v"(P[CUR][0][1]), "v"(P[CUR][1][0]), "v"(P[CUR][1][1]));
    float rs0 = (part0[0] + part0[1]) + (part0[2] + part0[3]);
    float rs1 = (part1[0] + part1[1]) + (part1[2] + part1[3]);
    // keep limit: the lane's accumulated sum, clamped to [1, 2^8]; the first
    // tile's blocks are all <= the reference (it is their row max), so they only
    // need the 2^8 guard (a row that saw none of them has no reference yet)
    const float lo = i < BPT ? SUM_LIMIT : 1.0f;
    const float keep0 = __builtin_amdgcn_fmed3f(l_run[0], lo, SUM_LIMIT);
    const float keep1 = __builtin_amdgcn_fmed3f(l_run[1], lo, SUM_LIMIT);
    if (__builtin_amdgcn_ballot_w64(rs0 > keep0 || rs1 > keep1) != 0) {  // wave-uniform, rare
      f32x16 Sb[SUB];
      if constexpr (J == 3) {
        const int key = min(i * 32 + l32, Lk - 1);
        const unsigned off = ((unsigned)(key * kstride) + half * 8) * 2u;
        scores2(Sb, i, [&](int ks) { return *reinterpret_cast<const bf16x8*>(kgb + off + ks * 32); });
      } else {
        scores2(Sb, i, [&](int ks) { return kread(ks, Int<J>{}); });
      }
      raise_reference(lane_max(Sb[0]), Int<0>{});
      raise_reference(lane_max(Sb[1]), Int<1>{});
      exps_half(Sb[0], P[CUR][0][0], part0, Int<0>{}, Int<0>{});
      exps_half(Sb[0], P[CUR][0][1], part0, Int<1>{}, Int<0>{});
      exps_half(Sb[1], P[CUR][1][0], part1, Int<0>{}, Int<1>{});
      exps_half(Sb[1], P[CUR][1][1], part1, Int<1>{}, Int<1>{});
      rs0 = (part0[0] + part0[1]) + (part0[2] + part0[3]);
      rs1 = (part1[0] + part1[1]) + (part1[2] + part1[3]);
      // the next block's scores are recomputed too, so they need no registers
      // while this path runs (its mask, if any, is applied at its own step)
      S[NXT][0] = f32x16{};
      S[NXT][1] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kk = kread(ks, Int<(J + 1) & 3>{});
        S[NXT][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, qr[0][ks], S[NXT][0], 0, 0, 0);
        S[NXT][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, qr[1][ks], S[NXT][1], 0, 0, 0);
      }
    }
    l_run[0] += rs0;
    l_run[1] += rs1;
  };
  // ---- prologue: tile 0 landed, tile 1 in flight, scores of block 0.
  // Step 0 also multiplies the values of block 3 of tile 0 by an all-zero P
  // (there is no block -1), and the last step computes scores of a block past
  // the end from whatever the key buffer holds; both results are unused.
#pragma unroll
  for (int sb = 0; sb < SUB; ++sb) {
    P[1][sb][0] = bf16x8{};
    P[1][sb][1] = bf16x8{};
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) vnext[k] = bf16x8{};
  if (nblk > 0) {
    copy_tile(0);
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): the queries and this wave's share of tile 0
    __syncthreads();
    if (ntile > 1) copy_tile(1);
    // the row max over the first tile is the first reference, so its blocks
    // take the kept path with every weight <= 1 (rows that see none of it keep
    // -inf); block 0's scores are computed last and stay in S[0]
    static_assert(BPT == 4, "the first reference spans the four blocks of a tile");
    float mx0 = -INFINITY, mx1 = -INFINITY;
    auto first_scores = [&](auto b_tag) __attribute__((always_inline)) {
      constexpr int B = decltype(b_tag)::value;
      scores2(S[0], B, [&](int ks) { return kread(ks, Int<B>{}); });
      mx0 = fmaxf(mx0, lane_max(S[0][0]));
      mx1 = fmaxf(mx1, lane_max(S[0][1]));
    };
    first_scores(Int<3>{});
    first_scores(Int<2>{});
    first_scores(Int<1>{});
    first_scores(Int<0>{});
    raise_reference(mx0, Int<0>{});
    raise_reference(mx1, Int<1>{});
  }
  if (nblk > 0) {
    for (int i0 = 0; i0 < nblk; i0 += 4) {
      step(Int<0>{}, i0);
      step(Int<1>{}, i0 + 1);
      step(Int<2>{}, i0 + 2);
      step(Int<3>{}, i0 + 3);
    }
    // O += V^T P^T of the last block (its values were read at the end of its step)
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb)
          acc[sb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vnext[2 * st + db], P[1][sb][st], acc[sb][db],
                                                                0, 0, 0);
  }

  // ---- epilogue, per sub-tile: O = acc / l, LSE = (m + log2 l) * ln 2; written,
  // or merged into the running state (o, lse) by their log-sum-exps (rows that
  // saw no key here leave the state as it is)
  // (the lane index is taken afresh from the exec mask, so no lane-derived value
  // has to stay live across the loop)
  const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int half_e = lane_e >> 5;
#pragma unroll
  for (int sb = 0; sb < SUB; ++sb) {
    const float l_tot = sum_halves(l_run[sb]);
    const float inv = l_tot > 0.f ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
    const int row = rw0 + 32 * sb + (lane_e & 31);
    if (row < Lq) {
      const size_t grow = (size_t)(p.q_row0[s] + row);
      float* dst = p.o + (grow * p.hq + head) * D + half_e * 4;
      float* lse_dst = p.lse + (size_t)head * p.total_q + grow;
      const float lse_b = l_tot > 0.f ? (m_run[sb] + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
      if (!p.merge) {
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f32x4 v4;
            v4[0] = acc[sb][db][i * 4 + 0] * inv;
            v4[1] = acc[sb][db][i * 4 + 1] * inv;
            v4[2] = acc[sb][db][i * 4 + 2] * inv;
            v4[3] = acc[sb][db][i * 4 + 3] * inv;
            *reinterpret_cast<f32x4*>(dst + db * 32 + i * 8) = v4;
          }
        if (half_e == 0) *lse_dst = lse_b;
      } else if (l_tot > 0.f) {
        // the running state's O and LSE are loaded together, before the weights
        // need the LSE (both halves read the LSE before half 0 writes it)
        f32x4 oa[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) oa[k] = *reinterpret_cast<const f32x4*>(dst + (k >> 2) * 32 + (k & 3) * 8);
        const float la = *lse_dst;
        float lse, wa, wb;
        lse_merge_weights(la, lse_b, &lse, &wa, &wb);
        const float wbi = wb * inv;  // this block's weight times its normaliser
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int db = k >> 2, i = k & 3;
          f32x4 o4;
          o4[0] = fmaf(wbi, acc[sb][db][i * 4 + 0], wa * oa[k][0]);
          o4[1] = fmaf(wbi, acc[sb][db][i * 4 + 1], wa * oa[k][1]);
          o4[2] = fmaf(wbi, acc[sb][db][i * 4 + 2], wa * oa[k][2]);
          o4[3] = fmaf(wbi, acc[sb][db][i * 4 + 3], wa * oa[k][3]);
          *reinterpret_cast<f32x4*>(dst + db * 32 + i * 8) = o4;
        }
        if (half_e == 0) *lse_dst = lse;
      }
    }
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, const Bf16Geometry& geo, int n_units,
                           hipStream_t stream) {
  const dim3 grid(n_units * p.n_head_groups), block(geo.waves * 64);
  switch (geo.heads_per_group) {
    case 4: hipLaunchKernelGGL((fwd_bf16_kernel<4>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((fwd_bf16_kernel<2>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((fwd_bf16_kernel<1>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace attnring
