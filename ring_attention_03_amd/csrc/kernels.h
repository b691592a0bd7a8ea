// Internal interface between the C ABI (abi.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnring {

constexpr int kHeadDim = 64;
constexpr int kMaxSeqs = 64;

// Everything a forward launch needs, passed by value in the kernel arguments.
// Sequences appear in processing order (heaviest first); `unit_off` is the
// prefix count of row tiles over that order.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;
  int32_t total_q;
  int32_t hq;
  int32_t hkv;
  int32_t causal;
  int32_t merge;     // 1: fold this block's result into (o, lse) in place instead of writing it
  float scale_log2;  // softmax scale times log2(e): scores are exponentiated base 2
  int32_t nseq;
  int32_t n_head_groups;  // workgroups per row tile (one per group of heads sharing K/V)
  int32_t rows_per_tile;  // query rows one workgroup covers
  int32_t q_row0[kMaxSeqs];
  int32_t q_len[kMaxSeqs];
  int32_t k_row0[kMaxSeqs];
  int32_t k_len[kMaxSeqs];
  int32_t q_pos0[kMaxSeqs];
  int32_t k_pos0[kMaxSeqs];
  int32_t unit_off[kMaxSeqs + 1];
};

// Tile geometry of the bf16 MFMA kernel, shared with the host planner.
constexpr int kBf16Waves = 4;        // waves per workgroup
constexpr int kBf16RowsPerWave = 64; // query rows per wave (two 32-row sub-tiles)

struct Bf16Geometry {
  int waves;           // waves per workgroup
  int heads_per_group; // query heads per workgroup (all share one kv head)
  int rows_per_wave;   // query rows per wave
  int rows_per_tile() const { return rows_per_wave * (waves / heads_per_group); }
};

// Heads per workgroup: the largest of 4, 2, 1 dividing the GQA group size.
inline Bf16Geometry bf16_geometry(int hq, int hkv) {
  const int group = hq / hkv;
  Bf16Geometry g;
  g.waves = kBf16Waves;
  g.rows_per_wave = kBf16RowsPerWave;
  g.heads_per_group = (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1;
  return g;
}

hipError_t launch_fwd_bf16(const FwdParams& p, const Bf16Geometry& geo, int n_units,
                           hipStream_t stream);

constexpr int kF32RowsPerTile = 64;
hipError_t launch_fwd_f32(const FwdParams& p, int n_units, hipStream_t stream);

hipError_t launch_merge(int32_t total_q, int32_t hq, float* o_acc, float* lse_acc,
                        const float* o_part, const float* lse_part, hipStream_t stream);

}  // namespace attnring
