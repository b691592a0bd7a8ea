// Issue-rate probes for the instruction mix of the attention kernel's softmax
// (measurement only, not part of the attention ABI).
//
// At head_dim 64 every score costs 256 matrix-core flops and about four vector
// instructions (scale-and-shift FMA, base-2 exponential, row-sum add, half a
// bf16 pack), and the MFMA operands come from LDS; how fast a SIMD issues that
// mix bounds the kernel.  Each probe runs one instruction mix in a loop on
// every SIMD of the chip with w waves per SIMD: one workgroup of 4*w waves
// per CU (its 84 KiB of LDS keeps any other workgroup off the CU).  Every wave
// records the shader-clock cycles (s_memtime) its loop took, the real-time
// counter's ticks over the same loop and its start.  Waves sharing a SIMD do
// not progress evenly (the oldest issues first), so the host takes a SIMD's
// time as its slowest wave's.
//
// Probes (mode):
//   0 fma     v_fma_f32             8 independent chains
//   1 exp     v_exp_f32             8 chains
//   2 add     v_add_f32             8 chains
//   3 cvt     v_cvt_pk_bf16_f32     8 chains
//   4 dot2    v_dot2c_f32_bf16      8 chains
//   5 max3    v_max3_f32            8 chains
//   6 mfma32  v_mfma_f32_32x32x16_bf16, 4 independent accumulators
//   7 mfma16  v_mfma_f32_16x16x32_bf16, 4 independent accumulators
//   8 mix     one 32-key softmax block's worth per iteration, all independent:
//             8 MFMA 32x32x16 + 16 exp + 16 fma + 16 add + 8 cvt, interleaved
//   9 mix_noexp  the same with the 16 exponentials left out
//  10 mix_nomfma the same with the 8 MFMAs left out
//  11 mfma+fma  8 MFMA 32x32x16 + 32 independent FMAs, interleaved
//  12 mfma+exp  8 MFMA 32x32x16 + 16 independent exponentials, interleaved
//  13 mfma+fma64  8 MFMA 32x32x16 + 64 independent FMAs, interleaved
//  14 (retired)
//  15 mix_poly  the block mix with every exponential computed by a cubic
//               polynomial on the FMA unit instead of v_exp_f32
//  16 mix16     the block mix with the matrix work as 16 v_mfma_f32_16x16x32_bf16
//  17 mfma_agpr+fma  8 MFMA 32x32x16 accumulating in AGPRs + 32 FMAs
//  18 mix_agpr   the block mix with the MFMAs accumulating in AGPRs
//  19 mfma16+fma 16 MFMA 16x16x32 + 32 FMAs
//  20 mfma_ab_agpr+fma  8 MFMA 32x32x16 with A, B and C in AGPRs + 32 FMAs
//  21 mix_ab_agpr  the block mix with the MFMAs' A, B and C in AGPRs
//  22 mix_a_agpr   the block mix with A and C in AGPRs, B in VGPRs
//  23 mix_lds      the block mix with the attention kernel's LDS reads: the
//                  MFMAs' A operands come from 4 ds_read_b128 and 8
//                  ds_read_b64_tr_b16 per iteration, as in the kernel
//  24 mix_lds_free the same reads issued, but the MFMAs use register operands
//                  (the reads' results are only kept alive)
//  25 mix_lds_b128 as 23, with the value operands read by 4 ds_read_b128
//                  (the same bytes in 8 instead of 12 reads)
//  26 mix_lds_2tile two query sub-tiles per wave share every LDS operand:
//                  per iteration 16 MFMAs, twice the vector work, 12 reads
//  27 mul     v_mul_f32             8 chains
//  28 fmamk   v_fmamk_f32 (a multiplier given as a literal) 8 chains
//  29 fmac    v_fmac_f32 (the accumulator is the destination) 8 chains
//  30 mix_lit      the block mix with the exponent's scale as a literal (v_fmamk_f32)
//  31 mix_lds_lit  the LDS-fed block mix (23) with the scale as a literal
//  32 mix_lds_2tile_random  probe 26 on random operands: the LDS tile, the query
//                  operands and the scores drawn from a counter hash (bf16
//                  operands uniform in (-2, 2)), so the matrix cores draw the
//                  power of real data and the board sets its clock accordingly
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int CH = 8;  // independent chains of the vector probes

__device__ __forceinline__ float lane_value(int salt) {
  return 0.25f + 0.001f * (float)((__builtin_amdgcn_workitem_id_x() * 7 + salt) & 127);
}

__device__ __forceinline__ uint32_t hash32(uint32_t x) {  // xorshift-multiply rounds
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
// uniform in (lo, lo + width) from the hash of counter `n`
__device__ __forceinline__ float hashed_value(uint32_t n, float lo, float width) {
  return lo + (float)(hash32(n) >> 8) * (width / 16777216.0f);
}

template <int MODE>
__device__ __forceinline__ float vector_probe(int iters) {
  float x[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) x[c] = lane_value(c);
  const float a = lane_value(100), b = lane_value(101);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if constexpr (MODE == 0) {
          x[c] = fmaf(x[c], a, b);
        } else if constexpr (MODE == 1) {
          x[c] = __builtin_amdgcn_exp2f(-x[c]);  // stays in [0.5, 1]
        } else if constexpr (MODE == 2) {
          x[c] = x[c] + a;
        } else if constexpr (MODE == 3) {
          // (written out so no repacking instructions surround it)
          asm volatile("v_cvt_pk_bf16_f32 %0, %0, %1" : "+v"(x[c]) : "v"(a));
        } else if constexpr (MODE == 27) {
          x[c] = x[c] * a;
        } else if constexpr (MODE == 28) {
          x[c] = fmaf(x[c], 0.18033688f, b);
        } else if constexpr (MODE == 29) {
          x[c] = fmaf(a, b, x[c]);
        } else if constexpr (MODE == 4) {
          const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
          x[c] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, __float_as_uint(b)), ones, x[c], false);
        } else {
          x[c] = fmaxf(fmaxf(x[c], a), b);
        }
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) s += x[c];
  return s;
}

// x * scale + shift; with LIT the scale is the literal log2(e)/8 in a v_fmamk_f32
// (written out: with the literal used many times the compiler keeps it in a
// register and emits v_fma_f32)
template <bool LIT>
__device__ __forceinline__ float scale_shift(float x, float scale, float shift) {
  if constexpr (LIT) {
    float r;
    asm("v_fmamk_f32 %0, %1, 0x3e38aa3b, %2" : "=v"(r) : "v"(x), "v"(shift));
    return r;
  } else {
    return fmaf(x, scale, shift);
  }
}

template <int MODE>
__device__ __forceinline__ float matrix_probe(int iters) {
  bf16x8 r0, r1;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    r0[j] = (__bf16)lane_value(j);
    r1[j] = (__bf16)lane_value(j + 8);
  }
  f32x16 c[4] = {};
  f32x4 d[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (MODE == 6)
          c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r0, r1, c[k], 0, 0, 0);
        else
          d[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r0, r1, d[k], 0, 0, 0);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    s += c[k][0] + c[k][15];
    s += d[k][0] + d[k][3];
  }
  return s;
}

// One 32-key block's worth of softmax-shaped vector work beside its 8 MFMAs,
// every instruction independent of the others within the iteration, with the
// vector instructions spread evenly between the MFMAs.
template <int MODE>
__device__ __forceinline__ float mix_probe(int iters) {
  bf16x8 r0, r1;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    r0[j] = (__bf16)lane_value(j);
    r1[j] = (__bf16)lane_value(j + 8);
  }
  constexpr bool MF = MODE != 10, EX = MODE != 9;
  constexpr bool ONLY_FMA = MODE == 11 || MODE == 13 || MODE == 17 || MODE == 19 || MODE == 20;
  constexpr int NFMA = MODE == 13 ? 8 : 4;
  constexpr bool ONLY_EXP = MODE == 12;
  constexpr bool POLY = MODE == 15;
  constexpr bool LIT = MODE == 30;  // the scale as a compile-time literal
  // matrix work: 0 = 8 x 32x32x16 (VGPR accumulators), 1 = 16 x 16x16x32, 2 = 8 x 32x32x16 in AGPRs
  // 3 = A, B, C in AGPRs; 4 = A, C in AGPRs
  constexpr int MK = (MODE == 16 || MODE == 19) ? 1 : (MODE == 17 || MODE == 18) ? 2
                     : (MODE == 20 || MODE == 21) ? 3 : MODE == 22 ? 4 : 0;
  f32x4 c4[4] = {};
  f32x16 ca[2] = {};
  f32x16 c[2] = {};
  float s[16], e[16], acc[4] = {0.f, 0.f, 0.f, 0.f};
  float f[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) s[j] = lane_value(j + 20);
  unsigned pk[8];
  (void)pk;
  const float cs = lane_value(50), nm = -lane_value(51);
  for (int it = 0; it < iters; ++it) {
    // the scores change every iteration as far as the compiler knows (no instruction)
#pragma unroll
    for (int j = 0; j < 16; ++j) asm volatile("" : "+v"(s[j]));
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if constexpr (MF && MK == 0) c[k & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r0, r1, c[k & 1], 0, 0, 0);
      if constexpr (MF && MK == 1) {
        c4[(2 * k) & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r0, r1, c4[(2 * k) & 3], 0, 0, 0);
        c4[(2 * k + 1) & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r0, r1, c4[(2 * k + 1) & 3], 0, 0, 0);
      }
      if constexpr (MF && MK == 2)  // accumulator in AGPRs; read only after the loop, behind explicit waits
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(ca[k & 1]) : "v"(r0), "v"(r1));
      if constexpr (MF && MK == 3)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(ca[k & 1]) : "a"(r0), "a"(r1));
      if constexpr (MF && MK == 4)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(ca[k & 1]) : "a"(r0), "v"(r1));
      if constexpr (ONLY_FMA) {
#pragma unroll
        for (int j = 0; j < NFMA; ++j) s[(NFMA * k + j) & 15] = fmaf(s[(NFMA * k + j) & 15], cs, nm);
      } else if constexpr (ONLY_EXP) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          e[2 * k + j] = __builtin_amdgcn_exp2f(s[2 * k + j]);
          asm volatile("" ::"v"(e[2 * k + j]));
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int i = 2 * k + j;
          f[i] = scale_shift<LIT>(s[i], cs, nm);
          if constexpr (POLY) {
            // 2^x = 2^n * 2^r, n = round(x), r in [-1/2, 1/2]: the magic constant
            // rounds x into the low mantissa bits of t; cubic in r
            const float xc = fmaxf(f[i], -126.f);
            const float t = xc + 12582912.0f;
            const float r = xc - (t - 12582912.0f);
            const float pr = fmaf(fmaf(fmaf(0.0555041f, r, 0.2402265f), r, 0.6931472f), r, 1.0f);
            e[i] = __int_as_float(__float_as_int(pr) + (__float_as_int(t) << 23));
          } else {
            e[i] = EX ? __builtin_amdgcn_exp2f(f[i]) : f[i];
          }
          acc[i & 3] += e[i];
        }
        const bf16x2 p2 = {(__bf16)e[2 * k], (__bf16)e[2 * k + 1]};
        pk[k] = __builtin_bit_cast(unsigned, p2);
        asm volatile("" ::"v"(pk[k]));  // the packed probabilities are used
      }
      if constexpr (MF && MK >= 2) __builtin_amdgcn_sched_barrier(0);  // (asm is not a schedule group)
      if constexpr (MF && MK < 2) {
        __builtin_amdgcn_sched_group_barrier(0x008, MK == 1 ? 2 : 1, 0);  // the MFMA(s)
        __builtin_amdgcn_sched_group_barrier(0x002, ONLY_FMA ? NFMA : ONLY_EXP ? 2 : POLY ? 23 : LIT ? 5 : (EX ? 7 : 5),
                                             0);  // its vector share (the literal FMAs are asm: not counted)
      }
    }
  }
  if constexpr (MK >= 2) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::);  // MFMA results settle before reads
  float t = acc[0] + acc[1] + acc[2] + acc[3] + c[0][0] + c[1][5] + c4[0][0] + c4[3][1] + ca[0][0] + ca[1][3];
#pragma unroll
  for (int j = 0; j < 16; ++j) t += s[j];
  return t;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// The block mix fed from LDS like the attention kernel: per iteration 4 A
// operands by ds_read_b128 (keys) and 8 half-operands by ds_read_b64_tr_b16
// (values), addresses inside the 16 KiB at `lds`.
template <bool FEED, bool VB128 = false, int TILES = 1, bool LIT = false, bool RND = false>
__device__ __forceinline__ float mix_lds_probe(int iters, const __attribute__((address_space(3))) char* lds) {
  // with RND the query operands and the scores are random, per thread of the grid
  const uint32_t gid = __builtin_amdgcn_workgroup_id_x() * __builtin_amdgcn_workgroup_size_x() +
                       __builtin_amdgcn_workitem_id_x();
  bf16x8 r1, r2;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    r1[j] = (__bf16)(RND ? hashed_value(gid * 64u + j, -2.f, 4.f) : lane_value(j + 8));
    r2[j] = (__bf16)(RND ? hashed_value(gid * 64u + 8 + j, -2.f, 4.f) : lane_value(j + 9));
  }
  const int lane = __builtin_amdgcn_workitem_id_x() & 63;
  // lane-linear addresses: conflict-free, like the kernel's swizzled tile reads
  const int ka = lane * 16;
  const int va = lane * 8;
  f32x16 c[2 * TILES] = {};
  float s[16], e[16], acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 16; ++j) s[j] = RND ? hashed_value(gid * 64u + 16 + j, -8.f, 8.f) : lane_value(j + 20);
  unsigned pk[8];
  const float cs = lane_value(50), nm = -lane_value(51), nm2 = -lane_value(52);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) asm volatile("" : "+v"(s[j]));
    bf16x8 kop[4], vop[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      kop[k] = *(const __attribute__((address_space(3))) bf16x8*)(lds + ka + k * 1024 + (it & 1) * 4096);
      if constexpr (VB128) {
        vop[k] = *(const __attribute__((address_space(3))) bf16x8*)(lds + 8192 + ka + k * 1024);
      } else {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + 8192 + va + k * 1024));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + 8192 + va + k * 1024 + 512));
        vop[k] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
#pragma unroll
    for (int k = 0; k < 8 * TILES; ++k) {
      const int kk = k % 8, tl = k / 8;
      const bf16x8 a = kk < 4 ? vop[kk] : kop[kk - 4];
      if constexpr (FEED) {
        c[(k & 1) + 2 * tl] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, tl ? r2 : r1, c[(k & 1) + 2 * tl], 0, 0, 0);
      } else {
        asm volatile("" ::"v"(a));
        c[k & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r1, r1, c[k & 1], 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = 2 * kk + j;
        e[i] = __builtin_amdgcn_exp2f(scale_shift<LIT>(s[i], cs, tl ? nm2 : nm));
        acc[i & 3] += e[i];
      }
      const bf16x2 p2 = {(__bf16)e[2 * kk], (__bf16)e[2 * kk + 1]};
      pk[kk] = __builtin_bit_cast(unsigned, p2);
      asm volatile("" ::"v"(pk[kk]));
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, LIT ? 5 : 7, 0);
    }
  }
  float t = acc[0] + acc[1] + acc[2] + acc[3] + c[0][0] + c[1][5] + c[2 * TILES - 1][3];
#pragma unroll
  for (int j = 0; j < 16; ++j) t += s[j];
  return t;
}

template <int MODE>
__global__ __launch_bounds__(1024) void probe_valu_kernel(float* sink, unsigned long long* cycles,
                                                          unsigned long long* realtime, unsigned long long* starts,
                                                          int iters) {
  __shared__ float pad[84 * 256];
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  float r;
  if constexpr (MODE <= 5 || (MODE >= 27 && MODE <= 29)) {
    r = vector_probe<MODE>(iters);
  } else if constexpr (MODE <= 7) {
    r = matrix_probe<MODE>(iters);
  } else if constexpr ((MODE >= 23 && MODE <= 26) || MODE == 31 || MODE == 32) {
    // 16 KiB of this workgroup's LDS as the operand source (contents arbitrary but
    // finite; for probe 32, pairs of random bf16 in (-2, 2))
    const int tid = __builtin_amdgcn_workitem_id_x();
    const uint32_t salt = 0x10000u * (1u + __builtin_amdgcn_workgroup_id_x());
    for (int i = tid; i < 4096; i += __builtin_amdgcn_workgroup_size_x()) {
      if constexpr (MODE == 32) {
        const bf16x2 two = {(__bf16)hashed_value(salt + 2 * i, -2.f, 4.f),
                            (__bf16)hashed_value(salt + 2 * i + 1, -2.f, 4.f)};
        pad[i] = __builtin_bit_cast(float, two);
      } else {
        pad[i] = 0.001f * (float)(i & 255);
      }
    }
    __syncthreads();
    const auto* lds = (const __attribute__((address_space(3))) char*)(const __attribute__((address_space(3))) float*)pad;
    if constexpr (MODE == 25)
      r = mix_lds_probe<true, true>(iters, lds);
    else if constexpr (MODE == 26)
      r = mix_lds_probe<true, false, 2>(iters, lds);
    else if constexpr (MODE == 31)
      r = mix_lds_probe<true, false, 1, true>(iters, lds);
    else if constexpr (MODE == 32)
      r = mix_lds_probe<true, false, 2, false, true>(iters, lds);
    else
      r = mix_lds_probe<MODE == 23>(iters, lds);
  } else {
    r = mix_probe<MODE>(iters);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int gid = __builtin_amdgcn_workgroup_id_x() * __builtin_amdgcn_workgroup_size_x() + tid;
  pad[tid] = r;
  __syncthreads();
  sink[gid] = pad[tid ^ 1];
  if ((tid & 63) == 0) {
    cycles[gid >> 6] = t1 - t0;
    realtime[gid >> 6] = r1 - r0;
    starts[gid >> 6] = r0;
  }
}

template <int MODE>
hipError_t launch(float* sink, unsigned long long* cycles, unsigned long long* realtime, unsigned long long* starts,
                  int cus, int w, int iters, hipStream_t s) {
  hipLaunchKernelGGL(probe_valu_kernel<MODE>, dim3(cus), dim3(256 * w), 0, s, sink, cycles, realtime, starts, iters);
  return hipGetLastError();
}

}  // namespace

// Instructions of each probe per loop iteration (per wave), for the host's arithmetic:
// vector probes 32 (4 unrolled x 8 chains); matrix probes 16 MFMAs; mix probes one block.
extern "C" int attn_probe_valu_modes(void) { return 33; }

// Run probe `mode` on `cus` CUs with `waves_per_simd` (1, 2 or 4) waves per
// SIMD for `iters` iterations: cus workgroups of 256 * waves_per_simd threads.
// `sink` must hold cus*waves_per_simd*256 floats; `cycles`, `realtime` and
// `starts` cus*waves_per_simd*4 counters each (one per wave: its loop's
// s_memtime and s_memrealtime deltas, and its start on the real-time counter).
// Returns 0 or a HIP error code (invalid arguments: hipErrorInvalidValue,
// nothing launched).
extern "C" int attn_probe_valu(float* sink, unsigned long long* cycles, unsigned long long* realtime,
                               unsigned long long* starts, int mode, int cus, int waves_per_simd, int iters,
                               hipStream_t stream) {
  if (!sink || !cycles || !realtime || !starts || cus < 1 || iters < 1 ||
      (waves_per_simd != 1 && waves_per_simd != 2 && waves_per_simd != 4) || mode == 14)
    return (int)hipErrorInvalidValue;
  const int w = waves_per_simd;
  hipError_t e;
  switch (mode) {
    case 0: e = launch<0>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 1: e = launch<1>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 2: e = launch<2>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 3: e = launch<3>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 4: e = launch<4>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 5: e = launch<5>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 6: e = launch<6>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 7: e = launch<7>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 8: e = launch<8>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 9: e = launch<9>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 10: e = launch<10>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 11: e = launch<11>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 12: e = launch<12>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 13: e = launch<13>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 15: e = launch<15>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 16: e = launch<16>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 17: e = launch<17>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 18: e = launch<18>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 19: e = launch<19>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 20: e = launch<20>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 21: e = launch<21>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 22: e = launch<22>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 23: e = launch<23>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 24: e = launch<24>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 25: e = launch<25>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 26: e = launch<26>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 27: e = launch<27>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 28: e = launch<28>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 29: e = launch<29>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 30: e = launch<30>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 31: e = launch<31>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    case 32: e = launch<32>(sink, cycles, realtime, starts, cus, w, iters, stream); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)e;
}
