// Matrix-core rate probe (measurement only, not part of the attention ABI).
//
// Every wave runs `iters` iterations of 16 independent-chain bf16 MFMAs
// (v_mfma_f32_32x32x16_bf16 into four accumulators) over eight operand
// registers.  With `random` set the operands are uniform in (-2, 2), drawn from
// a counter hash per lane; otherwise every operand is the same constant.  The
// two rates differ because the matrix cores' power depends on the data they
// switch: on random data the board lowers its clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ inline uint32_t mix(uint32_t x) {  // a 32-bit integer hash (xorshift-multiply rounds)
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(256) void probe_mfma_kernel(float* out, int random, int iters) {
  const uint32_t base = (blockIdx.x * 256u + threadIdx.x) * 64u;
  bf16x8 r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float u = random ? (float)(mix(base + i * 8 + j) >> 8) * (4.0f / 16777216.0f) - 2.0f : 0.5f;
      r[i][j] = (__bf16)u;
    }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[0], r[1], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[2], r[3], c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[4], r[5], c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[6], r[7], c3, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[1], r[2], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[3], r[4], c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[5], r[6], c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[7], r[0], c3, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[2], r[5], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[3], r[6], c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[4], r[7], c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[0], r[1], c3, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[6], r[3], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[7], r[2], c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[0], r[5], c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[1], r[4], c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * 256u + threadIdx.x] = s;
}

}  // namespace

// Launch `blocks` workgroups of 256 threads (4 waves, one per SIMD) on `stream`;
// `out` must hold blocks * 256 floats.  Returns 0, or the HIP error code.
extern "C" int attn_probe_mfma(float* out, int blocks, int random, int iters, hipStream_t stream) {
  if (!out || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(256), 0, stream, out, random, iters);
  return (int)hipGetLastError();
}
