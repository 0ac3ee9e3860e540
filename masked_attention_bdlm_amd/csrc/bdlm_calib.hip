// Calibration kernel (diagnostics, not part of the attention path): the bf16
// MFMA rate the chip sustains for a given operand and instruction mix.
//
// The published dense bf16 peak assumes every SIMD's matrix core busy at the
// 2.4 GHz peak engine clock.  Under load the chip holds its power limit by
// lowering the clock, and MFMA power depends on the operand bits that toggle:
// with constant operands the clock stays near the peak, with random operands
// (as attention data are) it does not.  This kernel keeps the matrix cores
// busy for a whole launch and records, per wave, shader-clock cycles and
// 100 MHz real-time ticks, from which the caller derives the clock and the
// achieved rate.  See bdlm_calib_mfma in include/bdlm_attn.h for the modes.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/bdlm_attn.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;            // 8 waves: two per SIMD
constexpr int kLdsWords = 6144;          // 96 KB of LDS: one workgroup per CU

__device__ inline uint32_t mix32(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
  return x;
}
// Eight bf16 values uniform in [-0.5, 0.5) from a 32-bit seed (or a constant).
__device__ inline bf16x8 operand(uint32_t seed, bool random) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t h = random ? mix32(seed * 8u + (uint32_t)i) : 0x4000u * (uint32_t)(i + 1);
    v[i] = (__bf16)((float)(h & 0xFFFFu) * (1.0f / 65536.0f) - 0.5f);
  }
  return v;
}

// Every wave runs `iters` steps of 4 MFMAs (v_mfma_f32_32x32x16_bf16, four
// independent accumulators, 128 matrix-core cycles per step), plus per MODE:
//   0  constant operands;
//   1  random operands, 8 register sets in rotation;
//   2  mode 1 plus one 16-byte LDS read per lane per MFMA (1 KB per wave, the
//      attention kernels' LDS operand traffic), each consumed 4 MFMAs later;
//   3  mode 1 plus 4 FMAs per MFMA.
template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void calib_mfma_kernel(int64_t* cycles, float* sink, int iters) {
  __shared__ u32x4 lds[kLdsWords];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  for (int i = tid; i < kLdsWords; i += kThreads)
    lds[i] = u32x4{mix32(i), mix32(i + 7), mix32(i + 13), mix32(i + 29)};
  __syncthreads();
  const uint32_t seed = (uint32_t)(blockIdx.x * kThreads + tid);
  bf16x8 A[8], B[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    A[j] = operand(seed * 16u + (uint32_t)j, MODE != 0);
    B[j] = operand(seed * 16u + 8u + (uint32_t)j, MODE != 0);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  float x[4] = {1e-3f, 2e-3f, 3e-3f, 4e-3f};
  const float k = 0.999f;
  u32x4 ring[4] = {}, acc = {};
  const int64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (MODE == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc ^= ring[q];
          ring[q] = lds[(lane + 64 * ((it * 4 + u * 4 + q) & 63)) % kLdsWords];
        }
      }
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[4 * u + 0], B[4 * u + 0], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[4 * u + 1], B[4 * u + 1], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[4 * u + 2], B[4 * u + 2], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[4 * u + 3], B[4 * u + 3], c3, 0, 0, 0);
      if (MODE == 3) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = __builtin_fmaf(x[i], k, k);
      }
    }
  }
  const int64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
  for (int q = 0; q < 4; ++q) acc ^= ring[q];
  float t = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) + x[0] + x[1] + x[2] + x[3];
#pragma unroll
  for (int i = 0; i < 16; ++i) t += c0[i] + c1[i] + c2[i] + c3[i];
  sink[(int64_t)blockIdx.x * kThreads + tid] = t;
  if (lane == 0) {
    cycles[((int64_t)blockIdx.x * 8 + w) * 2] = t1 - t0;
    cycles[((int64_t)blockIdx.x * 8 + w) * 2 + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" int bdlm_calib_mfma(int32_t mode, int32_t workgroups, int32_t iters, int64_t* cycles, float* sink,
                               hipStream_t stream) {
  if (mode < 0 || mode > 3 || workgroups < 1 || workgroups > 65536 || iters < 2 || (iters & 1) || !cycles ||
      !sink)
    return BDLM_ERR_INVALID_ARG;
  const dim3 grid(workgroups), block(kThreads);
  switch (mode) {
    case 0: calib_mfma_kernel<0><<<grid, block, 0, stream>>>(cycles, sink, iters); break;
    case 1: calib_mfma_kernel<1><<<grid, block, 0, stream>>>(cycles, sink, iters); break;
    case 2: calib_mfma_kernel<2><<<grid, block, 0, stream>>>(cycles, sink, iters); break;
    default: calib_mfma_kernel<3><<<grid, block, 0, stream>>>(cycles, sink, iters); break;
  }
  return hipGetLastError() == hipSuccess ? BDLM_OK : BDLM_ERR_HIP;
}
