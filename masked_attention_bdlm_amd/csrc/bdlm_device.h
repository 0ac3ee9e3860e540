// Device-side building blocks: element traits, MFMA wrappers, fragment loads.
//
// MFMA shapes used (CDNA4 / gfx950):
//   bf16: v_mfma_f32_32x32x16_bf16  A 32x16, B 16x32, C 32x32 fp32
//   fp32: v_mfma_f32_32x32x2_f32    A 32x2,  B 2x32,  C 32x32 fp32
// Operand layout (wave64): lane l supplies row (A) / column (B) l%32 and the
// KPL consecutive k values starting at KPL*(l/32).  The 32x32 fp32 result gives
// lane l column l%32 and rows 8*(i/4) + 4*(l/32) + i%4 for its 16 values i.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bdlm_common.h"

namespace bdlm {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T> struct Elt;

template <> struct Elt<bf16> {
  static constexpr int KPL = 8;    // k values per lane per MFMA
  static constexpr int VEC = 8;    // elements per 16-byte access
  static constexpr int PAD = 8;    // LDS row padding (elements)
  using Frag = bf16x8;
  __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Elt<float> {
  static constexpr int KPL = 1;
  static constexpr int VEC = 4;
  static constexpr int PAD = 4;
  using Frag = float;
  __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// 16-byte vector of VEC elements.
struct alignas(16) Vec16 { uint32_t w[4]; };

__device__ inline Vec16 ld16(const void* p) { return *reinterpret_cast<const Vec16*>(p); }
__device__ inline void st16(void* p, const Vec16& v) { *reinterpret_cast<Vec16*>(p) = v; }
__device__ inline Vec16 zero16() { Vec16 v; v.w[0] = v.w[1] = v.w[2] = v.w[3] = 0u; return v; }

template <typename T> __device__ inline T elem_of(const Vec16& v, int j) {
  return reinterpret_cast<const T*>(&v)[j];
}

// KPL contiguous elements at p (A/B fragment along k).
template <typename T> __device__ inline typename Elt<T>::Frag ld_frag(const T* p);
template <> __device__ inline bf16x8 ld_frag<bf16>(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <> __device__ inline float ld_frag<float>(const float* p) { return *p; }

// Fragment whose k values are the C-layout rows c_row(i, hh) for
// i = ci*KPL .. ci*KPL+KPL-1 of a 32-row tile starting at `row0`, read from a
// row of a k-major (transposed) LDS buffer.  For bf16 (KPL=8) these are two
// runs of 4 consecutive rows: 16*(ci) + 4*hh + 0..3 and 16*ci + 8 + 4*hh + 0..3.
template <typename T> __device__ inline typename Elt<T>::Frag ld_frag_crows(const T* row, int ci, int hh);
template <> __device__ inline bf16x8 ld_frag_crows<bf16>(const bf16* row, int ci, int hh) {
  const bf16* p = row + 16 * ci + 4 * hh;
  bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
  bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 8);
  bf16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}
template <> __device__ inline float ld_frag_crows<float>(const float* row, int ci, int hh) {
  return row[c_row(ci, hh)];
}

// Pack C-layout values acc[ci*KPL .. ci*KPL+KPL) into an MFMA fragment.
template <typename T> __device__ inline typename Elt<T>::Frag pack_frag(const float* v);
template <> __device__ inline bf16x8 pack_frag<bf16>(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = static_cast<bf16>(v[j]);
  return r;
}
template <> __device__ inline float pack_frag<float>(const float* v) { return v[0]; }

template <typename T> __device__ inline T to_elt(float x) { return static_cast<T>(x); }

__device__ inline float wave_swap32(float x) { return __shfl_xor(x, 32, 64); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace bdlm
