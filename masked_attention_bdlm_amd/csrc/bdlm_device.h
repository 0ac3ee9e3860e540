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
typedef uint32_t Vec16 __attribute__((ext_vector_type(4)));

__device__ inline Vec16 ld16(const void* p) { return *reinterpret_cast<const Vec16*>(p); }
__device__ inline void st16(void* p, const Vec16& v) { *reinterpret_cast<Vec16*>(p) = v; }
__device__ inline Vec16 zero16() { return Vec16{0u, 0u, 0u, 0u}; }

template <typename T> __device__ inline T elem_of(const Vec16& v, int j);
template <> __device__ inline bf16 elem_of<bf16>(const Vec16& v, int j) {
  return __builtin_bit_cast(bf16x8, v)[j];
}
template <> __device__ inline float elem_of<float>(const Vec16& v, int j) {
  return __builtin_bit_cast(f32x4, v)[j];
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

// ---- fragments read "down" a row-major LDS tile (k = tile rows, lane = column)
//
// ds_read_b64_tr_b16 (gfx950): in each 16-lane group, lane r supplies the
// address of 4 consecutive 16-bit elements, forming a 16x4 matrix M[r][c];
// lane i receives M[4j + i/4][i%4] for j = 0..3.  If lane r addresses
// tile[r0 + r/4][c0 + 4*(r%4)], lane i receives tile[r0 + j][c0 + i], j=0..3:
// column c0 + i of rows r0..r0+3.
typedef short s16x4 __attribute__((ext_vector_type(4)));

// The transpose-read builtin carries no alias information of its own, so the
// compiler makes it wait for every global->LDS DMA still in flight, including
// the one filling the other half of a double buffer.  Inlining through a
// restrict-qualified parameter attaches alias scopes to the read, which lifts
// that wait; the kernels order their own DMA waits and barriers explicitly.
__device__ __forceinline__ s16x4 ds_read_tr16(const void* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) void*)(p));
}
__device__ inline bf16x4 ld_tr4(const bf16* tile, int stride, int r0, int c0, int i16) {
  const bf16* p = tile + (r0 + (i16 >> 2)) * stride + c0 + 4 * (i16 & 3);
  return __builtin_bit_cast(bf16x4, ds_read_tr16(p));
}

__device__ inline bf16x8 cat44(bf16x4 lo, bf16x4 hi) {
  bf16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// MFMA fragment for column col0 + lane%32 whose k values are the tile rows
// row0 + c_row(ci*KPL + j, hh), j < KPL (the C-layout row order of chunk ci).
template <typename T> __device__ inline typename Elt<T>::Frag ld_frag_kcrow(const T* tile, int stride, int row0,
                                                                         int ci, int lane, int col0);
template <> __device__ inline bf16x8 ld_frag_kcrow<bf16>(const bf16* tile, int stride, int row0, int ci, int lane,
                                                        int col0) {
  const int r = row0 + 16 * ci + 4 * (lane >> 5);
  const int c = col0 + ((lane >> 4) & 1) * 16;
  return cat44(ld_tr4(tile, stride, r, c, lane & 15), ld_tr4(tile, stride, r + 8, c, lane & 15));
}
template <> __device__ inline float ld_frag_kcrow<float>(const float* tile, int stride, int row0, int ci, int lane,
                                                        int col0) {
  return tile[(row0 + c_row(ci, lane >> 5)) * stride + col0 + (lane & 31)];
}

// Same with the natural k order: rows row0 + KPL*hh + j, j < KPL.
template <typename T> __device__ inline typename Elt<T>::Frag ld_frag_knat(const T* tile, int stride, int row0,
                                                                        int lane, int col0);
template <> __device__ inline bf16x8 ld_frag_knat<bf16>(const bf16* tile, int stride, int row0, int lane, int col0) {
  const int r = row0 + 8 * (lane >> 5);
  const int c = col0 + ((lane >> 4) & 1) * 16;
  return cat44(ld_tr4(tile, stride, r, c, lane & 15), ld_tr4(tile, stride, r + 4, c, lane & 15));
}
template <> __device__ inline float ld_frag_knat<float>(const float* tile, int stride, int row0, int lane, int col0) {
  return tile[(row0 + (lane >> 5)) * stride + col0 + (lane & 31)];
}

// ---- unpadded row-major tiles with XOR-swizzled 16-byte chunks
//
// Row r of a D-column tile is D*sizeof(T) bytes = CH chunks of 16 bytes;
// logical chunk c of row r is stored at chunk c ^ f(r).  A row block of 1 KB
// stays contiguous, so a wave's global->LDS DMA (64 lanes x 16 bytes) fills
// 64/CH whole rows whatever f is.  f is chosen for the two read patterns on
// gfx950's 64-bank LDS (16 bank groups of 16 bytes):
//  - a fragment read, 16 lanes reading one logical chunk of 16 consecutive
//    rows, needs f to take 16 distinct bank groups over those rows;
//  - a transpose read (ds_read_b64_tr_b16), half a wave reading 4 aligned
//    chunks of 4 aligned consecutive rows, needs the 4 rows to land on 4
//    different aligned 4-chunk groups.
// bf16, D = 128 (CH = 16): f(r) swaps the two 2-bit halves of r mod 16.
// bf16, D = 64 (CH = 8, two rows per 256 bytes): f(r) = g(r/2 mod 8) with g
// moving bit 0 to bit 2.  fp32 tiles (reference precision) use f(r) = r mod CH.
template <typename T, int D>
struct Swz {
  static constexpr int EPC = 16 / (int)sizeof(T);   // elements per chunk
  static constexpr int CH = D / EPC;                // chunks per row
  static constexpr int RPB = 64 / CH;               // rows per 1 KB DMA block
  __host__ __device__ static inline int f(int r) {
    if constexpr (sizeof(T) == 2 && CH == 16) {
      return ((r & 3) << 2) | ((r >> 2) & 3);
    } else if constexpr (sizeof(T) == 2 && CH == 8) {
      const int x = (r >> 1) & 7;
      return ((x & 1) << 2) | (x >> 1);
    } else {
      return r & (CH - 1);
    }
  }
  __host__ __device__ static inline int idx(int r, int col) {
    return r * D + (((col / EPC) ^ f(r)) * EPC) + (col % EPC);
  }
};

template <typename T, int D> __device__ inline typename Elt<T>::Frag ld_frag_s(const T* tile, int r, int col) {
  return ld_frag<T>(tile + Swz<T, D>::idx(r, col));
}

template <int D> __device__ inline bf16x4 ld_tr4_s(const bf16* tile, int r0, int c0, int i16) {
  const bf16* p = tile + Swz<bf16, D>::idx(r0 + (i16 >> 2), c0 + 4 * (i16 & 3));
  return __builtin_bit_cast(bf16x4, ds_read_tr16(p));
}

// ld_frag_kcrow / ld_frag_knat on a swizzled tile.
template <typename T, int D> __device__ inline typename Elt<T>::Frag ld_frag_kcrow_s(const T* tile, int row0, int ci,
                                                                                   int lane, int col0);
template <> __device__ inline bf16x8 ld_frag_kcrow_s<bf16, 128>(const bf16* tile, int row0, int ci, int lane, int col0) {
  const int r = row0 + 16 * ci + 4 * (lane >> 5), c = col0 + ((lane >> 4) & 1) * 16;
  return cat44(ld_tr4_s<128>(tile, r, c, lane & 15), ld_tr4_s<128>(tile, r + 8, c, lane & 15));
}
template <> __device__ inline bf16x8 ld_frag_kcrow_s<bf16, 64>(const bf16* tile, int row0, int ci, int lane, int col0) {
  const int r = row0 + 16 * ci + 4 * (lane >> 5), c = col0 + ((lane >> 4) & 1) * 16;
  return cat44(ld_tr4_s<64>(tile, r, c, lane & 15), ld_tr4_s<64>(tile, r + 8, c, lane & 15));
}
template <> __device__ inline float ld_frag_kcrow_s<float, 128>(const float* tile, int row0, int ci, int lane, int col0) {
  return tile[Swz<float, 128>::idx(row0 + c_row(ci, lane >> 5), col0 + (lane & 31))];
}
template <> __device__ inline float ld_frag_kcrow_s<float, 64>(const float* tile, int row0, int ci, int lane, int col0) {
  return tile[Swz<float, 64>::idx(row0 + c_row(ci, lane >> 5), col0 + (lane & 31))];
}

// ---- bf16 fragment reads at precomputed per-lane byte offsets
//
// On a swizzled bf16 tile the lane-dependent part of a fragment address
// repeats every 16 rows, so it can be computed once per kernel; the 32-row
// sub-tile, the 16-row chunk and the buffer go in the instruction's
// immediate offset or one add per tile.
//   offA[c]            row-fragment read: row lane%32, k = 16c + 8(lane/32) .. +7
//   offT[2 dt + h]     transpose read h of ld_frag_kcrow_s(tile, 0, 0, lane, 32 dt)
template <int D>
__device__ inline void bf16_frag_offsets(int lane, uint32_t* offA, uint32_t* offT) {
  using S = Swz<bf16, D>;
  const int ln = lane & 31, hh = lane >> 5, i16 = lane & 15;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) offA[c] = 2u * (uint32_t)S::idx(ln, (2 * c + hh) * 8);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int r = 4 * hh + 8 * h2 + (i16 >> 2);
      const int col = dt * 32 + 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
      offT[2 * dt + h2] = 2u * (uint32_t)S::idx(r, col);
    }
  }
}
// Row fragment: rows r0 + lane%32 (r0 a multiple of 16) of the tile at `tile`.
__device__ __forceinline__ bf16x8 ld_fragA(const char* tile, uint32_t off, int r0_bytes) {
  return *reinterpret_cast<const bf16x8*>(tile + off + r0_bytes);
}
// ld_frag_kcrow_s(tile, row0, ci, lane, 32 dt) with row0 + 16 ci in bytes.
__device__ __forceinline__ bf16x8 ld_fragT(const char* tile, const uint32_t* offT, int dt, int r_bytes) {
  return cat44(__builtin_bit_cast(bf16x4, ds_read_tr16(tile + offT[2 * dt] + r_bytes)),
               __builtin_bit_cast(bf16x4, ds_read_tr16(tile + offT[2 * dt + 1] + r_bytes)));
}

// Global -> LDS DMA of rows [k0, k0+NR) of a [rows, heads, D] array (row
// stride rs elements, pointer at the head) into a swizzled tile.  Wave `wave`
// of NW issues every NW-th 1 KB block; each lane moves one 16-byte chunk.
// Rows at or past kmax re-read row kmax-1 (finite data; callers mask them).
template <typename T, int NR, int D, int NW = 4>
__device__ inline void dma_rows(T* tile, const T* base, int64_t rs, int k0, int kmax, int wave, int lane) {
  using S = Swz<T, D>;
  constexpr int NBLK = NR / S::RPB;
  static_assert(NR % S::RPB == 0, "tile rows must fill whole DMA blocks");
  static_assert(NBLK % NW == 0, "every wave issues the same number of blocks");
  const int lr = lane / S::CH, pc = lane % S::CH;
  // Every address is one wave-uniform base (row k0, scalar registers) plus a
  // 32-bit per-lane byte offset: the instruction then takes the scalar-base
  // form, whose per-lane address is 4 bytes instead of 8, which the memory
  // pipeline accepts faster.  The empty asm keeps the compiler from widening
  // the (loop-invariant) offset into a 64-bit per-lane address.
  const char* tb = reinterpret_cast<const char*>(base + (int64_t)k0 * rs);
  if (k0 + NR <= kmax) {   // whole tile inside the array: fixed per-lane offsets
#pragma unroll
    for (int j = 0; j < NBLK / NW; ++j) {
      const int bb = wave + j * NW;
      const int r = bb * S::RPB + lr;
      const int c = pc ^ S::f(r);
      uint32_t off = ((uint32_t)r * (uint32_t)rs + (uint32_t)(c * S::EPC)) * (uint32_t)sizeof(T);
      asm volatile("" : "+v"(off));
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(tb + off),
                                       (__attribute__((address_space(3))) void*)(tile + bb * S::RPB * D), 16, 0, 0);
    }
  } else {                 // the tile crosses the array end: rows clamped to kmax - 1
#pragma unroll
    for (int j = 0; j < NBLK / NW; ++j) {
      const int bb = wave + j * NW;
      const int r = bb * S::RPB + lr;
      const int c = pc ^ S::f(r);
      const int rr = min(r, kmax - 1 - k0);
      uint32_t off = ((uint32_t)rr * (uint32_t)rs + (uint32_t)(c * S::EPC)) * (uint32_t)sizeof(T);
      asm volatile("" : "+v"(off));
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(tb + off),
                                       (__attribute__((address_space(3))) void*)(tile + bb * S::RPB * D), 16, 0, 0);
    }
  }
}

// Return v unchanged but opaque to the compiler, held in scalar registers.
// Kernel arguments are otherwise re-loaded from memory wherever they are used
// (the compiler treats those loads as free to repeat), which inside a loop
// adds a scalar-memory round trip per use.
template <typename V> __device__ __forceinline__ V pin_sgpr(V v) {
  asm volatile("" : "+s"(v));
  return v;
}

// Workgroup barrier that orders LDS only: waits for this wave's own LDS
// reads and writes (lgkmcnt(0)), not for its outstanding global->LDS DMA, so
// prefetches stay in flight across it.  __syncthreads() would also wait for
// the DMA (its release fence must cover every LDS write, DMA included).  A
// tile written by DMA is published by its issuing wave waiting for it
// (s_waitcnt vmcnt) before the barrier.  The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt(63) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until this wave's outstanding vector-memory operations (including
// global->LDS DMA) have completed: s_waitcnt vmcnt(0).
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Pack C-layout values acc[ci*KPL .. ci*KPL+KPL) into an MFMA fragment.
template <typename T> __device__ inline typename Elt<T>::Frag pack_frag(const float* v);
template <> __device__ inline bf16x8 pack_frag<bf16>(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = static_cast<bf16>(v[j]);
  return r;
}
template <> __device__ inline float pack_frag<float>(const float* v) { return v[0]; }

// Store the KPL values of fragment f (C-layout rows c_row(ci*KPL + j, hh) of a
// 32-row tile) into one row of a k-major LDS buffer (`row` points at the
// tile's first row): bf16 as two 8-byte runs of 4 consecutive rows.
template <typename T> __device__ inline void store_crow_run(T* row, int ci, int hh, typename Elt<T>::Frag f);
template <> __device__ inline void store_crow_run<bf16>(bf16* row, int ci, int hh, bf16x8 f) {
  bf16* p = row + 16 * ci + 4 * hh;
  bf16x4 lo, hi;
  lo[0] = f[0]; lo[1] = f[1]; lo[2] = f[2]; lo[3] = f[3];
  hi[0] = f[4]; hi[1] = f[5]; hi[2] = f[6]; hi[3] = f[7];
  *reinterpret_cast<bf16x4*>(p) = lo;
  *reinterpret_cast<bf16x4*>(p + 8) = hi;
}
template <> __device__ inline void store_crow_run<float>(float* row, int ci, int hh, float f) {
  row[c_row(ci, hh)] = f;
}

template <typename T> __device__ inline T to_elt(float x) { return static_cast<T>(x); }

// Combine the two 32-lane halves of a wave64 lane by lane: lane l gets
// op(x[l mod 32], x[l mod 32 + 32]).  v_permlane32_swap exchanges 32 lanes
// between its two register operands; with x in both, one result holds the
// lower half twice and the other the upper half twice, so a symmetric op of
// the two results needs no lane select (and no LDS round trip, unlike a
// ds_bpermute shuffle).
__device__ inline float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace bdlm
