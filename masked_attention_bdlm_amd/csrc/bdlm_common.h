// Shared definitions of the BDLM attention kernels (gfx950 / CDNA4).
//
// The visibility rule of block diffusion LM attention over [x0 ; xt]
// ("Block Parallelism For Efficient Distributed Long-Context Diffusion Language
// Model Training", abstract): blocks of B tokens, autoregressive across blocks,
// bidirectional inside a corrupted block, clean K/V shared by later blocks.
// Every query row's visible keys form at most two contiguous ranges, one in the
// clean K/V array and one in the corrupted (or rank-local) K/V array, so the
// kernels never test a dense mask: a tile is either inside both ranges of all
// its rows (no mask), outside them (never scheduled), or on a range edge
// (element test against the row's [lo, hi)).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bdlm {

constexpr int kMaxLocalBlocks = 256;
constexpr int kMaxMergeParts = 64;
constexpr int kWave = 64;

// Runtime problem shape, passed by value to every kernel.
struct Problem {
  int batch, L, B, hq, hkv, group, D;
  int bshift;         // log2(B) when B is a power of two, else -1
  int gshift;         // log2(group) when group is a power of two, else -1
  int mode;           // 0 = full [x0 ; xt], 1 = CSBP share (local corrupted blocks)
  int rows[2];        // query rows per stream array: full {L, L}; share {0, n*B}
  int klen[2];        // key rows per key array:      full {L, L}; share {L, n*B}
  int kv_begin, kv_end, own_block;
  int incl;           // share mode: 1 = local blocks are clean queries (prefix includes the block)
  int nlocal;
  int block_ids[kMaxLocalBlocks];
};

// r / B and x / group, with shifts when the divisor is a power of two (the
// branch is uniform across a wave).
__host__ __device__ inline int div_b(const Problem& p, int r) { return p.bshift >= 0 ? (r >> p.bshift) : r / p.B; }
__host__ __device__ inline int div_g(const Problem& p, int x) { return p.gshift >= 0 ? (x >> p.gshift) : x / p.group; }
__host__ __device__ inline int mod_g(const Problem& p, int x) {
  return p.gshift >= 0 ? (x & (p.group - 1)) : x % p.group;
}

// Visible key range [lo, hi) of query row r of stream s (0 clean, 1 corrupted /
// local) inside key array a (0 clean, 1 corrupted / local).  lo and hi are
// non-decreasing in r, which the schedule relies on.
__host__ __device__ inline void row_keys(const Problem& p, int s, int r, int a, int& lo, int& hi) {
  if (p.mode == 0) {
    const int b = div_b(p, r);
    if (s == 0) {            // clean query: clean blocks <= b
      lo = 0;
      hi = (a == 0) ? (b + 1) * p.B : 0;
    } else if (a == 0) {     // corrupted query, clean keys: blocks < b
      lo = 0;
      hi = b * p.B;
    } else {                 // corrupted query, corrupted keys: its own block
      lo = b * p.B;
      hi = (b + 1) * p.B;
    }
  } else {
    const int i = div_b(p, r);   // local block index
    if (a == 0) {            // clean window cut to the block's clean prefix
      lo = p.kv_begin;       // (strict for corrupted blocks, inclusive for clean ones)
      int e = (p.block_ids[i] + p.incl) * p.B;
      hi = e < p.kv_end ? e : p.kv_end;
      if (hi < lo) hi = lo;
    } else if (p.own_block) {
      lo = i * p.B;
      hi = lo + p.B;
    } else {
      lo = hi = 0;
    }
  }
  if (hi <= lo) lo = hi = 0;   // empty range
}

// Rows [r_lo, r_hi) of stream s that see at least one key of [k0, k1) in key
// array a.  Binary search over blocks (ranges are constant inside a block and
// non-decreasing across blocks).
__host__ __device__ inline void query_span(const Problem& p, int s, int a, int k0, int k1,
                                           int& r_lo, int& r_hi) {
  const int nb = div_b(p, p.rows[s]);
  int lo, hi;
  // first block whose range ends after k0
  int x = 0, y = nb;
  while (x < y) {
    int m = (x + y) >> 1;
    row_keys(p, s, m * p.B, a, lo, hi);
    if (hi > k0) y = m; else x = m + 1;
  }
  const int ja = x;
  // first block (>= ja) whose range starts at or after k1, or is empty-and-after
  x = ja; y = nb;
  while (x < y) {
    int m = (x + y) >> 1;
    row_keys(p, s, m * p.B, a, lo, hi);
    if (hi > lo && lo < k1) x = m + 1; else y = m;
  }
  r_lo = ja * p.B;
  r_hi = x * p.B;
  if (r_hi < r_lo) r_hi = r_lo;
}

// Range of keys of array `a` seen by any valid row of [r0, r1) (stream s), and
// the range [flo, fhi) seen by every row (empty rows make it empty).
__host__ __device__ inline void tile_ranges(const Problem& p, int s, int a, int r0, int r1,
                                   int& klo, int& khi, int& flo, int& fhi) {
  klo = 0x7fffffff; khi = 0; flo = 0; fhi = 0x7fffffff;
  for (int bb = div_b(p, r0); bb * p.B < r1; ++bb) {
    int lo, hi;
    row_keys(p, s, bb * p.B, a, lo, hi);
    if (hi > lo) { klo = klo < lo ? klo : lo; khi = khi > hi ? khi : hi; }
    flo = flo > lo ? flo : lo;
    fhi = fhi < hi ? fhi : hi;
  }
  if (fhi < flo) fhi = flo;
}

// Key row of C-layout element i (0..15) held by lane half hh in a 32x32 MFMA
// output tile: rows 8*(i/4) + 4*hh + (i%4).
__host__ __device__ inline int c_row(int i, int hh) { return ((i >> 2) << 3) + (hh << 2) + (i & 3); }

// Map a linear work-item order onto workgroup ids so that items that share K/V
// (same batch and kv head) run on the same XCD: consecutive workgroup ids are
// dispatched round-robin over the 8 XCDs, each with its own L2.
struct XcdMap {
  int nbg;        // (batch, kv-head) groups
  int per_bg;     // items per group
  int by_xcd;     // 1 if nbg % 8 == 0
  __host__ __device__ void decode(int wg, int& bg, int& item) const {
    if (by_xcd) {
      const int xcd = wg & 7, slot = wg >> 3;
      const int groups = nbg >> 3;            // groups per XCD
      item = slot / groups;                   // heavy items first on every XCD
      bg = xcd * groups + slot % groups;
    } else {
      item = wg / nbg;
      bg = wg % nbg;
    }
  }
};

}  // namespace bdlm
