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

// Whether key tile [k0, k0 + N) leaves the range [flo, fhi) that every row of
// a query tile sees (then its elements are tested against each row's range).
__host__ __device__ inline bool key_tile_partial(int k0, int N, int flo, int fhi) {
  return !(k0 >= flo && k0 + N <= fhi);
}
// The same, or a short query tile (rows [r0, r1) with rows past the stream end).
__host__ __device__ inline bool qmajor_tile_masked(int k0, int N, int flo, int fhi, int r0, int r1, int M) {
  return key_tile_partial(k0, N, flo, fhi) || (r1 - r0 < M);
}

// Iteration order of a key-major backward workgroup (keys [k0, k1) of array
// a): query tiles of M rows descending; at each tile position the (up to two)
// query streams that see the keys, then the q heads of the GQA group, so the
// workgroups of one kv head sweep the same query tiles together.
struct BwdOrder {
  int s0, s1, thi0, thi1, inter, tb, slow, nboth, n0, total;

  __host__ __device__ inline void init(const Problem& p, int a, int ns0, int k0, int k1, int M) {
    int tlo0 = 0, tlo1 = 0, nseg = 0;
    s0 = s1 = thi0 = thi1 = 0;
    for (int s = (a == 0 ? ns0 : 1); s < 2; ++s) {
      if (p.rows[s] == 0) continue;
      int rlo, rhi;
      query_span(p, s, a, k0, k1, rlo, rhi);
      if (rlo >= rhi) continue;
      if (nseg == 0) { s0 = s; tlo0 = rlo / M; thi0 = (rhi - 1) / M; }
      else { s1 = s; tlo1 = rlo / M; thi1 = (rhi - 1) / M; }
      ++nseg;
    }
    const int G = p.group;
    inter = (nseg == 2 && thi0 == thi1) ? 1 : 0;
    tb = inter ? (tlo0 > tlo1 ? tlo0 : tlo1) : 0;
    slow = tlo0 <= tlo1 ? s0 : s1;
    nboth = inter ? (thi0 - tb + 1) * 2 * G : 0;
    n0 = nseg > 0 ? (thi0 - tlo0 + 1) * G : 0;
    total = inter ? nboth + (tb - (tlo0 < tlo1 ? tlo0 : tlo1)) * G
                  : n0 + (nseg > 1 ? (thi1 - tlo1 + 1) * G : 0);
  }

  // Stream s, query tile t and head-in-group hg of iteration it.
  __host__ __device__ inline void decode(const Problem& p, int it, int& s, int& t, int& hg) const {
    if (inter) {
      if (it < nboth) {
        const int u = div_g(p, it);
        t = thi0 - (u >> 1);
        s = (u & 1) ? s1 : s0;
        hg = mod_g(p, it);
      } else {
        const int r = it - nboth;
        t = tb - 1 - div_g(p, r);
        s = slow;
        hg = mod_g(p, r);
      }
    } else if (it < n0) {
      t = thi0 - div_g(p, it);
      s = s0;
      hg = mod_g(p, it);
    } else {
      const int r = it - n0;
      t = thi1 - div_g(p, r);
      s = s1;
      hg = mod_g(p, r);
    }
  }
};

// Packed state of key-major iteration it: query tile | stream << 19 |
// element-mask flag << 20 | head-in-group << 21.  The flag is set when the key
// tile [k0, k0 + N) is not inside the range every row of the query tile sees,
// or the query tile is short (rows past the stream end).
__host__ __device__ inline unsigned bwd_entry(const Problem& p, const BwdOrder& o, int a, int k0, int N, int M,
                                              int it) {
  int s, t, hg;
  o.decode(p, it, s, t, hg);
  const int q0 = t * M;
  const int q1 = q0 + M < p.rows[s] ? q0 + M : p.rows[s];
  int klo, khi, flo, fhi;
  tile_ranges(p, s, a, q0, q1, klo, khi, flo, fhi);
  const unsigned m = qmajor_tile_masked(k0, N, flo, fhi, q0, q1, M) ? 1u : 0u;
  return (unsigned)t | ((unsigned)s << 19) | (m << 20) | ((unsigned)hg << 21);
}
__host__ __device__ inline int entry_tile(unsigned e) { return (int)(e & 0x7FFFFu); }
__host__ __device__ inline int entry_stream(unsigned e) { return (int)((e >> 19) & 1u); }
__host__ __device__ inline bool entry_masked(unsigned e) { return (e >> 20) & 1u; }
__host__ __device__ inline int entry_head(unsigned e) { return (int)(e >> 21); }

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
