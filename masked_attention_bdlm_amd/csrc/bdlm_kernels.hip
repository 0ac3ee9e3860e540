// HIP kernels of BDLM masked attention for gfx950 (CDNA4).
//
// Forward: one workgroup (4 waves) per (batch, q-head, stream, 128-row q tile).
// Each wave owns 32 query rows and computes S^T = K Q^T with the rows of K as
// the MFMA A operand, so a lane's accumulator values all belong to ONE query:
// the online softmax (max, exp2, sum, rescale) is lane-local except one swap
// between the two lane halves.  P^T then feeds O^T += V^T P^T directly from
// registers (its k order is the C-layout row order, which the V^T fragment
// loads reproduce), so P never touches LDS.  K and V tiles are staged
// row-major in LDS; V^T fragments are read with the gfx950 LDS transpose
// load.  Only key tiles inside a row's visible ranges are visited; tiles on a
// range edge test each element against [lo, hi).
//
// Backward (stored-LSE recompute, "dK/dV accumulated per key tile"), two
// kernels after a row pass that forms D = rowsum(dO * O) and LSE * log2(e):
//  - dK/dV, key-major: one workgroup per (batch, kv-head, key array, 128-key
//    tile); each key's K, V and dK, dV accumulators stay in registers while
//    the workgroup sweeps the visible query tiles of every q head of the GQA
//    group.  Producer waves compute S, dP, P and dS; consumer waves accumulate
//    dV += P^T dO and dK += dS^T Q with dO / Q read transposed out of LDS.
//  - dQ, query-major (the forward's decomposition): per key tile it recomputes
//    S^T and dP^T and accumulates dQ^T += K^T dS^T in registers.
// Every output element is written once by one lane: no atomics.

#include <hip/hip_runtime.h>

#include "bdlm_common.h"
#include "bdlm_device.h"
#include "bdlm_kernels.h"

namespace bdlm {

// ------------------------------------------------------------------ staging
// Copy rows [k0, k0+NR) of a [rows, heads, D] array (row stride `rs` elements,
// pointer already at the head) into LDS.  Rows >= kmax are zero-filled.
template <typename T, int NR, int D, int ST>
__device__ inline void stage_rows(T* lds, const T* base, int64_t rs, int k0, int kmax, int tid) {
  constexpr int VEC = Elt<T>::VEC;
  constexpr int VPR = D / VEC;                    // 16-byte vectors per row
  constexpr int NV = NR * VPR;
#pragma unroll
  for (int j = 0; j < (NV + 255) / 256; ++j) {
    const int vi = tid + 256 * j;
    if (NV % 256 == 0 || vi < NV) {
      const int row = vi / VPR, col = (vi % VPR) * VEC;
      const int k = k0 + row;
      Vec16 v = (k < kmax) ? ld16(base + (int64_t)k * rs + col) : zero16();
      st16(lds + row * ST + col, v);
    }
  }
}

// Copy rows [k0, k0+NR) transposed into LDS: lds[d * ST + row].  Each thread
// reads RPT consecutive rows x VEC columns and writes VEC runs of RPT elements.
template <typename T, int NR, int D, int ST>
__device__ inline void stage_rows_t(T* lds, const T* base, int64_t rs, int k0, int kmax, int tid) {
  constexpr int VEC = Elt<T>::VEC;
  constexpr int RPT = NR * D / (256 * VEC);       // rows per thread
  static_assert(RPT >= 1 && NR * D == 256 * VEC * RPT, "tile/thread mismatch");
  constexpr int RG = NR / RPT;                    // row groups
  const int rg = tid % RG, dc = tid / RG;
  const int col = dc * VEC;
  T vals[RPT][VEC];
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int k = k0 + rg * RPT + j;
    Vec16 v = (k < kmax) ? ld16(base + (int64_t)k * rs + col) : zero16();
#pragma unroll
    for (int e = 0; e < VEC; ++e) vals[j][e] = elem_of<T>(v, e);
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    T* dst = lds + (col + e) * ST + rg * RPT;
#pragma unroll
    for (int j = 0; j < RPT; ++j) dst[j] = vals[j][e];
  }
}

// Copy rows [k0, k0+NR) into LDS twice from one global read: row-major
// (lds_r[row * ST + d]) and transposed (lds_t[d * STT + row]).
template <typename T, int NR, int D, int ST, int STT>
__device__ inline void stage_rows_dual(T* lds_r, T* lds_t, const T* base, int64_t rs, int k0, int kmax,
                                       int tid) {
  constexpr int VEC = Elt<T>::VEC;
  constexpr int RPT = NR * D / (256 * VEC);
  static_assert(RPT >= 1 && NR * D == 256 * VEC * RPT, "tile/thread mismatch");
  constexpr int RG = NR / RPT;
  const int rg = tid % RG, dc = tid / RG;
  const int col = dc * VEC;
  Vec16 v[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int k = k0 + rg * RPT + j;
    v[j] = (k < kmax) ? ld16(base + (int64_t)k * rs + col) : zero16();
  }
#pragma unroll
  for (int j = 0; j < RPT; ++j) st16(lds_r + (rg * RPT + j) * ST + col, v[j]);
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    T* dst = lds_t + (col + e) * STT + rg * RPT;
#pragma unroll
    for (int j = 0; j < RPT; ++j) dst[j] = elem_of<T>(v[j], e);
  }
}

// ================================================================= forward
template <typename T, int D, bool OUT_F32>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void fwd_kernel(FwdArgs args) {
  using E = Elt<T>;
  using Frag = typename E::Frag;
  constexpr int M = 128, N = 64;
  constexpr int KPL = E::KPL, KC = 2 * KPL;
  constexpr int DCH = D / KC;          // k-chunks over head_dim
  constexpr int CPS = 32 / KC;         // k-chunks per 32-key subtile
  // K and V tiles, double-buffered, filled by global->LDS DMA (swizzled rows)
  __shared__ __attribute__((aligned(16))) T kv_lds[2][2][N * D];

  const Problem& p = args.p;
  int bg, item;
  args.map.decode(blockIdx.x, bg, item);
  const int b = bg / p.hkv, g = bg % p.hkv;
  const int hg = item % p.group;
  const int rest = item / p.group;
  const int nstr = 2 - args.ns0;
  const int s = args.ns0 + rest % nstr;
  const int t = args.nqt[s] - 1 - rest / nstr;
  const int h = g * p.group + hg;
  const int R = p.rows[s];
  const int r0 = t * M;
  const int r1 = min(r0 + M, R);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform per wave
  const int ln = lane & 31, hh = lane >> 5;
  const int r = r0 + 32 * w + ln;
  const bool valid = r < r1;

  // Q^T fragments (MFMA B operand): column = this lane's query.
  Frag qf[DCH];
  {
    const T* qrow = reinterpret_cast<const T*>(args.q[s]) +
                    ((int64_t)b * R + (valid ? r : r0)) * p.hq * D + (int64_t)h * D;
#pragma unroll
    for (int c = 0; c < DCH; ++c) {
      qf[c] = ld_frag<T>(qrow + c * KC + hh * KPL);
      if (!valid) qf[c] = Frag{};
    }
  }

  // key tiles: array 0 (clean) then array 1 (corrupted / local)
  int klo[2], khi[2], flo[2], fhi[2], nt[2], lo[2], hi[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    tile_ranges(p, s, a, r0, r1, klo[a], khi[a], flo[a], fhi[a]);
    nt[a] = klo[a] < khi[a] ? (khi[a] - klo[a] + N - 1) / N : 0;
    if (valid) row_keys(p, s, r, a, lo[a], hi[a]); else lo[a] = hi[a] = 0;
  }
  const int total = nt[0] + nt[1];
  const int64_t rs = (int64_t)p.hkv * D;
  const T* kb[2];
  const T* vb[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    kb[a] = reinterpret_cast<const T*>(args.k[a]) + (int64_t)b * p.klen[a] * rs + (int64_t)g * D;
    vb[a] = reinterpret_cast<const T*>(args.v[a]) + (int64_t)b * p.klen[a] * rs + (int64_t)g * D;
  }
  if (total > 0) {
    const int a0 = nt[0] > 0 ? 0 : 1;
    dma_rows<T, N, D>(kv_lds[0][0], kb[a0], rs, klo[a0], khi[a0], w, lane);
    dma_rows<T, N, D>(kv_lds[0][1], vb[a0], rs, klo[a0], khi[a0], w, lane);
  }

  // bf16: per-lane fragment offsets, computed once (see bf16_frag_offsets)
  constexpr bool OFFS = sizeof(T) == 2;
  uint32_t offA[OFFS ? D / 16 : 1], offT[OFFS ? D / 16 : 1];
  if constexpr (OFFS) bf16_frag_offsets<D>(lane, offA, offT);

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};

  for (int it = 0; it < total; ++it) {
    const int a = it < nt[0] ? 0 : 1;
    const int k0 = klo[a] + (it - (a ? nt[0] : 0)) * N;
    wait_vmem();
    __syncthreads();   // tile `it` is in buffer it&1; buffer (it+1)&1 is free
    const T* k_lds = kv_lds[it & 1][0];
    const T* v_lds = kv_lds[it & 1][1];
    const bool need_mask = key_tile_partial(k0, N, flo[a], fhi[a]);
    const int mylo = a ? lo[1] : lo[0], myhi = a ? hi[1] : hi[0];

    // S^T[key][query] for the N keys of the tile; K fragments are read in
    // batches of 4 k-chunks one batch ahead of the MFMAs that use them.
    f32x16 sacc[N / 32];
    {
      constexpr int BT = DCH < 4 ? DCH : 4;
      constexpr int NB = (N / 32) * (DCH / BT);       // batches over (sub, chunk)
      Frag ka[2][BT];
#pragma unroll
      for (int c = 0; c < BT; ++c) {
        if constexpr (OFFS) ka[0][c] = ld_fragA(reinterpret_cast<const char*>(k_lds), offA[c], 0);
        else ka[0][c] = ld_frag_s<T, D>(k_lds, ln, c * KC + hh * KPL);
      }
#pragma unroll
      for (int sub = 0; sub < N / 32; ++sub) sacc[sub] = f32x16{};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (nb + 1 < NB) {
          const int sub2 = (nb + 1) / (DCH / BT), cb2 = (nb + 1) % (DCH / BT);
#pragma unroll
          for (int c = 0; c < BT; ++c) {
            if constexpr (OFFS)
              ka[(nb + 1) & 1][c] = ld_fragA(reinterpret_cast<const char*>(k_lds), offA[OFFS ? cb2 * BT + c : 0],
                                             sub2 * 32 * D * 2);
            else
              ka[(nb + 1) & 1][c] = ld_frag_s<T, D>(k_lds, sub2 * 32 + ln, (cb2 * BT + c) * KC + hh * KPL);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        const int sub = nb / (DCH / BT), cb = nb % (DCH / BT);
#pragma unroll
        for (int c = 0; c < BT; ++c) sacc[sub] = E::mma(ka[nb & 1][c], qf[cb * BT + c], sacc[sub]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Next tile's DMA, issued behind the S^T MFMAs: a wave stalls while the
    // memory pipeline accepts its DMA instructions, which then overlaps the
    // matrix core working through those MFMAs.
    if (it + 1 < total) {
      const int a2 = it + 1 < nt[0] ? 0 : 1;
      const int k02 = klo[a2] + (it + 1 - (a2 ? nt[0] : 0)) * N;
      dma_rows<T, N, D>(kv_lds[(it + 1) & 1][0], kb[a2], rs, k02, khi[a2], w, lane);
      dma_rows<T, N, D>(kv_lds[(it + 1) & 1][1], vb[a2], rs, k02, khi[a2], w, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    // The V^T fragments of the first two d-tiles do not depend on P: read
    // them now, so that their latency hides behind the softmax.
    Frag va[3][N / KC];
    auto rd_va = [&](int dt) {
#pragma unroll
      for (int cc = 0; cc < N / KC; ++cc) {
        if constexpr (OFFS)
          va[dt % 3][cc] = ld_fragT(reinterpret_cast<const char*>(v_lds), offT, OFFS ? dt : 0,
                                    ((cc / CPS) * 32 + 16 * (cc % CPS)) * D * 2);
        else
          va[dt % 3][cc] = ld_frag_kcrow_s<T, D>(v_lds, (cc / CPS) * 32, cc % CPS, lane, dt * 32);
      }
    };
    rd_va(0);
    if (D / 32 > 1) rd_va(1);

    // Edge tiles only (one uniform branch): keys outside the row's range.
    if (need_mask) {
#pragma unroll
      for (int sub = 0; sub < N / 32; ++sub) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = k0 + sub * 32 + c_row(i, hh);
          if (kk < mylo || kk >= myhi) sacc[sub][i] = -INFINITY;
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < N / 32; ++sub) {
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[sub][i]);
    }
    mx = halves_max(mx);
    // Lazy rescaling: O and l stay relative to the reference m_run until some
    // row's max exceeds it by more than 8 (log2 units); the exponentials are
    // then at most 2^8, harmless for fp32 sums and bf16 operands, and the
    // final O = acc / l and LSE = m_run + log2 l are unchanged.  The rescale
    // is skipped for the whole wave when no row needs it.
    const float m_new = fmaxf(m_run, mx * args.scale_log2);
    const bool grow = m_new > m_run + 8.f;
    if (__ballot(grow)) {
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;   // 0 while m_run = -inf
      if (grow) m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

    float pv[N / 32][16];
#pragma unroll
    for (int sub = 0; sub < N / 32; ++sub) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(sacc[sub][i] * args.scale_log2 - m_use);
        pv[sub][i] = e;
        l_run += e;
      }
    }

    // O^T[d][query] += V^T[d][key] P^T[key][query]; the V^T fragments of each
    // d-tile are read two d-tiles ahead of its MFMAs (3-slot ring)
    Frag pb[N / KC];
#pragma unroll
    for (int cc = 0; cc < N / KC; ++cc) pb[cc] = pack_frag<T>(&pv[cc / CPS][(cc % CPS) * KPL]);
    {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        if (dt + 2 < D / 32) rd_va(dt + 2);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int cc = 0; cc < N / KC; ++cc) oacc[dt] = E::mma(va[dt % 3][cc], pb[cc], oacc[dt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  const float l_tot = halves_sum(l_run);
  if (valid) {
    float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float lse_out = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    using OT = typename std::conditional<OUT_F32, float, T>::type;
    OT* orow = reinterpret_cast<OT*>(args.o[s]) + ((int64_t)b * R + r) * p.hq * D + (int64_t)h * D;
    float* lrow = &args.lse[s][((int64_t)b * p.hq + h) * R + r];
    bool write = true;
    float w_old = 0.f;
    if constexpr (OUT_F32) {
      // Running merge of this call's partial into the held one (fp32 O): both
      // are normalised attention outputs over disjoint key sets, so
      // LSE = logsumexp(LSE_old, LSE_new) and O = sum_j exp(LSE_j - LSE) O_j.
      // A row that sees no key here keeps the held result unchanged.
      if (args.accum) {
        if (l_tot > 0.f) {
          const float lse_old = *lrow;
          const float m = fmaxf(lse_old, lse_out);
          const float a_old = __expf(lse_old - m);   // 0 when nothing is held yet
          const float a_new = __expf(lse_out - m);
          const float sum = a_old + a_new;
          w_old = a_old / sum;
          inv *= a_new / sum;
          lse_out = m + __logf(sum);
        } else {
          write = false;
        }
      }
    }
    if (write) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          OT* dst = orow + dt * 32 + g4 * 8 + hh * 4;
          if constexpr (OUT_F32) {
            if (w_old != 0.f) {   // only while merging into a held result
              const f32x4 old = *reinterpret_cast<const f32x4*>(dst);
#pragma unroll
              for (int j = 0; j < 4; ++j) dst[j] = w_old * old[j] + oacc[dt][g4 * 4 + j] * inv;
              continue;
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) dst[j] = static_cast<OT>(oacc[dt][g4 * 4 + j] * inv);
        }
      }
      if (hh == 0) *lrow = lse_out;
    }
  }
}

// ============================================================ backward: D
// delta[b][h][r] = <dO, O> over head_dim, and lse2[b][h][r] = LSE * log2(e).
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdPreArgs args) {
  constexpr int VEC = Elt<T>::VEC;
  constexpr int LPR = D / VEC;               // lanes per (row, head)
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t unit = gid / LPR;            // (b, r, h) triple
  const int part = (int)(gid % LPR);
  const int s = args.stream;
  const int64_t nunits = (int64_t)args.batch * args.rows * args.hq;
  const bool ok = unit < nunits;
  float acc = 0.f;
  int64_t u = ok ? unit : 0;
  const T* o = reinterpret_cast<const T*>(args.o) + u * D + part * VEC;
  const T* d = reinterpret_cast<const T*>(args.dout) + u * D + part * VEC;
  if (ok) {
    Vec16 vo = ld16(o), vd = ld16(d);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc += (float)elem_of<T>(vo, e) * (float)elem_of<T>(vd, e);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (ok && part == 0) {
    const int h = (int)(u % args.hq);
    const int64_t br = u / args.hq;
    const int r = (int)(br % args.rows);
    const int bb = (int)(br / args.rows);
    const int64_t ri = ((int64_t)bb * args.hq + h) * args.rows + r;
    args.delta[ri] = acc;
    args.lse2[ri] = args.lse[ri] * kLog2e;
  }
  (void)s;
}

// ==================================================== backward: dK/dV kernel
// Key-major dK/dV: one workgroup per (batch, kv-head, key array, 128-key
// tile); wave w owns 32 keys and keeps K_w, V_w (MFMA B operands) and its dK_w,
// dV_w accumulators in registers while it sweeps the visible 64-row query
// tiles of every q head of the GQA group.  S = Q K_w^T and dP = dO V_w^T put
// the key on the lane, so P and dS are directly the A operands of
// dV += P^T dO and dK += dS^T Q; their dO / Q operands are read transposed out
// of the row-major tiles.  Q/dO tiles and the per-row LSE / D are
// double-buffered in LDS and filled by global->LDS DMA one iteration ahead.
template <typename T, int D>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BwdArgs args) {
  using E = Elt<T>;
  using Frag = typename E::Frag;
  constexpr int N = 128;                                   // keys per workgroup
  constexpr int M = sizeof(T) == 2 ? 64 : 32;              // query rows per iteration
  constexpr int QS = M / 32;
  constexpr int KPL = E::KPL, KC = 2 * KPL;
  constexpr int DCH = D / KC;
  constexpr int CPS = 32 / KC;
  // One LDS object (a kernel with several makes the compiler wait for every
  // in-flight DMA into an object before any read of it, which would serialise
  // the double buffer): [buffer][Q, dO] tiles, then [buffer][LSE, D] rows.
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * M * D * sizeof(T) + 2 * 2 * 64 * sizeof(float)];
  T (*qd_lds)[2][M * D] = reinterpret_cast<T (*)[2][M * D]>(smem);
  float (*row_l)[2][64] = reinterpret_cast<float (*)[2][64]>(smem + 2 * 2 * M * D * sizeof(T));

  const Problem& p = args.p;
  // Per-stream values read once: indexing the argument block with the
  // iteration's stream number would re-load them from memory every iteration.
  const int rows0 = pin_sgpr(p.rows[0]), rows1 = pin_sgpr(p.rows[1]);
  const T* const q_0 = pin_sgpr(reinterpret_cast<const T*>(args.q[0]));
  const T* const q_1 = pin_sgpr(reinterpret_cast<const T*>(args.q[1]));
  const T* const do_0 = pin_sgpr(reinterpret_cast<const T*>(args.dout[0]));
  const T* const do_1 = pin_sgpr(reinterpret_cast<const T*>(args.dout[1]));
  const float* const l2_0 = pin_sgpr(args.lse2[0]);
  const float* const l2_1 = pin_sgpr(args.lse2[1]);
  const float* const dl_0 = pin_sgpr(args.delta[0]);
  const float* const dl_1 = pin_sgpr(args.delta[1]);
  int bg, item;
  args.map.decode(blockIdx.x, bg, item);
  const int b = bg / p.hkv, g = bg % p.hkv;
  const int a = item < args.nkt[0] ? 0 : 1;
  const int j = a == 0 ? item : item - args.nkt[0];
  const int k0 = args.kbase[a] + j * N;
  const int k1 = min(k0 + N, args.kend[a]);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform per wave
  const int ln = lane & 31, hh = lane >> 5;
  const int kk = k0 + 32 * w + ln;           // this lane's key (MFMA column)
  const bool kvalid = kk < k1;

  const int64_t krs = (int64_t)p.hkv * D;
  const T* kbase = reinterpret_cast<const T*>(args.k[a]) + (int64_t)b * p.klen[a] * krs + (int64_t)g * D;
  const T* vbase = reinterpret_cast<const T*>(args.v[a]) + (int64_t)b * p.klen[a] * krs + (int64_t)g * D;

  Frag kf[DCH], vf[DCH];
#pragma unroll
  for (int c = 0; c < DCH; ++c) {
    const int64_t off = (int64_t)(kvalid ? kk : k0) * krs + c * KC + hh * KPL;
    kf[c] = ld_frag<T>(kbase + off);
    vf[c] = ld_frag<T>(vbase + off);
    if (!kvalid) { kf[c] = Frag{}; vf[c] = Frag{}; }
  }

  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) { dkacc[dt] = f32x16{}; dvacc[dt] = f32x16{}; }

  BwdOrder ord;
  ord.init(p, a, args.ns0, k0, k1, M);
  const int total = ord.total;
  const int G = p.group;
  const int64_t qrs = (int64_t)p.hq * D;

  // Per-iteration state (bwd_entry), decoded 64 iterations at a time (one per
  // lane, as vector code).  An iteration then costs two lane reads instead of
  // the branchy scalar decode, which all waves of the CU would otherwise run
  // on the shared scalar unit.
#define DKDV_ENTRY(idx, out) out = bwd_entry(p, ord, a, k0, N, M, (idx))
  unsigned ent0 = 0, ent1 = 0;
  int ent_base = 0;
  if (total > 0) {
    DKDV_ENTRY(min(lane, total - 1), ent0);
    DKDV_ENTRY(min(64 + lane, total - 1), ent1);
  }
#define DKDV_GET(x)                                                                \
  ((x) - ent_base < 64 ? (unsigned)__builtin_amdgcn_readlane((int)ent0, (x) - ent_base) \
                       : (unsigned)__builtin_amdgcn_readlane((int)ent1, (x) - ent_base - 64))

  // DMA of iteration `it`'s Q/dO tiles and row data into buffer `buf`; rows past
  // the stream end re-read its last row and are masked in the main block.
#define DKDV_ISSUE(it, buf)                                                                      \
  do {                                                                                           \
    const unsigned e_ = DKDV_GET(it);                                                            \
    const int s_ = (int)((e_ >> 19) & 1u);                                                       \
    const int q0_ = (int)(e_ & 0x7FFFFu) * M;                                                    \
    const int h_ = g * G + (int)(e_ >> 21);                                                      \
    const int R_ = s_ ? rows1 : rows0;                                                                   \
    const int q1_ = min(q0_ + M, R_);                                                            \
    const int64_t hb_ = (int64_t)b * R_ * qrs + (int64_t)h_ * D;                                 \
    dma_rows<T, M, D>(qd_lds[buf][0], (s_ ? q_1 : q_0) + hb_, qrs, q0_, q1_,                    \
                      w, lane);                                                                  \
    dma_rows<T, M, D>(qd_lds[buf][1], (s_ ? do_1 : do_0) + hb_, qrs, q0_,                        \
                      q1_, w, lane);                                                          \
    if (w < 2) {                                                                                 \
      const int64_t ri_ = ((int64_t)b * p.hq + h_) * R_ + min(q0_ + lane, q1_ - 1);              \
      const float* src_ = (w == 0 ? (s_ ? l2_1 : l2_0) : (s_ ? dl_1 : dl_0)) + ri_;                \
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src_,      \
                                       (__attribute__((address_space(3))) void*)(row_l[buf][w]), 4, 0, 0); \
    }                                                                                            \
  } while (0)

  if (total > 0) DKDV_ISSUE(0, 0);
  const float sl2 = args.scale_log2;
  for (int it = 0; it < total; ++it) {
    const int cur = it & 1;
    if (it - ent_base == 64) {   // next 64 decoded iterations
      ent0 = ent1;
      ent_base += 64;
      DKDV_ENTRY(min(ent_base + 64 + lane, total - 1), ent1);
    }
    const unsigned e = DKDV_GET(it);
    const int s = (int)((e >> 19) & 1u);
    const int q0 = (int)(e & 0x7FFFFu) * M;
    const int R = s ? rows1 : rows0;
    const int q1 = min(q0 + M, R);
    const bool need_mask = (e >> 20) & 1u;
    wait_vmem();
    __syncthreads();   // buffer `cur` holds iteration it; buffer cur^1 is free
    if (it + 1 < total) DKDV_ISSUE(it + 1, cur ^ 1);
    const T* qt = qd_lds[cur][0];
    const T* dot = qd_lds[cur][1];
    const float* lse_r = row_l[cur][0];
    const float* dl_r = row_l[cur][1];

    // One 32-row query sub-tile at a time: S = Q K_w^T and dP = dO V_w^T
    // (rows = queries, column = this lane's key), then P and dS, then their
    // contributions to dV_w and dK_w.
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      {
        constexpr int BT = DCH < 4 ? DCH : 4;
        Frag qa[2][BT], da[2][BT];
#pragma unroll
        for (int c = 0; c < BT; ++c) {
          qa[0][c] = ld_frag_s<T, D>(qt, qs * 32 + ln, c * KC + hh * KPL);
          da[0][c] = ld_frag_s<T, D>(dot, qs * 32 + ln, c * KC + hh * KPL);
        }
#pragma unroll
        for (int cb = 0; cb < DCH / BT; ++cb) {
          if (cb + 1 < DCH / BT) {
#pragma unroll
            for (int c = 0; c < BT; ++c) {
              const int cc = (cb + 1) * BT + c;
              qa[(cb + 1) & 1][c] = ld_frag_s<T, D>(qt, qs * 32 + ln, cc * KC + hh * KPL);
              da[(cb + 1) & 1][c] = ld_frag_s<T, D>(dot, qs * 32 + ln, cc * KC + hh * KPL);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int c = 0; c < BT; ++c) {
            sacc = E::mma(qa[cb & 1][c], kf[cb * BT + c], sacc);
            pacc = E::mma(da[cb & 1][c], vf[cb * BT + c], pacc);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // P = exp(S - LSE), dS = P (dP - D); masked pairs get P = 0.  Both are
      // packed into MFMA fragments right away (k = queries in C-row order).
      float pe[16], de[16];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int rr0 = qs * 32 + c_row(4 * i4, hh);      // 4 consecutive rows
        // one 16-byte vector read each (a typed vector load keeps the alias
        // information that lets the compiler skip waiting for in-flight DMA)
        const f32x4 lv = *reinterpret_cast<const f32x4*>(lse_r + rr0);
        const f32x4 dv = *reinterpret_cast<const f32x4*>(dl_r + rr0);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int i = 4 * i4 + jj;
          const float e = fast_exp2(sacc[i] * sl2 - lv[jj]);
          pe[i] = e;
          de[i] = dv[jj];
        }
      }
      if (need_mask) {   // edge tiles only: visible range of each row, rows past the end masked
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int row = q0 + qs * 32 + c_row(4 * i4, hh);   // 4 rows of one block
          int lo = 0, hi = 0;
          row_keys(p, s, min(row, R - 1), a, lo, hi);
          const bool kin = kk >= lo && kk < hi;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            if (!kin || row + jj >= q1) pe[4 * i4 + jj] = 0.f;
        }
      }
      Frag pfr[CPS], sfr[CPS];
#pragma unroll
      for (int ci = 0; ci < CPS; ++ci) {
        float d8[KPL];
#pragma unroll
        for (int jj = 0; jj < KPL; ++jj) {
          const int i = ci * KPL + jj;
          d8[jj] = pe[i] * (pacc[i] - de[i]);
        }
        pfr[ci] = pack_frag<T>(&pe[ci * KPL]);
        sfr[ci] = pack_frag<T>(d8);
      }
      // dV_w += P^T dO ; dK_w += dS^T Q  (the dO / Q fragments are read
      // transposed out of the row-major tiles)
      {
        Frag ob[2][CPS], qb2[2][CPS];
#pragma unroll
        for (int ci = 0; ci < CPS; ++ci) {
          ob[0][ci] = ld_frag_kcrow_s<T, D>(dot, qs * 32, ci, lane, 0);
          qb2[0][ci] = ld_frag_kcrow_s<T, D>(qt, qs * 32, ci, lane, 0);
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          if (dt + 1 < D / 32) {
#pragma unroll
            for (int ci = 0; ci < CPS; ++ci) {
              ob[(dt + 1) & 1][ci] = ld_frag_kcrow_s<T, D>(dot, qs * 32, ci, lane, (dt + 1) * 32);
              qb2[(dt + 1) & 1][ci] = ld_frag_kcrow_s<T, D>(qt, qs * 32, ci, lane, (dt + 1) * 32);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ci = 0; ci < CPS; ++ci) {
            dvacc[dt] = E::mma(pfr[ci], ob[dt & 1][ci], dvacc[dt]);
            dkacc[dt] = E::mma(sfr[ci], qb2[dt & 1][ci], dkacc[dt]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
#undef DKDV_ISSUE
#undef DKDV_GET
#undef DKDV_ENTRY

  // dK = scale * sum dS^T Q, dV = sum P^T dO for the wave's 32 keys.
  T* dkb = reinterpret_cast<T*>(args.dk[a]) + (int64_t)b * p.klen[a] * krs + (int64_t)g * D;
  T* dvb = reinterpret_cast<T*>(args.dv[a]) + (int64_t)b * p.klen[a] * krs + (int64_t)g * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = k0 + 32 * w + c_row(i, hh);
      if (key < k1) {
        const int64_t off = (int64_t)key * krs + dt * 32 + ln;
        dkb[off] = to_elt<T>(dkacc[dt][i] * args.scale);
        dvb[off] = to_elt<T>(dvacc[dt][i]);
      }
    }
  }
}

// ================================= backward: dK/dV kernel, bf16, two roles
// Eight waves, two per SIMD, in four pairs; pair w owns keys k0 + 32w .. +31
// of the workgroup's 128-key tile.  The producer wave (w) keeps K_w, V_w in
// registers and, per 32-row query sub-tile, computes S = Q K_w^T and
// dP = dO V_w^T (MFMA), then P = exp2(S * scale * log2e - LSE * log2e) and
// dS = P (dP - D) (VALU), and hands P and dS, already packed as bf16 MFMA
// operands, to its consumer wave (w + 4) through LDS.  The consumer keeps dK_w
// and dV_w in registers and accumulates dV += P^T dO and dK += dS^T Q with dO
// and Q read transposed out of the tiles.  Step j runs the producers on
// sub-tile j and the consumers on sub-tile j - 1, so on each SIMD one wave's
// exponentials overlap the other's MFMAs; a workgroup barrier ends each step.
// Q/dO tiles with their LSE and D rows are triple-buffered; the consumers'
// global->LDS DMA fills tile i during steps 2i-3 .. 2i-1.
template <int D>
struct DkdvWs {
  static constexpr int M = 64;                         // query rows per tile
  static constexpr int DCH = D / 16;                   // 16-wide k chunks
  static constexpr int DT = D / 32;                    // 32-column blocks
  static constexpr int TILE = M * D * 2;               // one Q or dO tile (bytes)
  static constexpr int BUFB = 2 * TILE + 512;          // Q, dO, LSE*log2e[64], D[64]
  static constexpr int NBUF = 3;
  static constexpr int PDS = NBUF * BUFB;              // P/dS exchange area
  static constexpr int SLOT = 4 * 4 * 1024;            // 4 pairs x {P0, P1, dS0, dS1} x 64 lanes x 16 B
  static constexpr int BYTES = PDS + 2 * SLOT;
};

template <int D>
__global__ __launch_bounds__(512, 1) void dkdv_ws_kernel(BwdArgs args) {
  using L = DkdvWs<D>;
  constexpr int N = 128, M = L::M;
  static_assert(L::BYTES <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

  const Problem& p = args.p;
  const int rows0 = pin_sgpr(p.rows[0]), rows1 = pin_sgpr(p.rows[1]);
  const bf16* const q_0 = pin_sgpr(reinterpret_cast<const bf16*>(args.q[0]));
  const bf16* const q_1 = pin_sgpr(reinterpret_cast<const bf16*>(args.q[1]));
  const bf16* const do_0 = pin_sgpr(reinterpret_cast<const bf16*>(args.dout[0]));
  const bf16* const do_1 = pin_sgpr(reinterpret_cast<const bf16*>(args.dout[1]));
  const float* const l2_0 = pin_sgpr(args.lse2[0]);
  const float* const l2_1 = pin_sgpr(args.lse2[1]);
  const float* const dl_0 = pin_sgpr(args.delta[0]);
  const float* const dl_1 = pin_sgpr(args.delta[1]);
  int bg, item;
  args.map.decode(blockIdx.x, bg, item);
  const int b = bg / p.hkv, g = bg % p.hkv;
  const int a = item < args.nkt[0] ? 0 : 1;
  const int jt = a == 0 ? item : item - args.nkt[0];
  const int k0 = args.kbase[a] + jt * N;
  const int k1 = min(k0 + N, args.kend[a]);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = w & 3;
  const bool producer = w < 4;
  const int ln = lane & 31, hh = lane >> 5;
  const int kk = k0 + 32 * pair + ln;        // this lane's key (MFMA column)
  const bool kvalid = kk < k1;
  const int64_t krs = (int64_t)p.hkv * D;
  const int64_t qrs = (int64_t)p.hq * D;

  BwdOrder ord;
  ord.init(p, a, args.ns0, k0, k1, M);
  const int total = ord.total;
  const int G = p.group;

  // Iteration (tile) i's state (bwd_entry), decoded 64 at a time, one per lane.
  unsigned ent = 0;
  int ent_base = 0;
#define WS_ENTRY(idx, out) out = bwd_entry(p, ord, a, k0, N, M, (idx))
  // entry of tile x; x never decreases between calls of one wave
#define WS_GET(x, out)                                                                           \
  do {                                                                                           \
    if ((x) - ent_base >= 64) {                                                                  \
      ent_base = (x);                                                                            \
      WS_ENTRY(min(ent_base + lane, total - 1), ent);                                            \
    }                                                                                            \
    out = (unsigned)__builtin_amdgcn_readlane((int)ent, (x) - ent_base);                         \
  } while (0)
  if (total > 0) WS_ENTRY(min(lane, total - 1), ent);

  if (producer) {
    // ------------------------------------------------------------ producer
    const bf16* kbase = reinterpret_cast<const bf16*>(args.k[a]) + (int64_t)b * p.klen[a] * krs + (int64_t)g * D;
    const bf16* vbase = reinterpret_cast<const bf16*>(args.v[a]) + (int64_t)b * p.klen[a] * krs + (int64_t)g * D;
    bf16x8 kf[L::DCH], vf[L::DCH];
#pragma unroll
    for (int c = 0; c < L::DCH; ++c) {
      const int64_t off = (int64_t)(kvalid ? kk : k0) * krs + c * 16 + hh * 8;
      kf[c] = ld_frag<bf16>(kbase + off);
      vf[c] = ld_frag<bf16>(vbase + off);
      if (!kvalid) { kf[c] = bf16x8{}; vf[c] = bf16x8{}; }
    }
    uint32_t offA[L::DCH];
#pragma unroll
    for (int c = 0; c < L::DCH; ++c) offA[c] = 2u * (uint32_t)Swz<bf16, D>::idx(ln, (2 * c + hh) * 8);
    const float sl2 = args.scale_log2;
    barrier_lds();                                  // tile 0 has landed
    for (int j = 0; j <= 2 * total; ++j) {
      if (j < 2 * total) {
        const int it = j >> 1, qs = j & 1;
        const char* tb = smem + (it % L::NBUF) * L::BUFB;
        unsigned e;
        WS_GET(it, e);
        // S and dP for rows qs*32 .. +31 (rows = queries, column = this lane's key)
        f32x16 sacc = f32x16{}, pacc = f32x16{};
        // Q / dO fragments read three k-chunks ahead of their MFMAs (4-slot ring)
        bf16x8 qa[4], da[4];
        auto rd = [&](int c) {
          const char* ap = tb + offA[c] + qs * 32 * D * 2;
          qa[c % 4] = *reinterpret_cast<const bf16x8*>(ap);
          da[c % 4] = *reinterpret_cast<const bf16x8*>(ap + L::TILE);
        };
        // The rows' LSE and D values (C-layout rows of this lane) are read in
        // the middle of the MFMA chain, so that they have landed at its end.
        const char* rb = tb + 2 * L::TILE;
        f32x4 lv[4], dv[4];
        auto rd_rows = [&]() {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int rr = qs * 32 + 8 * i4 + 4 * hh;
            lv[i4] = *reinterpret_cast<const f32x4*>(rb + rr * 4);
            dv[i4] = *reinterpret_cast<const f32x4*>(rb + 256 + rr * 4);
          }
        };
        rd(0);
        if (L::DCH > 1) rd(1);
        if (L::DCH > 2) rd(2);
#pragma unroll
        for (int c = 0; c < L::DCH; ++c) {
          if (c + 3 < L::DCH) rd(c + 3);
          if (c == L::DCH / 2 - 1) rd_rows();
          __builtin_amdgcn_sched_barrier(0);
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[c % 4], kf[c], sacc, 0, 0, 0);
          pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[c % 4], vf[c], pacc, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // P and dS in the C layout (k of the consumer's MFMAs = queries)
        float pe[16], de[16];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int i = 4 * i4 + jj;
            const float ex = fast_exp2(__builtin_fmaf(sacc[i], sl2, -lv[i4][jj]));
            pe[i] = ex;
            de[i] = ex * (pacc[i] - dv[i4][jj]);
          }
        }
        if ((e >> 20) & 1u) {   // edge tile: each row's visible keys; rows past the stream end
          const int s = (int)((e >> 19) & 1u);
          const int q0 = (int)(e & 0x7FFFFu) * M;
          const int R = s ? rows1 : rows0;
          const int q1 = min(q0 + M, R);
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int row = q0 + qs * 32 + 8 * i4 + 4 * hh;
            int lo = 0, hi = 0;
            row_keys(p, s, min(row, R - 1), a, lo, hi);
            const bool kin = kk >= lo && kk < hi;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              if (!kin || row + jj >= q1) { pe[4 * i4 + jj] = 0.f; de[4 * i4 + jj] = 0.f; }
          }
        }
        char* pd = smem + L::PDS + (j & 1) * L::SLOT + pair * 4096 + lane * 16;
#pragma unroll
        for (int ci = 0; ci < 2; ++ci) {
          *reinterpret_cast<bf16x8*>(pd + ci * 1024) = pack_frag<bf16>(&pe[8 * ci]);
          *reinterpret_cast<bf16x8*>(pd + 2048 + ci * 1024) = pack_frag<bf16>(&de[8 * ci]);
        }
      }
      barrier_lds();
    }
  } else {
    // ------------------------------------------------------------ consumer
    const int wy = w - 4;
    uint32_t offT[2 * L::DT];
    {
      const int i16 = lane & 15;
#pragma unroll
      for (int dt = 0; dt < L::DT; ++dt) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int r = 4 * hh + 8 * h2 + (i16 >> 2);
          const int col = dt * 32 + 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
          offT[2 * dt + h2] = 2u * (uint32_t)Swz<bf16, D>::idx(r, col);
        }
      }
    }
    f32x16 dkacc[L::DT], dvacc[L::DT];
#pragma unroll
    for (int dt = 0; dt < L::DT; ++dt) { dkacc[dt] = f32x16{}; dvacc[dt] = f32x16{}; }
    // DMA of tile i: 4 Q blocks, 4 dO blocks per wave (+ the LSE / D row for
    // consumers 0 and 1); rows past the stream end re-read its last row.
#define WS_ISSUE(i)                                                                              \
  do {                                                                                           \
    unsigned e_;                                                                                 \
    WS_GET(i, e_);                                                                               \
    const int s_ = (int)((e_ >> 19) & 1u);                                                       \
    const int q0_ = (int)(e_ & 0x7FFFFu) * M;                                                    \
    const int h_ = g * G + (int)(e_ >> 21);                                                      \
    const int R_ = s_ ? rows1 : rows0;                                                           \
    const int q1_ = min(q0_ + M, R_);                                                            \
    const int64_t hb_ = (int64_t)b * R_ * qrs + (int64_t)h_ * D;                                 \
    bf16* tq_ = reinterpret_cast<bf16*>(smem + ((i) % L::NBUF) * L::BUFB);                       \
    dma_rows<bf16, M, D>(tq_, (s_ ? q_1 : q_0) + hb_, qrs, q0_, q1_, wy, lane);                  \
    dma_rows<bf16, M, D>(tq_ + M * D, (s_ ? do_1 : do_0) + hb_, qrs, q0_, q1_, wy, lane);        \
    if (wy < 2) {                                                                                \
      const float* rb_ = (wy == 0 ? (s_ ? l2_1 : l2_0) : (s_ ? dl_1 : dl_0)) +                   \
                         (((int64_t)b * p.hq + h_) * R_ + q0_);                                  \
      uint32_t ro_ = 4u * (uint32_t)min(lane, q1_ - 1 - q0_);                                    \
      asm volatile("" : "+v"(ro_));                                                              \
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)           \
                                       (reinterpret_cast<const char*>(rb_) + ro_),               \
                                       (__attribute__((address_space(3))) void*)(smem +          \
                                           ((i) % L::NBUF) * L::BUFB + 2 * L::TILE + wy * 256), 4, 0, 0); \
    }                                                                                            \
  } while (0)
    // vector-memory operations one tile's DMA leaves outstanding in this wave
#define WS_WAIT_BUT_ONE_TILE()                                                                   \
  do {                                                                                           \
    if (wy < 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * (M / Swz<bf16, D>::RPB) / 4 + 1));      \
    else __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * (M / Swz<bf16, D>::RPB) / 4));                 \
  } while (0)
    if (total > 0) WS_ISSUE(0);
    if (total > 1) { WS_ISSUE(1); WS_WAIT_BUT_ONE_TILE(); } else wait_vmem();
    barrier_lds();                                  // tile 0 has landed
    for (int j = 0; j <= 2 * total; ++j) {
      if ((j & 1) && (j + 3) / 2 < total) WS_ISSUE((j + 3) / 2);
      if (j >= 1) {
        const int jj = j - 1;
        const int qs = jj & 1;
        const char* tb = smem + ((jj >> 1) % L::NBUF) * L::BUFB;
        const char* pd = smem + L::PDS + (jj & 1) * L::SLOT + pair * 4096 + lane * 16;
        bf16x8 pfr[2], sfr[2];
#pragma unroll
        for (int ci = 0; ci < 2; ++ci) {
          pfr[ci] = *reinterpret_cast<const bf16x8*>(pd + ci * 1024);
          sfr[ci] = *reinterpret_cast<const bf16x8*>(pd + 2048 + ci * 1024);
        }
        // dV_w += P^T dO ; dK_w += dS^T Q.  The transposed dO / Q fragments of
        // each column block are read two blocks ahead of its MFMAs (3-slot ring).
        bf16x8 ob[3][2], qb[3][2];
        auto read_t = [&](int dt, bf16x8 (&o)[2], bf16x8 (&q)[2]) {
#pragma unroll
          for (int ci = 0; ci < 2; ++ci) {
            const int imm = (qs * 32 + 16 * ci) * D * 2;
            const char* b0 = tb + offT[2 * dt] + imm;
            const char* b1 = tb + offT[2 * dt + 1] + imm;
            o[ci] = cat44(__builtin_bit_cast(bf16x4, ds_read_tr16(b0 + L::TILE)),
                          __builtin_bit_cast(bf16x4, ds_read_tr16(b1 + L::TILE)));
            q[ci] = cat44(__builtin_bit_cast(bf16x4, ds_read_tr16(b0)),
                          __builtin_bit_cast(bf16x4, ds_read_tr16(b1)));
          }
        };
        read_t(0, ob[0], qb[0]);
#pragma unroll
        for (int dt = 0; dt < L::DT; ++dt) {
          if (dt >= 1 && dt + 2 < L::DT) read_t(dt + 2, ob[(dt + 2) % 3], qb[(dt + 2) % 3]);
          __builtin_amdgcn_sched_barrier(0);
          dvacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pfr[0], ob[dt % 3][0], dvacc[dt], 0, 0, 0);
          dkacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sfr[0], qb[dt % 3][0], dkacc[dt], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          if (dt == 0 && L::DT > 1) read_t(1, ob[1], qb[1]);
          if (dt == 0 && L::DT > 2) read_t(2, ob[2], qb[2]);
          __builtin_amdgcn_sched_barrier(0);
          dvacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pfr[1], ob[dt % 3][1], dvacc[dt], 0, 0, 0);
          dkacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sfr[1], qb[dt % 3][1], dkacc[dt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j & 1) {                                    // tile (j+1)/2 is read from step j+1 on
        const int i = (j + 1) / 2;
        if (i < total) {
          if (i + 1 < total) WS_WAIT_BUT_ONE_TILE(); else wait_vmem();
        }
      }
      barrier_lds();
    }
#undef WS_ISSUE
#undef WS_WAIT_BUT_ONE_TILE
    // dK = scale * sum dS^T Q, dV = sum P^T dO for the pair's 32 keys
    bf16* dkb = reinterpret_cast<bf16*>(args.dk[a]) + (int64_t)b * p.klen[a] * krs + (int64_t)g * D;
    bf16* dvb = reinterpret_cast<bf16*>(args.dv[a]) + (int64_t)b * p.klen[a] * krs + (int64_t)g * D;
#pragma unroll
    for (int dt = 0; dt < L::DT; ++dt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 32 * pair + c_row(i, hh);
        if (key < k1) {
          const int64_t off = (int64_t)key * krs + dt * 32 + ln;
          dkb[off] = to_elt<bf16>(dkacc[dt][i] * args.scale);
          dvb[off] = to_elt<bf16>(dvacc[dt][i]);
        }
      }
    }
  }
#undef WS_GET
#undef WS_ENTRY
}

// ======================================================== backward: dQ kernel
// Query-major: one workgroup per (batch, q-head, stream, 128-row query tile),
// the forward's decomposition.  Per key tile it recomputes S^T = K Q^T and
// dP^T = V dO^T (lane = query), forms dS^T = P^T (dP^T - D) with
// P^T = exp(S^T - LSE) in registers, and accumulates dQ^T += K^T dS^T with dS^T
// as the MFMA B operand straight from registers and K^T read transposed out of
// the row-major K tile.  Each dQ row is written once: no atomics.
template <typename T, int D, bool ADD_F32>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void dq_kernel(DqArgs args) {
  using E = Elt<T>;
  using Frag = typename E::Frag;
  constexpr int M = 128, N = 64;
  constexpr int KPL = E::KPL, KC = 2 * KPL;
  constexpr int DCH = D / KC;
  constexpr int CPS = 32 / KC;
  // K and V tiles, double-buffered, filled by global->LDS DMA (swizzled rows)
  __shared__ __attribute__((aligned(16))) T kv_lds[2][2][N * D];

  const Problem& p = args.p;
  int bg, item;
  args.map.decode(blockIdx.x, bg, item);
  const int b = bg / p.hkv, g = bg % p.hkv;
  const int hg = item % p.group;
  const int rest = item / p.group;
  const int nstr = 2 - args.ns0;
  const int s = args.ns0 + rest % nstr;
  const int t = args.nqt[s] - 1 - rest / nstr;
  const int h = g * p.group + hg;
  const int R = p.rows[s];
  const int r0 = t * M;
  const int r1 = min(r0 + M, R);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform per wave
  const int ln = lane & 31, hh = lane >> 5;
  const int r = r0 + 32 * w + ln;
  const bool valid = r < r1;
  const int64_t qrs = (int64_t)p.hq * D;

  // Q^T and dO^T fragments (MFMA B operands): column = this lane's query.
  Frag qf[DCH], df[DCH];
  {
    const int64_t off = ((int64_t)b * R + (valid ? r : r0)) * qrs + (int64_t)h * D + hh * KPL;
    const T* qrow = reinterpret_cast<const T*>(args.q[s]) + off;
    const T* drow = reinterpret_cast<const T*>(args.dout[s]) + off;
#pragma unroll
    for (int c = 0; c < DCH; ++c) {
      qf[c] = ld_frag<T>(qrow + c * KC);
      df[c] = ld_frag<T>(drow + c * KC);
      if (!valid) { qf[c] = Frag{}; df[c] = Frag{}; }
    }
  }
  float lse2 = 0.f, dd = 0.f;
  if (valid) {
    const int64_t ri = ((int64_t)b * p.hq + h) * R + r;
    lse2 = args.lse2[s][ri];
    dd = args.delta[s][ri];
  }
  int klo[2], khi[2], flo[2], fhi[2], nt[2], lo[2], hi[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    tile_ranges(p, s, a, r0, r1, klo[a], khi[a], flo[a], fhi[a]);
    nt[a] = klo[a] < khi[a] ? (khi[a] - klo[a] + N - 1) / N : 0;
    if (valid) row_keys(p, s, r, a, lo[a], hi[a]); else lo[a] = hi[a] = 0;
  }
  const int total = nt[0] + nt[1];
  const int64_t rs = (int64_t)p.hkv * D;
  const T* kb[2];
  const T* vb[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    kb[a] = reinterpret_cast<const T*>(args.k[a]) + (int64_t)b * p.klen[a] * rs + (int64_t)g * D;
    vb[a] = reinterpret_cast<const T*>(args.v[a]) + (int64_t)b * p.klen[a] * rs + (int64_t)g * D;
  }
  if (total > 0) {
    const int a0 = nt[0] > 0 ? 0 : 1;
    dma_rows<T, N, D>(kv_lds[0][0], kb[a0], rs, klo[a0], khi[a0], w, lane);
    dma_rows<T, N, D>(kv_lds[0][1], vb[a0], rs, klo[a0], khi[a0], w, lane);
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  // bf16: per-lane fragment offsets, computed once (see bf16_frag_offsets)
  constexpr bool OFFS = sizeof(T) == 2;
  uint32_t offA[OFFS ? D / 16 : 1], offT[OFFS ? D / 16 : 1];
  if constexpr (OFFS) bf16_frag_offsets<D>(lane, offA, offT);

  for (int it = 0; it < total; ++it) {
    const int a = it < nt[0] ? 0 : 1;
    const int k0 = klo[a] + (it - (a ? nt[0] : 0)) * N;
    wait_vmem();
    __syncthreads();   // tile `it` is in buffer it&1; buffer (it+1)&1 is free
    const T* k_lds = kv_lds[it & 1][0];
    const T* v_lds = kv_lds[it & 1][1];
    const bool need_mask = qmajor_tile_masked(k0, N, flo[a], fhi[a], r0, r1, M);
    const int mylo = a ? lo[1] : lo[0], myhi = a ? hi[1] : hi[0];

    // per 32-key sub-tile: S^T = K Q^T and dP^T = V dO^T, then
    // dS^T = P^T (dP^T - D) with P^T = exp(S^T - LSE), then dQ^T += K^T dS^T
#pragma unroll
    for (int sub = 0; sub < N / 32; ++sub) {
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      {
        constexpr int BT = DCH < 2 ? DCH : 2;
        Frag ka[2][BT], va[2][BT];
#pragma unroll
        for (int c = 0; c < BT; ++c) {
          if constexpr (OFFS) {
            ka[0][c] = ld_fragA(reinterpret_cast<const char*>(k_lds), offA[c], sub * 32 * D * 2);
            va[0][c] = ld_fragA(reinterpret_cast<const char*>(v_lds), offA[c], sub * 32 * D * 2);
          } else {
            ka[0][c] = ld_frag_s<T, D>(k_lds, sub * 32 + ln, c * KC + hh * KPL);
            va[0][c] = ld_frag_s<T, D>(v_lds, sub * 32 + ln, c * KC + hh * KPL);
          }
        }
#pragma unroll
        for (int cb = 0; cb < DCH / BT; ++cb) {
          if (cb + 1 < DCH / BT) {
#pragma unroll
            for (int c = 0; c < BT; ++c) {
              const int cc = (cb + 1) * BT + c;
              if constexpr (OFFS) {
                ka[(cb + 1) & 1][c] = ld_fragA(reinterpret_cast<const char*>(k_lds), offA[OFFS ? cc : 0], sub * 32 * D * 2);
                va[(cb + 1) & 1][c] = ld_fragA(reinterpret_cast<const char*>(v_lds), offA[OFFS ? cc : 0], sub * 32 * D * 2);
              } else {
                ka[(cb + 1) & 1][c] = ld_frag_s<T, D>(k_lds, sub * 32 + ln, cc * KC + hh * KPL);
                va[(cb + 1) & 1][c] = ld_frag_s<T, D>(v_lds, sub * 32 + ln, cc * KC + hh * KPL);
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int c = 0; c < BT; ++c) {
            sacc = E::mma(ka[cb & 1][c], qf[cb * BT + c], sacc);
            pacc = E::mma(va[cb & 1][c], df[cb * BT + c], pacc);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // The K^T fragments of the first two d-tiles do not depend on dS: read
      // them now, so that their latency hides behind the DMA issue and the
      // exponentials; the others are read two d-tiles ahead (3-slot ring).
      Frag kt[3][CPS];
      auto rd_kt = [&](int dt) {
#pragma unroll
        for (int ci = 0; ci < CPS; ++ci) {
          if constexpr (OFFS)
            kt[dt % 3][ci] = ld_fragT(reinterpret_cast<const char*>(k_lds), offT, OFFS ? dt : 0, (sub * 32 + 16 * ci) * D * 2);
          else
            kt[dt % 3][ci] = ld_frag_kcrow_s<T, D>(k_lds, sub * 32, ci, lane, dt * 32);
        }
      };
      rd_kt(0);
      if (D / 32 > 1) rd_kt(1);
      // Next tile's DMA, issued behind the first sub-tile's S^T / dP^T MFMAs
      // (a wave stalls while the memory pipeline accepts DMA instructions).
      if (sub == 0 && it + 1 < total) {
        const int a2 = it + 1 < nt[0] ? 0 : 1;
        const int k02 = klo[a2] + (it + 1 - (a2 ? nt[0] : 0)) * N;
        dma_rows<T, N, D>(kv_lds[(it + 1) & 1][0], kb[a2], rs, k02, khi[a2], w, lane);
        dma_rows<T, N, D>(kv_lds[(it + 1) & 1][1], vb[a2], rs, k02, khi[a2], w, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
      float pe[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) pe[i] = fast_exp2(sacc[i] * args.scale_log2 - lse2);
      // Edge tiles only (one uniform branch): keys outside the row's range.
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = k0 + sub * 32 + c_row(i, hh);
          if (kk < mylo || kk >= myhi) pe[i] = 0.f;
        }
      }
      Frag dsf[CPS];
#pragma unroll
      for (int ci = 0; ci < CPS; ++ci) {
        float de[KPL];
#pragma unroll
        for (int jj = 0; jj < KPL; ++jj) de[jj] = pe[ci * KPL + jj] * (pacc[ci * KPL + jj] - dd);
        dsf[ci] = pack_frag<T>(de);
      }
      // dQ^T[d][query] += K^T[d][key] dS^T[key][query]
      {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          if (dt + 2 < D / 32) rd_kt(dt + 2);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ci = 0; ci < CPS; ++ci) acc[dt] = E::mma(kt[dt % 3][ci], dsf[ci], acc[dt]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  if (valid && (total > 0 || !ADD_F32)) {
    using OT = typename std::conditional<ADD_F32, float, T>::type;
    OT* orow = reinterpret_cast<OT*>(args.dq[s]) + ((int64_t)b * R + r) * qrs + (int64_t)h * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        OT* dst = orow + dt * 32 + g4 * 8 + hh * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = acc[dt][g4 * 4 + j] * args.scale;
          if (ADD_F32) dst[j] = static_cast<OT>(static_cast<float>(dst[j]) + v);
          else dst[j] = static_cast<OT>(v);
        }
      }
    }
  }
}

// ============================================================ partial merge
// One group of D/4 lanes per (batch, token, head) row; each lane owns 4 floats.
template <typename OT, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs args) {
  constexpr int LPR = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / LPR;                 // (b, t, h) in [b][t][h] order
  const int part = (int)(gid % LPR);
  const int64_t nrows = (int64_t)args.batch * args.tokens * args.heads;
  if (row >= nrows) return;
  const int h = (int)(row % args.heads);
  const int64_t bt = row / args.heads;
  const int64_t t = bt % args.tokens;
  const int64_t bb = bt / args.tokens;
  const int64_t li = (bb * args.heads + h) * args.tokens + t;
  const int64_t oi = row * D + part * 4;

  // Pass 1: the row's LPR lanes read the parts' LSEs in parallel (lane `part`
  // reads parts part, part + LPR, ...), then a shuffle reduction gives the max
  // and a ballot the set of live parts (LSE > -inf).  The LSE values stay
  // cached for pass 2.
  const int lane = threadIdx.x & 63;
  const int gbase = lane & ~(LPR - 1);          // first lane of this row's group
  float m = -INFINITY;
  uint64_t live = 0;
#pragma unroll
  for (int k = 0; k < kMaxMergeParts / LPR; ++k) {
    const int jj = part + k * LPR;
    const float l = jj < args.nparts ? args.lse[jj][li] : -INFINITY;
    m = fmaxf(m, l);
    const uint64_t bal = __ballot(l != -INFINITY);
    live |= ((bal >> gbase) & ((LPR == 64) ? ~0ull : ((1ull << LPR) - 1))) << (k * LPR);
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  // In place (output aliases part 0): a row where every other part is empty
  // keeps its values, so it is neither read nor written.
  if (args.inplace && (live & ~1ull) == 0) return;
  // Pass 2: live parts PB at a time, their loads issued together (one
  // dependent load per part would leave the row latency-bound); empty parts
  // have weight 0 and their O is not read.
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float tot = 0.f;
  constexpr int PB = 8;
  // Takes the next (up to) PB live parts out of `set` and adds them in.
  auto merge_batch = [&](uint64_t& set) {
    int idx[PB];
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      idx[u] = set ? __builtin_ctzll(set) : -1;
      set &= set ? set - 1 : 0ull;
    }
    float l[PB];
    float4 v[PB];
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      if (idx[u] >= 0) {
        l[u] = args.lse[idx[u]][li];
        v[u] = *reinterpret_cast<const float4*>(args.o[idx[u]] + oi);
      }
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      if (idx[u] >= 0) {
        const float wj = __expf(l[u] - m);
        tot += wj;
        acc.x += wj * v[u].x; acc.y += wj * v[u].y; acc.z += wj * v[u].z; acc.w += wj * v[u].w;
      }
    }
  };
  // The rows of a wave almost always share their live set (they belong to one
  // block); then the part index is wave-uniform and the parts' pointers are
  // scalar loads instead of per-lane pointer gathers ahead of every data load.
  const uint64_t wlive = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)live)) |
                         ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(live >> 32)) << 32);
  if (__all(live == wlive)) {
    uint64_t lv = wlive;
    while (lv) merge_batch(lv);
  } else {
    while (live) merge_batch(live);
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  OT* dst = reinterpret_cast<OT*>(args.o_out) + oi;
  if constexpr (sizeof(OT) == 2) {
    bf16x4 pk;
    pk[0] = static_cast<bf16>(acc.x * inv); pk[1] = static_cast<bf16>(acc.y * inv);
    pk[2] = static_cast<bf16>(acc.z * inv); pk[3] = static_cast<bf16>(acc.w * inv);
    *reinterpret_cast<bf16x4*>(dst) = pk;
  } else {
    *reinterpret_cast<float4*>(dst) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  if (part == 0) args.lse_out[li] = tot > 0.f ? m + __logf(tot) : -INFINITY;
}

// ================================================================ launchers
template <typename T, int D, bool OUT_F32>
hipError_t launch_fwd_t(const FwdArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((fwd_kernel<T, D, OUT_F32>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int grid, int is_bf16, int out_f32, hipStream_t st) {
  const int D = a.p.D;
  if (is_bf16) {
    if (D == 128) return out_f32 ? launch_fwd_t<bf16, 128, true>(a, grid, st) : launch_fwd_t<bf16, 128, false>(a, grid, st);
    if (D == 64) return out_f32 ? launch_fwd_t<bf16, 64, true>(a, grid, st) : launch_fwd_t<bf16, 64, false>(a, grid, st);
  } else {
    if (D == 128) return launch_fwd_t<float, 128, true>(a, grid, st);
    if (D == 64) return launch_fwd_t<float, 64, true>(a, grid, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_pre(const BwdPreArgs& a, int is_bf16, hipStream_t st) {
  const int VEC = is_bf16 ? 8 : 4;
  const int64_t threads = (int64_t)a.batch * a.rows * a.hq * (a.D / VEC);
  const int grid = (int)((threads + 255) / 256);
  if (grid == 0) return hipSuccess;
  if (is_bf16) {
    if (a.D == 128) hipLaunchKernelGGL((bwd_pre_kernel<bf16, 128>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((bwd_pre_kernel<bf16, 64>), dim3(grid), dim3(256), 0, st, a);
  } else {
    if (a.D == 128) hipLaunchKernelGGL((bwd_pre_kernel<float, 128>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((bwd_pre_kernel<float, 64>), dim3(grid), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_dkdv(const BwdArgs& a, int grid, int is_bf16, hipStream_t st) {
  const int D = a.p.D;
  if (is_bf16) {
    if (D == 128) hipLaunchKernelGGL((dkdv_ws_kernel<128>), dim3(grid), dim3(512), 0, st, a);
    else hipLaunchKernelGGL((dkdv_ws_kernel<64>), dim3(grid), dim3(512), 0, st, a);
  } else {
    if (D == 128) hipLaunchKernelGGL((dkdv_kernel<float, 128>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((dkdv_kernel<float, 64>), dim3(grid), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dq_t(const DqArgs& a, int grid, int add_f32, hipStream_t st) {
  if (add_f32) hipLaunchKernelGGL((dq_kernel<T, D, true>), dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((dq_kernel<T, D, false>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dq(const DqArgs& a, int grid, int is_bf16, int add_f32, hipStream_t st) {
  const int D = a.p.D;
  if (is_bf16) return D == 128 ? launch_dq_t<bf16, 128>(a, grid, add_f32, st) : launch_dq_t<bf16, 64>(a, grid, add_f32, st);
  return D == 128 ? launch_dq_t<float, 128>(a, grid, add_f32, st) : launch_dq_t<float, 64>(a, grid, add_f32, st);
}

hipError_t launch_merge(const MergeArgs& a, int out_bf16, hipStream_t st) {
  const int64_t threads = (int64_t)a.batch * a.tokens * a.heads * (a.D / 4);
  const int64_t grid = (threads + 255) / 256;
  if (grid == 0) return hipSuccess;
  if (a.D == 128) {
    if (out_bf16) hipLaunchKernelGGL((merge_kernel<bf16, 128>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((merge_kernel<float, 128>), dim3(grid), dim3(256), 0, st, a);
  } else {
    if (out_bf16) hipLaunchKernelGGL((merge_kernel<bf16, 64>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((merge_kernel<float, 64>), dim3(grid), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace bdlm
