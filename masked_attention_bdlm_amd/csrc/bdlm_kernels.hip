// HIP kernels of BDLM masked attention for gfx950 (CDNA4).
//
// Forward: one workgroup (4 waves) per (batch, q-head, stream, 128-row q tile).
// Each wave owns 32 query rows and computes S^T = K Q^T with the rows of K as
// the MFMA A operand, so a lane's accumulator values all belong to ONE query:
// the online softmax (max, exp2, sum, rescale) is lane-local except one swap
// between the two lane halves.  P^T then feeds O^T += V^T P^T directly from
// registers (its k order is the C-layout row order, which the V^T fragment
// loads reproduce), so P never touches LDS.  K tiles are staged row-major in
// LDS, V tiles transposed.  Only key tiles inside a row's visible ranges are
// visited; tiles on a range edge test each element against [lo, hi).
//
// Backward (stored-LSE recompute, "dK/dV accumulated per key tile"): one
// workgroup per (batch, kv-head, key array, 128-key tile); wave w owns 32 keys
// and keeps K_w, V_w and its dK_w, dV_w accumulators in registers while it loops
// over the visible query tiles of every q head of the GQA group.  S and dP are
// computed with the query as MFMA row, so P and dS (lane = key) are directly the
// A operands of dV += P^T dO and dK += dS^T Q; dO^T and Q^T come from LDS tiles
// staged transposed.  dS goes through LDS once more for dQ^T = K^T dS^T, which
// is added into an fp32 accumulator with hardware float atomics.

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
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs args) {
  using E = Elt<T>;
  using Frag = typename E::Frag;
  constexpr int M = 128, N = 64;
  constexpr int KPL = E::KPL, KC = 2 * KPL;
  constexpr int DCH = D / KC;          // k-chunks over head_dim
  constexpr int CPS = 32 / KC;         // k-chunks per 32-key subtile
  constexpr int KST = D + E::PAD;      // K tile row stride
  constexpr int VST = N + E::PAD;      // V^T tile row stride
  __shared__ __attribute__((aligned(16))) T k_lds[N * KST];
  __shared__ __attribute__((aligned(16))) T vt_lds[D * VST];

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

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
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

  int lo[2], hi[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    if (valid) row_keys(p, s, r, a, lo[a], hi[a]); else lo[a] = hi[a] = 0;
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};

  for (int a = 0; a < 2; ++a) {
    int klo, khi, flo, fhi;
    tile_ranges(p, s, a, r0, r1, klo, khi, flo, fhi);
    if (klo >= khi) continue;
    const int64_t rs = (int64_t)p.hkv * D;
    const T* kbase = reinterpret_cast<const T*>(args.k[a]) + (int64_t)b * p.klen[a] * rs + (int64_t)g * D;
    const T* vbase = reinterpret_cast<const T*>(args.v[a]) + (int64_t)b * p.klen[a] * rs + (int64_t)g * D;
    const int mylo = lo[a], myhi = hi[a];

    for (int k0 = klo; k0 < khi; k0 += N) {
      __syncthreads();
      stage_rows<T, N, D, KST>(k_lds, kbase, rs, k0, khi, tid);
      stage_rows_t<T, N, D, VST>(vt_lds, vbase, rs, k0, khi, tid);
      __syncthreads();
      const bool need_mask = !(k0 >= flo && k0 + N <= fhi);

      // S^T[key][query] for the N keys of the tile.
      f32x16 sacc[N / 32];
#pragma unroll
      for (int sub = 0; sub < N / 32; ++sub) {
        sacc[sub] = f32x16{};
#pragma unroll
        for (int c = 0; c < DCH; ++c) {
          Frag ka = ld_frag<T>(k_lds + (sub * 32 + ln) * KST + c * KC + hh * KPL);
          sacc[sub] = E::mma(ka, qf[c], sacc[sub]);
        }
      }

      float mx = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < N / 32; ++sub) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float v = sacc[sub][i];
          if (need_mask) {
            const int kk = k0 + sub * 32 + c_row(i, hh);
            if (kk < mylo || kk >= myhi) v = -INFINITY;
          }
          sacc[sub][i] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, wave_swap32(mx));
      const float m_new = fmaxf(m_run, mx * args.scale_log2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;

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

      // O^T[d][query] += V^T[d][key] P^T[key][query]
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int cc = 0; cc < N / KC; ++cc) {
          const int sub = cc / CPS, ci = cc % CPS;
          Frag va = ld_frag_crows<T>(vt_lds + (dt * 32 + ln) * VST + sub * 32, ci, hh);
          Frag pb = pack_frag<T>(&pv[sub][ci * KPL]);
          oacc[dt] = E::mma(va, pb, oacc[dt]);
        }
      }
    }
  }

  const float l_tot = l_run + wave_swap32(l_run);
  if (valid) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    using OT = typename std::conditional<OUT_F32, float, T>::type;
    OT* orow = reinterpret_cast<OT*>(args.o[s]) + ((int64_t)b * R + r) * p.hq * D + (int64_t)h * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        OT* dst = orow + dt * 32 + g4 * 8 + hh * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = static_cast<OT>(oacc[dt][g4 * 4 + j] * inv);
      }
    }
    if (hh == 0) {
      args.lse[s][((int64_t)b * p.hq + h) * R + r] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

// ========================================================== backward: D and zero
// delta[s][b][h][r] = <dO, O> over head_dim; zero the fp32 dQ accumulator rows.
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
    if (args.dq_acc) {
      float* z = args.dq_acc + u * D + part * VEC;
#pragma unroll
      for (int e = 0; e < VEC; ++e) z[e] = 0.f;
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (ok && part == 0) {
    const int h = (int)(u % args.hq);
    const int64_t br = u / args.hq;
    const int r = (int)(br % args.rows);
    const int bb = (int)(br / args.rows);
    args.delta[((int64_t)bb * args.hq + h) * args.rows + r] = acc;
  }
  (void)s;
}

// ======================================================= backward: main kernel
template <typename T, int D>
__global__ __launch_bounds__(256, 1) void bwd_kernel(BwdArgs args) {
  using E = Elt<T>;
  using Frag = typename E::Frag;
  constexpr int N = 128;                                   // keys per workgroup
  constexpr int M = sizeof(T) == 2 ? 64 : 32;              // query rows per iteration
  constexpr int QS = M / 32;
  constexpr int KPL = E::KPL, KC = 2 * KPL;
  constexpr int DCH = D / KC;
  constexpr int CPS = 32 / KC;
  constexpr int QST = D + E::PAD;      // q / dO row-major stride
  constexpr int QTST = M + E::PAD;     // q^T / dO^T stride
  constexpr int DSST = N + E::PAD;     // dS [query][key] stride
  constexpr int KTST = N + E::PAD;     // K^T [d][key] stride
  __shared__ __attribute__((aligned(16))) T q_lds[M * QST];
  __shared__ __attribute__((aligned(16))) T do_lds[M * QST];
  __shared__ __attribute__((aligned(16))) T qt_lds[D * QTST];
  __shared__ __attribute__((aligned(16))) T dot_lds[D * QTST];
  __shared__ __attribute__((aligned(16))) T ds_lds[M * DSST];
  __shared__ __attribute__((aligned(16))) T kt_lds[D * KTST];
  __shared__ __attribute__((aligned(16))) float lse_l[M];
  __shared__ __attribute__((aligned(16))) float dl_l[M];
  __shared__ int lo_l[M], hi_l[M];

  const Problem& p = args.p;
  int bg, item;
  args.map.decode(blockIdx.x, bg, item);
  const int b = bg / p.hkv, g = bg % p.hkv;
  const int a = item < args.nkt[0] ? 0 : 1;
  const int j = a == 0 ? item : item - args.nkt[0];
  const int k0 = args.kbase[a] + j * N;
  const int k1 = min(k0 + N, args.kend[a]);

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
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
  stage_rows_t<T, N, D, KTST>(kt_lds, kbase, krs, k0, k1, tid);

  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) { dkacc[dt] = f32x16{}; dvacc[dt] = f32x16{}; }

  const float sl2 = args.scale_log2;
  for (int s = (a == 0 ? args.ns0 : 1); s < 2; ++s) {
    const int R = p.rows[s];
    if (R == 0) continue;
    int rlo, rhi;
    query_span(p, s, a, k0, k1, rlo, rhi);
    if (rlo >= rhi) continue;
    const int64_t qrs = (int64_t)p.hq * D;
    for (int t = (rhi - 1) / M; t >= rlo / M; --t) {
      const int q0 = t * M;
      const int q1 = min(q0 + M, R);
      int klo, khi, flo, fhi;
      tile_ranges(p, s, a, q0, q1, klo, khi, flo, fhi);
      const bool need_mask = !(k0 >= flo && k0 + N <= fhi);
      for (int hg = 0; hg < p.group; ++hg) {
        const int h = g * p.group + hg;
        const T* qb = reinterpret_cast<const T*>(args.q[s]) + (int64_t)b * R * qrs + (int64_t)h * D;
        const T* db = reinterpret_cast<const T*>(args.dout[s]) + (int64_t)b * R * qrs + (int64_t)h * D;
        __syncthreads();
        stage_rows_dual<T, M, D, QST, QTST>(q_lds, qt_lds, qb, qrs, q0, q1, tid);
        stage_rows_dual<T, M, D, QST, QTST>(do_lds, dot_lds, db, qrs, q0, q1, tid);
        if (tid < M) {
          const int rr = q0 + tid;
          int lo = 0, hi = 0;
          float l2 = 0.f, dd = 0.f;
          if (rr < q1) {
            row_keys(p, s, rr, a, lo, hi);
            const int64_t ri = ((int64_t)b * p.hq + h) * R + rr;
            l2 = args.lse[s][ri] * kLog2e;
            dd = args.delta[s][ri];
          }
          lo_l[tid] = lo; hi_l[tid] = hi; lse_l[tid] = l2; dl_l[tid] = dd;
        }
        __syncthreads();

        // S = Q K_w^T and dP = dO V_w^T (rows = queries, column = this lane's key)
        f32x16 sacc[QS], pacc[QS];
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
          sacc[qs] = f32x16{};
          pacc[qs] = f32x16{};
#pragma unroll
          for (int c = 0; c < DCH; ++c) {
            Frag qa = ld_frag<T>(q_lds + (qs * 32 + ln) * QST + c * KC + hh * KPL);
            Frag da = ld_frag<T>(do_lds + (qs * 32 + ln) * QST + c * KC + hh * KPL);
            sacc[qs] = E::mma(qa, kf[c], sacc[qs]);
            pacc[qs] = E::mma(da, vf[c], pacc[qs]);
          }
        }
        // P = exp(S - LSE), dS = P (dP - D)
        float pv[QS][16], dsv[QS][16];
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int rr0 = qs * 32 + c_row(4 * i4, hh);      // 4 consecutive rows
            const float4 l4 = *reinterpret_cast<const float4*>(lse_l + rr0);
            const float4 d4 = *reinterpret_cast<const float4*>(dl_l + rr0);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
            const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int i = 4 * i4 + j;
              float pe = fast_exp2(sacc[qs][i] * sl2 - lv[j]);
              if (need_mask && !(kk >= lo_l[rr0 + j] && kk < hi_l[rr0 + j])) pe = 0.f;
              pv[qs][i] = pe;
              dsv[qs][i] = pe * (pacc[qs][i] - dv[j]);
            }
          }
        }
        // dV_w += P^T dO ; dK_w += dS^T Q   (k = queries in C-row order)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
          for (int cc = 0; cc < M / KC; ++cc) {
            const int qs = cc / CPS, ci = cc % CPS;
            Frag pa = pack_frag<T>(&pv[qs][ci * KPL]);
            Frag sa = pack_frag<T>(&dsv[qs][ci * KPL]);
            Frag ob = ld_frag_crows<T>(dot_lds + (dt * 32 + ln) * QTST + qs * 32, ci, hh);
            Frag qb2 = ld_frag_crows<T>(qt_lds + (dt * 32 + ln) * QTST + qs * 32, ci, hh);
            dvacc[dt] = E::mma(pa, ob, dvacc[dt]);
            dkacc[dt] = E::mma(sa, qb2, dkacc[dt]);
          }
        }
        // dS -> LDS as [query][key]
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            ds_lds[(qs * 32 + c_row(i, hh)) * DSST + 32 * w + ln] = to_elt<T>(dsv[qs][i]);
          }
        }
        __syncthreads();
        // dQ[query][d] = dS[query][key] K[key][d], added into fp32 dQ
        float* dqb = args.dq_acc[s] + (int64_t)b * R * qrs + (int64_t)h * D;
        constexpr int TILES = (D / 32) * QS;
        for (int tt = w; tt < TILES; tt += 4) {
          const int dt = tt % (D / 32), qs = tt / (D / 32);
          // rows = queries (A = dS from LDS), columns = head_dim (B = K^T from LDS):
          // each lane owns one d, so an atomic instruction covers 2 x 32
          // consecutive floats of two dQ rows.
          f32x16 acc = f32x16{};
#pragma unroll
          for (int c = 0; c < N / KC; ++c) {
            Frag sa = ld_frag<T>(ds_lds + (qs * 32 + ln) * DSST + c * KC + hh * KPL);
            Frag kb2 = ld_frag<T>(kt_lds + (dt * 32 + ln) * KTST + c * KC + hh * KPL);
            acc = E::mma(sa, kb2, acc);
          }
          float* dst = dqb + dt * 32 + ln;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int rr = q0 + qs * 32 + c_row(i, hh);
            if (rr < q1) unsafeAtomicAdd(dst + (int64_t)rr * qrs, acc[i] * args.scale);
          }
        }
      }
    }
  }

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

// ===================================================== backward: dQ fp32 -> T
template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ src, T* __restrict__ dst,
                                                      int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float4 v = reinterpret_cast<const float4*>(src)[i];
  T* d = dst + i * 4;
  d[0] = to_elt<T>(v.x); d[1] = to_elt<T>(v.y); d[2] = to_elt<T>(v.z); d[3] = to_elt<T>(v.w);
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

  float m = -INFINITY;
  int live = 0;
  for (int j = 0; j < args.nparts; ++j) {
    const float l = args.lse[j][li];
    m = fmaxf(m, l);
    live += (j > 0 && l != -INFINITY);
  }
  // In place (output aliases part 0): a row where every other part is empty
  // keeps its values, so it is neither read nor written.
  if (args.inplace && live == 0) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float tot = 0.f;
  if (m != -INFINITY) {
    for (int j = 0; j < args.nparts; ++j) {
      const float l = args.lse[j][li];
      if (l == -INFINITY) continue;              // weight 0: O_j is not read
      const float wj = __expf(l - m);
      const float4 v = *reinterpret_cast<const float4*>(args.o[j] + oi);
      tot += wj;
      acc.x += wj * v.x; acc.y += wj * v.y; acc.z += wj * v.z; acc.w += wj * v.w;
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  OT* dst = reinterpret_cast<OT*>(args.o_out) + oi;
  dst[0] = static_cast<OT>(acc.x * inv);
  dst[1] = static_cast<OT>(acc.y * inv);
  dst[2] = static_cast<OT>(acc.z * inv);
  dst[3] = static_cast<OT>(acc.w * inv);
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

hipError_t launch_bwd(const BwdArgs& a, int grid, int is_bf16, hipStream_t st) {
  const int D = a.p.D;
  if (is_bf16) {
    if (D == 128) hipLaunchKernelGGL((bwd_kernel<bf16, 128>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((bwd_kernel<bf16, 64>), dim3(grid), dim3(256), 0, st, a);
  } else {
    if (D == 128) hipLaunchKernelGGL((bwd_kernel<float, 128>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((bwd_kernel<float, 64>), dim3(grid), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_convert(const float* src, void* dst, int64_t n, int is_bf16, hipStream_t st) {
  const int64_t n4 = n / 4;
  const int grid = (int)((n4 + 255) / 256);
  if (grid == 0) return hipSuccess;
  if (is_bf16) hipLaunchKernelGGL((convert_kernel<bf16>), dim3(grid), dim3(256), 0, st, src, (bf16*)dst, n4);
  else hipLaunchKernelGGL((convert_kernel<float>), dim3(grid), dim3(256), 0, st, src, (float*)dst, n4);
  return hipGetLastError();
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
