// C ABI of the BDLM attention library: argument validation, work decomposition
// and kernel dispatch.  See include/bdlm_attn.h for the contract of each call.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <algorithm>
#include <vector>

#include "../../include/bdlm_attn.h"
#include "bdlm_common.h"
#include "bdlm_kernels.h"

using namespace bdlm;

namespace {

// ------------------------------------------------------------- profiling
struct ProfEntry { const char* name; hipEvent_t a, b; };
struct ProfState {
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<ProfEntry> used;
  size_t next = 0;
};
ProfState g_prof;

struct ProfScope {
  hipStream_t st;
  ProfEntry* e = nullptr;
  ProfScope(const char* name, hipStream_t s) : st(s) {
    if (!g_prof.on || g_prof.next + 2 > g_prof.pool.size()) return;
    g_prof.used.push_back({name, g_prof.pool[g_prof.next], g_prof.pool[g_prof.next + 1]});
    g_prof.next += 2;
    e = &g_prof.used.back();
    (void)hipEventRecord(e->a, st);
  }
  ~ProfScope() {
    if (e) (void)hipEventRecord(e->b, st);
  }
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int check_desc(const bdlm_attn_desc* d) {
  if (!d) return BDLM_ERR_INVALID_ARG;
  if (d->batch < 1 || d->seqlen < 1 || d->block < 16 || d->block % 16 != 0) return BDLM_ERR_INVALID_ARG;
  if (d->seqlen % d->block != 0) return BDLM_ERR_INVALID_ARG;
  if (d->num_q_heads < 1 || d->num_kv_heads < 1 || d->num_q_heads % d->num_kv_heads != 0)
    return BDLM_ERR_INVALID_ARG;
  if (d->dtype != BDLM_F32 && d->dtype != BDLM_BF16) return BDLM_ERR_INVALID_ARG;
  if (!(std::isfinite(d->softmax_scale) && d->softmax_scale > 0.f)) return BDLM_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return BDLM_ERR_UNSUPPORTED;
  // element counts must keep every row index inside int32 and every offset in int64
  const int64_t maxh = d->num_q_heads > d->num_kv_heads ? d->num_q_heads : d->num_kv_heads;
  if ((int64_t)d->batch * d->seqlen * maxh * d->head_dim > (int64_t(1) << 46)) return BDLM_ERR_UNSUPPORTED;
  if (d->num_local_blocks < 0) return BDLM_ERR_INVALID_ARG;
  if (d->num_local_blocks > 0) {
    if (d->num_local_blocks > BDLM_MAX_LOCAL_BLOCKS) return BDLM_ERR_UNSUPPORTED;
    if (!d->block_ids) return BDLM_ERR_INVALID_ARG;
    const int nb = d->seqlen / d->block;
    for (int i = 0; i < d->num_local_blocks; ++i) {
      const int id = d->block_ids[i];
      if (id < 0 || id >= nb) return BDLM_ERR_INVALID_ARG;
      if (i > 0 && id <= d->block_ids[i - 1]) return BDLM_ERR_INVALID_ARG;
    }
    if (d->kv_begin < 0 || d->kv_begin > d->kv_end || d->kv_end > d->seqlen) return BDLM_ERR_INVALID_ARG;
    if (d->own_block != 0 && d->own_block != 1) return BDLM_ERR_INVALID_ARG;
    if (d->clean_queries != 0 && d->clean_queries != 1) return BDLM_ERR_INVALID_ARG;
    if (d->clean_queries && d->own_block) return BDLM_ERR_INVALID_ARG;
    if (d->accumulate != 0 && d->accumulate != 1) return BDLM_ERR_INVALID_ARG;
    if (d->kv_staged != 0 && d->kv_staged != 1) return BDLM_ERR_INVALID_ARG;
  } else if (d->clean_queries != 0 || d->accumulate != 0 || d->kv_staged != 0) {
    return BDLM_ERR_INVALID_ARG;
  }
  return BDLM_OK;
}

Problem make_problem(const bdlm_attn_desc* d) {
  Problem p;
  std::memset(&p, 0, sizeof(p));
  p.batch = d->batch; p.L = d->seqlen; p.B = d->block;
  p.hq = d->num_q_heads; p.hkv = d->num_kv_heads; p.group = p.hq / p.hkv; p.D = d->head_dim;
  auto log2_exact = [](int x) { int s = 0; while ((1 << s) < x) ++s; return (1 << s) == x ? s : -1; };
  p.bshift = log2_exact(p.B);
  p.gshift = log2_exact(p.group);
  if (d->num_local_blocks == 0) {
    p.mode = 0;
    p.rows[0] = p.rows[1] = p.L;
    p.klen[0] = p.klen[1] = p.L;
    p.kv_begin = 0; p.kv_end = p.L; p.own_block = 1;
  } else {
    p.mode = 1;
    p.nlocal = d->num_local_blocks;
    p.rows[0] = 0; p.rows[1] = p.nlocal * p.B;
    // a staged window holds only rows [kv_begin, kv_end) per batch
    p.klen[0] = d->kv_staged ? d->kv_end - d->kv_begin : p.L;
    p.klen[1] = p.nlocal * p.B;
    p.kv_begin = d->kv_begin; p.kv_end = d->kv_end; p.own_block = d->own_block;
    p.incl = d->clean_queries;
    for (int i = 0; i < p.nlocal; ++i) p.block_ids[i] = d->block_ids[i];
  }
  return p;
}

XcdMap make_map(int nbg, int per_bg) {
  XcdMap m;
  m.nbg = nbg;
  m.per_bg = per_bg;
  m.by_xcd = (nbg % 8 == 0) ? 1 : 0;
  return m;
}

size_t elt_size(int dtype) { return dtype == BDLM_BF16 ? 2 : 4; }

// Address that clean-key row 0 would have in a staged window buffer: the
// kernels index array-0 rows by their clean-sequence position k, and a staged
// buffer holds row k at k - kv_begin.  Only rows of the window are ever read
// or written, so no access lands below the buffer.
template <typename P> P stage_shift(P ptr, const bdlm_attn_desc* d) {
  if (!ptr || d->num_local_blocks == 0 || !d->kv_staged) return ptr;
  const uintptr_t row = (uintptr_t)d->num_kv_heads * d->head_dim * elt_size(d->dtype);
  return reinterpret_cast<P>(reinterpret_cast<uintptr_t>(ptr) - row * (uintptr_t)d->kv_begin);
}

// Backward workspace: per query stream, D = rowsum(dO * O) and LSE * log2(e),
// fp32 [batch, Hq, rows] each.
struct BwdLayout { size_t delta_off[2], lse2_off[2], total; };

BwdLayout bwd_layout(const bdlm_attn_desc* d) {
  BwdLayout l{};
  const int64_t B = d->batch, H = d->num_q_heads;
  size_t off = 0;
  if (d->num_local_blocks == 0) {
    const int64_t L = d->seqlen;
    for (int s = 0; s < 2; ++s) {
      l.delta_off[s] = off; off = align256(off + sizeof(float) * B * H * L);
      l.lse2_off[s] = off; off = align256(off + sizeof(float) * B * H * L);
    }
  } else {
    const int64_t T = (int64_t)d->num_local_blocks * d->block;
    l.delta_off[0] = l.delta_off[1] = off;
    off = align256(off + sizeof(float) * B * H * T);
    l.lse2_off[0] = l.lse2_off[1] = off;
    off = align256(off + sizeof(float) * B * H * T);
  }
  l.total = off;
  return l;
}

}  // namespace

extern "C" {

const char* bdlm_status_str(int s) {
  switch (s) {
    case BDLM_OK: return "ok";
    case BDLM_ERR_INVALID_ARG: return "invalid argument";
    case BDLM_ERR_UNSUPPORTED: return "unsupported configuration";
    case BDLM_ERR_WORKSPACE: return "workspace missing or too small";
    case BDLM_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int bdlm_attn_version(void) { return 110; }

int bdlm_attn_check_desc(const bdlm_attn_desc* desc) { return check_desc(desc); }

size_t bdlm_attn_workspace_bytes(const bdlm_attn_desc* desc, int for_bwd) {
  if (check_desc(desc) != BDLM_OK) return 0;
  if (!for_bwd) return 0;
  return bwd_layout(desc).total;
}

int bdlm_attn_fwd(const bdlm_attn_desc* desc, const void* qc, const void* kc, const void* vc,
                  const void* qx, const void* kx, const void* vx, void* oc, void* ox,
                  float* lse_c, float* lse_x, void* ws, size_t ws_bytes, hipStream_t stream) {
  (void)ws; (void)ws_bytes;
  int st = check_desc(desc);
  if (st != BDLM_OK) return st;
  const bool share = desc->num_local_blocks > 0;
  if (share) {
    if (qc || oc || lse_c) return BDLM_ERR_INVALID_ARG;
    // without own_block no local K/V is read: NULL kx/vx stand in as kc/vc
    if (!desc->own_block && !kx && !vx) { kx = kc; vx = vc; }
  } else {
    if (!qc || !oc || !lse_c || !aligned16(qc) || !aligned16(oc) || !aligned4(lse_c)) return BDLM_ERR_INVALID_ARG;
  }
  const void* need[] = {kc, vc, qx, kx, vx, ox};
  for (const void* ptr : need) if (!ptr || !aligned16(ptr)) return BDLM_ERR_INVALID_ARG;
  if (!lse_x || !aligned4(lse_x)) return BDLM_ERR_INVALID_ARG;

  FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.p = make_problem(desc);
  a.q[0] = qc; a.q[1] = qx;
  a.k[0] = stage_shift(kc, desc); a.k[1] = kx;
  a.v[0] = stage_shift(vc, desc); a.v[1] = vx;
  a.o[0] = oc; a.o[1] = ox;
  a.lse[0] = lse_c; a.lse[1] = lse_x;
  a.scale_log2 = desc->softmax_scale * 1.4426950408889634f;
  a.ns0 = share ? 1 : 0;
  a.accum = share ? desc->accumulate : 0;
  for (int s = 0; s < 2; ++s) a.nqt[s] = (a.p.rows[s] + kFwdTileM - 1) / kFwdTileM;
  const int nstr = 2 - a.ns0;
  const int per_bg = a.nqt[1] * nstr * a.p.group;
  const int nbg = a.p.batch * a.p.hkv;
  a.map = make_map(nbg, per_bg);
  const int64_t grid = (int64_t)nbg * per_bg;
  if (grid <= 0) return BDLM_OK;
  if (grid > 0x7fffffff) return BDLM_ERR_UNSUPPORTED;
  ProfScope ps("bdlm_fwd", stream);
  hipError_t e = launch_fwd(a, (int)grid, desc->dtype == BDLM_BF16, share ? 1 : (desc->dtype == BDLM_F32), stream);
  return e == hipSuccess ? BDLM_OK : BDLM_ERR_HIP;
}

}  // extern "C"

namespace {

// The backward behind bdlm_attn_bwd and bdlm_attn_bwd_noalloc.  `ws_of` is
// called once every argument has been validated, with the workspace size the
// call needs; it returns the workspace (or NULL with *err set).
template <typename WsOf>
int bwd_impl(const bdlm_attn_desc* desc, const void* qc, const void* kc, const void* vc,
             const void* qx, const void* kx, const void* vx, const void* oc, const void* ox,
             const float* lse_c, const float* lse_x, const void* doc, const void* dox,
             void* dqc, void* dkc, void* dvc, void* dqx, void* dkx, void* dvx,
             WsOf ws_of, hipStream_t stream) {
  int st = check_desc(desc);
  if (st != BDLM_OK) return st;
  const bool share = desc->num_local_blocks > 0;
  if (share) {
    if (qc || oc || lse_c || doc || dqc) return BDLM_ERR_INVALID_ARG;
    if (desc->own_block) {
      if (!dkx || !dvx || !aligned16(dkx) || !aligned16(dvx)) return BDLM_ERR_INVALID_ARG;
    } else if (!kx && !vx) {
      kx = kc; vx = vc;   // never read without own_block
    }
  } else {
    const void* need[] = {qc, oc, doc, dqc, dkx, dvx};
    for (const void* ptr : need) if (!ptr || !aligned16(ptr)) return BDLM_ERR_INVALID_ARG;
    if (!lse_c || !aligned4(lse_c)) return BDLM_ERR_INVALID_ARG;
  }
  const void* need2[] = {kc, vc, qx, kx, vx, ox, dox, dkc, dvc, dqx};
  for (const void* ptr : need2) if (!ptr || !aligned16(ptr)) return BDLM_ERR_INVALID_ARG;
  if (!lse_x || !aligned4(lse_x)) return BDLM_ERR_INVALID_ARG;
  const BwdLayout lay = bwd_layout(desc);
  int ws_err = BDLM_OK;
  void* ws = ws_of(lay.total, &ws_err);
  if (ws_err != BDLM_OK) return ws_err;

  const int bf = desc->dtype == BDLM_BF16;
  const Problem p = make_problem(desc);
  char* wsb = reinterpret_cast<char*>(ws);
  float* delta[2] = {reinterpret_cast<float*>(wsb + lay.delta_off[0]), reinterpret_cast<float*>(wsb + lay.delta_off[1])};
  float* lse2[2] = {reinterpret_cast<float*>(wsb + lay.lse2_off[0]), reinterpret_cast<float*>(wsb + lay.lse2_off[1])};
  const float* lses[2] = {lse_c, lse_x};
  const int nbg = p.batch * p.hkv;

  // Every launch's arguments and grid are built and checked before the first
  // launch, so an unsupported size enqueues nothing.
  // 1) D = rowsum(dO * O) and LSE * log2(e)
  const void* os[2] = {oc, ox};
  const void* dos[2] = {doc, dox};
  BwdPreArgs pre[2];
  for (int s = share ? 1 : 0; s < 2; ++s) {
    BwdPreArgs& pa = pre[s];
    pa.batch = p.batch; pa.rows = p.rows[s]; pa.hq = p.hq; pa.D = p.D; pa.stream = s;
    pa.o = os[s]; pa.dout = dos[s]; pa.delta = delta[s];
    pa.lse = lses[s]; pa.lse2 = lse2[s];
  }
  // 2) dK, dV: key-major
  BwdArgs ka;
  std::memset(&ka, 0, sizeof(ka));
  ka.p = p;
  ka.q[0] = qc; ka.q[1] = qx;
  ka.k[0] = stage_shift(kc, desc); ka.k[1] = kx;
  ka.v[0] = stage_shift(vc, desc); ka.v[1] = vx;
  ka.dout[0] = doc; ka.dout[1] = dox;
  ka.lse2[0] = lse2[0]; ka.lse2[1] = lse2[1];
  ka.delta[0] = delta[0]; ka.delta[1] = delta[1];
  ka.dk[0] = stage_shift(dkc, desc); ka.dk[1] = dkx;
  ka.dv[0] = stage_shift(dvc, desc); ka.dv[1] = dvx;
  ka.scale = desc->softmax_scale;
  ka.scale_log2 = desc->softmax_scale * 1.4426950408889634f;
  ka.ns0 = share ? 1 : 0;
  if (share) {
    ka.kbase[0] = p.kv_begin; ka.kend[0] = p.kv_end;
    ka.nkt[0] = (p.kv_end - p.kv_begin + kBwdTileN - 1) / kBwdTileN;
    ka.kbase[1] = 0; ka.kend[1] = p.klen[1];
    ka.nkt[1] = p.own_block ? (p.klen[1] + kBwdTileN - 1) / kBwdTileN : 0;
  } else {
    for (int k = 0; k < 2; ++k) {
      ka.kbase[k] = 0; ka.kend[k] = p.L;
      ka.nkt[k] = (p.L + kBwdTileN - 1) / kBwdTileN;
    }
  }
  ka.map = make_map(nbg, ka.nkt[0] + ka.nkt[1]);
  const int64_t kgrid = (int64_t)nbg * (ka.nkt[0] + ka.nkt[1]);
  // 3) dQ: query-major, no atomics (share mode adds into the fp32 dqx)
  DqArgs qa;
  std::memset(&qa, 0, sizeof(qa));
  qa.p = p;
  qa.q[0] = qc; qa.q[1] = qx;
  qa.k[0] = stage_shift(kc, desc); qa.k[1] = kx;
  qa.v[0] = stage_shift(vc, desc); qa.v[1] = vx;
  qa.dout[0] = doc; qa.dout[1] = dox;
  qa.lse2[0] = lse2[0]; qa.lse2[1] = lse2[1];
  qa.delta[0] = delta[0]; qa.delta[1] = delta[1];
  qa.dq[0] = dqc; qa.dq[1] = dqx;
  qa.scale = desc->softmax_scale;
  qa.scale_log2 = desc->softmax_scale * 1.4426950408889634f;
  qa.ns0 = share ? 1 : 0;
  for (int s = 0; s < 2; ++s) qa.nqt[s] = (p.rows[s] + kFwdTileM - 1) / kFwdTileM;
  const int qper_bg = qa.nqt[1] * (2 - qa.ns0) * p.group;
  qa.map = make_map(nbg, qper_bg);
  const int64_t qgrid = (int64_t)nbg * qper_bg;
  if (kgrid > 0x7fffffff || qgrid > 0x7fffffff) return BDLM_ERR_UNSUPPORTED;
  for (int s = share ? 1 : 0; s < 2; ++s) {
    const int64_t threads = (int64_t)pre[s].batch * pre[s].rows * pre[s].hq * (pre[s].D / (bf ? 8 : 4));
    if ((threads + 255) / 256 > 0x7fffffff) return BDLM_ERR_UNSUPPORTED;
  }

  // From here on a HIP launch error leaves the launches before it enqueued.
  for (int s = share ? 1 : 0; s < 2; ++s) {
    ProfScope ps("bdlm_bwd_pre", stream);
    if (launch_bwd_pre(pre[s], bf, stream) != hipSuccess) return BDLM_ERR_HIP;
  }
  if (kgrid > 0) {
    ProfScope ps("bdlm_dkdv", stream);
    if (launch_dkdv(ka, (int)kgrid, bf, stream) != hipSuccess) return BDLM_ERR_HIP;
  }
  if (qgrid > 0) {
    ProfScope ps("bdlm_dq", stream);
    if (launch_dq(qa, (int)qgrid, bf, share ? 1 : 0, stream) != hipSuccess) return BDLM_ERR_HIP;
  }
  return BDLM_OK;
}

// ------------------------------------------------ scratch of the no-alloc call
// The workspace of bdlm_attn_bwd_noalloc: one array per GPU, part of the
// library's device image (no allocation call), held until the process ends.
// Host code never uses the array's name as an address: the device address of
// each GPU's copy comes from hipGetSymbolAddress with that GPU current.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's scratch copy (looked up once per device).
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BDLM_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BDLM_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BDLM_OK;
}

}  // namespace

extern "C" {

int bdlm_attn_bwd(const bdlm_attn_desc* desc, const void* qc, const void* kc, const void* vc,
                  const void* qx, const void* kx, const void* vx, const void* oc, const void* ox,
                  const float* lse_c, const float* lse_x, const void* doc, const void* dox,
                  void* dqc, void* dkc, void* dvc, void* dqx, void* dkx, void* dvx,
                  void* ws, size_t ws_bytes, hipStream_t stream) {
  auto ws_of = [&](size_t need, int* err) -> void* {
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) *err = BDLM_ERR_WORKSPACE;
    return ws;
  };
  return bwd_impl(desc, qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x, doc, dox, dqc, dkc, dvc, dqx, dkx, dvx,
                  ws_of, stream);
}

size_t bdlm_attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

int bdlm_attn_bwd_noalloc(const bdlm_attn_desc* desc, const void* qc, const void* kc, const void* vc,
                          const void* qx, const void* kx, const void* vx, const void* oc, const void* ox,
                          const float* lse_c, const float* lse_x, const void* doc, const void* dox,
                          void* dqc, void* dkc, void* dvc, void* dqx, void* dkx, void* dvx,
                          hipStream_t stream) {
  auto ws_of = [&](size_t need, int* err) -> void* {
    if (need > kScratchBytes) { *err = BDLM_ERR_UNSUPPORTED; return nullptr; }
    void* p = nullptr;
    *err = scratch_of_current_device(&p);
    return p;
  };
  return bwd_impl(desc, qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x, doc, dox, dqc, dkc, dvc, dqx, dkx, dvx,
                  ws_of, stream);
}

int bdlm_attn_merge_partials(int32_t num_parts, int32_t batch, int64_t tokens, int32_t heads,
                             int32_t head_dim, const float* const* o_parts,
                             const float* const* lse_parts, void* o_out, int32_t out_dtype,
                             float* lse_out, hipStream_t stream) {
  if (num_parts < 1 || batch < 1 || tokens < 0 || heads < 1) return BDLM_ERR_INVALID_ARG;
  if (num_parts > BDLM_MAX_MERGE_PARTS) return BDLM_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return BDLM_ERR_UNSUPPORTED;
  if (out_dtype != BDLM_F32 && out_dtype != BDLM_BF16) return BDLM_ERR_INVALID_ARG;
  if (!o_parts || !lse_parts || !o_out || !lse_out) return BDLM_ERR_INVALID_ARG;
  if (!aligned16(o_out) || !aligned4(lse_out)) return BDLM_ERR_INVALID_ARG;
  if ((int64_t)batch * tokens * heads * head_dim > (int64_t(1) << 46)) return BDLM_ERR_UNSUPPORTED;
  MergeArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int j = 0; j < num_parts; ++j) {
    if (!o_parts[j] || !lse_parts[j] || !aligned16(o_parts[j]) || !aligned4(lse_parts[j])) return BDLM_ERR_INVALID_ARG;
    // only part 0 may alias the output (and then only for fp32 output)
    if (o_parts[j] == o_out && (j > 0 || out_dtype != BDLM_F32)) return BDLM_ERR_INVALID_ARG;
    if (lse_parts[j] == lse_out && j > 0) return BDLM_ERR_INVALID_ARG;
    a.o[j] = o_parts[j];
    a.lse[j] = lse_parts[j];
  }
  a.nparts = num_parts; a.batch = batch; a.tokens = tokens; a.heads = heads; a.D = head_dim;
  a.o_out = o_out; a.lse_out = lse_out;
  a.inplace = (o_parts[0] == o_out && lse_parts[0] == lse_out) ? 1 : 0;
  ProfScope ps("bdlm_merge", stream);
  return launch_merge(a, out_dtype == BDLM_BF16, stream) == hipSuccess ? BDLM_OK : BDLM_ERR_HIP;
}

int bdlm_attn_schedule_walk(const bdlm_attn_desc* desc, int for_bwd, uint8_t* cover, int64_t cover_len,
                            int64_t* stats) {
  int st = check_desc(desc);
  if (st != BDLM_OK) return st;
  if (for_bwd < 0 || for_bwd > 2) return BDLM_ERR_INVALID_ARG;
  // the walk reports clean keys by their position in the clean sequence,
  // whether or not the call's window is staged
  bdlm_attn_desc unstaged = *desc;
  unstaged.kv_staged = 0;
  const Problem p = make_problem(&unstaged);
  const int64_t nrows = (int64_t)p.rows[0] + p.rows[1];
  const int64_t nkeys = (int64_t)p.klen[0] + p.klen[1];
  if (cover && cover_len < nrows * nkeys) return BDLM_ERR_INVALID_ARG;
  int64_t wgs = 0, visits = 0, masked = 0, pairs = 0, bad = 0;
  const int roff[2] = {0, p.rows[0]};
  const int koff[2] = {0, p.klen[0]};
  auto mark = [&](int s, int r, int a, int k) {
    ++pairs;
    if (r < 0 || r >= p.rows[s] || k < 0 || k >= p.klen[a]) { ++bad; return; }
    if (cover) {
      uint8_t& c = cover[(roff[s] + (int64_t)r) * nkeys + koff[a] + k];
      if (c < 255) ++c;
    }
  };
  const int nbg = p.batch * p.hkv;
  if (for_bwd != 1) {   // forward and dQ kernels share the query-major decomposition
    const int ns0 = p.mode == 0 ? 0 : 1, nstr = 2 - ns0;
    int nqt[2];
    for (int s = 0; s < 2; ++s) nqt[s] = (p.rows[s] + kFwdTileM - 1) / kFwdTileM;
    const int per_bg = nqt[1] * nstr * p.group;
    const XcdMap map = make_map(nbg, per_bg);
    wgs = (int64_t)nbg * per_bg;
    std::vector<uint8_t> seen((size_t)wgs, 0);
    for (int64_t wg = 0; wg < wgs; ++wg) {
      int bg, item;
      map.decode((int)wg, bg, item);
      if (bg < 0 || bg >= nbg || item < 0 || item >= per_bg || seen[(size_t)bg * per_bg + item]++) { ++bad; continue; }
      const int hg = item % p.group, rest = item / p.group;
      const int s = ns0 + rest % nstr, t = nqt[s] - 1 - rest / nstr;
      if (bg != 0 || hg != 0) continue;
      const int r0 = t * kFwdTileM, r1 = std::min(r0 + kFwdTileM, p.rows[s]);
      for (int a = 0; a < 2; ++a) {
        int klo, khi, flo, fhi;
        tile_ranges(p, s, a, r0, r1, klo, khi, flo, fhi);
        if (klo >= khi) continue;
        for (int k0 = klo; k0 < khi; k0 += 64) {
          ++visits;
          // the forward and dQ kernels' own element-mask tests
          const bool need_mask = for_bwd == 0 ? key_tile_partial(k0, 64, flo, fhi)
                                              : qmajor_tile_masked(k0, 64, flo, fhi, r0, r1, kFwdTileM);
          masked += need_mask;
          for (int r = r0; r < r1; ++r) {
            int lo, hi;
            row_keys(p, s, r, a, lo, hi);
            for (int k = k0; k < k0 + 64; ++k) {
              if (need_mask ? (k >= lo && k < hi) : true) mark(s, r, a, k);
            }
          }
        }
      }
    }
  } else {
    // the dK/dV kernel's iteration order and packed per-iteration decode
    const int ns0 = p.mode == 0 ? 0 : 1;
    int nkt[2], kbase[2], kend[2];
    if (p.mode == 1) {
      kbase[0] = p.kv_begin; kend[0] = p.kv_end; nkt[0] = (p.kv_end - p.kv_begin + kBwdTileN - 1) / kBwdTileN;
      kbase[1] = 0; kend[1] = p.klen[1]; nkt[1] = p.own_block ? (p.klen[1] + kBwdTileN - 1) / kBwdTileN : 0;
    } else {
      for (int a = 0; a < 2; ++a) { kbase[a] = 0; kend[a] = p.L; nkt[a] = (p.L + kBwdTileN - 1) / kBwdTileN; }
    }
    const int per_bg = nkt[0] + nkt[1];
    const XcdMap map = make_map(nbg, per_bg);
    wgs = (int64_t)nbg * per_bg;
    std::vector<uint8_t> seen((size_t)wgs, 0);
    const int M = desc->dtype == BDLM_BF16 ? 64 : 32;
    for (int64_t wg = 0; wg < wgs; ++wg) {
      int bg, item;
      map.decode((int)wg, bg, item);
      if (bg < 0 || bg >= nbg || item < 0 || item >= per_bg || seen[(size_t)bg * per_bg + item]++) { ++bad; continue; }
      if (bg != 0) continue;
      const int a = item < nkt[0] ? 0 : 1;
      const int j = a == 0 ? item : item - nkt[0];
      const int k0 = kbase[a] + j * kBwdTileN, k1 = std::min(k0 + kBwdTileN, kend[a]);
      BwdOrder ord;
      ord.init(p, a, ns0, k0, k1, M);
      for (int it = 0; it < ord.total; ++it) {
        const unsigned e = bwd_entry(p, ord, a, k0, kBwdTileN, M, it);
        if (entry_head(e) != 0) continue;          // q-head 0 of kv head 0
        const int s = entry_stream(e);
        const int q0 = entry_tile(e) * M, q1 = std::min(q0 + M, p.rows[s]);
        const bool need_mask = entry_masked(e);
        ++visits;
        masked += need_mask;
        // unmasked: every row of the M-row tile and every key of the workgroup
        for (int r = q0; r < (need_mask ? q1 : q0 + M); ++r) {
          int lo = 0, hi = 0;
          if (r < p.rows[s]) row_keys(p, s, r, a, lo, hi);
          for (int k = k0; k < k1; ++k) {
            if (need_mask ? (k >= lo && k < hi) : true) mark(s, r, a, k);
          }
        }
      }
    }
  }
  if (stats) { stats[0] = wgs; stats[1] = visits; stats[2] = masked; stats[3] = pairs; stats[4] = bad; }
  return BDLM_OK;
}

int bdlm_attn_profile_begin(int32_t max_launches) {
  if (max_launches < 1) return BDLM_ERR_INVALID_ARG;
  if (g_prof.on) return BDLM_ERR_INVALID_ARG;
  g_prof.pool.assign(2 * (size_t)max_launches, nullptr);
  for (auto& e : g_prof.pool) {
    if (hipEventCreate(&e) != hipSuccess) {
      for (auto& x : g_prof.pool) if (x) (void)hipEventDestroy(x);
      g_prof.pool.clear();
      return BDLM_ERR_HIP;
    }
  }
  g_prof.used.clear();
  g_prof.used.reserve(max_launches);
  g_prof.next = 0;
  g_prof.on = true;
  return BDLM_OK;
}

int bdlm_attn_profile_end(bdlm_kernel_time* out, int32_t max_entries, int32_t* num_entries) {
  if (!g_prof.on) return BDLM_ERR_INVALID_ARG;
  g_prof.on = false;
  std::vector<bdlm_kernel_time> acc;
  int status = BDLM_OK;
  for (auto& e : g_prof.used) {
    float ms = 0.f;
    if (hipEventSynchronize(e.b) != hipSuccess || hipEventElapsedTime(&ms, e.a, e.b) != hipSuccess) {
      status = BDLM_ERR_HIP;
      continue;
    }
    bdlm_kernel_time* slot = nullptr;
    for (auto& x : acc) if (std::strncmp(x.name, e.name, sizeof(x.name)) == 0) slot = &x;
    if (!slot) {
      bdlm_kernel_time t;
      std::memset(&t, 0, sizeof(t));
      std::strncpy(t.name, e.name, sizeof(t.name) - 1);
      acc.push_back(t);
      slot = &acc.back();
    }
    slot->launches += 1;
    slot->total_ms += ms;
  }
  for (auto& e : g_prof.pool) (void)hipEventDestroy(e);
  g_prof.pool.clear();
  g_prof.used.clear();
  const int n = (int)acc.size() < max_entries ? (int)acc.size() : max_entries;
  for (int i = 0; i < n && out; ++i) out[i] = acc[i];
  if (num_entries) *num_entries = n;
  return status;
}

}  // extern "C"
