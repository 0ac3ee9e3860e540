// Kernel argument blocks and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bdlm_common.h"

namespace bdlm {

struct FwdArgs {
  Problem p;
  const void* q[2];     // per stream (0 clean, 1 corrupted/local)
  const void* k[2];     // per key array (0 clean, 1 corrupted/local)
  const void* v[2];
  void* o[2];
  float* lse[2];
  float scale_log2;     // softmax_scale * log2(e)
  int nqt[2];           // 128-row query tiles per stream
  int ns0;              // first stream with queries (0 full, 1 share)
  int accum;            // share mode: merge into the (O, LSE) already in o/lse (fp32 O)
  XcdMap map;
};

struct BwdPreArgs {
  int batch, rows, hq, D, stream;
  const void* o;
  const void* dout;
  float* delta;         // [batch, hq, rows]: rowsum(dO * O)
  const float* lse;     // [batch, hq, rows]: forward LSE (natural log)
  float* lse2;          // [batch, hq, rows]: LSE * log2(e)
};

struct BwdArgs {
  Problem p;
  const void* q[2];
  const void* k[2];
  const void* v[2];
  const void* dout[2];
  const float* lse2[2];   // LSE * log2(e) per query stream
  const float* delta[2];
  void* dk[2];
  void* dv[2];
  float scale, scale_log2;
  int nkt[2];           // 128-key tiles per key array
  int kbase[2];         // first key of tile 0
  int kend[2];          // one past the last key
  int ns0;
  XcdMap map;
};

struct DqArgs {
  Problem p;
  const void* q[2];
  const void* k[2];
  const void* v[2];
  const void* dout[2];
  const float* lse2[2];   // LSE * log2(e) per query stream
  const float* delta[2];
  void* dq[2];          // dtype (full mode) or fp32 to add into (share mode)
  float scale, scale_log2;
  int nqt[2];           // 128-row query tiles per stream
  int ns0;
  XcdMap map;
};

struct MergeArgs {
  int nparts, batch, heads, D;
  int inplace;          // 1: o_out/lse_out alias part 0
  int64_t tokens;
  const float* o[kMaxMergeParts];
  const float* lse[kMaxMergeParts];
  void* o_out;
  float* lse_out;
};

constexpr int kFwdTileM = 128;
constexpr int kBwdTileN = 128;

hipError_t launch_fwd(const FwdArgs& a, int grid, int is_bf16, int out_f32, hipStream_t st);
hipError_t launch_bwd_pre(const BwdPreArgs& a, int is_bf16, hipStream_t st);
hipError_t launch_dkdv(const BwdArgs& a, int grid, int is_bf16, hipStream_t st);
hipError_t launch_dq(const DqArgs& a, int grid, int is_bf16, int add_f32, hipStream_t st);
hipError_t launch_merge(const MergeArgs& a, int out_bf16, hipStream_t st);

}  // namespace bdlm
