// attn_launch.h - internal interface between the C ABI (attn_api.cpp) and the
// kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace attn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d;
  int causal;
  float scale;
  bool bf16;
  void* stream;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // [B][H][N] fp32 workspace: D = rowsum(dO * O)
  int B, H, N, d;
  int causal;
  float scale;
  void* stream;
};

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd(const BwdArgs& a);
// phase 0 = preprocess (D), 1 = dK and dV, 2 = dQ
hipError_t launch_bwd_phase(const BwdArgs& a, int phase);

// Workspace of the backward: the D vector, rounded up to 256 bytes.
size_t bwd_delta_bytes(int B, int H, int N);

}  // namespace attn
