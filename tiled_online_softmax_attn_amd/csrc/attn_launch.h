// attn_launch.h - internal interface between the C ABI (attn_api.cpp) and the
// kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Head dimensions the kernels are built for (every forward and the backward).
constexpr bool head_dim_supported(int d) {
  return d == 32 || d == 64 || d == 96 || d == 128 || d == 256;
}
constexpr bool bwd_head_dim_supported(int d) { return head_dim_supported(d); }

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

// Backward of Nq queries against Nk keys and values.  Square attention
// (attn_bwd) has Nq = Nk = N; the backward of attn_fwd_kv (attn_bwd_kv) has
// the queries at the last Nq positions, so under the causal mask query i
// sees keys 0 .. i + Nk - Nq.
struct BwdArgs {
  const void* q;     // [B][H][Nq][d]
  const void* k;     // [B][H][Nk][d]
  const void* v;     // [B][H][Nk][d]
  const void* o;     // [B][H][Nq][d]
  const void* dout;  // [B][H][Nq][d]
  const float* lse;  // [B][H][Nq]
  void* dq;          // [B][H][Nq][d]
  void* dk;          // [B][H][Nk][d]
  void* dv;          // [B][H][Nk][d]
  float* delta;  // [B][H][Nq] fp32 workspace: D = rowsum(dO * O)
  int B, H, Nq, Nk, d;
  int causal;
  float scale;
  void* stream;
  // dQ split over the keys (bwd_dq_split_plan): dq_splits chunks of dq_chunk
  // keys, fp32 partials [dq_splits][B*H*Nq][d] in dq_part, summed into dq.
  float* dq_part = nullptr;
  int dq_splits = 1;
  int dq_chunk = 0;
};

// How the dQ phase cuts the keys: with few queries (Nq < Nk) a head has too
// few 128-query workgroups to fill the chip, so `splits` workgroups share a
// query tile, each summing dS K over `chunk` keys (whole 64-key tiles) into
// an fp32 partial; part_bytes is their workspace, rounded up to 256.
struct BwdDqSplit {
  int splits;
  int chunk;
  size_t part_bytes;
};
BwdDqSplit bwd_dq_split_plan(int B, int H, int Nq, int Nk, int d);

// Nq queries (the last Nq positions) against Nk keys, the keys cut into
// chunks processed by separate workgroups and merged (attn_fwd_kv).
struct FwdKvArgs {
  const void* q;  // [B][H][Nq][d] bf16
  const void* k;  // [B][H][Nk][d] bf16
  const void* v;  // [B][H][Nk][d] bf16
  void* o;        // [B][H][Nq][d] bf16
  float* lse;     // [B][H][Nq]
  int B, H, Nq, Nk, d;
  int causal;
  float scale;
  int num_splits;   // 0 = chosen from the shape
  void* workspace;  // kv_split_plan(...).o_part_bytes + lse_part_bytes (0 for one chunk)
  void* stream;
};

// How attn_fwd_kv cuts the keys: `splits` chunks of `chunk` keys (a multiple
// of the 64-key tile; the last chunk may be shorter), and the workspace it
// needs for the partial results (none with one chunk).
struct KvSplit {
  int splits;
  int chunk;
  size_t o_part_bytes;    // fp32 [splits][B*H][Nq][d], rounded up to 256; 0 if splits == 1
  size_t lse_part_bytes;  // fp32 [splits][B*H][Nq], rounded up to 256; 0 if splits == 1
};
KvSplit kv_split_plan(int B, int H, int Nq, int Nk, int d, int num_splits);
// The forward kernel of attn_fwd over chunk `split` of the keys, for every
// chunk (B*H*ceil(Nq/128)*splits workgroups): each chunk's O_c (fp32,
// normalised by the chunk's own sum) and lse_c into o_part / lse_part.
hipError_t launch_fwd_kv_partial(const FwdKvArgs& a, const KvSplit& sp, float* o_part,
                                 float* lse_part);
// One chunk: the same kernel over all Nk keys (B*H*ceil(Nq/128) workgroups)
// writes bf16 O and lse itself; no partial results, no merge.
hipError_t launch_fwd_kv_whole(const FwdKvArgs& a);

// Forward with Q and K in MXFP8 (E4M3 codes, one E8M0 scale per 32 elements
// along d) and V in bf16 (attn_fwd_mx).
// With vt8 set (attn_fwd_fp8), V arrives transposed in MXFP8 instead: V^T
// E4M3 codes [B][H][d][ldv] with one E8M0 scale per 32 keys [B][H][d][ldv /
// 32], ldv = 64 ceil(N / 64); P is rounded to E4M3 for P V.
struct FwdMxArgs {
  const void* q8;       // [B][H][N][d] E4M3
  const void* q_scale;  // [B][H][N][d / 32] E8M0
  const void* k8;
  const void* k_scale;
  const void* v;        // [B][H][N][d] bf16 (attn_fwd_mx)
  const void* vt8;      // [B][H][d][ldv] E4M3 (attn_fwd_fp8), else null
  const void* vt_scale; // [B][H][d][ldv / 32] E8M0
  void* o;              // [B][H][N][d] bf16
  float* lse;           // [B][H][N]
  int B, H, N, d;
  int causal;
  float scale;
  void* stream;
};
hipError_t launch_fwd_mx(const FwdMxArgs& a);

// Row-wise softmax of an M x N row-major matrix (attn_softmax_rows).
struct SoftmaxArgs {
  const void* x;
  void* y;
  int64_t M;
  int N;
  bool bf16;
  void* stream;
};
hipError_t launch_softmax_rows(const SoftmaxArgs& a);

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_fwd_kv(const FwdKvArgs& a);
hipError_t launch_bwd(const BwdArgs& a);
// phase 0 = preprocess (D), 1 = dK and dV, 2 = dQ
hipError_t launch_bwd_phase(const BwdArgs& a, int phase);
// phase 1 alone (dK and dV; attn_bwd_dkdv.hip)
hipError_t launch_bwd_dkdv(const BwdArgs& a);

// Workspace of the backward: the D vector (one fp32 per query row), rounded
// up to 256 bytes.
size_t bwd_delta_bytes(int B, int H, int Nq);

}  // namespace attn
