// attn_api.cpp - the C ABI declared in include/attn.h: host-side argument
// validation, then dispatch to the kernel launchers on the caller's stream.
#include "attn.h"

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "attn_launch.h"

namespace {

constexpr int kAbiVersion = 9;

// Device scratch of attn_bwd_noalloc: the D vector (one fp32 per query row)
// that attn_bwd keeps in the caller's workspace.  16 MiB per GPU, so
// B * H * N <= 4,194,304 rows.  In host code `scratch` names a host-side
// stand-in, never the device address: that comes from hipGetSymbolAddress,
// once per device, and is what every kernel argument uses.
constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};  // device address of `scratch`, per device

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept for the life of the process.
int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// lse is read and written one float at a time
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// The pages scale Q K^T by 1/sqrt(d) before the softmax, a positive number;
// the kernels rely on scale > 0 (the row maximum is taken on the unscaled
// scores, and masked scores are -inf before the scaling).  Zero, -0.0,
// negative and non-finite scales are refused.
bool scale_ok(float scale) { return isfinite(scale) && scale > 0.f; }

// Shape checks shared by every entry point.  Element counts must fit in
// int64 offsets and the workgroup count in a 32-bit grid: the finest grid is
// the fp32 forward's and the preprocess's, one workgroup per 32 query rows.
int check_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
  if (!attn::head_dim_supported(d)) return ATTN_ERR_HEADDIM;
  const int64_t bh = (int64_t)B * (int64_t)H;
  if (bh > (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  const int64_t tiles = bh * (((int64_t)N + 31) / 32);
  if (tiles > (int64_t)INT32_MAX) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

namespace attn {
size_t bwd_delta_bytes(int B, int H, int Nq) {
  return round256((size_t)B * (size_t)H * (size_t)Nq * sizeof(float));
}
}  // namespace attn

extern "C" {

int attn_abi_version(void) { return kAbiVersion; }

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "B, H and N must be >= 1 and the sizes must fit 64-bit offsets";
    case ATTN_ERR_DTYPE: return "dtype not supported by this entry point";
    case ATTN_ERR_HEADDIM:
      return "head dimension d must be 32, 64, 96, 128 or 256 (attn_fwd_mx: 64 or 128)";
    case ATTN_ERR_ALIGN: return "pointers must be 16-byte aligned (lse: 4-byte)";
    case ATTN_ERR_SCALE: return "scale must be finite and > 0";
    case ATTN_ERR_WORKSPACE:
      return "workspace is NULL or smaller than the matching *_workspace_bytes()";
    case ATTN_ERR_HIP: return "the HIP runtime refused the kernel launch";
    case ATTN_ERR_SCRATCH:
      return "B*H*N exceeds the static scratch of attn_bwd_noalloc (4194304 query rows)";
    default: return "unknown attn status";
  }
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int N, int d, int causal, float scale, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  int rc = check_shape(B, H, N, d);
  if (rc != ATTN_OK) return rc;
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F32) return ATTN_ERR_DTYPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return ATTN_ERR_ALIGN;
  if (!scale_ok(scale)) return ATTN_ERR_SCALE;
  attn::FwdArgs a{q, k, v, o, lse, B, H, N, d, causal != 0, scale, dtype == ATTN_DTYPE_BF16,
                  stream};
  return attn::launch_fwd(a) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

size_t attn_bwd_workspace_bytes(int B, int H, int N, int d, int dtype) {
  if (check_shape(B, H, N, d) != ATTN_OK || !attn::bwd_head_dim_supported(d) ||
      dtype != ATTN_DTYPE_BF16)
    return 0;
  return attn::bwd_delta_bytes(B, H, N);
}

// Every check of the backward except the workspace.
static int bwd_check(int phase, const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, const void* dq, const void* dk,
                     const void* dv, int B, int H, int N, int d, float scale, int dtype) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_ERR_NULL;
  int rc = check_shape(B, H, N, d);
  if (rc != ATTN_OK) return rc;
  if (!attn::bwd_head_dim_supported(d)) return ATTN_ERR_HEADDIM;
  if (phase < -1 || phase > 3) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_DTYPE_BF16) return ATTN_ERR_DTYPE;
  const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_ALIGN;
  if (!aligned4(lse)) return ATTN_ERR_ALIGN;
  if (!scale_ok(scale)) return ATTN_ERR_SCALE;
  return ATTN_OK;
}

static int bwd_common(int phase, const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                      int causal, float scale, int dtype, void* stream) {
  int rc = bwd_check(phase, q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, dtype);
  if (rc != ATTN_OK) return rc;
  const size_t need = attn_bwd_workspace_bytes(B, H, N, d, dtype);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
  attn::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace, B, H, N, N, d,
                  causal != 0, scale, stream};
  const hipError_t e = phase < 0 ? attn::launch_bwd(a) : attn::launch_bwd_phase(a, phase);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, void* workspace,
             size_t workspace_bytes, int B, int H, int N, int d, int causal, float scale,
             int dtype, void* stream) {
  return bwd_common(-1, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N,
                    d, causal, scale, dtype, stream);
}

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                     int H, int N, int d, int causal, float scale, int dtype, void* stream) {
  int rc = bwd_check(-1, q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, dtype);
  if (rc != ATTN_OK) return rc;
  if ((size_t)B * (size_t)H * (size_t)N * sizeof(float) > kNoallocScratchBytes)
    return ATTN_ERR_SCRATCH;
  void* ws = nullptr;
  rc = noalloc_scratch(&ws);
  if (rc != ATTN_OK) return rc;
  // the same kernels as attn_bwd; the dQ kernel writes every D entry that
  // the dK/dV kernel reads, so nothing in the scratch needs clearing
  attn::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, (float*)ws, B, H, N, N, d, causal != 0,
                  scale, stream};
  return attn::launch_bwd(a) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_bwd_phase(int phase, const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                   int causal, float scale, int dtype, void* stream) {
  if (phase < 0 || phase > 3) return ATTN_ERR_SHAPE;
  return bwd_common(phase, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H,
                    N, d, causal, scale, dtype, stream);
}

// Sizes of attn_fwd_kv: both sequence lengths >= 1, the causal alignment
// needs Nk >= Nq, and the grid (B*H*ceil(Nq/128)*splits workgroups, at most
// B*H*ceil(Nq/128)*ceil(Nk/64)) must fit a 32-bit count.
static int check_kv_shape(int B, int H, int Nq, int Nk, int d, int causal, int num_splits) {
  if (Nq < 1 || Nk < 1 || num_splits < 0) return ATTN_ERR_SHAPE;
  if ((int64_t)Nq + (int64_t)Nk >= (int64_t)INT32_MAX) return ATTN_ERR_SHAPE;
  if (causal && Nk < Nq) return ATTN_ERR_SHAPE;
  int rc = check_shape(B, H, Nq > Nk ? Nq : Nk, d);
  if (rc != ATTN_OK) return rc;
  const int64_t wgs = (int64_t)B * H * (((int64_t)Nq + 127) / 128) * (((int64_t)Nk + 63) / 64);
  if (wgs > (int64_t)INT32_MAX) return ATTN_ERR_SHAPE;
  // the merge runs one workgroup per 4 query rows
  if (((int64_t)B * H * Nq + 3) / 4 > (int64_t)INT32_MAX) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

size_t attn_fwd_kv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits,
                                   int dtype) {
  if (check_kv_shape(B, H, Nq, Nk, d, 0, num_splits) != ATTN_OK || dtype != ATTN_DTYPE_BF16)
    return 0;
  const attn::KvSplit sp = attn::kv_split_plan(B, H, Nq, Nk, d, num_splits);
  return sp.o_part_bytes + sp.lse_part_bytes;
}

int attn_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int Nq, int Nk, int d, int causal, float scale, int dtype, int num_splits,
                void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  int rc = check_kv_shape(B, H, Nq, Nk, d, causal, num_splits);
  if (rc != ATTN_OK) return rc;
  if (dtype != ATTN_DTYPE_BF16) return ATTN_ERR_DTYPE;
  const void* ptrs[] = {q, k, v, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_ALIGN;
  if (!aligned4(lse)) return ATTN_ERR_ALIGN;
  if (!scale_ok(scale)) return ATTN_ERR_SCALE;
  const size_t need = attn_fwd_kv_workspace_bytes(B, H, Nq, Nk, d, num_splits, dtype);
  if (need > 0) {  // one chunk needs none and ignores the workspace arguments
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
  }
  attn::FwdKvArgs a{q, k, v, o, lse, B, H, Nq, Nk, d, causal != 0, scale, num_splits,
                    workspace, stream};
  return attn::launch_fwd_kv(a) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

size_t attn_bwd_kv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int dtype) {
  if (check_kv_shape(B, H, Nq, Nk, d, 0, 0) != ATTN_OK || !attn::bwd_head_dim_supported(d) ||
      dtype != ATTN_DTYPE_BF16)
    return 0;
  return attn::bwd_delta_bytes(B, H, Nq) + attn::bwd_dq_split_plan(B, H, Nq, Nk, d).part_bytes;
}

int attn_bwd_kv(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, void* workspace,
                size_t workspace_bytes, int B, int H, int Nq, int Nk, int d, int causal,
                float scale, int dtype, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_ERR_NULL;
  int rc = check_kv_shape(B, H, Nq, Nk, d, causal, 0);
  if (rc != ATTN_OK) return rc;
  if (!attn::bwd_head_dim_supported(d)) return ATTN_ERR_HEADDIM;
  if (dtype != ATTN_DTYPE_BF16) return ATTN_ERR_DTYPE;
  const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_ALIGN;
  if (!aligned4(lse)) return ATTN_ERR_ALIGN;
  if (!scale_ok(scale)) return ATTN_ERR_SCALE;
  const size_t need = attn_bwd_kv_workspace_bytes(B, H, Nq, Nk, d, dtype);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
  attn::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace, B, H, Nq, Nk, d,
                  causal != 0, scale, stream};
  const attn::BwdDqSplit sp = attn::bwd_dq_split_plan(B, H, Nq, Nk, d);
  if (sp.splits > 1) {
    a.dq_part = (float*)((char*)workspace + attn::bwd_delta_bytes(B, H, Nq));
    a.dq_splits = sp.splits;
    a.dq_chunk = sp.chunk;
  }
  return attn::launch_bwd(a) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd_mx(const void* q8, const void* q_scale, const void* k8, const void* k_scale,
                const void* v, void* o, float* lse, int B, int H, int N, int d, int causal,
                float scale, void* stream) {
  if (!q8 || !q_scale || !k8 || !k_scale || !v || !o || !lse) return ATTN_ERR_NULL;
  int rc = check_shape(B, H, N, d);
  if (rc != ATTN_OK) return rc;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return ATTN_ERR_ALIGN;
  // scale rows are d / 32 bytes, read as one 16- or 32-bit word
  const uintptr_t salign = d == 128 ? 3u : 1u;
  if ((reinterpret_cast<uintptr_t>(q_scale) & salign) || (reinterpret_cast<uintptr_t>(k_scale) & salign))
    return ATTN_ERR_ALIGN;
  if (!scale_ok(scale)) return ATTN_ERR_SCALE;
  attn::FwdMxArgs a{q8, q_scale, k8, k_scale, v, nullptr, nullptr, o, lse, B, H, N, d,
                    causal != 0, scale, stream};
  return attn::launch_fwd_mx(a) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd_fp8(const void* q8, const void* q_scale, const void* k8, const void* k_scale,
                 const void* vt8, const void* vt_scale, void* o, float* lse, int B, int H, int N,
                 int d, int causal, float scale, void* stream) {
  if (!q8 || !q_scale || !k8 || !k_scale || !vt8 || !vt_scale || !o || !lse) return ATTN_ERR_NULL;
  int rc = check_shape(B, H, N, d);
  if (rc != ATTN_OK) return rc;
  // V^T rows of 64 ceil(N / 64) bytes: 16 rows of them must stay within the
  // 32-bit offsets of one copy instruction
  if (N > (1 << 26)) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(vt8) || !aligned16(o) || !aligned4(lse))
    return ATTN_ERR_ALIGN;
  const uintptr_t salign = d == 128 ? 3u : 1u;
  if ((reinterpret_cast<uintptr_t>(q_scale) & salign) ||
      (reinterpret_cast<uintptr_t>(k_scale) & salign) ||
      (reinterpret_cast<uintptr_t>(vt_scale) & 1u))
    return ATTN_ERR_ALIGN;
  if (!scale_ok(scale)) return ATTN_ERR_SCALE;
  attn::FwdMxArgs a{q8, q_scale, k8, k_scale, nullptr, vt8, vt_scale, o, lse, B, H, N, d,
                    causal != 0, scale, stream};
  return attn::launch_fwd_mx(a) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_softmax_rows(const void* x, void* y, long long M, int N, int dtype, void* stream) {
  if (!x || !y) return ATTN_ERR_NULL;
  if (M < 1 || N < 1) return ATTN_ERR_SHAPE;
  // M * N elements (at most 2^48) must stay addressable with 64-bit offsets;
  // checked by division, since the product itself may overflow
  if (M > (1LL << 40) || (long long)N > (1LL << 48) / M) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_DTYPE;
  if (!aligned16(x) || !aligned16(y)) return ATTN_ERR_ALIGN;
  attn::SoftmaxArgs a{x, y, (int64_t)M, N, dtype == ATTN_DTYPE_BF16, stream};
  return attn::launch_softmax_rows(a) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
