// attn_fwd_kv.hip - forward of Nq queries against an Nk-key cache, split over
// the keys (decode- and prefill-shaped attention; gfx950, bf16 in and out).
//
// The queries are the last Nq positions of an Nk-token sequence (query i sits
// at position i + Nk - Nq; under the causal mask it sees keys 0 .. i + Nk -
// Nq).  With few queries a head has too little work to fill 256 CUs, and the
// pass is bound by reading K and V from HBM (one token per request and step
// reuses every loaded key once: CS336 Lecture 5 notes "GPUs, TPUs", section
// 5.3).  So the key range is cut into `splits` chunks that separate
// workgroups stream concurrently.  Each chunk gives a partial result for every
// query, its own softmax-normalised O_c and logsumexp lse_c over the chunk's
// keys, and a second kernel merges them with the blocked-softmax identity
// (CS149 Lecture 9 notes "Efficiently Evaluating DNNs on GPUs", section 9):
//   lse = ln sum_c e^{lse_c},   O = sum_c e^{lse_c - lse} O_c.
// Each chunk is walked by the forward kernel itself (attn_fwd.hip, its
// partial-result instantiation: section 8.3 of the CS336 notes, S^T = K Q^T
// on MFMA with the lane owning one query, a lazily moved reference maximum,
// base-2 exponentials and O^T += V^T P^T); this file holds the split plan and
// the merge.  A plan of one chunk (many query tiles already fill the chip)
// skips both: the forward kernel walks all keys and writes O and lse.
#include "device_common.h"
#include "attn_launch.h"

#include <algorithm>
#include <type_traits>

namespace attn {
namespace {

constexpr int kKvBQ = 128;  // queries per workgroup of the forward kernel
constexpr int kKvBK = 64;   // keys per K/V tile (chunks are whole tiles)

// Merge of the chunks' partial results, one wave per query row:
//   lse = m + ln sum_c e^{lse_c - m} (m = max_c lse_c),
//   O = sum_c e^{lse_c - lse} O_c, stored as bf16.
// Every query sees at least one key, so some lse_c is finite.
template <int D>
__global__ void __launch_bounds__(256)
attn_fwd_kv_merge_kernel(const float* __restrict__ o_part, const float* __restrict__ lse_part,
                         __bf16* __restrict__ o, float* __restrict__ lse, int64_t rows,
                         int splits) {
  constexpr int PER = (D + 63) / 64;  // columns per lane: lane, lane + 64, ...
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float m = -INFINITY;
  for (int c = 0; c < splits; ++c) m = fmaxf(m, lse_part[c * rows + row]);
  float wsum = 0.f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int c = 0; c < splits; ++c) {
    const float lc = lse_part[c * rows + row];
    const float w = lc == -INFINITY ? 0.f : fast_exp2((lc - m) * kLog2e);
    wsum += w;
    const float* src = o_part + (c * rows + row) * D + lane;
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (e * 64 + lane < D) acc[e] = fmaf(w, src[e * 64], acc[e]);
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (e * 64 + lane < D) o[row * D + e * 64 + lane] = (__bf16)(acc[e] * inv);
  if (lane == 0) lse[row] = m + kLn2 * fast_log2(wsum);
}

template <int D>
hipError_t launch_kv(const FwdKvArgs& a, const KvSplit& sp) {
  // one chunk: partials and a merge would only copy O through fp32 (B2 H16
  // N4096 d64, 1024 query tiles: 199 us that way, 179 direct; causal 120, 98)
  if (sp.splits == 1) return launch_fwd_kv_whole(a);
  const int BH = a.B * a.H;
  const hipStream_t s = (hipStream_t)a.stream;
  float* o_part = (float*)a.workspace;
  float* lse_part = (float*)((char*)a.workspace + sp.o_part_bytes);
  const hipError_t e = launch_fwd_kv_partial(a, sp, o_part, lse_part);
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)BH * a.Nq;
  hipLaunchKernelGGL((attn_fwd_kv_merge_kernel<D>), dim3((unsigned)((rows + 3) / 4)), dim3(256),
                     0, s, (const float*)o_part, (const float*)lse_part, (__bf16*)a.o, a.lse,
                     rows, sp.splits);
  return hipGetLastError();
}

}  // namespace

KvSplit kv_split_plan(int B, int H, int Nq, int Nk, int d, int num_splits) {
  KvSplit sp{};
  const int64_t BH = (int64_t)B * H;
  const int64_t n_qtiles = (Nq + kKvBQ - 1) / kKvBQ;
  const int64_t tiles = (Nk + kKvBK - 1) / kKvBK;
  int64_t want = num_splits;
  if (want <= 0) {
    // about two workgroups per CU in total (the forward kernel's occupancy),
    // each chunk at least four tiles: more chunks shorten every stream and
    // add partial-result traffic (decode B8 H32 Nq1 Nk8192 d128: 2 chunks
    // 181 us, 4 183, 8 191; prefill B2 H16 Nq512 Nk4096 d128: 4 chunks 51 us,
    // 8 67)
    const int64_t base = BH * n_qtiles;
    want = (512 + base - 1) / base;
    want = std::min<int64_t>(want, std::max<int64_t>(1, tiles / 4));
  }
  want = std::max<int64_t>(1, std::min<int64_t>(want, tiles));
  const int64_t tiles_per_chunk = (tiles + want - 1) / want;
  sp.chunk = (int)(tiles_per_chunk * kKvBK);
  sp.splits = (int)((tiles + tiles_per_chunk - 1) / tiles_per_chunk);
  if (sp.splits == 1) return sp;  // the forward kernel writes O and lse itself
  const size_t rows = (size_t)sp.splits * (size_t)BH * (size_t)Nq;
  sp.o_part_bytes = (rows * (size_t)d * sizeof(float) + 255) & ~(size_t)255;
  sp.lse_part_bytes = (rows * sizeof(float) + 255) & ~(size_t)255;
  return sp;
}

hipError_t launch_fwd_kv(const FwdKvArgs& a) {
  const KvSplit sp = kv_split_plan(a.B, a.H, a.Nq, a.Nk, a.d, a.num_splits);
  switch (a.d) {
    case 32: return launch_kv<32>(a, sp);
    case 64: return launch_kv<64>(a, sp);
    case 96: return launch_kv<96>(a, sp);
    case 128: return launch_kv<128>(a, sp);
    case 256: return launch_kv<256>(a, sp);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
