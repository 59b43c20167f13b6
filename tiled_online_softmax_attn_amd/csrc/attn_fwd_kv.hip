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
// Inside a chunk the computation is the forward kernel's (section 8.3 of the
// CS336 notes): S^T = K Q^T on MFMA with the lane owning one query, a lazily
// moved reference maximum, base-2 exponentials and O^T += V^T P^T, with K/V
// tiles copied global -> LDS one tile ahead.
#include "device_common.h"
#include "attn_launch.h"

#include <algorithm>
#include <type_traits>

namespace attn {
namespace {

constexpr int kKvThreads = 256;
constexpr int kKvBQ = 128;  // queries per workgroup (32 per wave)
constexpr int kKvBK = 64;   // keys per K/V tile
constexpr float kKvRescaleSlack = 8.f;  // log2 units: P never exceeds 2^8

// Partial results of chunk `split` for queries qt*128 .. qt*128+127 of head
// bh: o_part[split][bh][Nq][D] (fp32, normalised by the chunk's own sum) and
// lse_part[split][bh][Nq] (natural log; -inf when no key of the chunk is
// visible to the query, with O_c = 0).  Query i sees keys 0 .. i + off:
// off = Nk - Nq under the causal mask and off = Nk (every key) without it,
// so one code path serves both.
template <int D>
__global__ void __launch_bounds__(kKvThreads, D > 128 ? 1 : 2)
attn_fwd_kv_partial_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                           const __bf16* __restrict__ v, float* __restrict__ o_part,
                           float* __restrict__ lse_part, int BH, int Nq, int Nk, int off,
                           int n_qtiles, int chunk, float scale_log2) {
  using Tile = SwzTile<tile_width(D), D>;
  static_assert(kKvBK == Tile::kRows, "K/V tile is one SwzTile");
  constexpr int RB = Tile::kRowBytes;
  constexpr int KS = D / 16;  // k-steps of the S^T MFMA
  constexpr int DB = D / 32;  // 32-wide d blocks of O^T
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[Tile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[Tile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[Tile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[Tile::kBytes];
  auto k_lds = [&](auto par_tag) {
    return (ATTN_LDS unsigned char*)(decltype(par_tag)::value ? lds_k1 : lds_k0);
  };
  auto v_lds = [&](auto par_tag) {
    return (ATTN_LDS unsigned char*)(decltype(par_tag)::value ? lds_v1 : lds_v0);
  };
  using Par0 = std::integral_constant<int, 0>;
  using Par1 = std::integral_constant<int, 1>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // workgroup id -> (chunk, query tile, head); consecutive ids are different
  // heads, so the workgroups of one head are spread over the XCDs' turns
  // like the forward's
  const int bh = blockIdx.x % BH;
  const int rest = blockIdx.x / BH;
  const int qt = rest % n_qtiles;
  const int split = rest / n_qtiles;

  const int key_begin = split * chunk;  // a multiple of the tile size
  int key_end = min(Nk, key_begin + chunk);
  const int q_wave0 = qt * kKvBQ + wave * 32;  // first query of this wave
  const int qry = q_wave0 + l32;               // this lane's query
  const bool wave_live = q_wave0 < Nq;
  // keys past this bound are hidden from every query of the wave (of the
  // workgroup, for key_end)
  const int wave_key_end = min(key_end, min(Nq - 1, q_wave0 + 31) + off + 1);
  key_end = min(key_end, min(Nq - 1, qt * kKvBQ + kKvBQ - 1) + off + 1);

  const int64_t qhead = (int64_t)bh * Nq * D;
  const int64_t khead = (int64_t)bh * Nk * D;
  const __bf16* kh = k + khead;
  const __bf16* vh = v + khead;

  // Q^T fragments (B operand): lane holds Q[qry][16 s + 8 half + e].
  bf16x8 qf[KS];
  {
    const bf16x8 zero = {};
    const __bf16* qrow = q + qhead + (int64_t)(qry < Nq ? qry : 0) * D + half * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = (qry < Nq) ? *reinterpret_cast<const bf16x8*>(qrow + 16 * s) : zero;
  }

  const int t_begin = key_begin / kKvBK;
  const int t_end = key_end > key_begin ? (key_end + kKvBK - 1) / kKvBK : t_begin;
  auto load_tile = [&](const __bf16* src, int j, ATTN_LDS unsigned char* dst) {
    Tile::template load<kKvThreads / 64>(src, j * kKvBK, Nk, dst, wave, lane);
  };
  const int k_base = Tile::row_read_base(l32, half);
  const int v_base_lo = Tile::tr_read_base(lane, false);
  const int v_base_hi = Tile::tr_read_base(lane, true);

  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = f32x16{};
  float m_ref = -INFINITY;  // reference maximum (log2 units), moved lazily
  float l_run = 0.f;        // this lane's share of the running sum

  // one K/V tile: S^T, mask, reference maximum, P, O^T += V^T P^T
  auto step = [&](const int j, auto par_tag, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int key0 = j * kKvBK;
    const ATTN_LDS unsigned char* kbuf = k_lds(par_tag);
    f32x16 sc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int a_off = k_base ^ (32 * s);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const ATTN_LDS bf16x8*>(kbuf + a_off + kb * 32 * RB);
        sc[kb] = mfma_32x32x16(a, qf[s], sc[kb]);
      }
    }
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
          if (key >= key_end || key > qry + off) sc[kb][i] = -INFINITY;
        }
    }
    float mx = sc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][i]);
    mx = max_across_halves(mx) * scale_log2;
    if (wave_any(mx > m_ref + kKvRescaleSlack)) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[b][i] *= alpha;
    }
    const float m_off = (m_ref == -INFINITY) ? 0.f : m_ref;
    float psum = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(sc[kb][i], scale_log2, -m_off));
        psum += p;
        pf[kb][i >> 3][i & 7] = (__bf16)p;
      }
    l_run += psum;
    const ATTN_LDS unsigned char* vbuf = v_lds(par_tag);
#pragma unroll
    for (int u = 0; u < 4 * DB; ++u) {
      const int kt = u / DB, b = u % DB;
      const int roff = kt * 16 * RB;
      const bf16x8 va =
          concat4(lds_read_tr4((const ATTN_LDS __bf16*)(vbuf + (v_base_lo ^ (64 * b)) + roff)),
                  lds_read_tr4((const ATTN_LDS __bf16*)(vbuf + (v_base_hi ^ (64 * b)) + roff)));
      oacc[b] = mfma_32x32x16(va, pf[kt >> 1][kt & 1], oacc[b]);
    }
  };

  auto iteration = [&](const int j, auto par_tag) {
    using Other = std::integral_constant<int, 1 - decltype(par_tag)::value>;
    if (j + 1 < t_end) {
      load_tile(kh, j + 1, k_lds(Other{}));
      load_tile(vh, j + 1, v_lds(Other{}));
    }
    const int key0 = j * kKvBK;
    if (wave_live && key0 < wave_key_end) {
      const bool need_mask = key0 + kKvBK > wave_key_end || key0 + kKvBK - 1 > q_wave0 + off;
      if (need_mask) step(j, par_tag, std::true_type{});
      else step(j, par_tag, std::false_type{});
    }
    wait_vmem();
    __syncthreads();
  };

  if (t_begin < t_end) {
    load_tile(kh, t_begin, k_lds(Par0{}));
    load_tile(vh, t_begin, v_lds(Par0{}));
  }
  wait_vmem();
  __syncthreads();
  for (int j = t_begin; j < t_end; j += 2) {
    iteration(j, Par0{});
    if (j + 1 < t_end) iteration(j + 1, Par1{});
  }

  // ---- partial result of this chunk: O_c = O / l, lse_c = ln2 (m + log2 l)
  const float l_tot = sum_across_halves(l_run);
  if (qry < Nq) {
    const int64_t prow = ((int64_t)split * BH + bh) * Nq + qry;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* orow = o_part + prow * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = oacc[b][r * 4 + e] * inv;
        *reinterpret_cast<f32x4*>(orow + b * 32 + r * 8 + half * 4) = w;
      }
    if (half == 0) lse_part[prow] = l_tot > 0.f ? kLn2 * (m_ref + fast_log2(l_tot)) : -INFINITY;
  }
}

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
  const int BH = a.B * a.H;
  const int n_qtiles = (a.Nq + kKvBQ - 1) / kKvBQ;
  const hipStream_t s = (hipStream_t)a.stream;
  float* o_part = (float*)a.workspace;
  float* lse_part = (float*)((char*)a.workspace + sp.o_part_bytes);
  const int off = a.causal ? a.Nk - a.Nq : a.Nk;
  hipLaunchKernelGGL((attn_fwd_kv_partial_kernel<D>),
                     dim3((unsigned)((int64_t)BH * n_qtiles * sp.splits)), dim3(kKvThreads), 0, s,
                     (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, o_part, lse_part,
                     BH, a.Nq, a.Nk, off, n_qtiles, sp.chunk, a.scale * kLog2e);
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
    // about four workgroups per CU in total, each chunk at least four tiles
    const int64_t base = BH * n_qtiles;
    want = (1024 + base - 1) / base;
    want = std::min<int64_t>(want, std::max<int64_t>(1, tiles / 4));
  }
  want = std::max<int64_t>(1, std::min<int64_t>(want, tiles));
  const int64_t tiles_per_chunk = (tiles + want - 1) / want;
  sp.chunk = (int)(tiles_per_chunk * kKvBK);
  sp.splits = (int)((tiles + tiles_per_chunk - 1) / tiles_per_chunk);
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
