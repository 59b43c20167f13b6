// attn_bwd.hip - fused attention backward for gfx950 (bf16 in/out, fp32 math).
//
// Method (CS336 Lecture 5 notes "GPUs, TPUs", section 8.4 and Exercise 9):
// nothing N x N is stored by the forward; the backward recomputes it block by
// block from Q, K, V, O, the logsumexp L and dO:
//   P = e^{scale*S - L},  dV += P^T dO,  dP = dO V^T,
//   dS = P * (dP - D)  with  D_i = rowsum(dO_i * O_i),
//   dQ += scale * dS K,  dK += scale * dS^T Q.
// The loop order is key/value blocks outside, query blocks inside (the
// outer-K/V schedule of PDC notes Lecture 4, section 4.12), so dK and dV stay
// in registers for the whole kernel, and dQ, which every key block adds to,
// is accumulated with fp32 atomics (PDC notes Lecture 5, section 5.11) into a
// workspace that a last kernel rounds to bf16.  Three launches on one stream:
//   1. bwd_preprocess: D = rowsum(dO * O), dQ accumulator = 0
//   2. bwd_main:       one workgroup per (head, 128-key block)
//   3. bwd_dq_convert: dQ = bf16(accumulator)
// A kernel boundary is the global synchronisation between the steps (PDC
// notes Lecture 5, section 5.14).
//
// bwd_main layout (4 waves, 32 keys each; query tiles of 64 rows):
//   * S = Q K^T and dP = dO V^T use v_mfma_f32_32x32x16_bf16 with K^T and V^T
//     fragments held in registers; in their accumulators each lane owns one
//     key (column l % 32) and 16 queries.
//   * dV += P^T dO and dK += dS^T Q take P^T / dS^T straight from those
//     accumulators as the A operand; dO and Q come from LDS through the
//     transpose read ds_read_b64_tr_b16.
//   * dS^T is staged in LDS (bf16, key-major) so that the four waves can form
//     the 64 x d block of dQ over all 128 keys of the workgroup.
#include "device_common.h"
#include "attn_launch.h"

namespace attn {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kBwdBK = 128;  // keys per workgroup (32 per wave)
constexpr int kBwdBQ = 64;   // queries per inner step

template <int D>
struct BwdLds {
  static constexpr int kStrideQ = D + 16;        // Q and dO tiles, [query][d]
  static constexpr int kStrideK = D + 16;        // K block, [key][d]
  static constexpr int kStrideS = kBwdBQ + 16;   // dS^T, [key][query]
  static constexpr int kElemsQ = kBwdBQ * kStrideQ;
  // bf16 element offsets
  static constexpr int kOffQ = 0;                       // [2][BQ][strideQ]
  static constexpr int kOffDO = kOffQ + 2 * kElemsQ;    // [2][BQ][strideQ]
  static constexpr int kOffK = kOffDO + 2 * kElemsQ;    // [BK][strideK]
  static constexpr int kOffS = kOffK + kBwdBK * kStrideK;  // [BK][strideS]
  static constexpr int kElemsBf16 = kOffS + kBwdBK * kStrideS;
  // fp32 arrays after the bf16 region: L (log2 units) and D, [2][BQ] each
  static constexpr int kBytes = kElemsBf16 * 2 + 2 * 2 * kBwdBQ * 4;
  static constexpr int kChunks = kBwdBQ * D / 8;  // 16-byte chunks per Q (or dO) tile
  static constexpr int kChunksPerThread = kChunks / kBwdThreads;
  static_assert(kChunks % kBwdThreads == 0, "tile must split evenly over threads");
};

// ---------------------------------------------------------------- 1. preprocess
// 8 threads per row; each handles d/8 consecutive elements.
template <int D>
__global__ void __launch_bounds__(256)
bwd_preprocess_kernel(const __bf16* __restrict__ o, const __bf16* __restrict__ dout,
                      float* __restrict__ delta, float* __restrict__ dq_acc, int64_t rows) {
  constexpr int PER = D / 8;
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  float acc = 0.f;
  if (row < rows) {
    const __bf16* orow = o + row * D + part * PER;
    const __bf16* drow = dout + row * D + part * PER;
#pragma unroll
    for (int c = 0; c < PER; c += 8) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(orow + c);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(drow + c);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)a[e], (float)b[e], acc);
    }
    float* zrow = dq_acc + row * D + part * PER;
#pragma unroll
    for (int c = 0; c < PER; c += 4) *reinterpret_cast<float4*>(zrow + c) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < rows && part == 0) delta[row] = acc;
}

// ---------------------------------------------------------------- 3. dQ convert
__global__ void __launch_bounds__(256)
bwd_dq_convert_kernel(const float* __restrict__ dq_acc, __bf16* __restrict__ dq, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const float4 a = *reinterpret_cast<const float4*>(dq_acc + i * 8);
  const float4 b = *reinterpret_cast<const float4*>(dq_acc + i * 8 + 4);
  bf16x8 r;
  r[0] = (__bf16)a.x; r[1] = (__bf16)a.y; r[2] = (__bf16)a.z; r[3] = (__bf16)a.w;
  r[4] = (__bf16)b.x; r[5] = (__bf16)b.y; r[6] = (__bf16)b.z; r[7] = (__bf16)b.w;
  *reinterpret_cast<bf16x8*>(dq + i * 8) = r;
}

// ---------------------------------------------------------------- 2. main
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kBwdThreads, 1)
bwd_main_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                const __bf16* __restrict__ v, const __bf16* __restrict__ dout,
                const float* __restrict__ lse, const float* __restrict__ delta,
                float* __restrict__ dq_acc, __bf16* __restrict__ dk, __bf16* __restrict__ dv,
                int BH, int N, int n_kblocks, float scale, float scale_log2) {
  using L = BwdLds<D>;
  constexpr int KS = D / 16;  // k-steps over d
  constexpr int DB = D / 32;  // 32-wide d blocks
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  __bf16* smem = reinterpret_cast<__bf16*>(smem_raw);
  float* sm_l = reinterpret_cast<float*>(smem_raw + L::kElemsBf16 * 2);  // [2][BQ]
  float* sm_d = sm_l + 2 * kBwdBQ;                                      // [2][BQ]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int g16 = lane & 15;
  const int grp = lane >> 4;

  const int rank = blockIdx.x / BH;
  const int bh = blockIdx.x - rank * BH;
  const int kblk = rank;  // causal: low key blocks see the most queries, issue them first
  const int64_t head = (int64_t)bh * N * D;
  const __bf16* qh = q + head;
  const __bf16* doh = dout + head;
  const float* lse_h = lse + (int64_t)bh * N;
  const float* del_h = delta + (int64_t)bh * N;

  const int key_wg0 = kblk * kBwdBK;
  const int key_w0 = key_wg0 + wave * 32;  // first key of this wave
  const int key = key_w0 + l32;            // this lane's key (accumulator column)

  // K and V of this workgroup: LDS copy of K (for dQ), and per-wave K^T / V^T
  // fragments in registers (B operand: lane holds X[key][16 s + 8 half + e]).
  bf16x8 kf[KS], vf[KS];
  {
    const bf16x8 zero = {};
    const bool ok = key < N;
    const __bf16* krow = k + head + (int64_t)(ok ? key : 0) * D + half * 8;
    const __bf16* vrow = v + head + (int64_t)(ok ? key : 0) * D + half * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kf[s] = ok ? *reinterpret_cast<const bf16x8*>(krow + 16 * s) : zero;
      vf[s] = ok ? *reinterpret_cast<const bf16x8*>(vrow + 16 * s) : zero;
    }
    __bf16* ks = smem + L::kOffK;
    for (int c = tid; c < kBwdBK * D / 8; c += kBwdThreads) {
      const int row = c / (D / 8);
      const int col = (c % (D / 8)) * 8;
      const int kk = key_wg0 + row;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (kk < N) val = *reinterpret_cast<const uint4*>(k + head + (int64_t)kk * D + col);
      *reinterpret_cast<uint4*>(ks + row * L::kStrideK + col) = val;
    }
  }

  // query tiles this key block meets
  const int n_qtiles = (N + kBwdBQ - 1) / kBwdBQ;
  const int qt_begin = CAUSAL ? key_wg0 / kBwdBQ : 0;

  uint4 rq[L::kChunksPerThread], rdo[L::kChunksPerThread];
  float rl = 0.f, rd = 0.f;
  auto load_tile = [&](int qt) {
#pragma unroll
    for (int r = 0; r < L::kChunksPerThread; ++r) {
      const int c = tid + r * kBwdThreads;
      const int row = c / (D / 8);
      const int col = (c % (D / 8)) * 8;
      const int qq = qt * kBwdBQ + row;
      if (qq < N) {
        rq[r] = *reinterpret_cast<const uint4*>(qh + (int64_t)qq * D + col);
        rdo[r] = *reinterpret_cast<const uint4*>(doh + (int64_t)qq * D + col);
      } else {
        rq[r] = make_uint4(0, 0, 0, 0);
        rdo[r] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < kBwdBQ) {
      const int qq = qt * kBwdBQ + tid;
      rl = qq < N ? lse_h[qq] * kLog2e : 0.f;
      rd = qq < N ? del_h[qq] : 0.f;
    }
  };
  auto store_tile = [&](int st) {
    __bf16* qs = smem + L::kOffQ + st * L::kElemsQ;
    __bf16* ds = smem + L::kOffDO + st * L::kElemsQ;
#pragma unroll
    for (int r = 0; r < L::kChunksPerThread; ++r) {
      const int c = tid + r * kBwdThreads;
      const int row = c / (D / 8);
      const int col = (c % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(qs + row * L::kStrideQ + col) = rq[r];
      *reinterpret_cast<uint4*>(ds + row * L::kStrideQ + col) = rdo[r];
    }
    if (tid < kBwdBQ) {
      sm_l[st * kBwdBQ + tid] = rl;
      sm_d[st * kBwdBQ + tid] = rd;
    }
  };

  f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    dk_acc[b] = f32x16{};
    dv_acc[b] = f32x16{};
  }

  if (qt_begin < n_qtiles) {
    load_tile(qt_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int qt = qt_begin; qt < n_qtiles; ++qt) {
    const int st = (qt - qt_begin) & 1;
    if (qt + 1 < n_qtiles) load_tile(qt + 1);

    const ATTN_LDS __bf16* qs = (const ATTN_LDS __bf16*)(smem + L::kOffQ + st * L::kElemsQ);
    const ATTN_LDS __bf16* dos = (const ATTN_LDS __bf16*)(smem + L::kOffDO + st * L::kElemsQ);
    const float* lq = sm_l + st * kBwdBQ;
    const float* dq_d = sm_d + st * kBwdBQ;
    ATTN_LDS __bf16* sts = (ATTN_LDS __bf16*)(smem + L::kOffS);

    const int q0 = qt * kBwdBQ;
    // All 64 queries of the tile precede every key of this wave: nothing to do.
    const bool skip = CAUSAL && (q0 + kBwdBQ - 1 < key_w0);
    if (!skip) {
      const bool need_mask = (q0 + kBwdBQ > N) || (key_w0 + 32 > N) ||
                             (CAUSAL && q0 < key_w0 + 31);
      // ---- S = Q K^T and dP = dO V^T for two 32-query blocks
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        sacc[qb] = f32x16{};
        pacc[qb] = f32x16{};
        const ATTN_LDS __bf16* qrow = qs + (qb * 32 + l32) * L::kStrideQ + half * 8;
        const ATTN_LDS __bf16* drow = dos + (qb * 32 + l32) * L::kStrideQ + half * 8;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 a = *reinterpret_cast<const ATTN_LDS bf16x8*>(qrow + 16 * s);
          sacc[qb] = mfma_32x32x16(a, kf[s], sacc[qb]);
          const bf16x8 b = *reinterpret_cast<const ATTN_LDS bf16x8*>(drow + 16 * s);
          pacc[qb] = mfma_32x32x16(b, vf[s], pacc[qb]);
        }
      }
      // ---- P = 2^{S scale log2e - L log2e}; dS = P (dP - D)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qrow0 = qb * 32 + r * 8 + half * 4;  // 4 consecutive query rows
          const float4 l4 = *reinterpret_cast<const float4*>(lq + qrow0);
          const float4 d4 = *reinterpret_cast<const float4*>(dq_d + qrow0);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = r * 4 + e;
            float p = fast_exp2(fmaf(sacc[qb][i], scale_log2, -lv[e]));
            if (need_mask) {
              const int qq = q0 + qrow0 + e;
              if (qq >= N || key >= N || (CAUSAL && key > qq)) p = 0.f;
            }
            sacc[qb][i] = p;
            pacc[qb][i] = p * (pacc[qb][i] - dv4[e]);
          }
        }
      // ---- dV += P^T dO ; dK += dS^T Q   (A from the accumulators, B by transpose reads)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          bf16x8 pa, sa;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pa[e] = (__bf16)sacc[qb][t * 8 + e];
            sa[e] = (__bf16)pacc[qb][t * 8 + e];
          }
          const int row = qb * 32 + t * 16 + half * 4 + (g16 >> 2);
#pragma unroll
          for (int b = 0; b < DB; ++b) {
            const int col = b * 32 + (grp & 1) * 16 + 4 * (g16 & 3);
            const bf16x8 dob = concat4(lds_read_tr4(dos + row * L::kStrideQ + col),
                                       lds_read_tr4(dos + (row + 8) * L::kStrideQ + col));
            dv_acc[b] = mfma_32x32x16(pa, dob, dv_acc[b]);
            const bf16x8 qbv = concat4(lds_read_tr4(qs + row * L::kStrideQ + col),
                                       lds_read_tr4(qs + (row + 8) * L::kStrideQ + col));
            dk_acc[b] = mfma_32x32x16(sa, qbv, dk_acc[b]);
          }
        }
      // ---- stage dS^T (bf16) for the dQ product: sts[key][query]
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)pacc[qb][r * 4 + e];
          *reinterpret_cast<ATTN_LDS bf16x4*>(sts + (wave * 32 + l32) * L::kStrideS + qb * 32 +
                                              r * 8 + half * 4) = w;
        }
    } else {
      // this wave's keys contribute nothing to this query tile
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<ATTN_LDS bf16x4*>(sts + (wave * 32 + l32) * L::kStrideS + qb * 32 +
                                              r * 8 + half * 4) = bf16x4{};
    }
    __syncthreads();

    // ---- dQ[q0 .. q0+63][:] += scale * dS K over the 128 keys of the workgroup
    {
      const ATTN_LDS __bf16* ks = (const ATTN_LDS __bf16*)(smem + L::kOffK);
      const int qb = wave & 1;
      // causal: keys of this workgroup beyond the last query of the tile add nothing
      const int key_lim = CAUSAL ? min(kBwdBK, q0 + kBwdBQ - key_wg0) : kBwdBK;
      const int ksteps = (key_lim + 15) / 16;
#pragma unroll
      for (int bb = 0; bb < DB / 2 + (DB == 1); ++bb) {
        const int b = (wave >> 1) + 2 * bb;
        if (b >= DB) break;
        f32x16 acc = f32x16{};
        for (int ks16 = 0; ks16 < ksteps; ++ks16) {
          const int krow = ks16 * 16 + half * 8 + (g16 >> 2);
          // A = dS[query][keys]: transpose read of sts[key][query]
          const int qcol = qb * 32 + (grp & 1) * 16 + 4 * (g16 & 3);
          const bf16x8 a = concat4(lds_read_tr4(sts + krow * L::kStrideS + qcol),
                                   lds_read_tr4(sts + (krow + 4) * L::kStrideS + qcol));
          // B = K[keys][d]: transpose read of the K block
          const int dcol = b * 32 + (grp & 1) * 16 + 4 * (g16 & 3);
          const bf16x8 bk = concat4(lds_read_tr4(ks + krow * L::kStrideK + dcol),
                                    lds_read_tr4(ks + (krow + 4) * L::kStrideK + dcol));
          acc = mfma_32x32x16(a, bk, acc);
        }
        // acc lane: d column b*32 + l32, query rows (i/4)*8 + half*4 + i%4
        const int dd = b * 32 + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qq = q0 + qb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
          if (qq < N) atomicAdd(dq_acc + head + (int64_t)qq * D + dd, acc[i] * scale);
        }
      }
    }

    if (qt + 1 < n_qtiles) store_tile(st ^ 1);
    __syncthreads();
  }

  // ---- write dK = scale * acc and dV: lane holds d column b*32 + l32 and
  //      key rows (i/4)*8 + half*4 + i%4 of this wave's 32 keys
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = key_w0 + (i >> 2) * 8 + half * 4 + (i & 3);
      if (kk < N) {
        const int64_t off = head + (int64_t)kk * D + b * 32 + l32;
        dk[off] = (__bf16)(dk_acc[b][i] * scale);
        dv[off] = (__bf16)dv_acc[b][i];
      }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_main(const BwdArgs& a) {
  using L = BwdLds<D>;
  const int BH = a.B * a.H;
  const int n_kblocks = (a.N + kBwdBK - 1) / kBwdBK;
  auto kern = bwd_main_kernel<D, CAUSAL>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, L::kBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(BH * n_kblocks)), dim3(kBwdThreads), L::kBytes,
                     (hipStream_t)a.stream, (const __bf16*)a.q, (const __bf16*)a.k,
                     (const __bf16*)a.v, (const __bf16*)a.dout, a.lse, a.delta, a.dq_acc,
                     (__bf16*)a.dk, (__bf16*)a.dv, BH, a.N, n_kblocks, a.scale,
                     a.scale * kLog2e);
  return hipGetLastError();
}

template <int D>
hipError_t launch_phase(const BwdArgs& a, int phase) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  if (phase == 0) {
    hipLaunchKernelGGL(bwd_preprocess_kernel<D>, dim3((unsigned)((rows + 31) / 32)), dim3(256),
                       0, (hipStream_t)a.stream, (const __bf16*)a.o, (const __bf16*)a.dout,
                       a.delta, a.dq_acc, rows);
    return hipGetLastError();
  }
  if (phase == 1) return a.causal ? launch_main<D, true>(a) : launch_main<D, false>(a);
  const int64_t n8 = rows * D / 8;
  hipLaunchKernelGGL(bwd_dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0,
                     (hipStream_t)a.stream, a.dq_acc, (__bf16*)a.dq, n8);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_phase(const BwdArgs& a, int phase) {
  return a.d == 128 ? launch_phase<128>(a, phase) : launch_phase<64>(a, phase);
}

hipError_t launch_bwd(const BwdArgs& a) {
  for (int phase = 0; phase < 3; ++phase) {
    const hipError_t e = launch_bwd_phase(a, phase);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace attn
