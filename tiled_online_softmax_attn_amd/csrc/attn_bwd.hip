// attn_bwd.hip - fused attention backward for gfx950 (bf16 in/out, fp32 math).
//
// Method (CS336 Lecture 5 notes "GPUs, TPUs", section 8.4 and Exercise 9):
// nothing N x N is kept from the forward; the backward recomputes it block by
// block from Q, K, V, the logsumexp L and dO:
//   P = e^{scale*S - L},  dV += P^T dO,  dP = dO V^T,
//   dS = P * (dP - D)  with  D_i = rowsum(dO_i * O_i),
//   dQ += scale * dS K,  dK += scale * dS^T Q.
// Three launches on one stream (a kernel boundary is the global
// synchronisation between them, PDC notes Lecture 5, section 5.14):
//   phase 0  bwd_preprocess: D = rowsum(dO * O)                 (HBM-bound)
//   phase 1  bwd_dkdv:  key/value blocks outside, query blocks inside (the
//            outer-K/V schedule of PDC notes Lecture 4, section 4.12): dK and
//            dV of a 128-key block stay in registers for the whole kernel
//            (attn_bwd_dkdv.hip, its own compilation unit).
//   phase 2  bwd_dq:    query blocks outside, key/value blocks inside (the
//            forward's schedule): dQ of a 128-query block stays in registers.
// The queries may be the last Nq positions of an Nk-key sequence (the
// backward of attention over a key/value cache): query i then sees keys
// 0 .. i + off under the causal mask, off = Nk - Nq (0 for square attention).
//
// Splitting dQ from dK/dV recomputes S and dP once more (7 block products
// instead of 5) but removes every cross-workgroup reduction: on this chip a
// device-wide fp32 atomic add is carried out past the per-XCD L2, and the
// atomic form of dQ measured 2.3 GB of extra memory writes per launch at
// B=4, H=16, N=4096, d=128.  Both kernels write their results exactly once,
// so the backward is deterministic.
//
// Q/dO (dK/dV kernel) and K/V (dQ kernel) tiles of 64 rows go straight from
// global memory to LDS (SwzTile: unpadded, XOR-swizzled chunks, read both by
// rows and through the transpose read without bank conflicts).
//
// Register layout of bwd_dq (v_mfma_f32_32x32x16_bf16; see device_common.h):
// S^T = K Q^T and dP^T = V dO^T with Q^T / dO^T fragments resident; every
// lane owns one query.  dQ^T += K^T dS^T takes dS^T from the accumulator as
// the B operand and reads K^T through the transpose read.
#include "device_common.h"
#include "attn_launch.h"

#include <algorithm>

#include <type_traits>

namespace attn {
namespace {

constexpr int kBwdThreads = 256;

// ---------------------------------------------------------------- phase 0
// D_i = sum_k dO_ik O_ik; 8 threads per row, thread `part` over the 8-column
// chunks part, part + 8, ... of the row (adjacent threads, adjacent chunks).
template <int D>
__global__ void __launch_bounds__(256)
bwd_preprocess_kernel(const __bf16* __restrict__ o, const __bf16* __restrict__ dout,
                      float* __restrict__ delta, int64_t rows) {
  constexpr int CH = D / 8;  // chunks per row
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  float acc = 0.f;
  if (row < rows) {
    const __bf16* orow = o + row * D;
    const __bf16* drow = dout + row * D;
#pragma unroll
    for (int c = part; c < CH; c += 8) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(orow + c * 8);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(drow + c * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)a[e], (float)b[e], acc);
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < rows && part == 0) delta[row] = acc;
}

// ---------------------------------------------------------------- phase 2
constexpr int kDqBQ = 128;  // queries per workgroup (32 per wave)
constexpr int kDqBK = 64;   // keys per K/V tile (one SwzTile)

// PARTIAL: workgroup (split, query tile, head) sums dS K over key chunk
// `split` only (chunk keys, a multiple of the tile) and writes scale * that
// sum in fp32 to dq_part[split][bh][Nq][D] for bwd_dq_reduce_kernel.
// FORM_D: D = rowsum(dO * O) is formed here instead of read from the
// preprocess kernel's output, and written to `delta` for the dK/dV kernel,
// which then runs after this one (phase 3: phases 0 and 2 in one launch).
template <int D, bool CAUSAL, bool PARTIAL = false, bool FORM_D = false>
__global__ void __launch_bounds__(kBwdThreads, D > 128 ? 1 : 2)
bwd_dq_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
              const __bf16* __restrict__ v, const __bf16* __restrict__ dout,
              const __bf16* __restrict__ o, const float* __restrict__ lse,
              float* __restrict__ delta, __bf16* __restrict__ dq, int BH, int Nq, int Nk, int off,
              int n_qtiles, float scale, float scale_log2, float* __restrict__ dq_part, int chunk) {
  static_assert(!(PARTIAL && FORM_D), "a key chunk does not see the whole row of dO * O");
  using Tile = SwzTile<tile_width(D), D>;
  static_assert(kDqBK == Tile::kRows, "key tile is one SwzTile");
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr bool kPipelineHalves = (D <= 64) || CAUSAL;
  constexpr int RB = Tile::kRowBytes;
  // K and V tiles of 64 keys (SwzTile layout), two buffers each; K is read
  // both by rows (S^T) and transposed (dQ^T).  One LDS object per buffer, so
  // that the copies into one buffer do not make reads of the other wait.
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[Tile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[Tile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[Tile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[Tile::kBytes];
  auto k_lds = [&](auto buf_tag) {
    return (ATTN_LDS unsigned char*)(decltype(buf_tag)::value ? lds_k1 : lds_k0);
  };
  auto v_lds = [&](auto buf_tag) {
    return (ATTN_LDS unsigned char*)(decltype(buf_tag)::value ? lds_v1 : lds_v0);
  };
  using Buf0 = std::integral_constant<int, 0>;
  using Buf1 = std::integral_constant<int, 1>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // workgroup id -> (head, query tile[, key chunk]), heavy causal tiles first
  const int rank = blockIdx.x / BH;
  const int bh = blockIdx.x - rank * BH;
  const int split = PARTIAL ? rank / n_qtiles : 0;
  const int qrank = rank - split * n_qtiles;
  const int qt = CAUSAL ? (n_qtiles - 1 - qrank) : qrank;
  const int64_t qhead = (int64_t)bh * Nq * D;
  const int64_t khead = (int64_t)bh * Nk * D;
  const __bf16* kh = k + khead;
  const __bf16* vh = v + khead;

  const int q_wave0 = qt * kDqBQ + wave * 32;
  const int qry = q_wave0 + l32;
  const bool qok = qry < Nq;

  // Q^T and dO^T fragments (B operand): lane holds X[qry][16 s + 8 half + e]
  bf16x8 qf[KS], df[KS];
  {
    const bf16x8 zero = {};
    const int64_t roff = qhead + (int64_t)(qok ? qry : 0) * D + half * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = qok ? *reinterpret_cast<const bf16x8*>(q + roff + 16 * s) : zero;
      df[s] = qok ? *reinterpret_cast<const bf16x8*>(dout + roff + 16 * s) : zero;
    }
  }
  const float lq2 = qok ? lse[(int64_t)bh * Nq + qry] * kLog2e : 0.f;
  // D of the lane's query: read from the preprocess kernel's output, or
  // (FORM_D) formed below once the O rows of the workgroup are in LDS.
  float dlt = 0.f;
  if constexpr (!FORM_D) dlt = qok ? delta[(int64_t)bh * Nq + qry] : 0.f;

  // keys past the last one the workgroup's last query sees are not visited;
  // a split visits only its chunk (key tiles t_begin .. t_begin + n_tiles - 1)
  const int kv_all = CAUSAL ? (int)min((int64_t)Nk, (int64_t)(qt + 1) * kDqBQ + off) : Nk;
  const int key_begin = PARTIAL ? split * chunk : 0;
  const int kv_end = PARTIAL ? (int)min((int64_t)kv_all, (int64_t)key_begin + chunk) : kv_all;
  const int t_begin = key_begin / kDqBK;
  const int n_tiles = kv_end > key_begin ? (kv_end + kDqBK - 1) / kDqBK - t_begin : 0;

  auto load_tile = [&](int j, auto buf_tag) {
    Tile::template load<kBwdThreads / 64>(kh, j * kDqBK, Nk, k_lds(buf_tag), wave, lane);
    Tile::template load<kBwdThreads / 64>(vh, j * kDqBK, Nk, v_lds(buf_tag), wave, lane);
  };
  const int rd_base = Tile::row_read_base(l32, half);
  const int tr_lo = Tile::tr_read_base(lane, false);
  const int tr_hi = Tile::tr_read_base(lane, true);

  f32x16 dq_acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) dq_acc[b] = f32x16{};

  if (n_tiles > 0) load_tile(t_begin, Buf0{});
  if constexpr (FORM_D) {
    // the workgroup's 128 O rows into the second K / V buffers, which the
    // first copies of the loop fill only after the barrier below
    Tile::template load<kBwdThreads / 64>(o + qhead, qt * kDqBQ, Nq, k_lds(Buf1{}), wave, lane);
    Tile::template load<kBwdThreads / 64>(o + qhead, qt * kDqBQ + kDqBK, Nq, v_lds(Buf1{}), wave,
                                          lane);
  }
  wait_vmem();
  __syncthreads();
  if constexpr (FORM_D) {
    // D = rowsum(dO * O): the lane's dO^T fragments are in registers, and the
    // same columns of its query's O row are read from LDS with the row-read
    // pattern of the K tiles (query row 32 (wave & 1) + l32 of buffer
    // wave / 2); one add across the two lane halves (both halves get the same
    // sum), and half 0 stores D for the dK/dV kernel.
    const ATTN_LDS unsigned char* obuf = wave < 2 ? k_lds(Buf1{}) : v_lds(Buf1{});
    const int orow = (wave & 1) * 32 * RB;
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 of = *reinterpret_cast<const ATTN_LDS bf16x8*>(obuf + (rd_base ^ (32 * s)) + orow);
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf((float)of[e], (float)df[s][e], part);
    }
    dlt = sum_across_halves(part);
    if (qok && half == 0) delta[(int64_t)bh * Nq + qry] = dlt;
    __syncthreads();  // every wave has read its O rows before tile 1 is copied over them
  }
  // d <= 64: dP^T - D on the matrix unit.  One more k-step of dP^T = V dO^T
  // with an all-ones column pair in V (A operand) against -D split into two
  // bf16 parts in dO (B operand) subtracts D_hi + D_lo = D (to 2^-16
  // relative) from every entry of the lane's query, in place of 16 VALU
  // subtractions per 32-key half.
  constexpr bool kFoldD = D <= 64;
  bf16x8 ones_x = {}, negd_x = {};
  if (kFoldD && half == 0) {
    const __bf16 dhi = (__bf16)(-dlt);
    const __bf16 dlo = (__bf16)(-dlt - (float)dhi);
    ones_x[0] = (__bf16)1.f;
    ones_x[1] = (__bf16)1.f;
    negd_x[0] = dhi;
    negd_x[1] = dlo;
  }

  // One K/V tile t_begin + j, held in buffer CUR; the copies of the next go to
  // the other buffer meanwhile.
  auto tile = [&](const int j, auto cur_tag) {
    using Next = std::integral_constant<int, 1 - decltype(cur_tag)::value>;
    if (j + 1 < n_tiles) load_tile(t_begin + j + 1, Next{});
    const int key0 = (t_begin + j) * kDqBK;
    const bool skip = CAUSAL && key0 > q_wave0 + 31 + off;
    if (!skip) {
      const ATTN_LDS unsigned char* ks = k_lds(cur_tag);
      const ATTN_LDS unsigned char* vs = v_lds(cur_tag);
      const bool need_mask =
          (key0 + kDqBK > Nk) || (CAUSAL && key0 + kDqBK - 1 > q_wave0 + off);

      if constexpr (kPipelineHalves) {
        // The tile's 64 keys are two 32-key halves kb = 0, 1, software-
        // pipelined like the dK/dV kernel's query blocks (at d = 96 and 128
        // without the causal mask this order spills registers at two waves
        // per SIMD, so those take the plain order below):
        //   A  S^T, dP^T of half 0                       (MFMA)
        //   B  S^T, dP^T of half 1 |  P^T, dS^T of half 0 (VALU)
        //   C  dQ^T of half 0      |  P^T, dS^T of half 1
        //   D  dQ^T of half 1
        f32x16 sacc[2] = {f32x16{}, f32x16{}};
        f32x16 pacc[2] = {f32x16{}, f32x16{}};
        bf16x8 sf[2][2];

        // S^T = K Q^T and dP^T = V dO^T, k-step s of half kb
        auto sdp_step = [&](int kb, int s) {
          const int at = (rd_base ^ (32 * s)) + kb * 32 * RB;
          const bf16x8 a = *reinterpret_cast<const ATTN_LDS bf16x8*>(ks + at);
          sacc[kb] = mfma_32x32x16(a, qf[s], sacc[kb]);
          const bf16x8 b = *reinterpret_cast<const ATTN_LDS bf16x8*>(vs + at);
          if (kFoldD && s == 0) pacc[kb] = mfma_32x32x16(ones_x, negd_x, pacc[kb]);
          pacc[kb] = mfma_32x32x16(b, df[s], pacc[kb]);
        };
        // P^T = 2^{S^T scale log2e - L}, dS^T = P^T (dP^T - D) for accumulator
        // entries 4 r .. 4 r + 3 of half kb, as bf16 B operand
        auto soft_part = [&](int kb, int r, int e0, int e1, auto mask_tag) {
          constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
          for (int e = e0; e < e1; ++e) {
            const int i = r * 4 + e;
            float p = fast_exp2(fmaf(sacc[kb][i], scale_log2, -lq2));
            if constexpr (MASK) {
              const int kk = key0 + kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
              if (kk >= Nk || (CAUSAL && kk > qry + off)) p = 0.f;
            }
            // keep the exponential at this point of the issue order
            __asm__ volatile("" ::"v"(p));
            sf[kb][i >> 3][i & 7] = (__bf16)(p * (kFoldD ? pacc[kb][i] : pacc[kb][i] - dlt));
          }
        };
        // K^T fragment of dQ^T step g: steps 0 .. 2DB-1 are half 0 (C),
        // 2DB .. 4DB-1 half 1 (D); step u of a half covers 16 keys (t) and
        // 32 d rows (b)
        constexpr int UQ = 2 * DB;
        auto read_kt = [&](int g) {
          const int kb = g / UQ, u = g % UQ, t = u / DB, b = u % DB;
          const int roff = (kb * 32 + t * 16) * RB;
          return concat4(lds_read_tr4((const ATTN_LDS __bf16*)(ks + (tr_lo ^ (64 * b)) + roff)),
                         lds_read_tr4((const ATTN_LDS __bf16*)(ks + (tr_hi ^ (64 * b)) + roff)));
        };
        auto dq_step = [&](int g, const bf16x8& ka) {
          const int kb = g / UQ, u = g % UQ, t = u / DB, b = u % DB;
          dq_acc[b] = mfma_32x32x16(ka, sf[kb][t], dq_acc[b]);
        };
        // softmax entries [lo, hi) of half kb
        auto soft_range = [&](int kb, int lo, int hi, auto mask_tag) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int a = max(lo, 4 * r), z = min(hi, 4 * r + 4);
            if (a < z) soft_part(kb, r, a - 4 * r, z - 4 * r, mask_tag);
          }
        };

        auto body = [&](auto mask_tag) {
          // A
#pragma unroll
          for (int s = 0; s < KS; ++s) sdp_step(0, s);
          __builtin_amdgcn_sched_barrier(0);
          // B: entries 16s/KS .. 16(s+1)/KS of half 0's softmax per k-step.
          // Through B and C, the two phases that carry a softmax beside their
          // MFMAs, the wave takes issue priority over the other waves of its
          // SIMD (d = 64 .. 128), so that its matrix steps are not held behind
          // their MFMA-only phases (B4 H16 N4096 causal dQ forming D: d = 128
          // 395.1 -> 388.0 us, d = 64 110.7 -> 106.2 us).  At d = 32, three
          // waves per SIMD and a short softmax, it cost 142.1 against 129.6 us.
          if constexpr (D >= 64 && D <= 128) __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            sdp_step(1, s);
            soft_range(0, 16 * s / KS, 16 * (s + 1) / KS, mask_tag);
            __builtin_amdgcn_sched_barrier(0);
          }
          // C, D: dQ^T steps of half 0 then half 1, each step's K^T fragment
          // read one step ahead; C carries half 1's softmax, spread evenly
          bf16x8 kr[2];
          kr[0] = read_kt(0);
#pragma unroll
          for (int g = 0; g < 2 * UQ; ++g) {
            if (g + 1 < 2 * UQ) kr[(g + 1) & 1] = read_kt(g + 1);
            dq_step(g, kr[g & 1]);
            if (g < UQ) soft_range(1, 16 * g / UQ, 16 * (g + 1) / UQ, mask_tag);
            __builtin_amdgcn_sched_barrier(0);
            if (D >= 64 && D <= 128 && g == UQ - 1) __builtin_amdgcn_s_setprio(0);
          }
        };
        if (need_mask)
          body(std::true_type{});
        else
          body(std::false_type{});
      } else {
        // Plain order; every LDS operand is read one step ahead of its MFMAs.
        // ---- S^T = K Q^T and dP^T = V dO^T, step u = s * 2 + kb
        f32x16 sacc[2] = {f32x16{}, f32x16{}};
        f32x16 pacc[2] = {f32x16{}, f32x16{}};
        struct RowFrag { bf16x8 k, v; };
        auto read_row = [&](int u) {
          const int s = u >> 1, kb = u & 1;
          const int at = (rd_base ^ (32 * s)) + kb * 32 * RB;
          return RowFrag{*reinterpret_cast<const ATTN_LDS bf16x8*>(ks + at),
                         *reinterpret_cast<const ATTN_LDS bf16x8*>(vs + at)};
        };
        RowFrag rf[2];
        rf[0] = read_row(0);
#pragma unroll
        for (int u = 0; u < 2 * KS; ++u) {
          if (u + 1 < 2 * KS) rf[(u + 1) & 1] = read_row(u + 1);
          const int s = u >> 1, kb = u & 1;
          sacc[kb] = mfma_32x32x16(rf[u & 1].k, qf[s], sacc[kb]);
          pacc[kb] = mfma_32x32x16(rf[u & 1].v, df[s], pacc[kb]);
          __builtin_amdgcn_sched_barrier(0);
        }

        // ---- P^T = 2^{S^T scale log2e - L}; dS^T = P^T (dP^T - D), as bf16 B operand
        bf16x8 sf[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float p = fast_exp2(fmaf(sacc[kb][i], scale_log2, -lq2));
            if (need_mask) {
              const int kk = key0 + kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
              if (kk >= Nk || (CAUSAL && kk > qry + off)) p = 0.f;
            }
            sf[kb][i >> 3][i & 7] = (__bf16)(p * (pacc[kb][i] - dlt));
          }

        // ---- dQ^T += K^T dS^T, step u = (kb * 2 + t) * DB + b (K^T by
        // transpose reads of the K tile)
        auto read_kt = [&](int u) {
          const int kt = u / DB, b = u % DB;
          const int roff = kt * 16 * RB;
          return concat4(lds_read_tr4((const ATTN_LDS __bf16*)(ks + (tr_lo ^ (64 * b)) + roff)),
                         lds_read_tr4((const ATTN_LDS __bf16*)(ks + (tr_hi ^ (64 * b)) + roff)));
        };
        constexpr int US = 4 * DB;
        bf16x8 ka[2];
        ka[0] = read_kt(0);
#pragma unroll
        for (int u = 0; u < US; ++u) {
          if (u + 1 < US) ka[(u + 1) & 1] = read_kt(u + 1);
          const int kt = u / DB, b = u % DB;
          dq_acc[b] = mfma_32x32x16(ka[u & 1], sf[kt >> 1][kt & 1], dq_acc[b]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  };
  for (int j = 0; j < n_tiles; j += 2) {
    tile(j, Buf0{});
    if (j + 1 < n_tiles) tile(j + 1, Buf1{});
  }

  // ---- dQ = scale * acc: lane holds query qry, d rows b*32 + (i/4)*8 + half*4 + i%4
  if (PARTIAL && qok) {
    float* row = dq_part + (((int64_t)split * BH + bh) * Nq + qry) * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = dq_acc[b][r * 4 + e] * scale;
        *reinterpret_cast<f32x4*>(row + b * 32 + r * 8 + half * 4) = w;
      }
  } else if (qok) {
    __bf16* row = dq + qhead + (int64_t)qry * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(dq_acc[b][r * 4 + e] * scale);
        *reinterpret_cast<bf16x4*>(row + b * 32 + r * 8 + half * 4) = w;
      }
  }
}

// dQ = sum over the splits of the fp32 partials, in split order (so the
// result does not depend on which workgroup finished first), as bf16; eight
// consecutive elements per thread.
__global__ void __launch_bounds__(256)
bwd_dq_reduce_kernel(const float* __restrict__ part, __bf16* __restrict__ dq, int64_t n,
                     int splits) {
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e0 >= n) return;
  f32x4 a = {}, b = {};
  for (int s = 0; s < splits; ++s) {
    const float* src = part + (int64_t)s * n + e0;
    a += *reinterpret_cast<const f32x4*>(src);
    b += *reinterpret_cast<const f32x4*>(src + 4);
  }
  bf16x8 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w[e] = (__bf16)a[e];
    w[e + 4] = (__bf16)b[e];
  }
  *reinterpret_cast<bf16x8*>(dq + e0) = w;
}

// ---------------------------------------------------------------- launchers
template <int D>
hipError_t launch_phase(const BwdArgs& a, int phase) {
  const int BH = a.B * a.H;
  const hipStream_t s = (hipStream_t)a.stream;
  const int off = a.causal ? a.Nk - a.Nq : 0;
  if (phase == 0) {
    const int64_t rows = (int64_t)BH * a.Nq;
    hipLaunchKernelGGL(bwd_preprocess_kernel<D>, dim3((unsigned)((rows + 31) / 32)), dim3(256),
                       0, s, (const __bf16*)a.o, (const __bf16*)a.dout, a.delta, rows);
  } else if (phase == 1) {
    return launch_bwd_dkdv(a);
  } else {
    const bool form_d = phase == 3;
    if (form_d && a.dq_splits > 1) {
      // key chunks each see part of a row only: D from the preprocess kernel
      const hipError_t e = launch_phase<D>(a, 0);
      if (e != hipSuccess) return e;
      return launch_phase<D>(a, 2);
    }
    const int nqt = (a.Nq + kDqBQ - 1) / kDqBQ;
    // d = 256 without the mask runs the masked kernel with every key visible
    // (off = Nk): its unmasked instantiation spills registers there
    const int dq_off = a.causal ? off : a.Nk;
    if (a.dq_splits > 1) {
      // key chunks: the masked instantiation for either mask (off = Nk shows
      // every key), then the reduction
      hipLaunchKernelGGL((bwd_dq_kernel<D, true, true>), dim3((unsigned)((int64_t)BH * nqt * a.dq_splits)),
                         dim3(kBwdThreads), 0, s, (const __bf16*)a.q, (const __bf16*)a.k,
                         (const __bf16*)a.v, (const __bf16*)a.dout, (const __bf16*)a.o, a.lse,
                         a.delta, (__bf16*)a.dq, BH, a.Nq, a.Nk, dq_off, nqt, a.scale,
                         a.scale * kLog2e, a.dq_part, a.dq_chunk);
      const int64_t n = (int64_t)BH * a.Nq * D;
      hipLaunchKernelGGL(bwd_dq_reduce_kernel, dim3((unsigned)((n / 8 + 255) / 256)), dim3(256), 0, s,
                         (const float*)a.dq_part, (__bf16*)a.dq, n, a.dq_splits);
      return hipGetLastError();
    }
    auto kern = form_d ? bwd_dq_kernel<D, true, false, true> : bwd_dq_kernel<D, true>;
    if constexpr (D <= 128) {
      if (!a.causal) kern = form_d ? bwd_dq_kernel<D, false, false, true> : bwd_dq_kernel<D, false>;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(BH * nqt)), dim3(kBwdThreads), 0, s,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                       (const __bf16*)a.dout, (const __bf16*)a.o, a.lse, a.delta, (__bf16*)a.dq,
                       BH, a.Nq, a.Nk, dq_off, nqt, a.scale, a.scale * kLog2e, (float*)nullptr, 0);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_phase(const BwdArgs& a, int phase) {
  switch (a.d) {
    case 32: return launch_phase<32>(a, phase);
    case 64: return launch_phase<64>(a, phase);
    case 96: return launch_phase<96>(a, phase);
    case 128: return launch_phase<128>(a, phase);
    case 256: return launch_phase<256>(a, phase);
    default: return hipErrorInvalidValue;
  }
}

BwdDqSplit bwd_dq_split_plan(int B, int H, int Nq, int Nk, int d) {
  BwdDqSplit sp{1, 0, 0};
  if (Nq >= Nk) return sp;  // square calls run attn_bwd's kernels unchanged
  const int64_t base = (int64_t)B * H * ((Nq + kDqBQ - 1) / kDqBQ);
  const int64_t tiles = (Nk + kDqBK - 1) / kDqBK;
  // about two workgroups per CU in all, each chunk at least eight key tiles
  int64_t want = (512 + base - 1) / base;
  want = std::min<int64_t>(want, std::max<int64_t>(1, tiles / 8));
  if (want <= 1) return sp;
  const int64_t per = (tiles + want - 1) / want;
  sp.splits = (int)((tiles + per - 1) / per);
  if (sp.splits <= 1) return BwdDqSplit{1, 0, 0};
  sp.chunk = (int)(per * kDqBK);
  sp.part_bytes = ((size_t)sp.splits * (size_t)B * H * (size_t)Nq * (size_t)d * sizeof(float) + 255) &
                  ~(size_t)255;
  return sp;
}

// dQ forming D (phase 3), then dK/dV, which reads that D (phase 1)
hipError_t launch_bwd(const BwdArgs& a) {
  const hipError_t e = launch_bwd_phase(a, 3);
  if (e != hipSuccess) return e;
  return launch_bwd_phase(a, 1);
}

}  // namespace attn
