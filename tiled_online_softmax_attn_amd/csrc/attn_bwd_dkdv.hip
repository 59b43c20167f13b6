// attn_bwd_dkdv.hip - phase 1 of the fused attention backward for gfx950:
// dK and dV (bf16 in/out, fp32 math).
//
// Method (CS336 Lecture 5 notes "GPUs, TPUs", section 8.4): key/value blocks
// outside, query blocks inside (the outer-K/V schedule of PDC notes Lecture 4,
// section 4.12).  A workgroup owns 128 keys and keeps their dK and dV in
// registers while it walks the query tiles that see them, recomputing
//   S = Q K^T,  P = e^{scale*S - L},  dV += P^T dO,
//   dP = dO V^T,  dS = P * (dP - D),  dK += scale * dS^T Q
// from Q, dO, the saved logsumexp L and D = rowsum(dO * O) (formed by the dQ
// kernel, which runs first, or by the preprocess kernel; attn_bwd.hip).  Every
// dK / dV element is written once, by the workgroup that owns its key.
//
// Register layout (v_mfma_f32_32x32x16_bf16; see device_common.h): S = Q K^T
// and dP = dO V^T with K^T / V^T fragments resident in registers, so every
// lane owns one key.  dV += P^T dO and dK += dS^T Q take P^T / dS^T straight
// from those accumulators as the A operand and read dO / Q through the LDS
// transpose read.
//
// Own compilation unit: build.py compiles this file with the LLVM option
// -amdgpu-mfma-vgpr-form, which makes every MFMA write ordinary registers.
// At d >= 96 a wave needs more than the 256 ordinary registers; the compiler
// then keeps some values in accumulation registers as spill space, but S and
// dP stay in ordinary registers and the softmax reads them directly.  Without
// the option every MFMA of a kernel that uses accumulation registers writes
// them, and the softmax pays two v_accvgpr_read per entry: at d = 128 the
// option cuts the VALU instructions of a query tile by 15% (d = 96 19%), with
// bitwise the same results.  dQ (attn_bwd.hip) is built without it: its d = 256
// kernel is slower in that form.
#include "device_common.h"
#include "attn_launch.h"

#include <type_traits>

namespace attn {
namespace {

constexpr int kBwdThreads = 256;

constexpr int kKvBK = 128;  // keys per workgroup (32 per wave)
constexpr int kKvBQ = 64;   // queries per inner step (one SwzTile)

// Columns of dK and dV one workgroup accumulates.  Up to d = 128 all of
// them; at d = 256 the K^T / V^T fragments of S and dP (128 registers) and
// dK, dV of all 256 columns (256 accumulators) would not fit one wave's 512
// registers beside S and dP, so two workgroups share a key block, each
// accumulating 128 columns; both compute S and dP over the full d.
constexpr int bwd_out_cols(int d) { return d > 128 ? 128 : d; }

// d = 32 fits three waves per SIMD (168 registers each, a one-step operand
// ring below: 186.8 -> 172.1 us against two waves on B4 H16 N4096 d32
// causal), d = 64 two (256 registers each, a two-step ring); d = 96 and above
// need one wave's whole register file (ordinary registers, plus accumulation
// registers that the allocator uses as spill space).
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kBwdThreads, D <= 32 ? 3 : D <= 64 ? 2 : 1)
bwd_dkdv_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                const __bf16* __restrict__ v, const __bf16* __restrict__ dout,
                const float* __restrict__ lse, const float* __restrict__ delta,
                __bf16* __restrict__ dk, __bf16* __restrict__ dv, int BH, int Nq, int Nk,
                int off, float scale, float scale_log2) {
  using Tile = SwzTile<tile_width(D), D>;
  static_assert(kKvBQ == Tile::kRows, "query tile is one SwzTile");
  constexpr int KS = D / 16;  // k-steps over d
  constexpr int DO = bwd_out_cols(D);  // dK / dV columns of this workgroup
  constexpr int NH = D / DO;           // workgroups per key block
  constexpr int DB = DO / 32;          // 32-wide blocks of those columns
  constexpr int RB = Tile::kRowBytes;
  // One LDS object per buffer: the compiler then knows that the copies into
  // one buffer cannot alias reads of the other and does not wait for them.
  __shared__ __attribute__((aligned(1024))) unsigned char lds_q0[Tile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_q1[Tile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_do0[Tile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_do1[Tile::kBytes];
  // [buffer][L, D][query]; D is stored negated at d <= 64 (see kDpFromNegD)
  __shared__ __attribute__((aligned(16))) float lds_stats[2][2][kKvBQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // workgroup id -> (head, key block, column half); low key blocks meet the
  // most queries under the causal mask, so they are issued first
  const int kblk = blockIdx.x / (BH * NH);
  const int rem = blockIdx.x - kblk * (BH * NH);
  const int ohalf = NH > 1 ? rem / BH : 0;
  const int bh = rem - ohalf * BH;
  const int c0 = ohalf * DO;  // first dK / dV column of this workgroup
  const int64_t qhead = (int64_t)bh * Nq * D;
  const int64_t khead = (int64_t)bh * Nk * D;
  const __bf16* qh = q + qhead;
  const __bf16* doh = dout + qhead;
  const float* lse_h = lse + (int64_t)bh * Nq;
  const float* del_h = delta + (int64_t)bh * Nq;

  const int key_wg0 = kblk * kKvBK;
  const int key_w0 = key_wg0 + wave * 32;  // first key of this wave
  const int key = key_w0 + l32;            // this lane's key (accumulator column)

  // K^T and V^T fragments (B operand): lane holds X[key][16 s + 8 half + e].
  bf16x8 kf[KS], vf[KS];
  {
    const bf16x8 zero = {};
    const bool ok = key < Nk;
    const __bf16* krow = k + khead + (int64_t)(ok ? key : 0) * D + half * 8;
    const __bf16* vrow = v + khead + (int64_t)(ok ? key : 0) * D + half * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kf[s] = ok ? *reinterpret_cast<const bf16x8*>(krow + 16 * s) : zero;
      vf[s] = ok ? *reinterpret_cast<const bf16x8*>(vrow + 16 * s) : zero;
    }
  }

  const int n_qtiles = (Nq + kKvBQ - 1) / kKvBQ;
  // the first query that sees key key_wg0 is key_wg0 - off
  const int qt_begin = CAUSAL ? max(key_wg0 - off, 0) / kKvBQ : 0;

  // Q and dO tiles go straight to LDS buffer B; L and D pass through one
  // register each on the first 64 threads (L is scaled to log2 units only
  // when stored, so that nothing waits for the load before then).
  float rl = 0.f, rd = 0.f;
  auto q_lds = [&](auto buf_tag) {
    return (ATTN_LDS unsigned char*)(decltype(buf_tag)::value ? lds_q1 : lds_q0);
  };
  auto do_lds = [&](auto buf_tag) {
    return (ATTN_LDS unsigned char*)(decltype(buf_tag)::value ? lds_do1 : lds_do0);
  };
  auto load_tile = [&](int qt, auto buf_tag) {
    Tile::template load<kBwdThreads / 64>(qh, qt * kKvBQ, Nq, q_lds(buf_tag), wave, lane);
    Tile::template load<kBwdThreads / 64>(doh, qt * kKvBQ, Nq, do_lds(buf_tag), wave, lane);
    if (tid < kKvBQ) {
      const int qq = qt * kKvBQ + tid;
      rl = qq < Nq ? lse_h[qq] : 0.f;
      rd = qq < Nq ? del_h[qq] : 0.f;
    }
  };
  auto store_stats = [&](auto buf_tag) {
    if (tid < kKvBQ) {
      lds_stats[decltype(buf_tag)::value][0][tid] = rl * kLog2e;
      lds_stats[decltype(buf_tag)::value][1][tid] = D <= 64 ? -rd : rd;
    }
  };
  using Buf0 = std::integral_constant<int, 0>;
  using Buf1 = std::integral_constant<int, 1>;

  const int rd_base = Tile::row_read_base(l32, half);
  // transpose reads of this workgroup's columns: block b of them is global
  // block b + ohalf * DB, i.e. chunk offset 64 (b ^ ohalf DB) (no carries)
  const int tr_lo = Tile::tr_read_base(lane, false) ^ (64 * DB * ohalf);
  const int tr_hi = Tile::tr_read_base(lane, true) ^ (64 * DB * ohalf);

  f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    dk_acc[b] = f32x16{};
    dv_acc[b] = f32x16{};
  }

  if (qt_begin < n_qtiles) {
    load_tile(qt_begin, Buf0{});
    store_stats(Buf0{});
  }
  wait_vmem();
  __syncthreads();

  // One query tile; its Q / dO / L / D sit in buffer CUR, and the copies of
  // the next tile go to the other buffer meanwhile.
  auto tile = [&](const int qt, auto cur_tag) {
    constexpr int CUR = decltype(cur_tag)::value;
    using Next = std::integral_constant<int, 1 - CUR>;
    if (qt + 1 < n_qtiles) load_tile(qt + 1, Next{});

    const int q0 = qt * kKvBQ;
    // wave-uniform: no query of the tile sees any key of this wave
    const bool skip = CAUSAL && (q0 + kKvBQ - 1 + off < key_w0);
    if (!skip) {
      const ATTN_LDS unsigned char* qs = q_lds(cur_tag);
      const ATTN_LDS unsigned char* dos = do_lds(cur_tag);
      const float* lq = lds_stats[CUR][0];
      const float* dstat = lds_stats[CUR][1];  // -D at d <= 64, D above
      const bool need_mask =
          (q0 + kKvBQ > Nq) || (key_w0 + 32 > Nk) || (CAUSAL && q0 + off < key_w0 + 31);

      // The tile's 64 queries are two 32-query blocks qb = 0, 1.  The issue
      // order is software-pipelined across them so that MFMA and VALU work
      // of the one wave overlap:
      //   A  S, dP of block 0                      (MFMA)
      //   B  S, dP of block 1   |  P, dS of block 0 (VALU)
      //   C  dV, dK of block 0  |  P, dS of block 1
      //   D  dV, dK of block 1
      // Every LDS operand is read one step before the MFMAs that use it, and
      // each softmax part's L values one part ahead, so that with a single
      // wave per SIMD the LDS latency stays off the critical path.
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
      // d <= 64: dP = dO V^T accumulates on top of -D.  Entry i of block qb
      // belongs to query row qb*32 + (i/4)*8 + half*4 + i%4, so its four
      // consecutive entries 4r .. 4r+3 start from four consecutive -D values
      // of the LDS stats, and the matrix unit delivers dP - D itself: 32 VALU
      // subtractions fewer per tile (fp32 sums in another order than dP
      // first, then - D).  B4 H16 N4096 causal, one box: d = 64 145.2 ->
      // 142.1 us, d = 32 175.3 -> 167.1 us; at d = 128, one wave per SIMD,
      // 551.7 -> 561.3 us, so d >= 96 subtract in the softmax as before.
      constexpr bool kDpFromNegD = D <= 64;
      f32x16 pacc[2] = {f32x16{}, f32x16{}};
      auto init_dp = [&](int qb) {
        if constexpr (!kDpFromNegD) return;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float4 nd = *reinterpret_cast<const float4*>(dstat + qb * 32 + r * 8 + half * 4);
          pacc[qb][4 * r] = nd.x;
          pacc[qb][4 * r + 1] = nd.y;
          pacc[qb][4 * r + 2] = nd.z;
          pacc[qb][4 * r + 3] = nd.w;
        }
      };
      init_dp(0);
      bf16x8 pa[2][2], sa[2][2];

      struct RowFrag { bf16x8 q, d; };   // Q and dO rows: one k-step of one block
      struct TrFrag { bf16x8 d, q; };    // dO and Q transposed: one (t, b) step
      struct Stats { float4 l, d; };     // L (and D) of 4 query rows
      // k-step s of S = Q K^T and dP = dO V^T for block qb
      auto read_row = [&](int qb, int s) {
        const int at = (rd_base ^ (32 * s)) + qb * 32 * RB;
        return RowFrag{*reinterpret_cast<const ATTN_LDS bf16x8*>(qs + at),
                       *reinterpret_cast<const ATTN_LDS bf16x8*>(dos + at)};
      };
      auto mma_sdp = [&](int qb, int s, const RowFrag& f) {
        sacc[qb] = mfma_32x32x16(f.q, kf[s], sacc[qb]);
        pacc[qb] = mfma_32x32x16(f.d, vf[s], pacc[qb]);
      };
      // step u = t * DB + b of dV += P^T dO and dK += dS^T Q for block qb
      auto read_tr = [&](int qb, int u) {
        const int t = u / DB, b = u % DB;
        const int roff = (qb * 32 + t * 16) * RB;
        const int lo = (tr_lo ^ (64 * b)) + roff;
        const int hi = (tr_hi ^ (64 * b)) + roff;
        return TrFrag{concat4(lds_read_tr4((const ATTN_LDS __bf16*)(dos + lo)),
                              lds_read_tr4((const ATTN_LDS __bf16*)(dos + hi))),
                      concat4(lds_read_tr4((const ATTN_LDS __bf16*)(qs + lo)),
                              lds_read_tr4((const ATTN_LDS __bf16*)(qs + hi)))};
      };
      auto mma_dvdk = [&](int qb, int u, const TrFrag& f) {
        const int t = u / DB, b = u % DB;
        dv_acc[b] = mfma_32x32x16(pa[qb][t], f.d, dv_acc[b]);
        dk_acc[b] = mfma_32x32x16(sa[qb][t], f.q, dk_acc[b]);
      };
      // L (and D, where the softmax subtracts it) of query rows
      // qb*32 + r*8 + half*4 + e, e = 0..3
      auto read_stats = [&](int qb, int r) {
        const int qrow0 = qb * 32 + r * 8 + half * 4;
        Stats st;
        st.l = *reinterpret_cast<const float4*>(lq + qrow0);
        if constexpr (!kDpFromNegD) st.d = *reinterpret_cast<const float4*>(dstat + qrow0);
        return st;
      };
      // Entries [lo, hi) of block qb: P = 2^{S scale log2e - L log2e} and
      // dS = P (dP - D), each bf16 pair converted as soon as both are done.
      // Entry i belongs to query row qb*32 + (i/4)*8 + half*4 + i%4; its L
      // (and -D) are part i/4 of the block, held in sv[(i/4) & 1] and read one
      // part ahead (the last part of block 0 reads the first of block 1).
      Stats sv[2];
      auto soft_range = [&](int qb, int lo, int hi, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
        for (int i = lo; i < hi; ++i) {
          const int r = i >> 2, e = i & 3;
          if (e == 0) {
            if (r + 1 < 4) sv[(r + 1) & 1] = read_stats(qb, r + 1);
            else if (qb == 0) sv[0] = read_stats(1, 0);
          }
          const Stats& st4 = sv[r & 1];
          const float lv = e == 0 ? st4.l.x : e == 1 ? st4.l.y : e == 2 ? st4.l.z : st4.l.w;
          float p = fast_exp2(fmaf(sacc[qb][i], scale_log2, -lv));
          if constexpr (MASK) {
            const int qq = q0 + qb * 32 + r * 8 + half * 4 + e;
            if (qq >= Nq || key >= Nk || (CAUSAL && key > qq + off)) p = 0.f;
          }
          // keep the exponential at this point of the issue order
          __asm__ volatile("" ::"v"(p));
          sacc[qb][i] = p;
          if constexpr (kDpFromNegD) {
            pacc[qb][i] = p * pacc[qb][i];
          } else {
            const float dv1 = e == 0 ? st4.d.x : e == 1 ? st4.d.y : e == 2 ? st4.d.z : st4.d.w;
            pacc[qb][i] = p * (pacc[qb][i] - dv1);
          }
          if (i & 1) {
            pa[qb][i >> 3][(i & 7) - 1] = (__bf16)sacc[qb][i - 1];
            pa[qb][i >> 3][i & 7] = (__bf16)sacc[qb][i];
            sa[qb][i >> 3][(i & 7) - 1] = (__bf16)pacc[qb][i - 1];
            sa[qb][i >> 3][i & 7] = (__bf16)pacc[qb][i];
          }
        }
      };

      // The tile is one sequence of steps g: KS row steps of block 0 (A), KS
      // of block 1 (B), 2*DB transposed steps of block 0 (C) and of block 1
      // (D).  Both kinds read two bf16x8 fragments, so one ring of registers
      // holds the fragments of the next kPrefetch steps (one at d = 32 and two
      // at d = 64, where the other waves of the SIMD also hide LDS latency).
      // The softmax of block 0 is spread evenly over the steps of B and that
      // of block 1 over the steps of C, so that every step carries about the
      // same VALU work beside its two MFMAs.
      constexpr int US = 2 * DB;
      constexpr int NSTEPS = 2 * KS + 2 * US;
      constexpr int kPrefetch = D <= 32 ? 1 : D <= 64 ? 2 : D == 128 ? 1 : 3;
      auto read_step = [&](int g) {
        if (g < KS) { const RowFrag f = read_row(0, g); return TrFrag{f.q, f.d}; }
        if (g < 2 * KS) { const RowFrag f = read_row(1, g - KS); return TrFrag{f.q, f.d}; }
        if (g < 2 * KS + US) return read_tr(0, g - 2 * KS);
        return read_tr(1, g - 2 * KS - US);
      };
      auto body = [&](auto mask_tag) {
        TrFrag ring[kPrefetch + 1];
#pragma unroll
        for (int g = 0; g < kPrefetch; ++g) ring[g] = read_step(g);
#pragma clang loop unroll(full)
        for (int g = 0; g < NSTEPS; ++g) {
          if (g + kPrefetch < NSTEPS) ring[(g + kPrefetch) % (kPrefetch + 1)] = read_step(g + kPrefetch);
          const TrFrag& f = ring[g % (kPrefetch + 1)];
          if (g < KS) {
            // A: S, dP of block 0
            mma_sdp(0, g, RowFrag{f.d, f.q});
            if (g == KS - 1) {
              sv[0] = read_stats(0, 0);
              init_dp(1);
            }
          } else if (g < 2 * KS) {
            // B: S, dP of block 1 | entries 16s/KS .. 16(s+1)/KS of block 0
            const int s = g - KS;
            mma_sdp(1, s, RowFrag{f.d, f.q});
            soft_range(0, 16 * s / KS, 16 * (s + 1) / KS, mask_tag);
          } else if (g < 2 * KS + US) {
            // C: dV, dK of block 0 | entries 16u/US .. 16(u+1)/US of block 1
            const int u = g - 2 * KS;
            mma_dvdk(0, u, f);
            soft_range(1, 16 * u / US, 16 * (u + 1) / US, mask_tag);
          } else {
            // D: dV, dK of block 1
            mma_dvdk(1, g - 2 * KS - US, f);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (need_mask)
        body(std::true_type{});
      else
        body(std::false_type{});
    }

    if (qt + 1 < n_qtiles) store_stats(Next{});
    wait_vmem();
    __syncthreads();
  };
  for (int qt = qt_begin; qt < n_qtiles; qt += 2) {
    tile(qt, Buf0{});
    if (qt + 1 < n_qtiles) tile(qt + 1, Buf1{});
  }

  // ---- dK = scale * acc, dV: lane holds d column b*32 + l32 and key rows
  //      (i/4)*8 + half*4 + i%4 of this wave's 32 keys
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = key_w0 + (i >> 2) * 8 + half * 4 + (i & 3);
      if (kk < Nk) {
        const int64_t at = khead + (int64_t)kk * D + c0 + b * 32 + l32;
        dk[at] = (__bf16)(dk_acc[b][i] * scale);
        dv[at] = (__bf16)dv_acc[b][i];
      }
    }
}

template <int D>
hipError_t launch_dkdv(const BwdArgs& a) {
  const int BH = a.B * a.H;
  const hipStream_t s = (hipStream_t)a.stream;
  const int off = a.causal ? a.Nk - a.Nq : 0;
  const int nkb = (a.Nk + kKvBK - 1) / kKvBK * (D / bwd_out_cols(D));
  // d = 32 without the mask runs the masked kernel with every key visible
  // (off = Nk): its unmasked instantiation spills registers at three waves
  // per SIMD
  auto kern = bwd_dkdv_kernel<D, true>;
  int kv_off = a.causal ? off : a.Nk;
  if constexpr (D != 32) {
    if (!a.causal) {
      kern = bwd_dkdv_kernel<D, false>;
      kv_off = 0;
    }
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(BH * nkb)), dim3(kBwdThreads), 0, s,
                     (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                     (const __bf16*)a.dout, a.lse, a.delta, (__bf16*)a.dk, (__bf16*)a.dv, BH,
                     a.Nq, a.Nk, kv_off, a.scale, a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dkdv(const BwdArgs& a) {
  switch (a.d) {
    case 32: return launch_dkdv<32>(a);
    case 64: return launch_dkdv<64>(a);
    case 96: return launch_dkdv<96>(a);
    case 128: return launch_dkdv<128>(a);
    case 256: return launch_dkdv<256>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
