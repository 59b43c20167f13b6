// attn_fwd.hip - fused attention forward for gfx950.
//
// Method (CS336 Lecture 5 notes "GPUs, TPUs", section 8.3; CS149 Lecture 9
// notes "Efficiently Evaluating DNNs on GPUs", section 9): one workgroup owns
// a block of queries and streams the key/value blocks past it, keeping the
// running row maximum m, the running sum l and the output accumulator O on
// chip.  For each key block:
//   S = Q K^T * scale,  m' = max(m, rowmax S),  P = e^{S - m'},
//   l = e^{m - m'} l + rowsum P,  O = e^{m - m'} O + P V,  m = m'
// and at the end O /= l, lse = m + ln l.  Under the causal mask, key blocks
// wholly in the future of the query block are never visited (section 8.3).
//
// bf16 path (the throughput path):
//   * 256 threads = 4 waves; 128 queries per workgroup, 32 per wave.
//   * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so that in
//     the accumulator every lane owns ONE query (column l % 32) and 16 keys.
//     Row max / row sum are then in-lane plus one permlane32 swap.
//   * Q^T is held in registers for the whole kernel (B operand).
//   * O^T = V^T P^T: P^T feeds the B operand straight from the S^T
//     accumulator (bf16-rounded), and V^T comes from row-major V in LDS via
//     ds_read_b64_tr_b16.  The O^T accumulator keeps one query per lane, so
//     the e^{m - m'} rescale and the final 1/l are per-lane scalars.
//   * K and V tiles (64 keys) are double-buffered in LDS; the copies of the
//     next tiles are in flight while tile j is computed (at d = 96, 128 and
//     256, where S^T of tile j+1 is computed during the softmax of tile j, K
//     runs one tile ahead of V).
//   * The row sum runs on the matrix unit at d <= 64 (an all-ones operand
//     against P^T), on the VALU above.
//   * The exponentials run in base 2 with scale*log2(e) folded into one FMA.
//
// fp32 path: plain fp32 FMAs (no bf16 rounding anywhere), 8 threads per query.
#include "device_common.h"
#include "attn_launch.h"

#include <type_traits>

namespace attn {
namespace {

constexpr int kFwdThreads = 256;
constexpr int kFwdBQ = 128;  // queries per workgroup
constexpr int kFwdBK = 64;   // keys per K/V tile
constexpr float kRescaleSlack = 8.f;  // log2 units: P never exceeds 2^8

// Workgroup id -> (head, query tile).  Heavy causal tiles (late queries see
// more keys) are issued first.  With B*H a multiple of 8 every query tile of
// one head lands on the same XCD (ids are dealt round-robin over the 8 XCDs),
// so a head's K/V stay in one L2.
__device__ __forceinline__ void fwd_tile_coords(int bid, int BH, int n_qtiles, bool causal,
                                                int& bh, int& qt) {
  const int rank = bid / BH;
  bh = bid - rank * BH;
  qt = causal ? (n_qtiles - 1 - rank) : rank;
}

// Interleaved schedule of the pipelined forward (KS k-steps, exponentials of
// scores [32 s / KS, 32 (s + 1) / KS) in k-step s, two PV steps per k-step
// from kPvStart on): the part holding score e, and the first k-step from
// which every PV step issued in the loop finds the 8 scores of its 16 keys
// (kt = u / DB) exponentiated in an earlier k-step.
constexpr int exp_part_of(int e, int ks) {
  int p = 0;
  while (32 * (p + 1) / ks <= e) ++p;
  return p;
}
constexpr int pv_start(int ks, int db) {
  for (int start = 1; start < ks; ++start) {
    bool ok = true;
    for (int s = start; s < ks; ++s)
      for (int j = 0; j < 2; ++j)
        if (exp_part_of(8 * ((2 * (s - start) + j) / db) + 7, ks) >= s) ok = false;
    if (ok) return start;
  }
  return ks;
}
static_assert(pv_start(8, 4) == 2 && pv_start(16, 8) == 4 && pv_start(6, 3) == 2,
              "PV start of d = 128, 256 and 96");

// One code path serves both masks: query i sees keys j with j - i <= off,
// off = 0 under the causal mask and off = N without it (every key visible).
// A separate unmasked instantiation spilled registers at d = 96 and 128.
//
// PARTIAL: the same computation for Nq queries against Nk keys (the queries
// are the last Nq positions: off = Nk - Nq under the causal mask, Nk without
// it), with the keys cut into chunks of `chunk` keys (a multiple of the tile
// size).  Workgroup (split, query tile, head) walks chunk `split` only and
// writes that chunk's partial result for the merge: O_c normalised by the
// chunk's own sum (fp32, [split][bh][Nq][D]) and lse_c over the chunk's keys
// ([split][bh][Nq], natural log, -inf with O_c = 0 where no key of the chunk
// is visible).  Without PARTIAL: all Nk keys in one pass, bf16 O and lse
// (attn_fwd: Nq = Nk = N).
template <int D, bool PARTIAL>
__global__ void __launch_bounds__(kFwdThreads, D > 128 ? 1 : 2)
attn_fwd_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                     const __bf16* __restrict__ v, void* __restrict__ o_out,
                     float* __restrict__ lse, int BH, int Nq, int Nk, int n_qtiles, int off,
                     int chunk, float scale_log2) {
  using Tile = SwzTile<tile_width(D), D>;
  static_assert(kFwdBK == Tile::kRows, "K/V tile is one SwzTile");
  constexpr int RB = Tile::kRowBytes;
  constexpr int KS = D / 16;  // k-steps of the S^T MFMA
  constexpr int DB = D / 32;  // 32-wide d blocks of O^T
  // d >= 96: S^T of tile j+1 is computed during the softmax of tile j (the
  // MFMA work per tile is large enough to hide the exponentials; at d = 256,
  // one wave per SIMD, it is the only overlap there is).  d <= 64: S^T of a
  // tile is computed at the start of its own step, which keeps the register
  // count low enough for more waves per SIMD (measured faster there).
  constexpr bool kPipelineQK = (D == 96 || D == 128 || D == 256);
  // K and V tiles of 64 keys (SwzTile layout), two buffers each.  One LDS
  // object per buffer: the compiler then knows that the copies into one
  // buffer cannot alias reads of another and does not wait for them.
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[Tile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[Tile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[Tile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[Tile::kBytes];
  // buffer P of K / V (P a compile-time 0 or 1)
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

  // workgroup id -> (head, query tile, key chunk); heavy causal query tiles
  // first, consecutive ids on different heads (see fwd_tile_coords)
  const int rank = blockIdx.x / BH;
  const int bh = blockIdx.x - rank * BH;
  const int split = PARTIAL ? rank / n_qtiles : 0;
  const int qt = n_qtiles - 1 - (rank - split * n_qtiles);
  const int64_t qhead = (int64_t)bh * Nq * D;
  const int64_t khead = (int64_t)bh * Nk * D;
  const __bf16* qh = q + qhead;
  const __bf16* kh = k + khead;
  const __bf16* vh = v + khead;

  const int q_wave0 = qt * kFwdBQ + wave * 32;  // first query of this wave
  const int qry = q_wave0 + l32;                 // this lane's query

  // Q^T fragments (B operand): lane holds Q[qry][16 s + 8 half + e].
  bf16x8 qf[KS];
  {
    const bf16x8 zero = {};
    const __bf16* qrow = qh + (int64_t)(qry < Nq ? qry : 0) * D + half * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = (qry < Nq) ? *reinterpret_cast<const bf16x8*>(qrow + 16 * s) : zero;
  }

  // Key tiles t_begin .. t_begin + n_tiles - 1: the chunk's keys, up to the
  // last one the workgroup's last query sees.
  const int key_begin = PARTIAL ? split * chunk : 0;
  const int64_t chunk_end = PARTIAL ? min((int64_t)Nk, (int64_t)key_begin + chunk) : (int64_t)Nk;
  const int kv_end = (int)min(chunk_end, (int64_t)min(Nq, (qt + 1) * kFwdBQ) + off);
  const int t_begin = key_begin / kFwdBK;
  const int n_tiles = kv_end > key_begin ? (kv_end + kFwdBK - 1) / kFwdBK - t_begin : 0;

  auto load_tile = [&](const __bf16* src, int j, ATTN_LDS unsigned char* dst) {
    Tile::template load<kFwdThreads / 64>(src, j * kFwdBK, Nk, dst, wave, lane);
  };
  // per-lane LDS read offsets: K rows (A operand of S^T) and V transpose reads
  const int k_base = Tile::row_read_base(l32, half);
  const int v_base_lo = Tile::tr_read_base(lane, false);
  const int v_base_hi = Tile::tr_read_base(lane, true);

  // S^T = K Q^T for the two 32-key halves of the K tile in `kbuf` (two
  // independent MFMA chains).
  auto qk = [&](f32x16 (&sacc)[2], const ATTN_LDS unsigned char* kbuf) {
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
    auto read_k = [&](int s, int kb) {
      return *reinterpret_cast<const ATTN_LDS bf16x8*>(kbuf + (k_base ^ (32 * s)) + kb * 32 * RB);
    };
    if constexpr (D > 128) {
      // d = 256 runs one wave per SIMD with every register in use: read each
      // k-step's K fragments one step ahead instead of all at once
      bf16x8 a[2][2];
      a[0][0] = read_k(0, 0);
      a[0][1] = read_k(0, 1);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s + 1 < KS) {
          a[(s + 1) & 1][0] = read_k(s + 1, 0);
          a[(s + 1) & 1][1] = read_k(s + 1, 1);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sacc[kb] = mfma_32x32x16(a[s & 1][kb], qf[s], sacc[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sacc[kb] = mfma_32x32x16(read_k(s, kb), qf[s], sacc[kb]);
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = f32x16{};
  // Reference maximum of the exponentials, in log2 units (score * scale *
  // log2 e).  It only moves when a row maximum exceeds it by more than
  // kRescaleSlack, so P = 2^{s - m_ref} stays below 2^kRescaleSlack and the
  // e^{m - m'} rescale of O and l runs on few tiles.  Any reference value
  // gives the same O = (sum P V) / (sum P) and lse = m_ref + log2(l) in exact
  // arithmetic.
  float m_ref = -INFINITY;
  float l_run = 0.f;  // this lane's share of the running sum (its 32 keys per tile)
  // d <= 64: the row sum runs on the matrix unit instead of the VALU, which
  // is the busier of the two there (two to four exponentials per MFMA): an
  // all-ones A operand against P^T adds sum_k P[q][k] (the bf16 P the
  // numerator uses) to every row of lacc, four MFMAs per tile in place of 32
  // adds per lane.
  constexpr bool kSumOnMfma = (D <= 64);
  f32x16 lacc = {};
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;

  // Tile j of the softmax pipeline.  On entry `sc` holds S^T of tile j; the
  // step issues S^T of tile j+1 into `sn` (when NEXT) so that those MFMAs run
  // while the VALU evaluates the exponentials of tile j, then adds
  // V_j^T P_j^T to O^T.  MASK selects the path for tiles that straddle the
  // causal diagonal or the end of the sequence.
  auto step = [&](const int j, auto par_tag, f32x16 (&sc)[2], f32x16 (&sn)[2], auto mask_tag,
                  auto next_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool NEXT = kPipelineQK && decltype(next_tag)::value;
    using Other = std::integral_constant<int, 1 - decltype(par_tag)::value>;
    const int key0 = j * kFwdBK;
    if constexpr (!kPipelineQK) qk(sc, k_lds(par_tag));
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
          if (key >= Nk || key - qry > off) sc[kb][i] = -INFINITY;
        }
    }

    // ---- row maximum of this tile for the lane's query
    float mx = sc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][i]);
    mx = max_across_halves(mx) * scale_log2;

    // ---- move the reference maximum only when it is exceeded by the slack
    if (wave_any(mx > m_ref + kRescaleSlack)) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = (MASK && m_new == -INFINITY) ? 1.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
      if constexpr (kSumOnMfma) {
#pragma unroll
        for (int i = 0; i < 16; ++i) lacc[i] *= alpha;
      } else {
        l_run *= alpha;
      }
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[b][i] *= alpha;
    }
    const float m_off = (MASK && m_ref == -INFINITY) ? 0.f : m_ref;

    // ---- P = 2^{s * scale * log2 e - m_ref} (bf16 B operand) on the VALU,
    // interleaved in issue order with S^T of the next tile on the MFMA unit:
    // k-step s issues the two MFMAs of that step (its K fragments were read
    // one step earlier) and then the exponentials of 32 / KS scores.
    float psum = 0.f;
    bf16x8 pf[2][2];
    // the 32 scores of the lane in kExpParts parts (one per k-step of the
    // pipelined loop; of 5 or 6 scores at d = 96)
    constexpr int kExpParts = (32 % KS == 0 || kPipelineQK) ? KS : 8;
    auto exp_part = [&](int part) {
#pragma unroll
      for (int e = 32 * part / kExpParts; e < 32 * (part + 1) / kExpParts; ++e) {
        const int kb = e >> 4, i = e & 15;
        const float p = fast_exp2(fmaf(sc[kb][i], scale_log2, -m_off));
        // keep the exponential at this point of the issue order (it would
        // otherwise sink below the MFMAs it is meant to overlap with)
        __asm__ volatile("" ::"v"(p));
        if constexpr (!kSumOnMfma) psum += p;
        pf[kb][i >> 3][i & 7] = (__bf16)p;
      }
    };
    // V^T fragment for O^T += V^T P^T step u = (kb * 2 + t) * DB + b, which
    // covers 16 keys (kt = kb * 2 + t) and 32 d rows (b)
    const ATTN_LDS unsigned char* vbuf = v_lds(par_tag);
    auto read_v = [&](int u) {
      const int kt = u / DB, b = u % DB;
      const int roff = kt * 16 * RB;
      return concat4(lds_read_tr4((const ATTN_LDS __bf16*)(vbuf + (v_base_lo ^ (64 * b)) + roff)),
                     lds_read_tr4((const ATTN_LDS __bf16*)(vbuf + (v_base_hi ^ (64 * b)) + roff)));
    };
    auto pv = [&](int u, const bf16x8& vfrag) {
      const int kt = u / DB, b = u % DB;
      oacc[b] = mfma_32x32x16(vfrag, pf[kt >> 1][kt & 1], oacc[b]);
      if constexpr (kSumOnMfma) {
        if (b == DB - 1) lacc = mfma_32x32x16(ones, pf[kt >> 1][kt & 1], lacc);
      }
    };
    constexpr int US = 4 * DB;
    if constexpr (NEXT) {
      // k-step s issues the two MFMAs of S^T of tile j+1 for that step, the
      // exponentials of scores [32 s / KS, 32 (s + 1) / KS) of tile j and,
      // from s = kPvStart on, two steps of O^T += V^T P^T of tile j: PV step u
      // needs the 8 scores of its 16 keys kt = u / DB, and kPvStart is the
      // first k-step for which every PV step issued in the loop finds them
      // exponentiated in an earlier k-step (pv_start: 2 at d = 96 and 128, 4
      // at d = 256).  The last 2 kPvStart PV steps follow the loop.  MFMA and
      // VALU work are thus spread evenly over the step.
      static_assert(US == 2 * KS, "two PV steps per k-step");
      // While in this loop the wave takes issue priority over the other wave
      // of its SIMD (which may be issuing copies or a row maximum), so that
      // the matrix unit stays fed.
      __builtin_amdgcn_s_setprio(1);
      constexpr int kPvStart = pv_start(KS, DB);
      constexpr int kPvInLoop = 2 * (KS - kPvStart);
      const ATTN_LDS unsigned char* kbuf = k_lds(Other{});
      sn[0] = f32x16{};
      sn[1] = f32x16{};
      // K and V fragments are read two k-steps ahead of their MFMAs
      constexpr int PD = 2;
      bf16x8 a[PD + 1][2], va[PD + 1][2];
#pragma unroll
      for (int s0 = 0; s0 < PD; ++s0)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          a[s0][kb] = *reinterpret_cast<const ATTN_LDS bf16x8*>(kbuf + (k_base ^ (32 * s0)) + kb * 32 * RB);
#pragma unroll
      for (int s0 = 0; s0 < PD; ++s0)
        if (s0 >= kPvStart) {
          const int u0 = 2 * (s0 - kPvStart);
          va[s0 % (PD + 1)][0] = read_v(u0);
          va[s0 % (PD + 1)][1] = read_v(u0 + 1);
        }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s + PD < KS) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            a[(s + PD) % (PD + 1)][kb] = *reinterpret_cast<const ATTN_LDS bf16x8*>(
                kbuf + (k_base ^ (32 * (s + PD))) + kb * 32 * RB);
        }
        // V fragments of the PV steps of k-step s + PD
        if (s + PD >= kPvStart && s + PD < KS) {
          const int u0 = 2 * (s + PD - kPvStart);
          va[(s + PD) % (PD + 1)][0] = read_v(u0);
          va[(s + PD) % (PD + 1)][1] = read_v(u0 + 1);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sn[kb] = mfma_32x32x16(a[s % (PD + 1)][kb], qf[s], sn[kb]);
        exp_part(s);
        if (s >= kPvStart) {
          const int u0 = 2 * (s - kPvStart);
          pv(u0, va[s % (PD + 1)][0]);
          pv(u0 + 1, va[s % (PD + 1)][1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      l_run += psum;
      bf16x8 vt[2];
      vt[0] = read_v(kPvInLoop);
#pragma unroll
      for (int u = kPvInLoop; u < US; ++u) {
        if (u + 1 < US) vt[(u + 1) & 1] = read_v(u + 1);
        pv(u, vt[u & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int part = 0; part < kExpParts; ++part) exp_part(part);
      l_run += psum;
      // O^T += V^T P^T; consecutive steps go to different accumulators, and
      // each step's V^T fragment is read one step ahead.
      bf16x8 vt[2];
      vt[0] = read_v(0);
#pragma unroll
      for (int u = 0; u < US; ++u) {
        if (u + 1 < US) vt[(u + 1) & 1] = read_v(u + 1);
        pv(u, vt[u & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Last tile (counted from t_begin) this wave computes: under the causal
  // mask, later tiles lie wholly in the future of all of its queries; a wave
  // whose queries all lie past Nq computes none (wave-uniform).
  const int last_tile =
      q_wave0 >= Nq ? -1
                    : (int)min((int64_t)n_tiles - 1,
                               ((int64_t)min(Nq - 1, q_wave0 + 31) + off) / kFwdBK - t_begin);

  // One iteration of the workgroup loop.  Buffers, pipelined: in iteration j
  // the K tile j+1 and the V tile j are read; the copies of K tile j+2 (into
  // the buffer of K tile j, last read in iteration j-1) and V tile j+1 (into
  // the buffer of V tile j-1) are in flight meanwhile.  Not pipelined: K and
  // V tile j are read and the copies of K and V tile j+1 are in flight.  The
  // barrier at the end of every iteration publishes the copies.  par_tag is
  // the parity of j, so that every buffer is a compile-time choice.
  auto iteration = [&](const int j, auto par_tag, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    using Other = std::integral_constant<int, 1 - decltype(par_tag)::value>;
    if constexpr (kPipelineQK) {
      if (j + 2 < n_tiles) load_tile(kh, t_begin + j + 2, k_lds(par_tag));
    } else {
      if (j + 1 < n_tiles) load_tile(kh, t_begin + j + 1, k_lds(Other{}));
    }
    if (j + 1 < n_tiles) load_tile(vh, t_begin + j + 1, v_lds(Other{}));
    if (j <= last_tile) {
      const int jt = t_begin + j;  // tile index in the sequence
      const int key0 = jt * kFwdBK;
      const bool need_mask =
          (key0 + kFwdBK > Nk) || ((int64_t)key0 + kFwdBK - 1 > (int64_t)q_wave0 + off);
      const bool next = j < last_tile;
      if (need_mask) {
        if (next) step(jt, par_tag, sc, sn, std::true_type{}, std::true_type{});
        else step(jt, par_tag, sc, sn, std::true_type{}, std::false_type{});
      } else {
        if (next) step(jt, par_tag, sc, sn, std::false_type{}, std::true_type{});
        else step(jt, par_tag, sc, sn, std::false_type{}, std::false_type{});
      }
    }
    wait_vmem();
    __syncthreads();
  };

  // prologue: K tiles 0 and 1 and V tile 0 in LDS (and, pipelined, S^T of
  // tile 0 in registers)
  load_tile(kh, t_begin, k_lds(Par0{}));
  load_tile(vh, t_begin, v_lds(Par0{}));
  if (kPipelineQK && n_tiles > 1) load_tile(kh, t_begin + 1, k_lds(Par1{}));
  wait_vmem();
  __syncthreads();
  f32x16 s_even[2], s_odd[2];
  if constexpr (kPipelineQK) {
    qk(s_even, k_lds(Par0{}));
    __syncthreads();  // K buffer 0 is refilled in iteration 0
  }

  for (int j = 0; j < n_tiles; j += 2) {
    iteration(j, Par0{}, s_even, s_odd);
    if (j + 1 < n_tiles) iteration(j + 1, Par1{}, s_odd, s_even);
  }

  // ---- epilogue: O = O / l, lse = ln2 * (m + log2 l)
  const float l_tot = kSumOnMfma ? lacc[0] : sum_across_halves(l_run);
  const float m_run = m_ref;
  if (qry < Nq) {
    if constexpr (PARTIAL) {
      // chunk `split`'s partial result (l = 0: no key of the chunk visible)
      const int64_t prow = ((int64_t)split * BH + bh) * Nq + qry;
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      float* orow = (float*)o_out + prow * D;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = oacc[b][r * 4 + e] * inv;
          *reinterpret_cast<f32x4*>(orow + b * 32 + r * 8 + half * 4) = w;
        }
      if (half == 0) lse[prow] = l_tot > 0.f ? kLn2 * (m_run + fast_log2(l_tot)) : -INFINITY;
    } else {
      const float inv = 1.f / l_tot;
      __bf16* orow = (__bf16*)o_out + qhead + (int64_t)qry * D;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[b][r * 4 + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + b * 32 + r * 8 + half * 4) = w;
        }
      if (half == 0) lse[(int64_t)bh * Nq + qry] = kLn2 * (m_run + fast_log2(l_tot));
    }
  }
}

// ---------------------------------------------------------------- fp32 path
constexpr int kF32Threads = 256;
constexpr int kF32BK = 32;
// threads per query (each owns d / TPQ dims) and queries per workgroup: 8
// threads per query give the small fp32 shapes (one head of 256 queries) 8
// workgroups instead of 2, each thread a quarter of the serial work
template <int D> constexpr int kF32Tpq = 8;
template <int D> constexpr int kF32BQ = kF32Threads / kF32Tpq<D>;

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kF32Threads)
attn_fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                    const float* __restrict__ v, float* __restrict__ o,
                    float* __restrict__ lse, int BH, int N, int n_qtiles, float scale_log2) {
  constexpr int TPQ = kF32Tpq<D>;
  constexpr int BQ = kF32BQ<D>;
  constexpr int DH = D / TPQ;  // dims owned by each thread of a query
  __shared__ __attribute__((aligned(16))) float ks[kF32BK * D];
  __shared__ __attribute__((aligned(16))) float vs[kF32BK * D];

  const int tid = threadIdx.x;
  const int dpart = tid % TPQ;  // this thread's share of the query's dims
  int bh, qt;
  fwd_tile_coords(blockIdx.x, BH, n_qtiles, CAUSAL, bh, qt);
  const int64_t head = (int64_t)bh * N * D;
  const int qry = qt * BQ + tid / TPQ;
  const int q_block_last = min(N, (qt + 1) * BQ) - 1;

  float qr[DH], oa[DH];
  const float* qrow = q + head + (int64_t)(qry < N ? qry : 0) * D + dpart * DH;
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    qr[c] = (qry < N) ? qrow[c] : 0.f;
    oa[c] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;

  const int kv_end = CAUSAL ? q_block_last + 1 : N;
  for (int key0 = 0; key0 < kv_end; key0 += kF32BK) {
    __syncthreads();
    for (int c = tid; c < kF32BK * D / 4; c += kF32Threads) {
      const int row = c / (D / 4);
      const int col = (c % (D / 4)) * 4;
      const int key = key0 + row;
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
      if (key < N) {
        kk = *reinterpret_cast<const float4*>(k + head + (int64_t)key * D + col);
        vv = *reinterpret_cast<const float4*>(v + head + (int64_t)key * D + col);
      }
      *reinterpret_cast<float4*>(ks + row * D + col) = kk;
      *reinterpret_cast<float4*>(vs + row * D + col) = vv;
    }
    __syncthreads();

    float s[kF32BK];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kF32BK; ++jj) {
      const float* kr = ks + jj * D + dpart * DH;
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < DH; ++c) part = fmaf(qr[c], kr[c], part);
      float dot = part;
#pragma unroll
      for (int o = 1; o < TPQ; o <<= 1) dot += __shfl_xor(dot, o);
      const int key = key0 + jj;
      if (key >= N || (CAUSAL && key > qry)) dot = -INFINITY;
      s[jj] = dot;
      mx = fmaxf(mx, dot);
    }
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int c = 0; c < DH; ++c) oa[c] *= alpha;
#pragma unroll
    for (int jj = 0; jj < kF32BK; ++jj) {
      const float p = fast_exp2(fmaf(s[jj], scale_log2, -m_use));
      psum += p;
      const float* vr = vs + jj * D + dpart * DH;
#pragma unroll
      for (int c = 0; c < DH; ++c) oa[c] = fmaf(p, vr[c], oa[c]);
    }
    l_run = l_run * alpha + psum;
  }

  if (qry < N) {
    const float inv = 1.f / l_run;
    float* orow = o + head + (int64_t)qry * D + dpart * DH;
#pragma unroll
    for (int c = 0; c < DH; c += 4)
      *reinterpret_cast<float4*>(orow + c) =
          make_float4(oa[c] * inv, oa[c + 1] * inv, oa[c + 2] * inv, oa[c + 3] * inv);
    if (dpart == 0) lse[(int64_t)bh * N + qry] = kLn2 * (m_run + fast_log2(l_run));
  }
}

// All Nk keys in one pass per query tile: bf16 O and lse written directly.
template <int D>
hipError_t launch_whole(const void* q, const void* k, const void* v, void* o, float* lse,
                        int BH, int Nq, int Nk, int off, float scale, void* stream) {
  const int n_qtiles = (Nq + kFwdBQ - 1) / kFwdBQ;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false>), dim3((unsigned)(BH * n_qtiles)),
                     dim3(kFwdThreads), 0, (hipStream_t)stream, (const __bf16*)q,
                     (const __bf16*)k, (const __bf16*)v, o, lse, BH, Nq, Nk, n_qtiles, off, 0,
                     scale * kLog2e);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bf16(const FwdArgs& a) {
  return launch_whole<D>(a.q, a.k, a.v, a.o, a.lse, a.B * a.H, a.N, a.N, a.causal ? 0 : a.N,
                         a.scale, a.stream);
}

template <int D>
hipError_t launch_kv_whole(const FwdKvArgs& a) {
  return launch_whole<D>(a.q, a.k, a.v, a.o, a.lse, a.B * a.H, a.Nq, a.Nk,
                         a.causal ? a.Nk - a.Nq : a.Nk, a.scale, a.stream);
}

template <int D>
hipError_t launch_partial(const FwdKvArgs& a, const KvSplit& sp, float* o_part,
                          float* lse_part) {
  const int n_qtiles = (a.Nq + kFwdBQ - 1) / kFwdBQ;
  const int BH = a.B * a.H;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, true>),
                     dim3((unsigned)((int64_t)BH * n_qtiles * sp.splits)), dim3(kFwdThreads), 0,
                     (hipStream_t)a.stream, (const __bf16*)a.q, (const __bf16*)a.k,
                     (const __bf16*)a.v, (void*)o_part, lse_part, BH, a.Nq, a.Nk, n_qtiles,
                     a.causal ? a.Nk - a.Nq : a.Nk, sp.chunk, a.scale * kLog2e);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_f32(const FwdArgs& a) {
  const int n_qtiles = (a.N + kF32BQ<D> - 1) / kF32BQ<D>;
  const int BH = a.B * a.H;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)(BH * n_qtiles)),
                     dim3(kF32Threads), 0, (hipStream_t)a.stream, (const float*)a.q,
                     (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, BH, a.N,
                     n_qtiles, a.scale * kLog2e);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_d(const FwdArgs& a) {
  const bool c = a.causal != 0;
  if (a.bf16) return launch_bf16<D>(a);
  return c ? launch_f32<D, true>(a) : launch_f32<D, false>(a);
}

}  // namespace

hipError_t launch_fwd_kv_partial(const FwdKvArgs& a, const KvSplit& sp, float* o_part,
                                 float* lse_part) {
  switch (a.d) {
    case 32: return launch_partial<32>(a, sp, o_part, lse_part);
    case 64: return launch_partial<64>(a, sp, o_part, lse_part);
    case 96: return launch_partial<96>(a, sp, o_part, lse_part);
    case 128: return launch_partial<128>(a, sp, o_part, lse_part);
    case 256: return launch_partial<256>(a, sp, o_part, lse_part);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_kv_whole(const FwdKvArgs& a) {
  switch (a.d) {
    case 32: return launch_kv_whole<32>(a);
    case 64: return launch_kv_whole<64>(a);
    case 96: return launch_kv_whole<96>(a);
    case 128: return launch_kv_whole<128>(a);
    case 256: return launch_kv_whole<256>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd(const FwdArgs& a) {
  switch (a.d) {
    case 32: return launch_fwd_d<32>(a);
    case 64: return launch_fwd_d<64>(a);
    case 96: return launch_fwd_d<96>(a);
    case 128: return launch_fwd_d<128>(a);
    case 256: return launch_fwd_d<256>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
