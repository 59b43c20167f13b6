// attn_fwd_mx.hip - attention forward with Q and K in MXFP8 (gfx950).
//
// Q and K arrive in the microscaled FP8 format the CS336 Lecture 5 notes
// ("GPUs, TPUs", section 6.2) describe: E4M3 values with one E8M0 scale
// (a power of two) per 32 consecutive elements of a row, here along d.
// S = Q K^T contracts over d, the direction the blocks run in, so it runs on
// the gfx950 scaled FP8 matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4,
// which applies the block scales itself and accumulates in fp32: S is the
// exact product of the decoded values up to fp32 summation order, at twice
// the bf16 MFMA rate.  V and P stay bf16: P V contracts over the keys, and
// blocks along d do not survive that transpose (the same notes point this
// out: a transposed MX tensor has to be re-quantised), while an E4M3 P would
// carry a relative error of 2^-4 per probability.  The rest is the bf16
// forward (CS336 L5 notes section 8.3): one workgroup of 4 waves per 128
// queries, K/V tiles of 64 keys double-buffered in LDS and copied one tile
// ahead, S^T with the lane owning one query, a lazily moved reference
// maximum, base-2 exponentials, O^T += V^T P^T on bf16 MFMA.
//
// Layout of the scaled instruction (measured on gfx950 with one-hot probes):
//   A (32 rows x 64 k) and B (64 k x 32 cols): lane l holds row / col l % 32,
//     32 bytes; byte j of lane half h of A meets byte j of lane half h of B.
//   The scale of A row r for bytes 0-15 of both lane halves comes from lane
//     r, for bytes 16-31 from lane r + 32 (B likewise per column); the byte
//     of the 32-bit scale register is an immediate of the instruction.
// So with k-step s covering d = 64 s .. 64 s + 63, lane half h holds d =
// 64 s + 16 h + (0..15) in bytes 0-15 and 64 s + 32 + 16 h + (0..15) in
// bytes 16-31: bytes 0-15 of both halves are the MX block 2 s, bytes 16-31
// the block 2 s + 1, and lane half h supplies the scale of block 2 s + h.
#include "device_common.h"
#include "attn_launch.h"

#include <type_traits>

namespace attn {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kMxThreads = 256;
constexpr int kMxBQ = 128;  // queries per workgroup (32 per wave)
constexpr int kMxBK = 64;   // keys per K/V tile
constexpr float kMxRescaleSlack = 8.f;  // log2 units: P never exceeds 2^8

// C[32x32] += A[32x64] B[64x32] in E4M3 with E8M0 block scales; OPSEL picks
// the scale byte of sa / sb.
template <int OPSEL>
__device__ __forceinline__ f32x16 mfma_mx(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPSEL, sa, OPSEL, sb);
}

__device__ __forceinline__ i32x8 concat8(i32x4 lo, i32x4 hi) {
  i32x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// s_waitcnt with vmcnt = VM (at most VM of this wave's memory reads still in
// flight) and lgkmcnt = 0, then s_barrier; the asm statements keep the
// compiler from moving memory accesses across it.
template <int VM>
__device__ __forceinline__ void wait_copies_barrier() {
  static_assert(VM >= 0 && VM < 63, "vmcnt field");
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | ((VM >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Scales of a row's D / 32 blocks as one 32-bit word (byte b = block b).
template <int D>
__device__ __forceinline__ int load_scales(const unsigned char* row) {
  if constexpr (D == 128) return *reinterpret_cast<const int*>(row);
  else return (int)*reinterpret_cast<const unsigned short*>(row);
}

// Query i sees keys j with j - i <= off: off = 0 under the causal mask,
// off = N without it.
template <int D>
__global__ void __launch_bounds__(kMxThreads, 2)
attn_fwd_mx_kernel(const unsigned char* __restrict__ q8, const unsigned char* __restrict__ qs,
                   const unsigned char* __restrict__ k8, const unsigned char* __restrict__ ks,
                   const __bf16* __restrict__ v, __bf16* __restrict__ o,
                   float* __restrict__ lse, int BH, int N, int n_qtiles, int off,
                   float scale_log2) {
  static_assert(D == 64 || D == 128, "MX head dimensions");
  // K rows of D bytes held in LDS as rows of D / 2 two-byte elements
  using KTile = SwzTile<tile_width(D / 2), D / 2>;
  using VTile = SwzTile<tile_width(D), D>;
  static_assert(kMxBK == KTile::kRows && kMxBK == VTile::kRows, "tiles of 64 keys");
  constexpr int KRB = KTile::kRowBytes;
  constexpr int VRB = VTile::kRowBytes;
  constexpr int KS = D / 64;  // k-steps of the scaled S^T MFMA
  constexpr int DB = D / 32;  // 32-wide d blocks of O^T
  constexpr int NB = D / 32;  // MX blocks per row
  // rings of three buffers (tile t in buffer t mod 3): copies run two
  // iterations ahead of their use (K 8 KB and V 16 KB per buffer at d = 128,
  // 72 KB per workgroup, two workgroups per CU)
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[KTile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[KTile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k2[KTile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[VTile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[VTile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v2[VTile::kBytes];
  auto k_lds = [&](auto tag) {
    constexpr int b = decltype(tag)::value % 3;
    return (ATTN_LDS unsigned char*)(b == 0 ? lds_k0 : b == 1 ? lds_k1 : lds_k2);
  };
  auto v_lds = [&](auto tag) {
    constexpr int b = decltype(tag)::value % 3;
    return (ATTN_LDS unsigned char*)(b == 0 ? lds_v0 : b == 1 ? lds_v1 : lds_v2);
  };


  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // workgroup id -> (head, query tile), heavy causal tiles first
  const int rank = blockIdx.x / BH;
  const int bh = blockIdx.x - rank * BH;
  const int qt = n_qtiles - 1 - rank;
  const int64_t head = (int64_t)bh * N;  // first row of the head
  const unsigned char* kh = k8 + head * D;
  const unsigned char* ksh = ks + head * NB;
  const __bf16* vh = v + head * D;

  const int q_wave0 = qt * kMxBQ + wave * 32;  // first query of this wave
  const int qry = q_wave0 + l32;               // this lane's query
  const bool qok = qry < N;

  // Q^T fragments (B operand) and the lane's scale word, shifted so that
  // byte 2 s is the scale of block 2 s + half
  i32x8 qf[KS];
  int qsc;
  {
    const unsigned char* qrow = q8 + (head + (qok ? qry : 0)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const i32x4 zero = {};
      const i32x4 lo = qok ? *reinterpret_cast<const i32x4*>(qrow + 64 * s + 16 * half) : zero;
      const i32x4 hi = qok ? *reinterpret_cast<const i32x4*>(qrow + 64 * s + 32 + 16 * half) : zero;
      qf[s] = concat8(lo, hi);
    }
    qsc = load_scales<D>(qs + (head + (qok ? qry : 0)) * NB) >> (8 * half);
  }

  const int kv_end = (int)min((int64_t)N, (int64_t)(qt + 1) * kMxBQ + off);
  const int n_tiles = (kv_end + kMxBK - 1) / kMxBK;
  auto load_k = [&](int j, ATTN_LDS unsigned char* dst) {
    KTile::template load<kMxThreads / 64>((const __bf16*)kh, j * kMxBK, N, dst, wave, lane);
  };
  auto load_v = [&](int j, ATTN_LDS unsigned char* dst) {
    VTile::template load<kMxThreads / 64>(vh, j * kMxBK, N, dst, wave, lane);
  };
  // scale words of the lane's two keys of tile j (rows past the end re-read
  // the last row; the mask gives those keys weight 0), as loaded: the shift
  // by 8 half happens where they are used, so that nothing waits for the
  // load before then
  auto load_ksc = [&](int j, int (&dst)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = min(j * kMxBK + kb * 32 + l32, N - 1);
      dst[kb] = load_scales<D>(ksh + (int64_t)key * NB);
    }
  };
  const int k_base = KTile::row_read_base(l32, half);
  const int v_base_lo = VTile::tr_read_base(lane, false);
  const int v_base_hi = VTile::tr_read_base(lane, true);

  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = f32x16{};
  float m_ref = -INFINITY;  // reference maximum (log2 units), moved lazily
  float l_run = 0.f;        // this lane's share of the running sum
  int ksc[3][2];            // K scale words of tile t in ksc[t mod 3], [key half]

  // S^T of one tile (K buffer kbuf, scale words ks_) into sacc; `between(i)`
  // runs after the i-th of the 2 KS MFMAs
  auto read_k = [&](const ATTN_LDS unsigned char* kbuf, int s, int kb) {
    // chunks 4 s + half and 4 s + 2 + half of the key's row
    const int roff = kb * 32 * KRB;
    const i32x4 lo = *reinterpret_cast<const ATTN_LDS i32x4*>(kbuf + (k_base ^ (32 * (2 * s))) + roff);
    const i32x4 hi = *reinterpret_cast<const ATTN_LDS i32x4*>(kbuf + (k_base ^ (32 * (2 * s + 1))) + roff);
    return concat8(lo, hi);
  };
  auto qk_mfma = [&](f32x16 (&sacc)[2], const i32x8& a, int i, const int (&ks_)[2]) {
    const int s = i >> 1, kb = i & 1;
    const int ksw = ks_[kb] >> (8 * half);
    if (s == 0) sacc[kb] = mfma_mx<0>(a, qf[0], sacc[kb], ksw, qsc);
    else sacc[kb] = mfma_mx<2>(a, qf[KS - 1], sacc[kb], ksw, qsc);
  };
  auto qk = [&](f32x16 (&sacc)[2], const ATTN_LDS unsigned char* kbuf, const int (&ks_)[2]) {
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) qk_mfma(sacc, read_k(kbuf, i >> 1, i & 1), i, ks_);
  };

  // Tile j (tag T = j mod 3).  On entry `sc` holds S^T of tile j; with NEXT
  // the step forms S^T of tile j+1 into `sn` (K buffer and scale words
  // T + 1) while
  // the VALU exponentiates tile j, then adds V_j^T P_j^T.  Issue order, eight
  // slots: slot t issues S^T MFMA t (t < 2 KS), the exponentials of 4 scores
  // and, from slot 2 on, two of the 4 DB PV MFMAs whose 16 keys are already
  // exponentiated (PV step u needs exp parts 2 (u / DB) and 2 (u / DB) + 1);
  // the remaining PV MFMAs follow.
  auto step = [&](const int j, auto par_tag, f32x16 (&sc)[2], f32x16 (&sn)[2], auto mask_tag,
                  auto next_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr int T = decltype(par_tag)::value;
    const int key0 = j * kMxBK;
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
          if (key >= N || key - qry > off) sc[kb][i] = -INFINITY;
        }
    }
    float mx = sc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][i]);
    mx = max_across_halves(mx) * scale_log2;
    if (wave_any(mx > m_ref + kMxRescaleSlack)) {
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
    auto exp_part = [&](int part) {  // scores 4 part .. 4 part + 3
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = part * 4 + u;
        const int kb = e >> 4, i = e & 15;
        const float p = fast_exp2(fmaf(sc[kb][i], scale_log2, -m_off));
        // keep the exponential at this point of the issue order
        __asm__ volatile("" ::"v"(p));
        psum += p;
        pf[kb][i >> 3][i & 7] = (__bf16)p;
      }
    };
    const ATTN_LDS unsigned char* vbuf = v_lds(par_tag);
    auto read_v = [&](int u) {
      const int kt = u / DB, b = u % DB;
      const int roff = kt * 16 * VRB;
      return concat4(lds_read_tr4((const ATTN_LDS __bf16*)(vbuf + (v_base_lo ^ (64 * b)) + roff)),
                     lds_read_tr4((const ATTN_LDS __bf16*)(vbuf + (v_base_hi ^ (64 * b)) + roff)));
    };
    auto pv = [&](int u, const bf16x8& vfrag) {
      const int kt = u / DB, b = u % DB;
      oacc[b] = mfma_32x32x16(vfrag, pf[kt >> 1][kt & 1], oacc[b]);
    };
    constexpr int US = 4 * DB;
    constexpr int kSlots = 8;
    constexpr int kPvPerSlot = US / 8;  // 2 at d = 128, 1 at d = 64
    constexpr int kPvInLoop = kPvPerSlot * (kSlots - 2);
    if constexpr (NEXT) {
      using Next = std::integral_constant<int, (T + 1) % 3>;
      const ATTN_LDS unsigned char* kbuf = k_lds(Next{});
      sn[0] = f32x16{};
      sn[1] = f32x16{};
      i32x8 ka[2];
      ka[0] = read_k(kbuf, 0, 0);
      bf16x8 va[2][2];
#pragma unroll
      for (int t = 0; t < kSlots; ++t) {
        if (t + 1 < 2 * KS) ka[(t + 1) & 1] = read_k(kbuf, (t + 1) >> 1, (t + 1) & 1);
        if (t + 1 >= 2 && t + 1 < kSlots) {
#pragma unroll
          for (int w = 0; w < kPvPerSlot; ++w) va[(t + 1) & 1][w] = read_v(kPvPerSlot * (t - 1) + w);
        }
        if (t < 2 * KS) qk_mfma(sn, ka[t & 1], t, ksc[(T + 1) % 3]);
        exp_part(t);
        if (t >= 2) {
#pragma unroll
          for (int w = 0; w < kPvPerSlot; ++w) pv(kPvPerSlot * (t - 2) + w, va[t & 1][w]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
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
      for (int t = 0; t < kSlots; ++t) exp_part(t);
      l_run += psum;
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

  // last tile this wave computes: later tiles lie wholly past all its queries
  const int last_tile = (int)min((int64_t)n_tiles - 1, ((int64_t)q_wave0 + 31 + off) / kMxBK);
  // Iteration j (tag T = j mod 3) reads K tile j+1 and V tile j; it copies
  // K tile j+3 (into the buffer of K tile j, last read in iteration j-1), V
  // tile j+2 (into the buffer of V tile j-1) and the scale words of K tile
  // j+3, always the same number of copies (past the end they read zeros, or
  // the last key's scales), so that the wait at its end can leave exactly
  // this iteration's copies in flight.
  constexpr int kCopiesK = KTile::kRows / KTile::kRowsPerDma / (kMxThreads / 64);
  constexpr int kCopiesV = VTile::kRows / VTile::kRowsPerDma / (kMxThreads / 64);
  constexpr int kInFlight = kCopiesK + kCopiesV + 2;
  auto iteration = [&](const int j, auto T_tag, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    constexpr int T = decltype(T_tag)::value;
    load_k(j + 3, k_lds(std::integral_constant<int, T>{}));
    load_v(j + 2, v_lds(std::integral_constant<int, T + 2>{}));
    load_ksc(j + 3, ksc[T]);
    if (j <= last_tile) {
      const int key0 = j * kMxBK;
      const bool need_mask =
          (key0 + kMxBK > N) || ((int64_t)key0 + kMxBK - 1 > (int64_t)q_wave0 + off);
      const bool next = j < last_tile;
      if (need_mask) {
        if (next) step(j, T_tag, sc, sn, std::true_type{}, std::true_type{});
        else step(j, T_tag, sc, sn, std::true_type{}, std::false_type{});
      } else {
        if (next) step(j, T_tag, sc, sn, std::false_type{}, std::true_type{});
        else step(j, T_tag, sc, sn, std::false_type{}, std::false_type{});
      }
    }
    wait_copies_barrier<kInFlight>();
  };

  // prologue: K tiles 0..2, V tiles 0..1 and the scale words of K tiles 0..2
  // issued; K tiles 0, 1, V tile 0 and their scales landed; S^T of tile 0
  load_k(0, k_lds(std::integral_constant<int, 0>{}));
  load_ksc(0, ksc[0]);
  load_k(1, k_lds(std::integral_constant<int, 1>{}));
  load_ksc(1, ksc[1]);
  load_v(0, v_lds(std::integral_constant<int, 0>{}));
  load_k(2, k_lds(std::integral_constant<int, 2>{}));
  load_v(1, v_lds(std::integral_constant<int, 1>{}));
  load_ksc(2, ksc[2]);
  wait_copies_barrier<kCopiesK + kCopiesV + 2>();
  f32x16 s_cur[2], s_nxt[2];
  qk(s_cur, k_lds(std::integral_constant<int, 0>{}), ksc[0]);
  wait_copies_barrier<kCopiesK + kCopiesV + 2>();  // K buffer 0 is refilled in iteration 0
  auto advance = [&]() {  // S^T of the next tile becomes the current one
    s_cur[0] = s_nxt[0];
    s_cur[1] = s_nxt[1];
  };
  for (int j = 0; j < n_tiles; j += 3) {
    iteration(j, std::integral_constant<int, 0>{}, s_cur, s_nxt);
    advance();
    if (j + 1 < n_tiles) {
      iteration(j + 1, std::integral_constant<int, 1>{}, s_cur, s_nxt);
      advance();
    }
    if (j + 2 < n_tiles) {
      iteration(j + 2, std::integral_constant<int, 2>{}, s_cur, s_nxt);
      advance();
    }
  }
  wait_vmem();

  // ---- epilogue: O = O / l, lse = ln2 * (m + log2 l)
  const float l_tot = sum_across_halves(l_run);
  if (qok) {
    const float inv = 1.f / l_tot;
    __bf16* orow = o + (head + qry) * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[b][r * 4 + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + b * 32 + r * 8 + half * 4) = w;
      }
    if (half == 0) lse[head + qry] = kLn2 * (m_ref + fast_log2(l_tot));
  }
}

template <int D>
hipError_t launch_mx(const FwdMxArgs& a) {
  const int n_qtiles = (a.N + kMxBQ - 1) / kMxBQ;
  const int BH = a.B * a.H;
  hipLaunchKernelGGL((attn_fwd_mx_kernel<D>), dim3((unsigned)(BH * n_qtiles)), dim3(kMxThreads),
                     0, (hipStream_t)a.stream, (const unsigned char*)a.q8,
                     (const unsigned char*)a.q_scale, (const unsigned char*)a.k8,
                     (const unsigned char*)a.k_scale, (const __bf16*)a.v, (__bf16*)a.o, a.lse,
                     BH, a.N, n_qtiles, a.causal ? 0 : a.N, a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_mx(const FwdMxArgs& a) {
  switch (a.d) {
    case 64: return launch_mx<64>(a);
    case 128: return launch_mx<128>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
