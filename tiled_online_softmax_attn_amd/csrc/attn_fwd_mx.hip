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
//
// attn_fwd_fp8 (FP8V) also takes V in MXFP8, and runs P V on the same
// instruction.  P V contracts over the keys, so V arrives transposed, V^T
// with one scale per 32 keys of each of its d rows: the blocks then run along
// the contraction again (a V quantised along d would have to be re-quantised
// after the transpose, as the notes say).  O^T = V^T P^T per 64-key tile:
//   A = V^T (32 d rows x 64 keys): lane half h of row r reads keys 16 h ..
//     16 h + 15 and 32 + 16 h .. 32 + 16 h + 15 of the tile, two 16-byte
//     chunks of the row; the scale of keys 0-31 comes from lane r, of keys
//     32-63 from lane r + 32.
//   B = P^T: P is rounded to E4M3 straight from the S^T accumulator, where
//     lane (q, h) holds keys 32 kb + 8 a + 4 h + (0..3), a = 0..3, as four
//     32-bit groups of 4 codes per 32-key half kb; two v_permlane32_swap per
//     half exchange groups a = 0 <-> 2 and 1 <-> 3 between the lane halves,
//     after which lane half h holds keys 32 kb + 16 h + (0..15) in the order
//     the A operand expects.  P = 2^(s - m_ref) <= 2^8 (the lazy reference),
//     within E4M3's range, so P's block scale is 2^0.
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

// A 64-key tile of V^T in LDS: D rows (one per head dimension) of 64 E4M3
// codes, the four 16-byte chunks of row r XOR-swizzled by (r >> 2) & 3, so
// that the fragment reads (lane r of lane half h: chunks h and 2 + h of row
// 32 b + r) touch distinct 16-byte bank groups for any 16 consecutive lanes.
template <int D>
struct VtTile {
  static constexpr int kBytes = D * 64;
  static constexpr int kCopies = kBytes / 1024;  // wave instructions per tile
  static __device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }
  // Copy keys [key0, key0 + 64) of every row of `vt` (rows of ldv bytes, ldv
  // a multiple of 64) with the NW waves of the workgroup: instruction blk
  // fills rows 16 blk .. 16 blk + 15, lane l writing physical chunk l % 4 of
  // row l / 4, which holds the row's logical chunk (l % 4) ^ swz(row).  Each
  // instruction's resource starts at its first row and ends 64 bytes into
  // its last, so every offset stays inside it; with key0 >= ldv (a tile past
  // the end of the rows) the resource is empty and the tile reads as zeros.
  template <int NW>
  static __device__ __forceinline__ void load(const unsigned char* vt, int key0, int ldv,
                                              ATTN_LDS unsigned char* dst, int wave, int lane) {
    static_assert(kCopies % NW == 0, "tile must split over the waves");
    constexpr int kPerWave = kCopies / NW;
    const int w = __builtin_amdgcn_readfirstlane(wave);
    const bool live = key0 < ldv;
    const int k0 = __builtin_amdgcn_readfirstlane(live ? key0 : 0);
    const int records = __builtin_amdgcn_readfirstlane(live ? 15 * ldv + 64 : 0);
    const int row = lane >> 2;
    const int voff = row * ldv + (((lane & 3) ^ swz(row)) << 4);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int blk = w * kPerWave + i;
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(vt + (int64_t)(16 * blk) * ldv + k0), (short)0, records, kBufferRsrcWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (ATTN_LDS void*)(dst + blk * 1024), 16, voff,
                                                0, 0, 0);
    }
  }
  // byte offsets of lane (r = lane % 32, h = lane / 32)'s two chunks in row
  // r; row 32 b + r adds 2048 b
  static __device__ __forceinline__ int read_lo(int r, int h) { return r * 64 + ((h ^ swz(r)) << 4); }
  static __device__ __forceinline__ int read_hi(int r, int h) {
    return r * 64 + (((2 + h) ^ swz(r)) << 4);
  }
};

// E4M3 code of 2^0: the block scale of P (P <= 2^8 fits E4M3 unscaled)
constexpr int kScaleOne4 = 0x7F7F7F7F;

// Query i sees keys j with j - i <= off: off = 0 under the causal mask,
// off = N without it.  FP8V: V^T in MXFP8 (vt8, vts, rows of ldv bytes)
// instead of V in bf16, and P V on the scaled FP8 instruction.
template <int D, bool FP8V>
__global__ void __launch_bounds__(kMxThreads, 2)
attn_fwd_mx_kernel(const unsigned char* __restrict__ q8, const unsigned char* __restrict__ qs,
                   const unsigned char* __restrict__ k8, const unsigned char* __restrict__ ks,
                   const __bf16* __restrict__ v, const unsigned char* __restrict__ vt8,
                   const unsigned char* __restrict__ vts, int ldv, __bf16* __restrict__ o,
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
  // 72 KB per workgroup, two workgroups per CU; with FP8V the V^T buffers
  // hold 8 KB)
  constexpr int kVBytes = FP8V ? VtTile<D>::kBytes : VTile::kBytes;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[KTile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[KTile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k2[KTile::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[kVBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[kVBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v2[kVBytes];
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
  const __bf16* vh = FP8V ? nullptr : v + head * D;
  // FP8V: the head's V^T codes (D rows of ldv bytes) and scales (D rows of
  // ldv / 32 bytes)
  const unsigned char* vth = FP8V ? vt8 + (int64_t)bh * D * ldv : nullptr;
  const unsigned char* vtsh = FP8V ? vts + (int64_t)bh * D * (ldv / 32) : nullptr;

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
    if constexpr (FP8V) {
      // tiles past the end of the rows get an empty resource: zeros
      VtTile<D>::template load<kMxThreads / 64>(vth, j * kMxBK, ldv, dst, wave, lane);
    } else {
      VTile::template load<kMxThreads / 64>(vh, j * kMxBK, N, dst, wave, lane);
    }
  };
  // FP8V: the V^T scale the lane supplies for tile j and each of its rows
  // 32 b + l32: block 2 j + half (keys 64 j + 32 half ..); tiles past the
  // end re-read the last tile's (never used)
  auto load_vsc = [&](int j, int (&dst)[D / 32]) {
    const int jj = min(j, ldv / kMxBK - 1);
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
      dst[b] = (int)vtsh[(int64_t)(32 * b + l32) * (ldv / 32) + 2 * jj + half];
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
  // FP8V: V^T scale words of tile t in vsc[t mod 3], [d block]
  int vsc[FP8V ? 3 : 1][D / 32];

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

  // FP8V part of step j after the row maximum: exponentials of tile j (kept
  // in fp32 for the row sum, rounded to E4M3 for P V) interleaved with the
  // scaled S^T MFMAs of tile j+1 (NEXT); V^T fragments read in the last
  // slots; O^T += V^T P^T on the scaled FP8 instruction, one MFMA per
  // 32-row d block.
  const int vt_lo = VtTile<D>::read_lo(l32, half);
  const int vt_hi = VtTile<D>::read_hi(l32, half);

  auto step_fp8v = [&](const int j, auto par_tag, f32x16 (&sc)[2], f32x16 (&sn)[2], auto mask_tag,
                       auto next_tag, const float m_off, float& psum) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr int T = decltype(par_tag)::value;
    constexpr int kSlots = 8;
    const int key0 = j * kMxBK;
    // Exponentials of scores 4 part .. 4 part + 3: accumulator entries 4 a ..
    // 4 a + 3 of key half kb (a = part % 4, kb = part / 4), the keys 32 kb +
    // 8 a + 4 h + (0..3) of lane (q, h); rounded to E4M3 as one group of four
    // codes right away.
    int pg[2][4];  // E4M3 codes of P^T: [key half][group of four]
    auto exp_part = [&](int part) {
      const int kb = part >> 2, a = part & 3;
      float p[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        p[c] = fast_exp2(fmaf(sc[kb][4 * a + c], scale_log2, -m_off));
        __asm__ volatile("" ::"v"(p[c]));  // keep it at this point of the issue order
        psum += p[c];
      }
      // the first conversion writes bytes 0-1 and keeps bytes 2-3 of its
      // input, which the second one overwrites: any input does, so p[0]'s
      // own register (its last use) is passed rather than a zero to load
      const int r = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __builtin_bit_cast(int, p[0]), false);
      pg[kb][a] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], r, true);
    };
    // swapping groups 0 <-> 2 and 1 <-> 3 of key half kb across the lane
    // halves leaves keys 32 kb + 16 h + (0..15) in the order [0, 2, 1, 3]
    auto pack_half = [&](int kb) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const auto r = __builtin_amdgcn_permlane32_swap((unsigned)pg[kb][a], (unsigned)pg[kb][a + 2],
                                                        false, false);
        pg[kb][a] = (int)r[0];
        pg[kb][a + 2] = (int)r[1];
      }
    };
    const ATTN_LDS unsigned char* vbuf = v_lds(par_tag);
    auto read_vt = [&](int b) {
      const i32x4 lo = *reinterpret_cast<const ATTN_LDS i32x4*>(vbuf + vt_lo + b * 2048);
      const i32x4 hi = *reinterpret_cast<const ATTN_LDS i32x4*>(vbuf + vt_hi + b * 2048);
      return concat8(lo, hi);
    };
    // V^T fragments of the DB blocks, read in the last DB slots
    i32x8 vf[DB];
    constexpr int kVtSlot0 = kSlots - DB;
    if constexpr (NEXT) {
      using Next = std::integral_constant<int, (T + 1) % 3>;
      const ATTN_LDS unsigned char* kbuf = k_lds(Next{});
      sn[0] = f32x16{};
      sn[1] = f32x16{};
      i32x8 ka[2];
      ka[0] = read_k(kbuf, 0, 0);
#pragma unroll
      for (int t = 0; t < kSlots; ++t) {
        if (t + 1 < 2 * KS) ka[(t + 1) & 1] = read_k(kbuf, (t + 1) >> 1, (t + 1) & 1);
        if (t >= kVtSlot0) vf[t - kVtSlot0] = read_vt(t - kVtSlot0);
        if (t < 2 * KS) qk_mfma(sn, ka[t & 1], t, ksc[(T + 1) % 3]);
        exp_part(t);
        if (t == kSlots / 2 - 1) pack_half(0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int t = 0; t < kSlots; ++t) {
        if (t >= kVtSlot0) vf[t - kVtSlot0] = read_vt(t - kVtSlot0);
        exp_part(t);
        if (t == kSlots / 2 - 1) pack_half(0);
      }
    }
    pack_half(1);
    const i32x8 pb = {pg[0][0], pg[0][2], pg[0][1], pg[0][3],
                      pg[1][0], pg[1][2], pg[1][1], pg[1][3]};
    // on the tile that holds key N - 1 (a masked tile), the codes of keys
    // past N (whatever the caller left in the padding of the rows) become 0
    // and the scales of blocks wholly past N become 2^0: their P is 0
    // already, but a NaN code or scale would still poison the product
    int vmask[8];
    if constexpr (MASK) {
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kbase = key0 + (w < 4 ? 16 * half + 4 * w : 32 + 16 * half + 4 * (w - 4));
        const int cnt = min(max(N - kbase, 0), 4);
        vmask[w] = (cnt == 4) ? -1 : (int)((1u << (8 * cnt)) - 1u);
      }
    }
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      int vs = vsc[T][b];  // block 2 j + half
      if constexpr (MASK) {
#pragma unroll
        for (int w = 0; w < 8; ++w) vf[b][w] &= vmask[w];
        if (key0 + 32 * half >= N) vs = 127;
      }
      oacc[b] = mfma_mx<0>(vf[b], pb, oacc[b], vs, kScaleOne4);
    }
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
    if constexpr (FP8V) {
      step_fp8v(j, par_tag, sc, sn, mask_tag, next_tag, m_off, psum);
      l_run += psum;
      return;
    } else {
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
  constexpr int kCopiesV = FP8V ? VtTile<D>::kCopies / (kMxThreads / 64)
                                : VTile::kRows / VTile::kRowsPerDma / (kMxThreads / 64);
  // copies plus the scale-word loads of one iteration (K: 2; V^T: D / 32)
  constexpr int kInFlight = kCopiesK + kCopiesV + 2 + (FP8V ? D / 32 : 0);
  auto iteration = [&](const int j, auto T_tag, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    constexpr int T = decltype(T_tag)::value;
    load_k(j + 3, k_lds(std::integral_constant<int, T>{}));
    load_v(j + 2, v_lds(std::integral_constant<int, T + 2>{}));
    load_ksc(j + 3, ksc[T]);
    if constexpr (FP8V) load_vsc(j + 2, vsc[(T + 2) % 3]);
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
  if constexpr (FP8V) load_vsc(0, vsc[0]);
  load_k(2, k_lds(std::integral_constant<int, 2>{}));
  load_v(1, v_lds(std::integral_constant<int, 1>{}));
  load_ksc(2, ksc[2]);
  if constexpr (FP8V) load_vsc(1, vsc[1]);
  // leaves K tile 2, V tile 1 and their scale words in flight
  wait_copies_barrier<kInFlight>();
  f32x16 s_cur[2], s_nxt[2];
  qk(s_cur, k_lds(std::integral_constant<int, 0>{}), ksc[0]);
  wait_copies_barrier<kInFlight>();  // K buffer 0 is refilled in iteration 0
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

template <int D, bool FP8V>
hipError_t launch_mx(const FwdMxArgs& a) {
  const int n_qtiles = (a.N + kMxBQ - 1) / kMxBQ;
  const int BH = a.B * a.H;
  const int ldv = (a.N + kMxBK - 1) / kMxBK * kMxBK;  // V^T row length (FP8V)
  hipLaunchKernelGGL((attn_fwd_mx_kernel<D, FP8V>), dim3((unsigned)(BH * n_qtiles)),
                     dim3(kMxThreads), 0, (hipStream_t)a.stream, (const unsigned char*)a.q8,
                     (const unsigned char*)a.q_scale, (const unsigned char*)a.k8,
                     (const unsigned char*)a.k_scale, (const __bf16*)a.v,
                     (const unsigned char*)a.vt8, (const unsigned char*)a.vt_scale, ldv,
                     (__bf16*)a.o, a.lse, BH, a.N, n_qtiles, a.causal ? 0 : a.N, a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_mx(const FwdMxArgs& a) {
  switch (a.d) {
    case 64: return a.vt8 ? launch_mx<64, true>(a) : launch_mx<64, false>(a);
    case 128: return a.vt8 ? launch_mx<128, true>(a) : launch_mx<128, false>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
