// device_common.h - gfx950 building blocks shared by the attention kernels.
//
// Lane layouts used throughout (wave64, checked on gfx950 hardware):
//
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A operand: lane l holds A[l % 32][(l / 32) * 8 + e],  e = 0..7
//     B operand: lane l holds B[(l / 32) * 8 + e][l % 32],  e = 0..7
//     C/D:       lane l holds D[(i / 4) * 8 + (l / 32) * 4 + (i % 4)][l % 32],
//                i = 0..15
//
//   ds_read_b64_tr_b16 (LDS transpose read): inside each group of 16 lanes,
//     if lane j of the group points at 4 consecutive 16-bit elements L[j][0..3],
//     lane i of the group receives element e = L[4 e + i / 4][i % 4].
//     So when lane j points at row (r0 + j / 4), columns (c0 + 4 (j % 4)) of a
//     row-major tile, lane i receives column c0 + i of rows r0 .. r0 + 3.
//
//   v_permlane32_swap(x, x) returns {x of lanes 0-31 in both halves,
//     x of lanes 32-63 in both halves}.
//
//   buffer_load_dwordx4 ... lds (direct global -> LDS): lane l's 16 bytes
//     land at LDS address M0 + 16 l, so one wave instruction fills 1 KiB of
//     LDS in lane order.  The instruction's immediate offset moves the global
//     AND the LDS address, so it is kept at 0.
//
// LDS banks: 64 banks of 4 bytes.  A ds_read_b128 is served 8 lanes at a
// time and a ds_read_b64_tr_b16 16 lanes at a time; both are conflict-free
// when the lanes served together touch distinct 16-byte bank groups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define ATTN_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x with the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) with the hardware transcendental unit (v_log_f32).
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Transpose read of 4 bf16 from LDS (see the layout note above).
__device__ __forceinline__ bf16x4 lds_read_tr4(const ATTN_LDS __bf16* p) {
  short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS short4v*)p);
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 concat4(bf16x4 lo, bf16x4 hi) {
  bf16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// True on every lane when p holds on at least one active lane of the wave.
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// max of x over lanes l and l ^ 32.
__device__ __forceinline__ float max_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

// x of lane l plus x of lane l ^ 32.
__device__ __forceinline__ float sum_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Word 3 of a raw buffer resource on gfx9-family chips: 32-bit data format
// (any non-zero format enables untyped loads), everything else default.
constexpr int kBufferRsrcWord3 = 0x00020000;

// Wait until every outstanding global load of this wave (including LDS DMA)
// has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// XOR swizzle of the 16-byte chunks of a row-major bf16 tile of D columns
// stored without padding (rows of 2*D bytes).  Logical chunk c of row r sits
// at physical chunk c ^ tile_swizzle<D>(r).  The choice makes the two read
// patterns of the kernels conflict-free:
//   * ds_read_b128 of one chunk by 8 lanes on 8 consecutive rows, and
//   * ds_read_b64_tr_b16 by 16 lanes on 4 consecutive rows (first row a
//     multiple of 4) and 2 adjacent chunks (first chunk even).
// D = 128 (16 chunks, one row = all 64 banks) and D = 256 (32 chunks, two
// bank rows; the XOR only touches the low 4 bits of the chunk index, which
// select the bank group): 4 (r & 3) + ((r >> 2) & 3).
// D = 64 (8 chunks, two rows per 64 banks): bit-reverse of (r >> 1) & 7.
template <int D>
__device__ __forceinline__ int tile_swizzle(int r) {
  if constexpr (D >= 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    const int x = (r >> 1) & 7;
    return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1);
  }
}

// Width of the LDS layout that holds a row of head dimension d: d = 32 rows
// sit in the 64-wide layout and d = 96 rows in the 128-wide one, their upper
// chunks never written nor read.  The MFMA loops run over d itself (d / 16
// k-steps, d / 32 output blocks), so the padding costs LDS space only.
constexpr int tile_width(int d) { return d <= 64 ? 64 : d <= 128 ? 128 : 256; }

// A 64-row tile of a row-major [rows][D] bf16 matrix held in LDS in rows of
// LD columns without padding between rows, its 16-byte chunks XOR-swizzled by
// row (tile_swizzle<LD>).  Columns D .. LD - 1 of the layout are unused.
template <int LD, int D = LD>
struct SwzTile {
  static_assert(LD == 64 || LD == 128 || LD == 256, "layout widths with a swizzle");
  static_assert(D % 32 == 0 && D <= LD, "d must be a multiple of 32 within the layout");
  static constexpr int kRows = 64;
  static constexpr int kRowBytes = 2 * LD;
  static constexpr int kBytes = kRows * kRowBytes;
  static constexpr int kRowsPerDma = 1024 / kRowBytes;  // rows one wave instruction fills
  static constexpr int kChunksPerRow = LD / 8;
  static constexpr int kDataChunks = D / 8;             // chunks that hold data

  // Copy rows [row0, row0 + 64) of `src` (row stride D elements) into `dst`
  // using the NW waves of the workgroup.  Lane l of an instruction writes
  // physical chunk l % kChunksPerRow of its row, so it fetches the logical
  // chunk the swizzle maps there; lanes whose logical chunk lies past column
  // D issue nothing.  The copies are buffer loads whose resource starts at
  // row row0 and ends at row nrows (at most 64 rows on), so the per-lane
  // offsets are the same for every tile and need no address arithmetic in
  // the loop; rows at or past `nrows` fall outside the resource and read as
  // zeros (finite values that the callers' masks give weight 0).
  template <int NW>
  static __device__ __forceinline__ void load(const __bf16* src, int row0, int nrows,
                                              ATTN_LDS unsigned char* dst, int wave, int lane) {
    constexpr int kPerWave = kRows / kRowsPerDma / NW;
    static_assert(kRows % (kRowsPerDma * NW) == 0, "tile must split over the waves");
    const int r_in = lane / kChunksPerRow;
    const int chunk = lane % kChunksPerRow;
    const int w = __builtin_amdgcn_readfirstlane(wave);  // LDS destinations in SGPRs
    // (uniform; readfirstlane keeps the resource in SGPRs where a VALU min
    // or max would otherwise leave it in VGPRs behind a waterfall loop)
    const int rows_left = __builtin_amdgcn_readfirstlane(min(max(nrows - row0, 0), kRows));
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(src + (int64_t)row0 * D), (short)0, rows_left * D * 2, kBufferRsrcWord3);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int blk = w * kPerWave + i;
      const int row = blk * kRowsPerDma + r_in;
      const int logical = chunk ^ tile_swizzle<LD>(row);
      if (kDataChunks == kChunksPerRow || logical < kDataChunks)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (ATTN_LDS void*)(dst + blk * 1024), 16,
                                                  row * (2 * D) + logical * 16, 0, 0, 0);
    }
  }

  // Row reads (MFMA operand with one tile row per lane): lane reads row
  // rb * 32 + l32, logical chunk 2 s + half.  Byte offset:
  //   (row_read_base(l32, half) ^ (32 s)) + rb * 32 * kRowBytes.
  static __device__ __forceinline__ int row_read_base(int l32, int half) {
    return (l32 * kRowBytes) | (((half ^ tile_swizzle<LD>(l32)) & (kChunksPerRow - 1)) << 4);
  }

  // Transpose reads (ds_read_b64_tr_b16): lane (group grp = lane / 16,
  // g16 = lane % 16) points at row r0 + half * 4 + g16 / 4 (+ 8 for `hi`),
  // columns 32 b + 16 (grp & 1) + 4 (g16 & 3), for r0 a multiple of 16.
  // Byte offset: (tr_read_base(lane, hi) ^ (64 b)) + r0 * kRowBytes.
  static __device__ __forceinline__ int tr_read_base(int lane, bool hi) {
    const int g16 = lane & 15;
    const int grp = lane >> 4;
    const int row = (grp >> 1) * 4 + (g16 >> 2) + (hi ? 8 : 0);
    const int cpart = 2 * (grp & 1) + ((g16 & 3) >> 1);
    return row * kRowBytes + (((cpart ^ tile_swizzle<LD>(row)) & (kChunksPerRow - 1)) << 4) +
           8 * (g16 & 1);
  }
};

}  // namespace attn
