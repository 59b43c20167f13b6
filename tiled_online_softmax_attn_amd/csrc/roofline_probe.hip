// roofline_probe.hip - measured ceilings of the chip the attention kernels
// run on (libattn_probe.so, declared in include/attn_probe.h).
//
// The roofline of CS336 Lecture 5 notes "GPUs, TPUs" (section 5.1) takes
// attainable = min(peak compute, intensity x bandwidth); section 5.4 asks to
// measure the ceilings rather than trust the data sheet.  Three probes:
//   * the dense bf16 matrix rate (v_mfma_f32_32x32x16_bf16, four
//     independent accumulator chains per wave), optionally with E groups of
//     the softmax's per-score VALU work (an FMA for scale and maximum, the
//     exponential, the row-sum add) issued between the MFMAs, which is what
//     the attention forward asks of a SIMD;
//   * the v_exp_f32 rate alone (eight independent chains per lane);
//   * a plain HBM copy, 16 bytes per lane per access, nontemporal.
// Wave 0 of every workgroup records the shader clock (s_memtime) and the
// 100 MHz constant clock (s_memrealtime) before and after its loop, so the
// clock the chip actually ran at under that load is measured too.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void clock_mark(unsigned long long* clk, bool end,
                                           unsigned long long& t0, unsigned long long& r0) {
  if (threadIdx.x != 0) return;
  const unsigned long long t = __builtin_amdgcn_s_memtime();
  const unsigned long long r = __builtin_amdgcn_s_memrealtime();
  if (!end) {
    t0 = t;
    r0 = r;
  } else {
    clk[2 * blockIdx.x] = t - t0;
    clk[2 * blockIdx.x + 1] = r - r0;
  }
}

// E softmax groups (FMA, exponential, add) after each of the four MFMAs of
// a round; 4 E independent score chains per lane.
template <int E>
__global__ void __launch_bounds__(256) mfma_probe_kernel(float* __restrict__ out,
                                                         unsigned long long* __restrict__ clk,
                                                         int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)(threadIdx.x + e));
    b[e] = (__bf16)(0.002f * (float)e - 0.003f);
  }
  f32x16 c[4] = {};
  float x[4 * E + 1], sum = 0.f;
#pragma unroll
  for (int j = 0; j < 4 * E + 1; ++j) x[j] = 0.01f * (float)(threadIdx.x & 7) + 0.05f * (float)j;
  const float m = 0.75f, sc = 0.0883883f;
  unsigned long long t0 = 0, r0 = 0;
  clock_mark(clk, false, t0, r0);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      c[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[r], 0, 0, 0);
#pragma unroll
      for (int g = 0; g < E; ++g) {
        // p = 2^(x sc - m) lies in (0.59, 0.63] for x in [0, 1], and p is
        // the chain's next score
        const float p = __builtin_amdgcn_exp2f(fmaf(x[r * E + g], sc, -m));
        sum += p;
        x[r * E + g] = p;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  clock_mark(clk, true, t0, r0);
  float s = sum;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[r][e];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Eight independent chains x = 2^(-x) per lane (the negation is a free
// source modifier, so the loop is v_exp_f32 alone); x stays in [0.5, 1].
__global__ void __launch_bounds__(256) exp_probe_kernel(float* __restrict__ out,
                                                        unsigned long long* __restrict__ clk,
                                                        int iters) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.05f * (float)j + 0.001f * (float)(threadIdx.x & 31);
  unsigned long long t0 = 0, r0 = 0;
  clock_mark(clk, false, t0, r0);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
  }
  clock_mark(clk, true, t0, r0);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// dst = src, 16 bytes per lane per access: a workgroup copies 16 KiB, its
// four 4 KiB slices read one after another by its 256 lanes (all four loads
// in flight before the stores), with nontemporal hints (the data is touched
// once).  One workgroup per 16 KiB, no grid-stride loop.
__global__ void __launch_bounds__(256) copy_probe_kernel(const f32x4* __restrict__ src,
                                                         f32x4* __restrict__ dst, int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  f32x4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (base + u * 256 < n16) v[u] = __builtin_nontemporal_load(src + base + u * 256);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (base + u * 256 < n16) __builtin_nontemporal_store(v[u], dst + base + u * 256);
}

}  // namespace

extern "C" {

int attn_probe_mfma(float* out, unsigned long long* clk, int blocks, int iters,
                    int softmax_groups, void* stream) {
  if (!out || !clk || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  const hipStream_t s = (hipStream_t)stream;
  switch (softmax_groups) {
    case 0: hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3(blocks), dim3(256), 0, s, out, clk, iters); break;
    case 1: hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3(blocks), dim3(256), 0, s, out, clk, iters); break;
    case 2: hipLaunchKernelGGL(mfma_probe_kernel<2>, dim3(blocks), dim3(256), 0, s, out, clk, iters); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int attn_probe_exp(float* out, unsigned long long* clk, int blocks, int iters, void* stream) {
  if (!out || !clk || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(exp_probe_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, clk,
                     iters);
  return (int)hipGetLastError();
}

int attn_probe_copy(const void* src, void* dst, long long bytes, void* stream) {
  if (!src || !dst || bytes < 16 || (bytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15))
    return (int)hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  const int64_t blocks64 = (n16 + 1023) / 1024;
  if (blocks64 > 0x7fffffff) return (int)hipErrorInvalidValue;
  const unsigned blocks = (unsigned)blocks64;
  hipLaunchKernelGGL(copy_probe_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const f32x4*)src, (f32x4*)dst, n16);
  return (int)hipGetLastError();
}

}  // extern "C"
