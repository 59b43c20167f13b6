/*
 * attn_probe.h - C ABI of libattn_probe.so: measured ceilings of the GPU the
 * attention library runs on.  Not part of the attention path; bench.py
 * (--peak, and the peak_measured figures of its report line) calls these to
 * put the measured rates beside the data-sheet peaks, as the roofline
 * discussion of CS336 Lecture 5 notes "GPUs, TPUs" (sections 5.1 and 5.4)
 * asks: attainable = min(peak compute, intensity x bandwidth), with the
 * ceilings measured on the machine.
 *
 * All pointers are DEVICE pointers owned by the caller; the functions enqueue
 * one kernel on `stream` (a hipStream_t, NULL = default) and return a
 * hipError_t value (0 = hipSuccess; hipErrorInvalidValue for bad arguments).
 */
#ifndef ATTN_PROBE_H_
#define ATTN_PROBE_H_

#ifdef __cplusplus
extern "C" {
#endif

/* Dense bf16 matrix rate: `blocks` workgroups of 256 threads; every wave runs
 * `iters` rounds of four v_mfma_f32_32x32x16_bf16 on four independent
 * accumulators (4 x 32768 FLOP per round), and after each MFMA
 * `softmax_groups` (0, 1 or 2) groups of the attention softmax's per-score
 * VALU work (FMA, exponential, add) on independent chains.
 *   out : float[blocks * 256], written (keeps the work observable).
 *   clk : unsigned long long[blocks * 2], written: per workgroup, shader
 *         clock cycles (s_memtime) and 100 MHz ticks (s_memrealtime) spent
 *         by its first wave in the loop.
 * FLOPs of a launch = blocks * 4 * iters * 4 * 32768. */
int attn_probe_mfma(float* out, unsigned long long* clk, int blocks, int iters,
                    int softmax_groups, void* stream);

/* v_exp_f32 rate: `blocks` x 256 threads, each `iters` rounds of eight
 * independent exponentials (blocks * 256 * iters * 8 in all).  out and clk
 * as above. */
int attn_probe_exp(float* out, unsigned long long* clk, int blocks, int iters, void* stream);

/* Plain HBM copy dst = src of `bytes` bytes (a multiple of 16, >= 16; both
 * pointers 16-byte aligned, not overlapping), 16 bytes per lane per access
 * with nontemporal hints; moves 2 * bytes through HBM. */
int attn_probe_copy(const void* src, void* dst, long long bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H_ */
