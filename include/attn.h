/*
 * attn.h - C ABI of the MI355X (gfx950) fused attention library (libattn.so).
 *
 * The operation is scaled-dot-product attention computed with blocked online
 * softmax, never materialising the N x N score matrix:
 *
 *   forward   O = softmax(scale * Q K^T [+ causal mask]) V  and, per query
 *             row, the natural-log logsumexp lse_i = ln sum_j e^{scale q_i.k_j}
 *             over the keys the row sees.  (CS336 Lecture 5 notes "GPUs,
 *             TPUs", sections 8.1-8.3; CS149 Lecture 9 notes "Efficiently
 *             Evaluating DNNs on GPUs", sections 8-9; PDC notes Lecture 4,
 *             sections 4.8 and 4.13.)
 *   backward  from Q, K, V, O, lse and dO, recomputes P = e^{scale*S - lse}
 *             block by block and returns dQ, dK, dV of sum(dO * O), with
 *             D_i = rowsum(dO_i * O_i).  (CS336 L5 notes section 8.4 and
 *             Exercise 9.)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are DEVICE pointers to contiguous row-major arrays.  Q, K, V, O,
 *   dO, dQ, dK, dV have shape [B][H][N][d] (a head's rows are tokens); lse is
 *   float32 [B][H][N].  Element type is given by `dtype`; lse is always fp32.
 * - Q, K and V all have the same N (self-attention).  `causal` != 0 hides key
 *   j from query i when j > i (the diagonal is visible).  `scale` multiplies
 *   Q K^T before the softmax.  The pages scale by 1/sqrt(d) (CS336 L5 notes
 *   sections 8.1 and 8.3; PDC notes Lecture 4, section 4.8), a positive
 *   number, and the kernels are built for a positive scale: it must be finite
 *   and > 0, otherwise ATTN_ERR_SCALE (0, -0.0 and negative values included).
 *   Results are finite as long as scale * |q_i . k_j| fits fp32.
 * - N may be any value >= 1 (no tile multiple is required); d must be 32, 64,
 *   96, 128 or 256 (64 or 128 in the FP8 forwards attn_fwd_mx and
 *   attn_fwd_fp8).  bf16 is supported by every entry point; fp32 by the
 *   forward only.  B * H * ceil(N / 32) must not exceed 2^31 - 1 (the finest
 *   grid launched has one workgroup per 32 query rows); ATTN_ERR_SHAPE
 *   otherwise.
 * - The caller owns every buffer (including the backward workspace).  The
 *   library never allocates, frees or synchronises; it enqueues kernels on
 *   `stream` (a hipStream_t, NULL = the default stream) and returns.  Results
 *   are ready when that stream is synchronised.  Execution errors inside a
 *   kernel surface at that synchronisation, not in the return code.
 * - Arguments are validated on the host before anything is enqueued; on a
 *   non-zero return nothing was written.  Outputs must not alias inputs.
 * - Tensor pointers must be 16-byte aligned (the kernels use 128-bit
 *   accesses); lse, read and written one float at a time, 4-byte aligned.
 * - Calls are thread-safe: the library keeps no per-call global state (the
 *   device array of attn_bwd_noalloc aside, see there).
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V, O, dO, dQ, dK, dV. */
typedef enum {
  ATTN_DTYPE_F32 = 0,  /* float32 storage; the arithmetic is fp32 */
  ATTN_DTYPE_BF16 = 1  /* bfloat16 storage; bf16 MFMA with fp32 accumulation */
} attn_dtype_t;

/* Return codes. */
typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,      /* a required pointer is NULL */
  ATTN_ERR_SHAPE = -2,     /* B, H or N < 1, or sizes overflow 64-bit offsets */
  ATTN_ERR_DTYPE = -3,     /* unknown dtype, or dtype not supported by this entry point */
  ATTN_ERR_HEADDIM = -4,   /* d is not 32, 64, 96, 128 or 256 (attn_fwd_mx: 64, 128) */
  ATTN_ERR_ALIGN = -5,     /* a pointer is not 16-byte aligned (lse: 4-byte) */
  ATTN_ERR_SCALE = -6,     /* scale is not finite, or not > 0 */
  ATTN_ERR_WORKSPACE = -7, /* workspace NULL or smaller than attn_bwd_workspace_bytes() */
  ATTN_ERR_HIP = -8,       /* the HIP runtime refused a launch */
  ATTN_ERR_SCRATCH = -9    /* attn_bwd_noalloc: B*H*N above its static scratch */
} attn_status_t;

/* Forward pass (CS336 L5 notes section 8.3).
 *   q, k, v : [B][H][N][d] in `dtype`, read only.
 *   o       : [B][H][N][d] in `dtype`, written: softmax(scale*QK^T [mask]) V.
 *   lse     : [B][H][N] float32, written: per-row natural-log logsumexp of
 *             the scaled, masked scores.
 *   dtype   : ATTN_DTYPE_BF16 or ATTN_DTYPE_F32.
 *   stream  : hipStream_t to enqueue on (NULL = default stream).
 * Returns ATTN_OK or an attn_status_t error code. */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int d, int causal, float scale, int dtype,
             void* stream);

/* Bytes of device workspace attn_bwd needs for these sizes: the D vector
 * (B*H*N fp32), rounded up to a multiple of 256.  Returns 0 for invalid
 * sizes or an unsupported dtype. */
size_t attn_bwd_workspace_bytes(int B, int H, int N, int d, int dtype);

/* Backward pass (CS336 L5 notes section 8.4): recomputes attention from the
 * saved logsumexp and returns the gradients of sum(dout * O).  Every output
 * element is written exactly once (no atomics), so results are bitwise
 * reproducible.
 *   q, k, v     : forward inputs, [B][H][N][d] in `dtype`.
 *   o, lse      : the forward outputs for those inputs (o in `dtype`, lse
 *                 float32 [B][H][N]), as attn_fwd wrote them.
 *   dout        : [B][H][N][d] in `dtype`, the gradient flowing into O.
 *   dq, dk, dv  : [B][H][N][d] in `dtype`, written.
 *   workspace   : device scratch of at least attn_bwd_workspace_bytes()
 *                 bytes, owned by the caller; contents on entry are ignored.
 *   dtype       : ATTN_DTYPE_BF16 only (ATTN_ERR_DTYPE otherwise).
 * Calls that share a workspace must not overlap in time.
 * Returns ATTN_OK or an attn_status_t error code. */
int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const void* dout, const float* lse, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
             int causal, float scale, int dtype, void* stream);

/* attn_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and results, bit for bit, with the D vector kept in a static
 * device array of the library (16 MiB on each GPU it runs on, held until the
 * process ends) instead of a caller workspace.  It calls no hipMalloc or
 * hipFree; the array's device address is looked up (hipGetSymbolAddress) on
 * the first call made with a device current.  Arguments and errors are
 * those of attn_bwd without the workspace, plus ATTN_ERR_SCRATCH when
 * B * H * N exceeds 4,194,304 query rows.  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (two streams, two host
 * threads) race and give undefined results; calls in sequence on one
 * stream do not.  Call it with the device that holds the tensors current. */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                     int B, int H, int N, int d, int causal, float scale, int dtype,
                     void* stream);

/* One phase of the backward, for callers that schedule or time the phases
 * separately.  attn_bwd(...) is exactly phase 3 then phase 1 on one stream,
 * with the same arguments:
 *   0  preprocess: D = rowsum(dO * O) into the workspace (CS336 L5 notes
 *      section 8.4 and Exercise 9)
 *   1  dK and dV: key blocks outside, query blocks inside; writes dk, dv
 *   2  dQ: query blocks outside, key blocks inside; writes dq
 *   3  phases 0 and 2 in one launch: the dQ kernel forms each query's D from
 *      its own dO and O rows, writes it to the workspace and writes dq
 * Phases 1 and 2 read D from the workspace, as phase 0 or 3 left it, not
 * each other's output.  0, 1, 2 in order give the results of attn_bwd within
 * the fp32 rounding of D (phase 0 sums its terms in another order).
 * A phase reads what the earlier phases left in the workspace; running them
 * out of order gives undefined results (no fault).  Errors as attn_bwd, plus
 * ATTN_ERR_SHAPE for a phase outside 0..3. */
int attn_bwd_phase(int phase, const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                   int causal, float scale, int dtype, void* stream);

/* Bytes of device workspace attn_fwd_kv needs for these sizes and this
 * num_splits (0 = the library's choice, the same one attn_fwd_kv makes): fp32
 * partial O and lse of every key chunk, each part rounded up to a multiple of
 * 256, when the keys are cut into two or more chunks.  Returns 0 when they
 * are not (one chunk needs no workspace), and 0 for invalid sizes or an
 * unsupported dtype, which attn_fwd_kv reports with its own error code. */
size_t attn_fwd_kv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits,
                                   int dtype);

/* Forward of Nq queries against an Nk-token key/value cache: decode (Nq = 1)
 * and chunked prefill (PDC notes Lecture 4, section 4.9; CS336 L5 notes
 * section 5.3).  The queries are the last Nq positions of the sequence.
 *   q          : [B][H][Nq][d] bf16, read only.
 *   k, v       : [B][H][Nk][d] bf16, read only.
 *   o          : [B][H][Nq][d] bf16, written.
 *   lse        : [B][H][Nq] float32, written (natural log, as attn_fwd).
 *   causal     : != 0 hides key j from query i when j > i + Nk - Nq, and then
 *                requires Nk >= Nq; 0 lets every query see every key.
 *   num_splits : number of key chunks streamed by separate workgroups and
 *                merged with the blocked-softmax identity (CS149 L9 notes
 *                section 9); 0 = chosen from the shape; values above
 *                ceil(Nk / 64) are capped.  It changes rounding only.
 *   workspace  : device scratch of at least attn_fwd_kv_workspace_bytes()
 *                bytes with the same num_splits, caller-owned; contents on
 *                entry are ignored.  When that size is 0 (one chunk) the
 *                workspace and workspace_bytes are not read (NULL is fine).
 *   dtype      : ATTN_DTYPE_BF16 only (ATTN_ERR_DTYPE otherwise).
 * With one chunk the forward kernel of attn_fwd walks all keys and writes o
 * and lse itself (no merge); Nq = Nk then gives attn_fwd's results bit for
 * bit.  Calls that share a workspace must not overlap in time.  Returns
 * ATTN_OK or an error:
 * those of attn_fwd, plus ATTN_ERR_SHAPE for Nq or Nk < 1, Nk < Nq with
 * causal, or num_splits < 0, and ATTN_ERR_WORKSPACE. */
int attn_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int Nq, int Nk, int d, int causal, float scale, int dtype,
                int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace attn_bwd_kv needs: the D vector (B*H*Nq fp32),
 * rounded up to a multiple of 256, plus, when dQ is split over the keys,
 * s partial results (s*B*H*Nq*d fp32, rounded up to a multiple of 256).  dQ
 * is split when Nq < Nk and the w = B*H*ceil(Nq/128) query tiles are too few
 * for the chip: s = number of chunks of ceil(T / m) key tiles, T = ceil(Nk/64),
 * m = min(ceil(512 / w), max(1, floor(T / 8))), when that is above 1.
 * Returns 0 for invalid sizes, an unsupported d or dtype. */
size_t attn_bwd_kv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int dtype);

/* Backward of attn_fwd_kv (CS336 L5 notes section 8.4 with the mask of a
 * key/value cache, PDC notes Lecture 4, section 4.9): Nq queries at the last
 * Nq positions of an Nk-token sequence, the training step of chunked
 * prefill.  Returns the gradients of sum(dout * O), recomputing attention
 * from the saved lse as attn_bwd does.
 *   q, o, dout, dq : [B][H][Nq][d] bf16 (dq written).
 *   k, v, dk, dv   : [B][H][Nk][d] bf16 (dk, dv written).
 *   lse            : [B][H][Nq] float32, the forward's (attn_fwd_kv writes it).
 *   causal         : != 0 hides key j from query i when j > i + Nk - Nq, and
 *                    then requires Nk >= Nq; 0 lets every query see every key.
 *   workspace      : at least attn_bwd_kv_workspace_bytes() bytes, caller-
 *                    owned, contents on entry ignored.
 * Nq = Nk is attn_bwd, bit for bit (the same kernels).  bf16.
 * With few queries the dQ sums over the keys run in chunks on separate
 * workgroups and are added in chunk order, so results still do not depend on
 * timing.  Every output element is written once (no atomics).  Errors: those of
 * attn_fwd_kv and attn_bwd.  Calls that share a workspace must not overlap. */
int attn_bwd_kv(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, void* workspace,
                size_t workspace_bytes, int B, int H, int Nq, int Nk, int d, int causal,
                float scale, int dtype, void* stream);

/* Forward pass with Q and K in MXFP8 (CS336 L5 notes section 6.2: E4M3
 * values plus one E8M0 scale per 32 elements; here the blocks run along d,
 * the dimension S = Q K^T contracts) and V in bf16.  Computes exactly what
 * attn_fwd computes for the decoded Q and K:
 *   Q[b,h,i,c] = e4m3(q8[b,h,i,c]) * 2^(q_scale[b,h,i,c/32] - 127), K alike.
 *   q8, k8           : [B][H][N][d] E4M3 codes (OCP FP8: bias 7, no
 *                      infinities, S.1111.111 = NaN), 16-byte aligned.
 *   q_scale, k_scale : [B][H][N][d/32] E8M0 scale codes (2^(e-127); 255 =
 *                      NaN), 4-byte aligned for d = 128, 2-byte for d = 64.
 *   v                : [B][H][N][d] bf16.  o: bf16 [B][H][N][d].  lse: fp32.
 *   d                : 64 or 128.
 * S runs on the gfx950 scaled FP8 matrix instruction; P is rounded to bf16
 * for P V as in attn_fwd.  Returns the codes of attn_fwd (ATTN_ERR_HEADDIM for
 * d other than 64 or 128). */
int attn_fwd_mx(const void* q8, const void* q_scale, const void* k8, const void* k_scale,
                const void* v, void* o, float* lse, int B, int H, int N, int d, int causal,
                float scale, void* stream);

/* FP8 attention forward: Q, K and V all in MXFP8 (CS336 L5 notes section
 * 6.2: E4M3 values plus one E8M0 scale per 32 elements), S = Q K^T and
 * P V both on the gfx950 scaled FP8 matrix instruction.  Q and K as in
 * attn_fwd_mx (blocks along d, the contraction of S).  P V contracts over
 * the keys, and block scales do not survive a transpose (same section), so V
 * comes transposed and quantised along the keys:
 *   vt8      : [B][H][d][ldv] E4M3 codes of V^T, ldv = 64 * ceil(N / 64);
 *              row c holds V[0..N-1][c]; codes at keys N..ldv-1 are ignored
 *              (any value, NaN codes included).  16-byte aligned.
 *   vt_scale : [B][H][d][ldv / 32] E8M0 codes, one per 32 keys of a row:
 *              V[j][c] = e4m3(vt8[b,h,c,j]) * 2^(vt_scale[b,h,c,j/32] - 127);
 *              scales of blocks wholly past N are ignored.  2-byte aligned.
 * P = 2^(s - m) with m the running reference maximum is rounded to E4M3
 * (round to nearest even; P <= 2^8, so its block scale is 2^0) for P V; the
 * row sum and lse use P before rounding.  Per element that adds at most
 * 2^-4 P + 2^-10 (relative to the row's largest P) times |V| to O before
 * normalisation.  o: bf16 [B][H][N][d]; lse: fp32 [B][H][N].  d: 64 or 128;
 * N <= 2^26.  Other arguments and errors as attn_fwd_mx. */
int attn_fwd_fp8(const void* q8, const void* q_scale, const void* k8, const void* k_scale,
                 const void* vt8, const void* vt_scale, void* o, float* lse, int B, int H, int N,
                 int d, int causal, float scale, void* stream);

/* Row-wise softmax of an M x N row-major matrix x (PDC notes Lecture 5,
 * section 5.20, fused softmax; CS149 L9 notes section 8):
 *   y_ij = e^{x_ij - max_j x_ij} / sum_j e^{x_ij - max_j x_ij}.
 *   x, y   : device pointers to M*N elements of `dtype` (fp32 or bf16), rows
 *            contiguous; y may equal x (in place), otherwise they must not
 *            overlap.  Entries equal to -inf get probability 0; a row needs at
 *            least one finite entry.
 * Each row is read from HBM once and written once (twice read for rows of
 * more than 16384 elements).  Returns ATTN_OK, ATTN_ERR_NULL, ATTN_ERR_SHAPE
 * (M or N < 1, M above 2^40 or M * N above 2^48), ATTN_ERR_DTYPE, ATTN_ERR_ALIGN
 * (x or y not 16-byte aligned) or ATTN_ERR_HIP. */
int attn_softmax_rows(const void* x, void* y, long long M, int N, int dtype, void* stream);

/* Static, human-readable text for a return code (never NULL). */
const char* attn_status_str(int status);

/* Library ABI version; bumped when an entry point is added or a signature or
 * a calling contract changes (2: attn_fwd_kv and attn_fwd_kv_workspace_bytes;
 * 3: attn_softmax_rows, and head dimensions 32, 96 and 256; 4: attn_fwd_mx;
 * 5: attn_bwd_noalloc; 6: attn_bwd_kv and attn_bwd_kv_workspace_bytes;
 * 7: attn_fwd_fp8; 8: attn_fwd_kv with one key chunk needs no workspace;
 * 9: attn_bwd_phase 3, and attn_bwd as phase 3 then phase 1). */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
