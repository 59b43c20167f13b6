/*
 * attn_oracle.c - fp64 CPU oracle for scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite, the
 * smoke check in __graft_entry__.py and the CPU-baseline leg of bench.py may
 * load this library.  It shares no code, header, table or helper with the HIP
 * library under tiled_online_softmax_attn_amd/, and it includes nothing from
 * there.
 *
 * What it computes is the plain definition of attention, written out with
 * the N x N score matrix S and probability matrix P materialised:
 *
 *   S = scale * Q K^T                       (CS336 Lecture 5 notes "GPUs, TPUs",
 *                                            section 8.1; CS149 Lecture 9 notes
 *                                            "Efficiently Evaluating DNNs on
 *                                            GPUs", section 8)
 *   causal: S_ij = -inf for key j > query i  (query i sees keys 0..i)
 *   P = row softmax of S, with the row maximum subtracted
 *                                           (CS149 L9 notes section 8; PDC
 *                                            notes Lecture 4, section 4.13.2)
 *   O = P V                                 (CS149 L9 notes section 8)
 *   lse_i = m_i + ln(l_i)                   (CS336 L5 notes section 8.3: the
 *                                            logsumexp kept for the backward)
 *
 * and the exact gradient of sum(dO * O) with respect to Q, K, V, in the terms
 * of CS336 L5 notes section 8.4 and Exercise 9:
 *
 *   dV = P^T dO,  dP = dO V^T,  D_i = sum_k dO_ik O_ik,
 *   dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
 *
 * Everything is double precision.  Callers widen their inputs exactly (bf16
 * and fp32 values are exactly representable as doubles).  No blocking, no
 * online rescaling, no reordering: rows are independent, and OpenMP only
 * splits the rows of a matrix over threads, which does not change any sum.
 *
 * Every function returns 0 on success and a negative value on bad arguments
 * (-1 null pointer, -2 bad size, -3 allocation failure).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Thread count of later calls (timing on one thread); no effect on results. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Safe softmax of one row (CS149 L9 notes section 8; PDC notes 4.13.2):
 * m = max x, f = exp(x - m), l = sum f, p = f / l.  Entries equal to -inf
 * (masked) get p = 0.  At least one entry must be finite. */
int oracle_softmax_row(const double* x, int64_t n, double* p, double* m_out,
                       double* l_out) {
  if (!x || !p) return -1;
  if (n < 1) return -2;
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j)
    if (x[j] > m) m = x[j];
  double l = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    p[j] = exp(x[j] - m);
    l += p[j];
  }
  for (int64_t j = 0; j < n; ++j) p[j] = p[j] / l;
  if (m_out) *m_out = m;
  if (l_out) *l_out = l;
  return 0;
}

/* Score row i: s[j] = scale * <q_i, k_j>, or -inf where the causal mask hides
 * key j from query i. */
static void score_row(const double* q, const double* k, int64_t N, int64_t d,
                      int causal, double scale, int64_t i, double* s) {
  const double* qi = q + i * d;
  for (int64_t j = 0; j < N; ++j) {
    if (causal && j > i) {
      s[j] = -INFINITY;
      continue;
    }
    const double* kj = k + j * d;
    double dot = 0.0;
    for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];
    s[j] = scale * dot;
  }
}

/* Forward for one head.  q, k, v: [N][d]; o: [N][d]; lse: [N].
 * p_out, if not NULL, receives P as [N][N]. */
int oracle_attn_fwd_head(const double* q, const double* k, const double* v,
                         int64_t N, int64_t d, int causal, double scale,
                         double* o, double* lse, double* p_out) {
  if (!q || !k || !v || !o || !lse) return -1;
  if (N < 1 || d < 1) return -2;
  double* S = (double*)malloc(sizeof(double) * (size_t)N * (size_t)N);
  double* P = p_out ? p_out : (double*)malloc(sizeof(double) * (size_t)N * (size_t)N);
  if (!S || !P) {
    free(S);
    if (!p_out) free(P);
    return -3;
  }
  /* S = scale * Q K^T (+ mask) */
#pragma omp parallel for schedule(dynamic, 8)
  for (int64_t i = 0; i < N; ++i) score_row(q, k, N, d, causal, scale, i, S + i * N);
  /* P = softmax(S) row by row; lse = m + ln l */
#pragma omp parallel for schedule(dynamic, 8)
  for (int64_t i = 0; i < N; ++i) {
    double m, l;
    oracle_softmax_row(S + i * N, N, P + i * N, &m, &l);
    lse[i] = m + log(l);
  }
  /* O = P V */
#pragma omp parallel for schedule(dynamic, 8)
  for (int64_t i = 0; i < N; ++i) {
    double* oi = o + i * d;
    for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
    for (int64_t j = 0; j < N; ++j) {
      const double pij = P[i * N + j];
      const double* vj = v + j * d;
      for (int64_t c = 0; c < d; ++c) oi[c] += pij * vj[c];
    }
  }
  free(S);
  if (!p_out) free(P);
  return 0;
}

/* Forward for selected query rows of one head: the same definition, one row
 * at a time (S row, softmax, P row times V).  rows: nrows query indices in
 * [0, N); o_rows: [nrows][d]; lse_rows: [nrows]; p_rows, when not NULL,
 * [nrows][N] receives each row of P. */
int oracle_attn_fwd_rows(const double* q, const double* k, const double* v,
                         int64_t N, int64_t d, int causal, double scale,
                         const int64_t* rows, int64_t nrows, double* o_rows,
                         double* lse_rows, double* p_rows) {
  if (!q || !k || !v || !rows || !o_rows || !lse_rows) return -1;
  if (N < 1 || d < 1 || nrows < 0) return -2;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= N) return -2;
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
    double* p = (double*)malloc(sizeof(double) * (size_t)N);
    if (!s || !p) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows[r];
        double m, l;
        score_row(q, k, N, d, causal, scale, i, s);
        oracle_softmax_row(s, N, p, &m, &l);
        lse_rows[r] = m + log(l);
        if (p_rows) memcpy(p_rows + r * N, p, sizeof(double) * (size_t)N);
        double* orow = o_rows + r * d;
        for (int64_t c = 0; c < d; ++c) orow[c] = 0.0;
        for (int64_t j = 0; j < N; ++j) {
          const double* vj = v + j * d;
          for (int64_t c = 0; c < d; ++c) orow[c] += p[j] * vj[c];
        }
      }
    }
    free(s);
    free(p);
  }
  return failed ? -3 : 0;
}

/* dQ rows of the backward for selected query rows of one head (CS336 L5
 * notes section 8.4): row i of dQ depends only on row i of P and dP, so it
 * is computed alone, in O(N d):
 *   p = softmax of the (masked) score row, o = p V, D = dO_i . o,
 *   dp_j = dO_i . v_j, ds_j = p_j (dp_j - D), dQ_i = scale sum_j ds_j k_j.
 * rows: nrows indices in [0, N); dq_rows: [nrows][d]. */
int oracle_attn_bwd_dq_rows(const double* q, const double* k, const double* v,
                            const double* dout, int64_t N, int64_t d, int causal,
                            double scale, const int64_t* rows, int64_t nrows,
                            double* dq_rows) {
  if (!q || !k || !v || !dout || !rows || !dq_rows) return -1;
  if (N < 1 || d < 1 || nrows < 0) return -2;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= N) return -2;
  int failed = 0;
#pragma omp parallel
  {
    double* sr = (double*)malloc(sizeof(double) * (size_t)N);
    double* pr = (double*)malloc(sizeof(double) * (size_t)N);
    double* orow = (double*)malloc(sizeof(double) * (size_t)d);
    if (!sr || !pr || !orow) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < nrows; ++r) {
        const int64_t row_i = rows[r];
        const double* doi = dout + row_i * d;
        double mr, lr;
        score_row(q, k, N, d, causal, scale, row_i, sr);
        oracle_softmax_row(sr, N, pr, &mr, &lr);
        for (int64_t c = 0; c < d; ++c) {
          double acc = 0.0;
          for (int64_t t = 0; t < N; ++t) acc += pr[t] * v[t * d + c];
          orow[c] = acc;
        }
        double Di = 0.0;
        for (int64_t c = 0; c < d; ++c) Di += doi[c] * orow[c];
        double* dqi = dq_rows + r * d;
        for (int64_t c = 0; c < d; ++c) dqi[c] = 0.0;
        for (int64_t t = 0; t < N; ++t) {
          if (pr[t] == 0.0) continue;  /* masked keys (and underflow) add nothing */
          double dpt = 0.0;
          for (int64_t c = 0; c < d; ++c) dpt += doi[c] * v[t * d + c];
          const double dst = pr[t] * (dpt - Di);
          for (int64_t c = 0; c < d; ++c) dqi[c] += dst * k[t * d + c];
        }
        for (int64_t c = 0; c < d; ++c) dqi[c] *= scale;
      }
    }
    free(sr);
    free(pr);
    free(orow);
  }
  return failed ? -3 : 0;
}

/* Forward for Nq queries against Nk keys of one head (decode- and
 * prefill-shaped attention over a key/value cache: PDC notes Lecture 4,
 * section 4.9; CS336 L5 notes section 5.3).  The queries are the last Nq
 * positions of the sequence, so query i sits at position i + Nk - Nq; under
 * the causal mask it sees keys 0 .. i + Nk - Nq.  Nq = Nk is the square case
 * of oracle_attn_fwd_head.  q: [Nq][d], k, v: [Nk][d]; o: [Nq][d], lse: [Nq].
 * With causal, Nk >= Nq is required (every query then sees key 0).  Same
 * definition as above: score row, safe softmax, P row times V.  p_out, when
 * not NULL, [Nq][Nk] receives P. */
int oracle_attn_fwd_rect(const double* q, const double* k, const double* v,
                         int64_t Nq, int64_t Nk, int64_t d, int causal, double scale,
                         double* o, double* lse, double* p_out) {
  if (!q || !k || !v || !o || !lse) return -1;
  if (Nq < 1 || Nk < 1 || d < 1 || (causal && Nk < Nq)) return -2;
  const int64_t offset = Nk - Nq;
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Nk);
    double* p = (double*)malloc(sizeof(double) * (size_t)Nk);
    if (!s || !p) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t i = 0; i < Nq; ++i) {
        const double* qi = q + i * d;
        for (int64_t j = 0; j < Nk; ++j) {
          if (causal && j > i + offset) {
            s[j] = -INFINITY;
            continue;
          }
          const double* kj = k + j * d;
          double dot = 0.0;
          for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];
          s[j] = dot * scale;
        }
        double m, l;
        oracle_softmax_row(s, Nk, p, &m, &l);
        lse[i] = log(l) + m;
        if (p_out) memcpy(p_out + i * Nk, p, sizeof(double) * (size_t)Nk);
        double* oi = o + i * d;
        for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
        for (int64_t j = 0; j < Nk; ++j) {
          const double* vj = v + j * d;
          for (int64_t c = 0; c < d; ++c) oi[c] += p[j] * vj[c];
        }
      }
    }
    free(s);
    free(p);
  }
  return failed ? -3 : 0;
}

/* Backward for one head (CS336 L5 notes section 8.4): the exact gradient of
 * sum(dO * O).  Inputs q, k, v, dout: [N][d].  Outputs dq, dk, dv: [N][d].
 * o_out [N][d], lse_out [N] and D_out [N], when not NULL, receive the
 * oracle's own O, lse and D = rowsum(dO * O). */
int oracle_attn_bwd_head(const double* q, const double* k, const double* v,
                         const double* dout, int64_t N, int64_t d, int causal,
                         double scale, double* dq, double* dk, double* dv,
                         double* o_out, double* lse_out, double* D_out) {
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
  if (N < 1 || d < 1) return -2;
  const size_t nn = (size_t)N * (size_t)N;
  double* P = (double*)malloc(sizeof(double) * nn);
  double* dS = (double*)malloc(sizeof(double) * nn);
  double* O = (double*)malloc(sizeof(double) * (size_t)N * (size_t)d);
  double* L = (double*)malloc(sizeof(double) * (size_t)N);
  double* D = (double*)malloc(sizeof(double) * (size_t)N);
  if (!P || !dS || !O || !L || !D) {
    free(P); free(dS); free(O); free(L); free(D);
    return -3;
  }
  int rc = oracle_attn_fwd_head(q, k, v, N, d, causal, scale, O, L, P);
  if (rc != 0) {
    free(P); free(dS); free(O); free(L); free(D);
    return rc;
  }
  /* D_i = sum_k dO_ik O_ik */
  for (int64_t i = 0; i < N; ++i) {
    double acc = 0.0;
    for (int64_t c = 0; c < d; ++c) acc += dout[i * d + c] * O[i * d + c];
    D[i] = acc;
  }
  /* dP = dO V^T, then dS = P * (dP - D) */
#pragma omp parallel for schedule(dynamic, 8)
  for (int64_t i = 0; i < N; ++i) {
    for (int64_t j = 0; j < N; ++j) {
      double dp = 0.0;
      for (int64_t c = 0; c < d; ++c) dp += dout[i * d + c] * v[j * d + c];
      dS[i * N + j] = P[i * N + j] * (dp - D[i]);
    }
  }
  /* dQ = scale * dS K */
#pragma omp parallel for schedule(dynamic, 8)
  for (int64_t i = 0; i < N; ++i) {
    for (int64_t c = 0; c < d; ++c) dq[i * d + c] = 0.0;
    for (int64_t j = 0; j < N; ++j) {
      const double g = dS[i * N + j];
      for (int64_t c = 0; c < d; ++c) dq[i * d + c] += g * k[j * d + c];
    }
    for (int64_t c = 0; c < d; ++c) dq[i * d + c] *= scale;
  }
  /* dK = scale * dS^T Q and dV = P^T dO, one key row j at a time */
#pragma omp parallel for schedule(dynamic, 8)
  for (int64_t j = 0; j < N; ++j) {
    for (int64_t c = 0; c < d; ++c) {
      dk[j * d + c] = 0.0;
      dv[j * d + c] = 0.0;
    }
    for (int64_t i = 0; i < N; ++i) {
      const double g = dS[i * N + j];
      const double pij = P[i * N + j];
      for (int64_t c = 0; c < d; ++c) {
        dk[j * d + c] += g * q[i * d + c];
        dv[j * d + c] += pij * dout[i * d + c];
      }
    }
    for (int64_t c = 0; c < d; ++c) dk[j * d + c] *= scale;
  }
  if (o_out) memcpy(o_out, O, sizeof(double) * (size_t)N * (size_t)d);
  if (lse_out) memcpy(lse_out, L, sizeof(double) * (size_t)N);
  if (D_out) memcpy(D_out, D, sizeof(double) * (size_t)N);
  free(P); free(dS); free(O); free(L); free(D);
  return 0;
}

/* Backward of oracle_attn_fwd_rect: the exact gradient of sum(dO * O) for
 * Nq queries at the end of an Nk-key sequence (chunked prefill), in the terms
 * of CS336 L5 notes section 8.4 with the shifted causal mask of the forward
 * (query i sees keys 0 .. i + Nk - Nq).  q, dout: [Nq][d]; k, v: [Nk][d];
 * dq: [Nq][d]; dk, dv: [Nk][d].  o_out [Nq][d], lse_out [Nq] and D_out [Nq],
 * when not NULL, receive the oracle's own O, lse and D.  Written out
 * directly: P [Nq][Nk] row by row (scores, mask, safe softmax), then D,
 * dPr = dO V^T, dSr = P * (dPr - D), dQ, dK, dV. */
int oracle_attn_bwd_rect(const double* q, const double* k, const double* v,
                         const double* dout, int64_t Nq, int64_t Nk, int64_t d, int causal,
                         double scale, double* dq, double* dk, double* dv, double* o_out,
                         double* lse_out, double* D_out) {
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
  if (Nq < 1 || Nk < 1 || d < 1 || (causal && Nk < Nq)) return -2;
  const int64_t shift = Nk - Nq;
  const size_t nqk = (size_t)Nq * (size_t)Nk;
  double* Pr = (double*)malloc(sizeof(double) * nqk);
  double* dSr = (double*)malloc(sizeof(double) * nqk);
  double* Or = (double*)malloc(sizeof(double) * (size_t)Nq * (size_t)d);
  double* Lr = (double*)malloc(sizeof(double) * (size_t)Nq);
  double* Dr = (double*)malloc(sizeof(double) * (size_t)Nq);
  double* srow = (double*)malloc(sizeof(double) * (size_t)Nk);
  if (!Pr || !dSr || !Or || !Lr || !Dr || !srow) {
    free(Pr); free(dSr); free(Or); free(Lr); free(Dr); free(srow);
    return -3;
  }
  /* P = softmax(scale q k^T + mask) row by row, O = P V, lse = m + ln l */
  for (int64_t r = 0; r < Nq; ++r) {
    for (int64_t t = 0; t < Nk; ++t) {
      if (causal && t > r + shift) {
        srow[t] = -INFINITY;
        continue;
      }
      double qk = 0.0;
      for (int64_t c = 0; c < d; ++c) qk += q[r * d + c] * k[t * d + c];
      srow[t] = scale * qk;
    }
    double mr, lr;
    oracle_softmax_row(srow, Nk, Pr + r * Nk, &mr, &lr);
    Lr[r] = mr + log(lr);
    for (int64_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t t = 0; t < Nk; ++t) acc += Pr[r * Nk + t] * v[t * d + c];
      Or[r * d + c] = acc;
    }
    double dd = 0.0;
    for (int64_t c = 0; c < d; ++c) dd += dout[r * d + c] * Or[r * d + c];
    Dr[r] = dd;
  }
  /* dSr = P * (dO V^T - D) */
#pragma omp parallel for schedule(dynamic, 8)
  for (int64_t r = 0; r < Nq; ++r) {
    for (int64_t t = 0; t < Nk; ++t) {
      double dpr = 0.0;
      for (int64_t c = 0; c < d; ++c) dpr += dout[r * d + c] * v[t * d + c];
      dSr[r * Nk + t] = Pr[r * Nk + t] * (dpr - Dr[r]);
    }
  }
  /* dQ = scale * dSr K */
#pragma omp parallel for schedule(dynamic, 8)
  for (int64_t r = 0; r < Nq; ++r) {
    for (int64_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t t = 0; t < Nk; ++t) acc += dSr[r * Nk + t] * k[t * d + c];
      dq[r * d + c] = scale * acc;
    }
  }
  /* dK = scale * dSr^T Q and dV = P^T dO, one key row t at a time */
#pragma omp parallel for schedule(dynamic, 8)
  for (int64_t t = 0; t < Nk; ++t) {
    for (int64_t c = 0; c < d; ++c) {
      double ak = 0.0, av = 0.0;
      for (int64_t r = 0; r < Nq; ++r) {
        ak += dSr[r * Nk + t] * q[r * d + c];
        av += Pr[r * Nk + t] * dout[r * d + c];
      }
      dk[t * d + c] = scale * ak;
      dv[t * d + c] = av;
    }
  }
  if (o_out) memcpy(o_out, Or, sizeof(double) * (size_t)Nq * (size_t)d);
  if (lse_out) memcpy(lse_out, Lr, sizeof(double) * (size_t)Nq);
  if (D_out) memcpy(D_out, Dr, sizeof(double) * (size_t)Nq);
  free(Pr); free(dSr); free(Or); free(Lr); free(Dr); free(srow);
  return 0;
}

/* ---------------------------------------------------------------- MXFP8
 * Q and K given in the MXFP8 format the CS336 L5 notes (section 6.2) name:
 * E4M3 values plus one E8M0 scale for every 32 elements of a row.  The
 * formats (OCP FP8 and OCP microscaling):
 *   E4M3: sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent
 *         field 0 holds the subnormals m * 2^-9; S.1111.111 is NaN; there
 *         are no infinities (largest finite value 448).
 *   E8M0: an unsigned exponent, value 2^(e - 127); 0xFF is NaN.
 * The attention of MXFP8 inputs is the attention of their decoded values,
 * so the oracle only decodes (exactly, in double precision). */
static double e4m3_value(uint8_t b) {
  const int sign = b >> 7, e = (b >> 3) & 15, m = b & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
  return sign ? -mag : mag;
}

static double e8m0_value(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

/* rows x d E4M3 codes (row-major) with rows x (d / 32) E8M0 scales: element
 * (r, c) is e4m3(codes[r][c]) * e8m0(scales[r][c / 32]).  d must be a
 * multiple of 32. */
int oracle_mx_decode(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t d,
                     double* out) {
  if (!codes || !scales || !out) return -1;
  if (rows < 0 || d < 32 || d % 32 != 0) return -2;
  const int64_t nb = d / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < d; ++c)
      out[r * d + c] = e4m3_value(codes[r * d + c]) * e8m0_value(scales[r * nb + c / 32]);
  return 0;
}

