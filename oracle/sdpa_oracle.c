/*
 * sdpa_oracle.c - fp64 CPU oracle for scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark; never by the product library, with which
 * it shares no code.  Plain C, fp64 throughout, OpenMP over rows.
 *
 * Every formula below is the plain definition of attention
 * softmax(scale * Q K^T + mask) V (the AOTriton README, "Kernel Support",
 * names FlashAttention, which computes exactly this), with the mask of the
 * generalized sliding window (AOTriton 0.10b release notes, "Major Changes")
 * and the principal-diagonal choice (AOTriton 0.15b release notes,
 * "Bottom-Right Aligned Sliding Windows").  Where the pages are silent the
 * plainest reading is taken; each reading is named where it is used.
 */
#include "sdpa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- decoding */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int expo = (bits >> 10) & 0x1f;
  int frac = bits & 0x3ff;
  double mag;
  if (expo == 0)
    mag = ldexp((double)frac, -24);                 /* zero or subnormal */
  else if (expo == 31)
    mag = frac ? NAN : INFINITY;
  else
    mag = ldexp((double)(1024 + frac), expo - 25);  /* 1.frac * 2^(e-15) */
  return sign ? -mag : mag;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double oracle_decode_bf16(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int expo = (bits >> 7) & 0xff;
  int frac = bits & 0x7f;
  double mag;
  if (expo == 0)
    mag = ldexp((double)frac, -133);                /* zero or subnormal */
  else if (expo == 255)
    mag = frac ? NAN : INFINITY;
  else
    mag = ldexp((double)(128 + frac), expo - 134);  /* 1.frac * 2^(e-127) */
  return sign ? -mag : mag;
}

static double decode_at(int dtype, const void *base, int64_t idx) {
  if (dtype == ORACLE_F32) {
    float f;
    memcpy(&f, (const char *)base + idx * 4, 4);
    return (double)f;
  }
  uint16_t b;
  memcpy(&b, (const char *)base + idx * 2, 2);
  return dtype == ORACLE_F16 ? oracle_decode_f16(b) : oracle_decode_bf16(b);
}

/* -------------------------------------------------------------- visibility */

/*
 * Key j is visible to query i iff i - L <= j <= i + R (0-based, local to the
 * sequence).  A window whose sides are both finite is "numeric"; under the
 * bottom-right diagonal a numeric window becomes L = wl - d, R = wr + d with
 * d = sk - sq of that sequence.  A window with an unbounded side (a causal
 * sentinel) is never shifted.  Reading: "sentinel" is a property of the whole
 * window, so (INF, 0) stays top-left under BOTTOM_RIGHT.
 */
int oracle_visible(int64_t i, int64_t j, int64_t sq, int64_t sk,
                   int window_left, int window_right, int diag) {
  int left_inf = window_left == ORACLE_WINDOW_INF;
  int right_inf = window_right == ORACLE_WINDOW_INF;
  int64_t L = window_left, R = window_right;
  if (diag == ORACLE_BOTTOM_RIGHT && !left_inf && !right_inf) {
    int64_t d = sk - sq;
    L = L - d;
    R = R + d;
  }
  if (i < 0 || i >= sq || j < 0 || j >= sk) return 0;
  if (!left_inf && j < i - L) return 0;
  if (!right_inf && j > i + R) return 0;
  return 1;
}

/* ------------------------------------------------------------- addressing */

typedef struct {
  int64_t q0, sq;   /* first packed row and length of the query side */
  int64_t k0, sk;   /* same for the key side */
} seq_span;

static int check_problem(const oracle_problem *p) {
  if (!p || p->batch < 0 || p->heads <= 0 || p->head_dim <= 0) return -1;
  if (p->dtype < ORACLE_F32 || p->dtype > ORACLE_BF16) return -1;
  if (p->diag != ORACLE_TOP_LEFT && p->diag != ORACLE_BOTTOM_RIGHT) return -1;
  if (p->layout == ORACLE_DENSE) {
    if (p->seqlen_q < 0 || p->seqlen_k < 0) return -1;
    return 0;
  }
  if (p->layout != ORACLE_PACKED) return -1;
  if (!p->cu_seqlens_q || !p->cu_seqlens_k) return -1;
  if (p->cu_seqlens_q[0] != 0 || p->cu_seqlens_k[0] != 0) return -1;
  for (int b = 0; b < p->batch; ++b)
    if (p->cu_seqlens_q[b + 1] < p->cu_seqlens_q[b] ||
        p->cu_seqlens_k[b + 1] < p->cu_seqlens_k[b])
      return -1;
  return 0;
}

static seq_span span_of(const oracle_problem *p, int b) {
  seq_span s;
  if (p->layout == ORACLE_DENSE) {
    s.q0 = 0; s.sq = p->seqlen_q;
    s.k0 = 0; s.sk = p->seqlen_k;
  } else {
    s.q0 = p->cu_seqlens_q[b]; s.sq = p->cu_seqlens_q[b + 1] - s.q0;
    s.k0 = p->cu_seqlens_k[b]; s.sk = p->cu_seqlens_k[b + 1] - s.k0;
  }
  return s;
}

/* Flat element index of (sequence b, head h, local row r, dim d). */
static int64_t elem_index(const oracle_problem *p, int b, int h, int64_t row0,
                          int64_t r, int64_t seqlen, int d) {
  int64_t H = p->heads, D = p->head_dim;
  if (p->layout == ORACLE_DENSE)
    return (((int64_t)b * H + h) * seqlen + r) * D + d;
  return ((row0 + r) * H + h) * D + d;
}

/* Row-statistics index: dense [B][H][Sq]; packed [H][Tq]. */
static int64_t lse_index(const oracle_problem *p, int b, int h, int64_t i) {
  if (p->layout == ORACLE_DENSE)
    return ((int64_t)b * p->heads + h) * p->seqlen_q + i;
  return (int64_t)h * p->cu_seqlens_q[p->batch] + p->cu_seqlens_q[b] + i;
}

/* Decode rows [0, n) of one (b, h) slice into a dense fp64 [n][D] array. */
static void load_slice(const oracle_problem *p, const void *src, int b, int h,
                       int64_t row0, int64_t n, double *dst) {
  int D = p->head_dim;
  for (int64_t r = 0; r < n; ++r)
    for (int d = 0; d < D; ++d)
      dst[r * D + d] =
          decode_at(p->dtype, src, elem_index(p, b, h, row0, r, n, d));
}

static double dot(const double *a, const double *b, int n) {
  double s = 0.0;
  for (int t = 0; t < n; ++t) s += a[t] * b[t];
  return s;
}

/* ------------------------------------------------------------ one row, fwd */

/*
 * Row i of the forward pass, two passes over the visible keys:
 *   m = max_j S_ij, l = sum_j exp(S_ij - m), LSE = m + ln l (natural log),
 *   O_i = sum_j exp(S_ij - LSE) v_j.
 * A row with no visible key gets O_i = 0 and LSE_i = +inf, the early-exit
 * convention of the AOTriton 0.15b and 0.14b release notes ("Kernel Bug
 * Fixes": the early-exit zero store and the +inf LSE of fully masked rows).
 * s must hold sk doubles.
 */
static void row_forward(const oracle_problem *p, const double *Q,
                        const double *K, const double *V, int64_t i,
                        int64_t sq, int64_t sk, double *s, double *o_row,
                        double *lse_out) {
  int D = p->head_dim;
  int any = 0;
  double m = -INFINITY;
  for (int64_t j = 0; j < sk; ++j) {
    if (!oracle_visible(i, j, sq, sk, p->window_left, p->window_right,
                        p->diag))
      continue;
    s[j] = p->scale * dot(Q + i * D, K + j * D, D);
    if (s[j] > m) m = s[j];
    any = 1;
  }
  for (int d = 0; d < D; ++d) o_row[d] = 0.0;
  if (!any) {
    *lse_out = INFINITY;
    return;
  }
  double l = 0.0;
  for (int64_t j = 0; j < sk; ++j)
    if (oracle_visible(i, j, sq, sk, p->window_left, p->window_right,
                       p->diag))
      l += exp(s[j] - m);
  double lse = m + log(l);
  for (int64_t j = 0; j < sk; ++j) {
    if (!oracle_visible(i, j, sq, sk, p->window_left, p->window_right,
                        p->diag))
      continue;
    double pij = exp(s[j] - lse);
    for (int d = 0; d < D; ++d) o_row[d] += pij * V[j * D + d];
  }
  *lse_out = lse;
}

/* P_ij recomputed from the row's LSE; 0 when j is not visible to i or the
 * row is empty (LSE = +inf). */
static double prob(const oracle_problem *p, const double *Q, const double *K,
                   int64_t i, int64_t j, int64_t sq, int64_t sk, double lse) {
  if (!oracle_visible(i, j, sq, sk, p->window_left, p->window_right, p->diag))
    return 0.0;
  if (isinf(lse)) return 0.0;
  int D = p->head_dim;
  return exp(p->scale * dot(Q + i * D, K + j * D, D) - lse);
}

/* ------------------------------------------------------------ slice helper */

typedef struct {
  seq_span sp;
  double *Q, *K, *V, *dO; /* decoded slice */
} slice;

static int slice_load(const oracle_problem *p, const void *q, const void *k,
                      const void *v, const void *dout, int b, int h,
                      slice *sl) {
  int D = p->head_dim;
  sl->sp = span_of(p, b);
  int64_t sq = sl->sp.sq, sk = sl->sp.sk;
  sl->Q = (double *)malloc(sizeof(double) * (size_t)(sq * D + 1));
  sl->K = (double *)malloc(sizeof(double) * (size_t)(sk * D + 1));
  sl->V = (double *)malloc(sizeof(double) * (size_t)(sk * D + 1));
  sl->dO = dout ? (double *)malloc(sizeof(double) * (size_t)(sq * D + 1))
                : NULL;
  if (!sl->Q || !sl->K || !sl->V || (dout && !sl->dO)) return -1;
  load_slice(p, q, b, h, sl->sp.q0, sq, sl->Q);
  load_slice(p, k, b, h, sl->sp.k0, sk, sl->K);
  load_slice(p, v, b, h, sl->sp.k0, sk, sl->V);
  if (dout) load_slice(p, dout, b, h, sl->sp.q0, sq, sl->dO);
  return 0;
}

static void slice_free(slice *sl) {
  free(sl->Q); free(sl->K); free(sl->V); free(sl->dO);
}

/* Forward over all rows of a slice into dense [sq][D] / [sq] fp64 arrays. */
static int slice_forward(const oracle_problem *p, const slice *sl,
                         double *O, double *lse) {
  int64_t sq = sl->sp.sq, sk = sl->sp.sk;
  int fail = 0;
#pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)(sk + 1));
    if (!s) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 8)
    for (int64_t i = 0; i < sq; ++i)
      if (s)
        row_forward(p, sl->Q, sl->K, sl->V, i, sq, sk, s,
                    O + i * p->head_dim, lse + i);
    free(s);
  }
  return fail ? -1 : 0;
}

/* ------------------------------------------------------------ public: fwd */

int oracle_fwd(const oracle_problem *p, const void *q, const void *k,
               const void *v, double *o, double *lse) {
  if (check_problem(p)) return -1;
  int D = p->head_dim;
  for (int b = 0; b < p->batch; ++b)
    for (int h = 0; h < p->heads; ++h) {
      slice sl;
      if (slice_load(p, q, k, v, NULL, b, h, &sl)) { slice_free(&sl); return -1; }
      int64_t sq = sl.sp.sq;
      double *O = (double *)malloc(sizeof(double) * (size_t)(sq * D + 1));
      double *L = (double *)malloc(sizeof(double) * (size_t)(sq + 1));
      int rc = (O && L) ? slice_forward(p, &sl, O, L) : -1;
      if (!rc)
        for (int64_t i = 0; i < sq; ++i) {
          for (int d = 0; d < D; ++d)
            o[elem_index(p, b, h, sl.sp.q0, i, sq, d)] = O[i * D + d];
          lse[lse_index(p, b, h, i)] = L[i];
        }
      free(O); free(L); slice_free(&sl);
      if (rc) return -1;
    }
  return 0;
}

int oracle_fwd_rows(const oracle_problem *p, const void *q, const void *k,
                    const void *v, int b, int h, int nrows,
                    const int32_t *rows, double *o_rows, double *lse_rows) {
  if (check_problem(p) || b < 0 || b >= p->batch || h < 0 || h >= p->heads)
    return -1;
  slice sl;
  if (slice_load(p, q, k, v, NULL, b, h, &sl)) { slice_free(&sl); return -1; }
  int64_t sq = sl.sp.sq, sk = sl.sp.sk;
  int bad = 0;
  for (int r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= sq) bad = 1;
  if (!bad) {
#pragma omp parallel
    {
      double *s = (double *)malloc(sizeof(double) * (size_t)(sk + 1));
#pragma omp for schedule(dynamic, 1)
      for (int r = 0; r < nrows; ++r)
        if (s)
          row_forward(p, sl.Q, sl.K, sl.V, rows[r], sq, sk, s,
                      o_rows + (int64_t)r * p->head_dim, lse_rows + r);
      if (!s) {
#pragma omp atomic write
        bad = 1;
      }
      free(s);
    }
  }
  slice_free(&sl);
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------ backward */

/*
 * Explicit gradients of the scalar <dO, O>:
 *   dP_ij = <dO_i, v_j>,  Delta_i = <dO_i, O_i>  (the oracle's own fp64 O),
 *   dS_ij = P_ij (dP_ij - Delta_i),
 *   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
 *   dV_j = sum_i P_ij dO_i.
 * Delta is the row-sum term of the backward preprocess named in the AOTriton
 * 0.14b release notes ("bwd_preprocess").  Empty rows have P = 0 and so
 * contribute nothing; keys seen by no row get dK = dV = 0.
 */
static void row_dq(const oracle_problem *p, const slice *sl, int64_t i,
                   double lse_i, double delta_i, double *dq_row) {
  int D = p->head_dim;
  int64_t sq = sl->sp.sq, sk = sl->sp.sk;
  for (int d = 0; d < D; ++d) dq_row[d] = 0.0;
  for (int64_t j = 0; j < sk; ++j) {
    double pij = prob(p, sl->Q, sl->K, i, j, sq, sk, lse_i);
    if (pij == 0.0) continue;
    double dpij = dot(sl->dO + i * D, sl->V + j * D, D);
    double ds = pij * (dpij - delta_i);
    for (int d = 0; d < D; ++d) dq_row[d] += p->scale * ds * sl->K[j * D + d];
  }
}

static void col_dkdv(const oracle_problem *p, const slice *sl, int64_t j,
                     const double *lse, const double *delta, double *dk_row,
                     double *dv_row) {
  int D = p->head_dim;
  int64_t sq = sl->sp.sq, sk = sl->sp.sk;
  for (int d = 0; d < D; ++d) dk_row[d] = dv_row[d] = 0.0;
  for (int64_t i = 0; i < sq; ++i) {
    double pij = prob(p, sl->Q, sl->K, i, j, sq, sk, lse[i]);
    if (pij == 0.0) continue;
    double dpij = dot(sl->dO + i * D, sl->V + j * D, D);
    double ds = pij * (dpij - delta[i]);
    for (int d = 0; d < D; ++d) {
      dk_row[d] += p->scale * ds * sl->Q[i * D + d];
      dv_row[d] += pij * sl->dO[i * D + d];
    }
  }
}

/* Row statistics (O, LSE, Delta) of a whole slice. */
static int slice_stats(const oracle_problem *p, const slice *sl, double *O,
                       double *lse, double *delta) {
  int D = p->head_dim;
  if (slice_forward(p, sl, O, lse)) return -1;
  for (int64_t i = 0; i < sl->sp.sq; ++i)
    delta[i] = dot(sl->dO + i * D, O + i * D, D);
  return 0;
}

int oracle_bwd(const oracle_problem *p, const void *q, const void *k,
               const void *v, const void *dout, double *o, double *lse,
               double *dq, double *dk, double *dv) {
  if (check_problem(p)) return -1;
  int D = p->head_dim;
  for (int b = 0; b < p->batch; ++b)
    for (int h = 0; h < p->heads; ++h) {
      slice sl;
      if (slice_load(p, q, k, v, dout, b, h, &sl)) { slice_free(&sl); return -1; }
      int64_t sq = sl.sp.sq, sk = sl.sp.sk;
      double *O = (double *)malloc(sizeof(double) * (size_t)(sq * D + 1));
      double *L = (double *)malloc(sizeof(double) * (size_t)(sq + 1));
      double *De = (double *)malloc(sizeof(double) * (size_t)(sq + 1));
      double *dQ = (double *)malloc(sizeof(double) * (size_t)(sq * D + 1));
      double *dK = (double *)malloc(sizeof(double) * (size_t)(sk * D + 1));
      double *dV = (double *)malloc(sizeof(double) * (size_t)(sk * D + 1));
      int rc = (O && L && De && dQ && dK && dV) ? slice_stats(p, &sl, O, L, De)
                                                 : -1;
      if (!rc) {
#pragma omp parallel for schedule(dynamic, 8)
        for (int64_t i = 0; i < sq; ++i) row_dq(p, &sl, i, L[i], De[i], dQ + i * D);
#pragma omp parallel for schedule(dynamic, 8)
        for (int64_t j = 0; j < sk; ++j)
          col_dkdv(p, &sl, j, L, De, dK + j * D, dV + j * D);
        for (int64_t i = 0; i < sq; ++i) {
          for (int d = 0; d < D; ++d) {
            int64_t e = elem_index(p, b, h, sl.sp.q0, i, sq, d);
            dq[e] = dQ[i * D + d];
            if (o) o[e] = O[i * D + d];
          }
          if (lse) lse[lse_index(p, b, h, i)] = L[i];
        }
        for (int64_t j = 0; j < sk; ++j)
          for (int d = 0; d < D; ++d) {
            int64_t e = elem_index(p, b, h, sl.sp.k0, j, sk, d);
            dk[e] = dK[j * D + d];
            dv[e] = dV[j * D + d];
          }
      }
      free(O); free(L); free(De); free(dQ); free(dK); free(dV);
      slice_free(&sl);
      if (rc) return -1;
    }
  return 0;
}

int oracle_bwd_dq_rows(const oracle_problem *p, const void *q, const void *k,
                       const void *v, const void *dout, int b, int h,
                       int nrows, const int32_t *rows, double *dq_rows) {
  if (check_problem(p) || b < 0 || b >= p->batch || h < 0 || h >= p->heads)
    return -1;
  slice sl;
  if (slice_load(p, q, k, v, dout, b, h, &sl)) { slice_free(&sl); return -1; }
  int D = p->head_dim;
  int64_t sq = sl.sp.sq, sk = sl.sp.sk;
  int bad = 0;
  for (int r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= sq) bad = 1;
  if (!bad) {
#pragma omp parallel
    {
      double *s = (double *)malloc(sizeof(double) * (size_t)(sk + 1));
      double *orow = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
      for (int r = 0; r < nrows; ++r) {
        if (!s || !orow) continue;
        double lse_i;
        int64_t i = rows[r];
        row_forward(p, sl.Q, sl.K, sl.V, i, sq, sk, s, orow, &lse_i);
        double delta_i = dot(sl.dO + i * D, orow, D);
        row_dq(p, &sl, i, lse_i, delta_i, dq_rows + (int64_t)r * D);
      }
      if (!s || !orow) {
#pragma omp atomic write
        bad = 1;
      }
      free(s); free(orow);
    }
  }
  slice_free(&sl);
  return bad ? -1 : 0;
}

int oracle_bwd_dkdv_cols(const oracle_problem *p, const void *q,
                         const void *k, const void *v, const void *dout,
                         int b, int h, int ncols, const int32_t *cols,
                         double *dk_cols, double *dv_cols) {
  if (check_problem(p) || b < 0 || b >= p->batch || h < 0 || h >= p->heads)
    return -1;
  slice sl;
  if (slice_load(p, q, k, v, dout, b, h, &sl)) { slice_free(&sl); return -1; }
  int D = p->head_dim;
  int64_t sq = sl.sp.sq, sk = sl.sp.sk;
  int bad = 0;
  for (int c = 0; c < ncols; ++c)
    if (cols[c] < 0 || cols[c] >= sk) bad = 1;
  double *O = (double *)malloc(sizeof(double) * (size_t)(sq * D + 1));
  double *L = (double *)malloc(sizeof(double) * (size_t)(sq + 1));
  double *De = (double *)malloc(sizeof(double) * (size_t)(sq + 1));
  if (!O || !L || !De) bad = 1;
  if (!bad && slice_stats(p, &sl, O, L, De)) bad = 1;
  if (!bad) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int c = 0; c < ncols; ++c)
      col_dkdv(p, &sl, cols[c], L, De, dk_cols + (int64_t)c * D,
               dv_cols + (int64_t)c * D);
  }
  free(O); free(L); free(De);
  slice_free(&sl);
  return bad ? -1 : 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
