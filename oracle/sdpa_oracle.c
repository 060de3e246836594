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

/* ------------------------------------------------------------- Philox */

/*
 * Philox4x32-10 as published (Salmon et al., SC 2011): ten rounds of
 *   (hi0, lo0) = M0 * c0, (hi1, lo1) = M1 * c2   (32 x 32 -> 64-bit products)
 *   c = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
 * with the key bumped by the Weyl constants (W0, W1) before every round but
 * the first.
 */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t p0 = (uint64_t)M0 * c[0], p1 = (uint64_t)M1 * c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
  for (int t = 0; t < 4; ++t) out[t] = c[t];
}

/* Largest sequence length of one side (the counters' and bias rows'
 * stride), from the fields or, when they are 0, from the problem. */
static int64_t max_len(const oracle_problem *p, int q) {
  int64_t m = q ? p->max_seqlen_q : p->max_seqlen_k;
  if (m > 0) return m;
  if (p->layout == ORACLE_DENSE) return q ? p->seqlen_q : p->seqlen_k;
  const int32_t *cu = q ? p->cu_seqlens_q : p->cu_seqlens_k;
  m = 0;
  for (int b = 0; b < p->batch; ++b)
    if (cu[b + 1] - cu[b] > m) m = cu[b + 1] - cu[b];
  return m;
}

/* Threshold of the keep decision: floor(p * 2^32), in [0, 2^32). */
static uint32_t dropout_threshold(double pdrop) {
  double t = floor(pdrop * 4294967296.0);
  if (t < 0.0) t = 0.0;
  if (t > 4294967295.0) t = 4294967295.0;
  return (uint32_t)t;
}

int oracle_dropout_keep(const oracle_problem *p, int b, int h, int64_t i, int64_t j) {
  if (!(p->dropout_p > 0.0)) return 1;
  const int64_t sqm = max_len(p, 1), skm = max_len(p, 0);
  const uint64_t groups = (uint64_t)((skm + 3) / 4);
  const uint64_t row = ((uint64_t)b * (uint64_t)p->heads + (uint64_t)h) * (uint64_t)sqm + (uint64_t)i;
  const uint64_t n = p->philox_offset + row * groups + (uint64_t)(j / 4);
  const uint32_t ctr[4] = {(uint32_t)n, (uint32_t)(n >> 32), 0u, 0u};
  const uint32_t key[2] = {(uint32_t)p->philox_seed, (uint32_t)(p->philox_seed >> 32)};
  uint32_t out[4];
  oracle_philox4x32_10(ctr, key, out);
  return out[j % 4] >= dropout_threshold(p->dropout_p);
}

void oracle_dropout_mask(const oracle_problem *p, int b, int h, int64_t nq, int64_t nk, uint8_t *keep) {
  for (int64_t i = 0; i < nq; ++i)
    for (int64_t j = 0; j < nk; ++j) keep[i * nk + j] = (uint8_t)oracle_dropout_keep(p, b, h, i, j);
}

/* Multiplier of P_ij after dropout: keep / (1 - p). */
static double dropout_scale(const oracle_problem *p, int b, int h, int64_t i, int64_t j) {
  if (!(p->dropout_p > 0.0)) return 1.0;
  return oracle_dropout_keep(p, b, h, i, j) ? 1.0 / (1.0 - p->dropout_p) : 0.0;
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
  if (!p || p->batch < 0 || p->heads <= 0 || p->head_dim <= 0 || p->head_dim_v < 0) return -1;
  if (p->dtype < ORACLE_F32 || p->dtype > ORACLE_BF16) return -1;
  if (p->diag != ORACLE_TOP_LEFT && p->diag != ORACLE_BOTTOM_RIGHT) return -1;
  if (!(p->dropout_p >= 0.0 && p->dropout_p < 1.0)) return -1;
  if (p->max_seqlen_q < 0 || p->max_seqlen_k < 0) return -1;
  if (p->layout == ORACLE_DENSE) {
    if (p->seqlen_q < 0 || p->seqlen_k < 0) return -1;
    return 0;
  }
  if (p->layout != ORACLE_PACKED) return -1;
  if (!p->cu_seqlens_q || !p->cu_seqlens_k) return -1;
  if (p->cu_seqlens_q[0] != 0 || p->cu_seqlens_k[0] != 0) return -1;
  for (int b = 0; b < p->batch; ++b) {
    if (p->cu_seqlens_q[b + 1] < p->cu_seqlens_q[b] ||
        p->cu_seqlens_k[b + 1] < p->cu_seqlens_k[b])
      return -1;
    if ((p->max_seqlen_q && p->cu_seqlens_q[b + 1] - p->cu_seqlens_q[b] > p->max_seqlen_q) ||
        (p->max_seqlen_k && p->cu_seqlens_k[b + 1] - p->cu_seqlens_k[b] > p->max_seqlen_k))
      return -1;
  }
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

/* Head dim of V, O, dO and dV: head_dim_v, or head_dim when it is 0. */
static int dim_v(const oracle_problem *p) { return p->head_dim_v > 0 ? p->head_dim_v : p->head_dim; }

/* Flat element index of (sequence b, head h, local row r, dim d) in a
 * tensor whose rows hold D values. */
static int64_t elem_index(const oracle_problem *p, int b, int h, int64_t row0,
                          int64_t r, int64_t seqlen, int64_t D, int d) {
  int64_t H = p->heads;
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

/* Decode rows [0, n) of one (b, h) slice of a tensor with D values per row
 * into a dense fp64 [n][D] array. */
static void load_slice(const oracle_problem *p, const void *src, int b, int h,
                       int64_t row0, int64_t n, int D, double *dst) {
  for (int64_t r = 0; r < n; ++r)
    for (int d = 0; d < D; ++d)
      dst[r * D + d] =
          decode_at(p->dtype, src, elem_index(p, b, h, row0, r, n, D, d));
}

static double dot(const double *a, const double *b, int n) {
  double s = 0.0;
  for (int t = 0; t < n; ++t) s += a[t] * b[t];
  return s;
}

/* ------------------------------------------------------------ logits */

typedef struct {
  seq_span sp;
  int b, h;
  double *Q, *K, *V, *dO; /* decoded slice */
} slice;

/* Logit of the visible pair (i, j) of a slice: scale q_i.k_j, plus the
 * bias entry (decoded from its stored encoding) and the ALiBi term when the
 * problem has them. */
static double logit(const oracle_problem *p, const slice *sl, int64_t i, int64_t j) {
  int D = p->head_dim;
  double x = p->scale * dot(sl->Q + i * D, sl->K + j * D, D);
  if (p->bias)
    x += decode_at(p->dtype, p->bias,
                   sl->b * p->bias_stride[0] + sl->h * p->bias_stride[1] + i * p->bias_stride[2] + j);
  if (p->alibi_slopes) {
    const int64_t shift = sl->sp.sk - sl->sp.sq;
    x -= p->alibi_slopes[sl->h] * fabs((double)(i + shift - j));
  }
  return x;
}

static int visible_in(const oracle_problem *p, const slice *sl, int64_t i, int64_t j) {
  return oracle_visible(i, j, sl->sp.sq, sl->sp.sk, p->window_left, p->window_right, p->diag);
}

/* ------------------------------------------------------------ one row, fwd */

/*
 * Row i of the forward pass, two passes over the visible keys:
 *   m = max_j X_ij, l = sum_j exp(X_ij - m), LSE = m + ln l (natural log),
 *   O_i = sum_j exp(X_ij - LSE) M_ij v_j,
 * X the logits above and M_ij the dropout multiplier (1 without dropout).
 * A row with no visible key gets O_i = 0 and LSE_i = +inf, the early-exit
 * convention of the AOTriton 0.15b and 0.14b release notes ("Kernel Bug
 * Fixes": the early-exit zero store and the +inf LSE of fully masked rows).
 * So does a row whose every visible logit is -inf (a bias of -inf masks
 * like the window).  s must hold sk doubles.
 */
static void row_forward(const oracle_problem *p, const slice *sl, int64_t i, double *s, double *o_row,
                        double *lse_out) {
  int D = dim_v(p);
  int64_t sk = sl->sp.sk;
  double m = -INFINITY;
  for (int64_t j = 0; j < sk; ++j) {
    if (!visible_in(p, sl, i, j)) continue;
    s[j] = logit(p, sl, i, j);
    if (s[j] > m) m = s[j];
  }
  for (int d = 0; d < D; ++d) o_row[d] = 0.0;
  if (m == -INFINITY) {
    *lse_out = INFINITY;
    return;
  }
  double l = 0.0;
  for (int64_t j = 0; j < sk; ++j)
    if (visible_in(p, sl, i, j)) l += exp(s[j] - m);
  double lse = m + log(l);
  for (int64_t j = 0; j < sk; ++j) {
    if (!visible_in(p, sl, i, j)) continue;
    double w = exp(s[j] - lse) * dropout_scale(p, sl->b, sl->h, i, j);
    for (int d = 0; d < D; ++d) o_row[d] += w * sl->V[j * D + d];
  }
  *lse_out = lse;
}

/* P_ij recomputed from the row's LSE (the softmax before dropout); 0 when j
 * is not visible to i or the row is empty (LSE = +inf). */
static double prob(const oracle_problem *p, const slice *sl, int64_t i, int64_t j, double lse) {
  if (!visible_in(p, sl, i, j)) return 0.0;
  if (isinf(lse)) return 0.0;
  return exp(logit(p, sl, i, j) - lse);
}

/* ------------------------------------------------------------ slice helper */

static int slice_load(const oracle_problem *p, const void *q, const void *k,
                      const void *v, const void *dout, int b, int h,
                      slice *sl) {
  int D = p->head_dim, DV = dim_v(p);
  sl->sp = span_of(p, b);
  sl->b = b;
  sl->h = h;
  int64_t sq = sl->sp.sq, sk = sl->sp.sk;
  sl->Q = (double *)malloc(sizeof(double) * (size_t)(sq * D + 1));
  sl->K = (double *)malloc(sizeof(double) * (size_t)(sk * D + 1));
  sl->V = (double *)malloc(sizeof(double) * (size_t)(sk * DV + 1));
  sl->dO = dout ? (double *)malloc(sizeof(double) * (size_t)(sq * DV + 1))
                : NULL;
  if (!sl->Q || !sl->K || !sl->V || (dout && !sl->dO)) return -1;
  load_slice(p, q, b, h, sl->sp.q0, sq, D, sl->Q);
  load_slice(p, k, b, h, sl->sp.k0, sk, D, sl->K);
  load_slice(p, v, b, h, sl->sp.k0, sk, DV, sl->V);
  if (dout) load_slice(p, dout, b, h, sl->sp.q0, sq, DV, sl->dO);
  return 0;
}

static void slice_free(slice *sl) {
  free(sl->Q); free(sl->K); free(sl->V); free(sl->dO);
}

/* Forward over all rows of a slice into dense [sq][DV] / [sq] fp64 arrays. */
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
        row_forward(p, sl, i, s, O + i * dim_v(p), lse + i);
    free(s);
  }
  return fail ? -1 : 0;
}

/* ------------------------------------------------------------ public: fwd */

int oracle_fwd(const oracle_problem *p, const void *q, const void *k,
               const void *v, double *o, double *lse) {
  if (check_problem(p)) return -1;
  int DV = dim_v(p);
  for (int b = 0; b < p->batch; ++b)
    for (int h = 0; h < p->heads; ++h) {
      slice sl;
      if (slice_load(p, q, k, v, NULL, b, h, &sl)) { slice_free(&sl); return -1; }
      int64_t sq = sl.sp.sq;
      double *O = (double *)malloc(sizeof(double) * (size_t)(sq * DV + 1));
      double *L = (double *)malloc(sizeof(double) * (size_t)(sq + 1));
      int rc = (O && L) ? slice_forward(p, &sl, O, L) : -1;
      if (!rc)
        for (int64_t i = 0; i < sq; ++i) {
          for (int d = 0; d < DV; ++d)
            o[elem_index(p, b, h, sl.sp.q0, i, sq, DV, d)] = O[i * DV + d];
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
          row_forward(p, &sl, rows[r], s, o_rows + (int64_t)r * dim_v(p), lse_rows + r);
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
 * Explicit gradients of the scalar <dO, O>, with M_ij the dropout
 * multiplier and P the softmax before dropout:
 *   G_ij = <dO_i, v_j>,  Delta_i = <dO_i, O_i>  (the oracle's own fp64 O),
 *   dS_ij = P_ij (M_ij G_ij - Delta_i)   (= d loss / d logit_ij),
 *   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
 *   dV_j = sum_i P_ij M_ij dO_i.
 * Delta is the row-sum term of the backward preprocess named in the AOTriton
 * 0.14b release notes ("bwd_preprocess"); with dropout, sum_j P_ij M_ij G_ij
 * equals <dO_i, O_i>, so it stays that term.  Empty rows have P = 0 and so
 * contribute nothing; keys seen by no row get dK = dV = 0.
 */
static double dlogit(const oracle_problem *p, const slice *sl, int64_t i, int64_t j, double pij, double delta_i) {
  int DV = dim_v(p);
  double g = dot(sl->dO + i * DV, sl->V + j * DV, DV);
  return pij * (dropout_scale(p, sl->b, sl->h, i, j) * g - delta_i);
}

static void row_dq(const oracle_problem *p, const slice *sl, int64_t i,
                   double lse_i, double delta_i, double *dq_row) {
  int D = p->head_dim;
  int64_t sk = sl->sp.sk;
  for (int d = 0; d < D; ++d) dq_row[d] = 0.0;
  for (int64_t j = 0; j < sk; ++j) {
    double pij = prob(p, sl, i, j, lse_i);
    if (pij == 0.0) continue;
    double ds = dlogit(p, sl, i, j, pij, delta_i);
    for (int d = 0; d < D; ++d) dq_row[d] += p->scale * ds * sl->K[j * D + d];
  }
}

static void col_dkdv(const oracle_problem *p, const slice *sl, int64_t j,
                     const double *lse, const double *delta, double *dk_row,
                     double *dv_row) {
  int D = p->head_dim, DV = dim_v(p);
  int64_t sq = sl->sp.sq;
  for (int d = 0; d < D; ++d) dk_row[d] = 0.0;
  for (int d = 0; d < DV; ++d) dv_row[d] = 0.0;
  for (int64_t i = 0; i < sq; ++i) {
    double pij = prob(p, sl, i, j, lse[i]);
    if (pij == 0.0) continue;
    double ds = dlogit(p, sl, i, j, pij, delta[i]);
    double pm = pij * dropout_scale(p, sl->b, sl->h, i, j);
    for (int d = 0; d < D; ++d) dk_row[d] += p->scale * ds * sl->Q[i * D + d];
    for (int d = 0; d < DV; ++d) dv_row[d] += pm * sl->dO[i * DV + d];
  }
}

/* Row statistics (O, LSE, Delta) of a whole slice. */
static int slice_stats(const oracle_problem *p, const slice *sl, double *O,
                       double *lse, double *delta) {
  int DV = dim_v(p);
  if (slice_forward(p, sl, O, lse)) return -1;
  for (int64_t i = 0; i < sl->sp.sq; ++i)
    delta[i] = dot(sl->dO + i * DV, O + i * DV, DV);
  return 0;
}

int oracle_bwd(const oracle_problem *p, const void *q, const void *k,
               const void *v, const void *dout, double *o, double *lse,
               double *dq, double *dk, double *dv) {
  return oracle_bwd_dbias(p, q, k, v, dout, o, lse, dq, dk, dv, NULL);
}

int oracle_bwd_dbias(const oracle_problem *p, const void *q, const void *k,
                     const void *v, const void *dout, double *o, double *lse,
                     double *dq, double *dk, double *dv, double *dbias) {
  if (check_problem(p)) return -1;
  int D = p->head_dim, DV = dim_v(p);
  const int64_t sqm = max_len(p, 1), skm = max_len(p, 0);
  for (int b = 0; b < p->batch; ++b)
    for (int h = 0; h < p->heads; ++h) {
      slice sl;
      if (slice_load(p, q, k, v, dout, b, h, &sl)) { slice_free(&sl); return -1; }
      int64_t sq = sl.sp.sq, sk = sl.sp.sk;
      double *O = (double *)malloc(sizeof(double) * (size_t)(sq * DV + 1));
      double *L = (double *)malloc(sizeof(double) * (size_t)(sq + 1));
      double *De = (double *)malloc(sizeof(double) * (size_t)(sq + 1));
      double *dQ = (double *)malloc(sizeof(double) * (size_t)(sq * D + 1));
      double *dK = (double *)malloc(sizeof(double) * (size_t)(sk * D + 1));
      double *dV = (double *)malloc(sizeof(double) * (size_t)(sk * DV + 1));
      int rc = (O && L && De && dQ && dK && dV) ? slice_stats(p, &sl, O, L, De)
                                                 : -1;
      if (!rc) {
#pragma omp parallel for schedule(dynamic, 8)
        for (int64_t i = 0; i < sq; ++i) row_dq(p, &sl, i, L[i], De[i], dQ + i * D);
#pragma omp parallel for schedule(dynamic, 8)
        for (int64_t j = 0; j < sk; ++j)
          col_dkdv(p, &sl, j, L, De, dK + j * D, dV + j * DV);
        for (int64_t i = 0; i < sq; ++i) {
          for (int d = 0; d < D; ++d) dq[elem_index(p, b, h, sl.sp.q0, i, sq, D, d)] = dQ[i * D + d];
          if (o)
            for (int d = 0; d < DV; ++d) o[elem_index(p, b, h, sl.sp.q0, i, sq, DV, d)] = O[i * DV + d];
          if (lse) lse[lse_index(p, b, h, i)] = L[i];
        }
        for (int64_t j = 0; j < sk; ++j) {
          for (int d = 0; d < D; ++d) dk[elem_index(p, b, h, sl.sp.k0, j, sk, D, d)] = dK[j * D + d];
          for (int d = 0; d < DV; ++d) dv[elem_index(p, b, h, sl.sp.k0, j, sk, DV, d)] = dV[j * DV + d];
        }
        if (dbias) {
          double *row0 = dbias + ((int64_t)b * p->heads + h) * sqm * skm;
#pragma omp parallel for schedule(dynamic, 8)
          for (int64_t i = 0; i < sq; ++i)
            for (int64_t j = 0; j < sk; ++j) {
              double pij = prob(p, &sl, i, j, L[i]);
              row0[i * skm + j] = pij == 0.0 ? 0.0 : dlogit(p, &sl, i, j, pij, De[i]);
            }
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
  int D = p->head_dim, DV = dim_v(p);
  int64_t sq = sl.sp.sq, sk = sl.sp.sk;
  int bad = 0;
  for (int r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= sq) bad = 1;
  if (!bad) {
#pragma omp parallel
    {
      double *s = (double *)malloc(sizeof(double) * (size_t)(sk + 1));
      double *orow = (double *)malloc(sizeof(double) * (size_t)DV);
#pragma omp for schedule(dynamic, 1)
      for (int r = 0; r < nrows; ++r) {
        if (!s || !orow) continue;
        double lse_i;
        int64_t i = rows[r];
        row_forward(p, &sl, i, s, orow, &lse_i);
        double delta_i = dot(sl.dO + i * DV, orow, DV);
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
  int D = p->head_dim, DV = dim_v(p);
  int64_t sq = sl.sp.sq, sk = sl.sp.sk;
  int bad = 0;
  for (int c = 0; c < ncols; ++c)
    if (cols[c] < 0 || cols[c] >= sk) bad = 1;
  double *O = (double *)malloc(sizeof(double) * (size_t)(sq * DV + 1));
  double *L = (double *)malloc(sizeof(double) * (size_t)(sq + 1));
  double *De = (double *)malloc(sizeof(double) * (size_t)(sq + 1));
  if (!O || !L || !De) bad = 1;
  if (!bad && slice_stats(p, &sl, O, L, De)) bad = 1;
  if (!bad) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int c = 0; c < ncols; ++c)
      col_dkdv(p, &sl, cols[c], L, De, dk_cols + (int64_t)c * D,
               dv_cols + (int64_t)c * DV);
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
