/*
 * sdpa_oracle.h - fp64 CPU oracle for scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes, links
 * or calls this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code with the GPU path.
 *
 * What it computes (plain definition, no blocking, no online rescaling):
 *   S_ij = scale * <q_i, k_j>  on the visible set J(i), P = softmax_j(S),
 *   O = P V, LSE_i = ln sum_{j in J(i)} exp(S_ij),
 * and the explicit gradients of <dO, O> with respect to Q, K and V.
 * FlashAttention (the one kernel family of the AOTriton README, section
 * "Kernel Support") reaches this same result; the oracle therefore writes the
 * definition out rather than the tiled algorithm.
 *
 * Visibility follows the generalized sliding-window rule of the AOTriton
 * 0.10b release notes (section "Major Changes": causal masking expressed as a
 * special case of the generalized window), with the diagonal choice of the
 * AOTriton 0.15b release notes, section "Bottom-Right Aligned Sliding
 * Windows".
 */
#ifndef SDPA_ORACLE_H
#define SDPA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Unbounded side of a window. */
#define ORACLE_WINDOW_INF 2147483647

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };
enum { ORACLE_DENSE = 0, ORACLE_PACKED = 1 };
enum { ORACLE_TOP_LEFT = 0, ORACLE_BOTTOM_RIGHT = 1 };

typedef struct {
  int dtype;      /* encoding of q, k, v, dout: ORACLE_F32 / _F16 / _BF16 */
  int layout;     /* ORACLE_DENSE: contiguous [B][H][S][D];
                     ORACLE_PACKED: contiguous [T][H][D] + cu_seqlens */
  int batch;      /* dense: batch; packed: number of sequences */
  int heads;
  int head_dim;
  int seqlen_q;   /* dense only */
  int seqlen_k;   /* dense only */
  const int32_t *cu_seqlens_q; /* packed only, host memory, batch+1 entries */
  const int32_t *cu_seqlens_k;
  int window_left;   /* ORACLE_WINDOW_INF = unbounded */
  int window_right;
  int diag;          /* ORACLE_TOP_LEFT / ORACLE_BOTTOM_RIGHT */
  double scale;
} oracle_problem;

/* 1 if key j is visible to query i in a sequence of sq queries, sk keys. */
int oracle_visible(int64_t i, int64_t j, int64_t sq, int64_t sk,
                   int window_left, int window_right, int diag);

/* Decoders of the stored input encodings, exposed for the pins. */
double oracle_decode_f16(uint16_t bits);
double oracle_decode_bf16(uint16_t bits);

/* Forward over the whole problem.  o: same shape as q (fp64);
 * lse: dense [B][H][Sq], packed [H][Tq] (fp64).  Fully masked rows give
 * o = 0 and lse = +inf.  Returns 0, or -1 on a malformed problem. */
int oracle_fwd(const oracle_problem *p, const void *q, const void *k,
               const void *v, double *o, double *lse);

/* Backward over the whole problem: dq, dk, dv shaped like q, k, v (fp64).
 * o and lse may be NULL; when given they receive the forward results. */
int oracle_bwd(const oracle_problem *p, const void *q, const void *k,
               const void *v, const void *dout, double *o, double *lse,
               double *dq, double *dk, double *dv);

/* Forward for selected query rows of one (sequence b, head h): rows[] are
 * sequence-local indices; o_rows is [nrows][D], lse_rows [nrows]. */
int oracle_fwd_rows(const oracle_problem *p, const void *q, const void *k,
                    const void *v, int b, int h, int nrows,
                    const int32_t *rows, double *o_rows, double *lse_rows);

/* dQ for selected query rows of one (b, h): dq_rows is [nrows][D]. */
int oracle_bwd_dq_rows(const oracle_problem *p, const void *q, const void *k,
                       const void *v, const void *dout, int b, int h,
                       int nrows, const int32_t *rows, double *dq_rows);

/* dK and dV for selected key rows of one (b, h): [ncols][D] each. */
int oracle_bwd_dkdv_cols(const oracle_problem *p, const void *q,
                         const void *k, const void *v, const void *dout,
                         int b, int h, int ncols, const int32_t *cols,
                         double *dk_cols, double *dv_cols);

/* Number of OpenMP threads the oracle uses. */
int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
