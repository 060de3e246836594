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
  /* Additive bias on the logits (NULL: none): logit_ij = scale q_i.k_j +
   * bias[b*bias_stride[0] + h*bias_stride[1] + i*bias_stride[2] + j], local
   * indices, stored in the inputs' encoding (dtype) and decoded exactly. */
  const void *bias;
  int64_t bias_stride[3];
  /* ALiBi (NULL: none): logit_ij gains -alibi_slopes[h] * |i + sk - sq - j|
   * with the sequence's own sq, sk (query i sits at key position
   * i + sk - sq, the bottom-right alignment of a query block that ends
   * where the keys end). */
  const double *alibi_slopes;
  /* Dropout (dropout_p = 0: none).  After the softmax, P_ij is multiplied by
   * keep_ij / (1 - dropout_p), keep_ij from oracle_dropout_keep below. */
  double dropout_p;
  uint64_t philox_seed;
  uint64_t philox_offset;
  /* Row length of the dropout counters and of the bias / dBias arrays: the
   * largest Sq / Sk (packed; the dense seqlen_q / seqlen_k otherwise). */
  int max_seqlen_q;
  int max_seqlen_k;
  /* Head dim of V (and so of O, dO and dV); 0 means head_dim.  Q and K
   * rows hold head_dim values, the scores use those; V rows hold
   * head_dim_v. */
  int head_dim_v;
} oracle_problem;

/* Philox4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel
 * random numbers: as easy as 1, 2, 3", SC 2011): the four output words of
 * counter ctr[4] under key key[2]; the generator the AOTriton 0.10b notes
 * name for dropout ("Philox32x4"). */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* Dropout decision for (sequence b, head h, local row i, local key j):
 * word j % 4 of Philox4x32-10 at counter (lo, hi 32 bits of
 * philox_offset + ((b*heads + h)*max_seqlen_q + i)*ceil(max_seqlen_k/4) +
 * j/4, 0, 0) and key (lo, hi 32 bits of philox_seed); the element is kept
 * iff that word is >= floor(dropout_p * 2^32).  The four words of one
 * counter serve four consecutive keys in generation order (the word order
 * fix of the AOTriton 0.14b notes, "Minor Changes"). */
int oracle_dropout_keep(const oracle_problem *p, int b, int h, int64_t i, int64_t j);

/* The keep decisions of rows [0, nq) and keys [0, nk) of (b, h) into
 * keep[nq][nk] (1 kept, 0 dropped). */
void oracle_dropout_mask(const oracle_problem *p, int b, int h, int64_t nq, int64_t nk, uint8_t *keep);

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

/* The same, with the gradient of the logits dS_ij (= d loss / d bias_ij)
 * into dbias [B][H][max_seqlen_q][max_seqlen_k] (fp64, 0 where no pair of
 * the sequence sits); dbias may be NULL. */
int oracle_bwd_dbias(const oracle_problem *p, const void *q, const void *k,
                     const void *v, const void *dout, double *o, double *lse,
                     double *dq, double *dk, double *dv, double *dbias);

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
