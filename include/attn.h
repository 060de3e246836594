/*
 * attn.h - C ABI of the MI355X (gfx950) fused scaled-dot-product attention
 * library: forward (O and the per-row logsumexp LSE) and backward (dQ, dK,
 * dV) under generalized sliding-window masks, for dense and packed
 * variable-length inputs.
 *
 * The operation is FlashAttention, the one kernel family of the AOTriton
 * README ("Kernel Support"):  O = softmax(scale * Q K^T + mask) V and
 * LSE_i = ln sum_{j visible} exp(scale * q_i . k_j).
 *
 * Mask (AOTriton 0.10b release notes, "Major Changes": generalized sliding
 * window, negative bounds allowed; AOTriton 0.15b release notes,
 * "Bottom-Right Aligned Sliding Windows"): with 0-based indices local to one
 * sequence, key j is visible to query i iff  i - L <= j <= i + R.  L and R
 * are window_left and window_right, except that under ATTN_BOTTOM_RIGHT a
 * window whose both sides are finite becomes L = wl - d, R = wr + d with
 * d = seqlen_k - seqlen_q of that sequence.  A window with an unbounded side
 * (ATTN_WINDOW_INF; causal is (ATTN_WINDOW_INF, 0)) is never shifted.
 *
 * Rows with no visible key get O = 0 (only the head_dim columns are written)
 * and LSE = +inf, as in the early-exit fixes of the AOTriton 0.15b and 0.14b
 * release notes ("Kernel Bug Fixes"); their dQ is 0, and keys seen by no row
 * get dK = dV = 0.
 *
 * Conventions shared by every entry point:
 *  - All pointers are device pointers, owned by the caller, and must stay
 *    valid until the work enqueued on `stream` has finished.  The library
 *    allocates nothing and keeps no pointer after returning.
 *  - Calls are asynchronous on `stream`; the device is the stream's device
 *    (hipStreamGetDevice), not the calling thread's current device (the
 *    AOTriton 0.14b release notes, "Runtime Bug Fixes").  The null stream
 *    means the current device's null stream.
 *  - Every output element is overwritten; nothing needs pre-zeroing.
 *  - A tensor with no elements (batch 0, or no rows on its side) touches no
 *    memory: its pointer may be NULL and takes part in no aliasing check.
 *  - Errors are returned, never printed: hipErrorInvalidValue for a malformed
 *    call (null required pointer, version or flags mismatch, negative or
 *    zero sizes where a size is needed, a pointer not aligned to its element
 *    size, workspace too small), hipErrorNotSupported for a well-formed call
 *    outside the built set (head_dim or head_dim_v above 256 for fp16 and
 *    bf16, above 128 for fp32), or the HIP error of the launch.  Validation makes no HIP call.  The contents of
 *    cu_seqlens arrays are a precondition (0 first, non-decreasing, last
 *    entry equal to total_q / total_k, every length <= the seqlen_q /
 *    seqlen_k maximum) and are not checked: reading them would need a sync.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Version of the params structs below (the versioned-params idea of the
 * AOTriton 0.15b release notes, "API Changes": kVersion fields, reserved bits
 * rejected).  Version 3 adds the per-side addressing fields at the end of
 * attn_fwd_params.  Structs of version 2 (the same layout without those
 * fields, and attn_bwd_params embedding that shorter struct) are still
 * accepted and translated, as the AOTriton 0.14b notes do for older params
 * ("ABI backward compatibility"); any other version is hipErrorInvalidValue. */
#define ATTN_PARAMS_VERSION 3u

/* Bits of attn_fwd_params.flags; every other bit must be 0.
 * ATTN_FLAG_LSE_TH (packed layout only): lse is [total_q, heads] (the "TH"
 *   layout of the AOTriton 0.14b VarlenBits LSE field) instead of
 *   [heads, total_q]. */
#define ATTN_FLAG_LSE_TH 1u
/* ATTN_FLAG_NO_SPLIT: never use the split paths that small grids otherwise
 *   take: the split mode of attn_bwd_workspace_size / attn_bwd below (the
 *   workspace then holds only Delta and LSE), and the forward's key-split
 *   workgroups (for a small grid, or for the last round of a grid of a few
 *   rounds); the forward then runs its plain grid. */
#define ATTN_FLAG_NO_SPLIT 2u

/* Unbounded side of a window. */
#define ATTN_WINDOW_INF 2147483647

/* Element type of q, k, v, o, dout, dq, dk, dv.  LSE and the workspace are
 * always fp32. */
#define ATTN_FP32 0
#define ATTN_FP16 1
#define ATTN_BF16 2

/* ATTN_BHSD:   dense [batch, heads, seq, head_dim] addressed with strides
 *              {batch, head, row}.
 * ATTN_THD:    packed [total, heads, head_dim]; sequence b owns rows
 *              cu_seqlens[b] .. cu_seqlens[b+1]-1 ("stacked" varlen of the
 *              AOTriton 0.14b release notes, "VarlenBits supersedes
 *              VarlenType"); strides {ignored, head, row}.
 * ATTN_VARLEN: each side addressed on its own by the mode byte of its side
 *              in `varlen` (below).  ATTN_BHSD is the mode 0 on both sides
 *              (plus ATTN_SEQ_LEN_ARRAY where seqused is given), ATTN_THD the
 *              mode ATTN_SEQ_STACKED | ATTN_SEQ_LEN_CUMSUM |
 *              ATTN_SEQ_POS_CUMSUM (LEN_ARRAY with seqused). */
#define ATTN_BHSD 0
#define ATTN_THD 1
#define ATTN_VARLEN 2

/* Mode byte of one side (VarlenMode of the AOTriton 0.14b VarlenBits: Q and
 * K decode independently along three axes).  Bit 0, storage:
 *   0 padded:  sequence b's rows start at b * stride[0] (a [batch, heads,
 *              seqlen, head_dim]-style tensor; seqlen rows of room each);
 *   ATTN_SEQ_STACKED: rows of every sequence in one [total, heads,
 *              head_dim] tensor (stride[0] ignored).
 * Bits 2:1, lengths:
 *   ATTN_SEQ_LEN_UNIFORM: every sequence has seqlen_q / seqlen_k rows;
 *   ATTN_SEQ_LEN_CUMSUM:  cu_seqlens[b+1] - cu_seqlens[b];
 *   ATTN_SEQ_LEN_ARRAY:   seqused[b] (seqused_q / seqused_k).
 * Bits 4:3, start row of sequence b in a stacked tensor (padded: 0):
 *   ATTN_SEQ_POS_UNIFORM: b * seqlen;
 *   ATTN_SEQ_POS_CUMSUM:  cu_seqlens[b];
 *   ATTN_SEQ_POS_ARRAY:   seqstart[b] (seqstart_q / seqstart_k).
 * A sequence's room is seqlen rows (padded, or stacked with POS_UNIFORM) or
 * its cu_seqlens range (stacked with POS_CUMSUM); with POS_ARRAY it is not
 * known.  LEN_ARRAY lengths are clamped to the room, or to seqlen when the
 * room is not known; rows of the room past the length are written as fully
 * masked rows (O = 0, LSE = +inf, gradients 0), rows outside every sequence
 * are never touched.  The sequences of one side must not overlap (outputs
 * are written per sequence).  Every row a mode addresses must lie in the
 * tensor: total rows (stacked) or batch * seqlen rows (padded).  The LSE
 * (and the backward's workspace) follows the Q side: [batch, heads,
 * seqlen_q] padded, [heads, total_q] (or [total_q, heads] with
 * ATTN_FLAG_LSE_TH) stacked. */
#define ATTN_SEQ_STACKED 0x01u
#define ATTN_SEQ_LEN_UNIFORM 0x00u
#define ATTN_SEQ_LEN_CUMSUM 0x02u
#define ATTN_SEQ_LEN_ARRAY 0x04u
#define ATTN_SEQ_POS_UNIFORM 0x00u
#define ATTN_SEQ_POS_CUMSUM 0x08u
#define ATTN_SEQ_POS_ARRAY 0x10u
/* `varlen` field of attn_fwd_params (ATTN_VARLEN only; 0 otherwise): Q's
 * mode byte in bits 7:0, K's in bits 15:8, the rest 0. */
#define ATTN_VARLEN_BITS(qmode, kmode) ((uint32_t)(qmode) | ((uint32_t)(kmode) << 8))

/* Principal diagonal (AOTriton 0.15b, VarlenPrincipalDiagonal). */
#define ATTN_TOP_LEFT 0
#define ATTN_BOTTOM_RIGHT 1

typedef struct {
  uint32_t version;        /* ATTN_PARAMS_VERSION */
  uint32_t flags;          /* ATTN_FLAG_LSE_TH (stacked Q only) and / or
                              ATTN_FLAG_NO_SPLIT, else 0 */
  int32_t dtype;           /* ATTN_FP32 / ATTN_FP16 / ATTN_BF16 */
  int32_t layout;          /* ATTN_BHSD / ATTN_THD / ATTN_VARLEN */
  int32_t batch;           /* BHSD: batch; THD: number of sequences (>= 1);
                              VARLEN: number of sequences (>= 1 if a side
                              is stacked) */
  int32_t heads;           /* >= 1; Q, K and V have the same head count */
  int32_t head_dim;        /* of Q and K (and of V, O, dO, dV when
                              head_dim_v is 0): 1..256 for fp16 / bf16,
                              1..128 for fp32.  32, 48, 64, 80, 96 and 128
                              (the multiples of 16 up to 128 the AOTriton
                              pages name or test, 48 and 80 among them, 0.10b
                              "Known Problems"), and 192 and 256 for fp16 /
                              bf16 (toward the larger heads of the 0.14b
                              notes, "Gfx950 Performance Boost"), run in
                              place; see "Repacked calls" for the others */
  int32_t seqlen_q;        /* BHSD: Sq (>= 0); THD: max sequence length of Q;
                              VARLEN: the Q side's uniform length / room,
                              and the largest length (>= 0) */
  int32_t seqlen_k;        /* the same for K */
  int32_t window_left;     /* any int32; ATTN_WINDOW_INF = unbounded */
  int32_t window_right;    /* any int32; ATTN_WINDOW_INF = unbounded */
  int32_t diag;            /* ATTN_TOP_LEFT / ATTN_BOTTOM_RIGHT */
  float scale;             /* any finite value, 0 and negatives included */
  int32_t reserved0;       /* must be 0 */
  int64_t total_q;         /* stacked Q side: rows of Q/O/dO (THD:
                              = cu_seqlens_q[batch]) */
  int64_t total_k;         /* stacked K side: rows of K/V */
  const void *q;           /* input */
  const void *k;           /* input */
  const void *v;           /* input */
  void *o;                 /* fwd: output; bwd: input (the forward's O) */
  float *lse;              /* fwd: output; bwd: input.  BHSD: contiguous
                              [batch, heads, seqlen_q]; THD: contiguous
                              [heads, total_q] (the "HT" layout), or
                              [total_q, heads] with ATTN_FLAG_LSE_TH. */
  const int32_t *cu_seqlens_q; /* device int32[batch+1]: THD, and VARLEN
                              with LEN_CUMSUM or POS_CUMSUM on Q; else NULL */
  const int32_t *cu_seqlens_k; /* the same for K */
  int64_t q_stride[3];     /* element strides {batch, head, row}; the */
  int64_t k_stride[3];     /* head_dim stride is 1.  A call whose base */
  int64_t v_stride[3];     /* pointers and strides keep every row 16-byte */
  int64_t o_stride[3];     /* aligned runs in place, any other is repacked.
                              A stride may be negative: the pointer is then
                              the address of index 0 on that axis, and the
                              operand reaches below it. */
  const int32_t *seqused_q; /* optional device int32[batch]: sequence b uses
                              only its first seqused_q[b] query rows (of
                              seqlen_q rows, BHSD, or of its cu_seqlens_q
                              range, THD); NULL = all rows */
  const int32_t *seqused_k; /* optional, the same for keys ("seqused_k" of
                              a packed KV cache, VarlenBits of the AOTriton
                              0.14b notes).  Rows past the used ones are
                              written as fully masked: O = 0, LSE = +inf,
                              dQ = dK = dV = 0.  0 <= seqused[b] <= the
                              sequence's rows is a precondition (values out
                              of range are clamped, never read past).  With
                              ATTN_VARLEN: the lengths of LEN_ARRAY, required
                              there and NULL otherwise. */
  /* Version 3. */
  uint32_t varlen;          /* ATTN_VARLEN: ATTN_VARLEN_BITS(qmode, kmode);
                              other layouts: 0 */
  int32_t reserved1;        /* must be 0 */
  const int32_t *seqstart_q; /* ATTN_VARLEN with POS_ARRAY on Q: device
                              int32[batch], start row of each sequence in
                              the stacked tensor; NULL otherwise */
  const int32_t *seqstart_k; /* the same for K */
  /* Optional features (version 3; a NULL pointer / 0 disables each).  The
   * logits become scale q_i.k_j + bias_ij + alibi_ij, and dropout scales the
   * softmax after it; a call with any of them runs on kernels built for
   * them (the plain kernels are unchanged).  Indices i, j are local to the
   * sequence (i < its Q length, j < its K length). */
  const void *bias;         /* additive bias in the dtype of q: element
                              (b, h, i, j) at b*bias_stride[0] +
                              h*bias_stride[1] + i*bias_stride[2] + j
                              (strides may be 0 to broadcast); converted to
                              fp32 before use (the AOTriton 0.14b notes,
                              "Kernel Bug Fixes"); -inf masks the pair */
  int64_t bias_stride[3];
  const float *alibi_slopes; /* device fp32[heads]: ALiBi adds
                              -slope_h * |i + sk - sq - j| with the
                              sequence's lengths sq, sk (query i at key
                              position i + sk - sq) */
  float dropout_p;          /* 0 (none) <= p < 1: pair (i, j) is kept iff word
                              j % 4 of Philox4x32-10 (the generator of the
                              AOTriton 0.10b notes) at counter (lo, hi 32 bits
                              of philox_offset + ((b*heads + h)*seqlen_q + i)
                              * ceil(seqlen_k / 4) + j / 4, 0, 0) and key
                              (lo, hi 32 bits of philox_seed) is >=
                              floor(p * 2^32) -- one counter for four
                              consecutive keys, words in generation order
                              (0.14b "Minor Changes"); kept probabilities are
                              scaled by 1 / (1 - p).  LSE is the softmax's,
                              before dropout. */
  int32_t head_dim_v;       /* head dim of V, O, dO and dV, as head_dim (Hdim_vo
                              of the AOTriton 0.15b notes, "Kernel Bug
                              Fixes"); 0 = head_dim.  A value other than
                              head_dim makes the call a repacked one. */
  uint64_t philox_seed;
  uint64_t philox_offset;
  void *workspace;          /* forward: device, caller-owned, 256-byte
                              aligned; needed by a repacked call, used by
                              the key-split tail when it holds
                              attn_fwd_workspace_size(this) bytes, NULL
                              allowed otherwise; ignored by the backward
                              calls (which take attn_bwd_params.workspace).
                              Calls that overlap on one workspace race. */
  uint64_t workspace_bytes;
} attn_fwd_params;

/* Repacked calls.  A call runs in place when head_dim is one of the built
 * dims (32, 48, 64, 80, 96, 128; 192 and 256 for fp16 / bf16), head_dim_v
 * equals it, and every operand row is 16-byte aligned (base pointers and
 * strides; for fp16 / bf16 also within the tile copies' 2 GiB span: 63 row
 * strides plus one row).  Any other call with supported head dims is
 * repacked: the library first copies its inputs,
 * each row zero-padded to Dp columns (the smallest built dim >= both head
 * dims), into the workspace, runs the in-place kernels there at head dim Dp
 * (zero columns add nothing to Q K^T, and give zero columns of O, dQ, dK
 * and dV), and copies the outputs' first head_dim (head_dim_v) columns
 * back, over the rows the in-place call would write.  LSE and dbias are
 * written directly.  The copies cost one read and one write of each
 * operand; the results equal those of the same problem zero-padded to Dp
 * by the caller. */

/* Forward workspace bytes a call can use; 0 when the problem is malformed.
 * Two parts, in this order:
 *  - needed (attn_fwd and attn_fwd_check reject a smaller workspace): for a
 *    repacked call, padded copies of q, k, v and o (rows of Dp elements; a
 *    stacked side's rows are total_q / total_k, a padded side's batch *
 *    seqlen), each rounded up to 256 bytes; nothing for an in-place call;
 *  - optional: the key-split tail's partial sums, for the in-place call it
 *    runs (at Dp when repacked) when that call is fp16 / bf16 at head_dim
 *    <= 128, has no optional feature and no ATTN_FLAG_NO_SPLIT, and its
 *    band is unbounded on a side or at least 1024 keys wide and spans at
 *    least 2 F keys (seqlen_k, or the band width + 255 if smaller; F = 512
 *    at head_dim <= 64, else 1024):
 *    256 * (2 if head_dim <= 64 else 1) slots of 8 * 64 * (4 * ceil(
 *    head_dim / 32) + 1) float4 (about 35 MiB at head_dim 128).
 * A workspace that holds both parts (and is 256-byte aligned) lets the
 * forward split the key axis of its grid's last, partly filled round over
 * more workgroups; without the second part it runs without that split.
 * The result differs between the two only by rounding. */
uint64_t attn_fwd_workspace_size(const attn_fwd_params *p);

typedef struct {
  attn_fwd_params fwd;     /* problem, inputs q/k/v and the forward's o/lse */
  const void *dout;        /* input, laid out like o (own strides) */
  void *dq;                /* outputs, laid out like q, k, v (own strides) */
  void *dk;
  void *dv;
  int64_t do_stride[3];
  int64_t dq_stride[3];
  int64_t dk_stride[3];
  int64_t dv_stride[3];
  void *workspace;         /* device, caller-owned, 256-byte aligned */
  uint64_t workspace_bytes;/* >= attn_bwd_workspace_size(this) */
  /* Version 3: optional output, fp32, the gradient of the loss with respect
   * to the logits (= d loss / d bias_ij): element (b, h, i, j) at
   * b*dbias_stride[0] + h*dbias_stride[1] + i*dbias_stride[2] + j, written
   * for every i < the sequence's Q length and j < its K length (0 where the
   * pair is masked), untouched elsewhere.  NULL: not computed. */
  float *dbias;
  int64_t dbias_stride[3];
} attn_bwd_params;

/* Forward: writes o and lse.  Enqueues on `stream` one forward kernel
 * over the query blocks (for fp16 / bf16 inputs with a band unbounded or at
 * least 1024 keys wide, the 256-row ping-pong kernel; in fp32 at head_dim
 * <= 64, a grid of at most half as many 64-row blocks as CUs runs on
 * workgroups that split the keys in two halves), then, only when seqused_q
 * is given, a small kernel that writes the rows past the used ones as
 * masked rows.  The ping-pong grid's last round, when partly filled:
 *  - with the key-split part of the workspace (attn_fwd_workspace_size),
 *    r blocks each run as np = min(8, round / r, band keys / F) >= 2
 *    ping-pong workgroups over near-equal runs of the block's key tiles,
 *    which store fp32 partials to the workspace, and a merge kernel
 *    combines each block's partials in a fixed order and writes its rows
 *    (a grid of fewer blocks than a round is all last round; one of at most
 *    a quarter as many blocks as CUs only when r np >= the CU count);
 *  - otherwise, with at most three full rounds and a last round at most a
 *    quarter full, a kernel that splits that round's blocks over four
 *    64-row workgroups, each over two key halves merged in LDS.
 * A grid of at most a quarter as many blocks as the device has CUs goes to
 * that last kernel whole.  ATTN_FLAG_NO_SPLIT keeps the plain grids.
 * attn_fwd_plan lists the kernels of a call. */
hipError_t attn_fwd(const attn_fwd_params *p, hipStream_t stream);

/* Backward: reads q, k, v, o, lse, dout; writes dq, dk, dv.  Enqueues, in
 * stream order, the row-sum preprocess Delta_i = sum_d dO_id O_id (the
 * "bwd_preprocess" of the AOTriton 0.14b release notes) into the workspace,
 * then the per-key-block dK/dV work and the per-query-block dQ work (the
 * split backward, "triton_split" in the same notes) as attn_bwd_dkdv_dq
 * does, then, only when seqused_q / seqused_k are given, the small kernels
 * that zero the gradient rows past the used ones.  The dK/dV and dQ sums are
 * computed without floating-point atomics: results are run-to-run
 * identical.
 *
 * Split mode (small and mid-size problems, unless ATTN_FLAG_NO_SPLIT): when
 * the call has no bias, ALiBi, dropout or dbias and the dK/dV or the dQ
 * grid (128 keys or queries per workgroup) would have fewer than 64
 * workgroups (at fp16 / bf16 head dims 96 and 128: a dK/dV grid of at most
 * 16), or, with seqlen_q and seqlen_k both at least 1024 (2048 at those
 * head dims), fewer than 200 (65 at those head dims), each grid is
 * repeated so that copy g of n walks the g-th of n contiguous shares of
 * the tiles it would visit (query tiles for dK/dV, key tiles for dQ), about
 * 256 workgroups in all (at most 8 copies, one per tile, fp32 partial sums
 * of at most 64 MiB); the copies store fp32 partial sums in the
 * workspace.  In fp32 each copy then counts itself in on an arrival
 * counter per block there, and the last copy of a block to arrive adds the
 * block's partials in copy order, scales, rounds and writes them (so the
 * result does not depend on which copy is last), and resets the counter; no
 * workgroup waits for another.  In fp16 / bf16 a last kernel does that sum
 * over the whole GPU.  The dK/dV and dQ copies run as one grid where both
 * kinds fit one workgroup's LDS (fp16 / bf16 up to head_dim 128, fp32 up to
 * 64).  The sums then group the tiles differently from the unsplit path
 * (results differ in rounding only, and stay run-to-run identical).
 * attn_bwd_preprocess zeroes the counters, so the step calls below need it
 * first, as they do anyway for Delta; repeated dK/dV or dQ calls on one
 * workspace are fine.  Split calls that overlap on one workspace race, as
 * any calls that share a workspace do. */
hipError_t attn_bwd(const attn_bwd_params *p, hipStream_t stream);

/* The three steps of attn_bwd as separate calls, for callers that schedule
 * or time them one by one.  Same parameters, validation and errors as
 * attn_bwd; each enqueues one kernel on `stream`, and attn_bwd_dkdv /
 * attn_bwd_dq also the row-zeroing kernel of their outputs when seqused
 * arrays are given (in split mode: their split grid, and in fp16 / bf16
 * the reduction of their outputs).  They must run in this order on one stream (or be
 * ordered by events): attn_bwd_dkdv and attn_bwd_dq read the Delta and LSE
 * log2(e) that attn_bwd_preprocess leaves in the workspace, which must not
 * be touched in between.
 *   attn_bwd_preprocess: Delta_i = sum_d dO_id O_id and LSE_i log2(e) into
 *                        the workspace.
 *   attn_bwd_dkdv:       dK and dV, one workgroup per block of keys.
 *   attn_bwd_dq:         dQ, one workgroup per block of queries. */
hipError_t attn_bwd_preprocess(const attn_bwd_params *p, hipStream_t stream);
hipError_t attn_bwd_dkdv(const attn_bwd_params *p, hipStream_t stream);
hipError_t attn_bwd_dq(const attn_bwd_params *p, hipStream_t stream);

/* dK, dV and dQ after attn_bwd_preprocess (same ordering rule as the two
 * calls above).  Where the build has it (fp16 and bf16 at head_dim 128) and
 * the problem gains from it (a band unbounded or at least 1024 keys wide,
 * and a separate dQ grid that would leave its last round on the device's
 * compute units at most a quarter full), one kernel whose workgroups are dK/dV
 * blocks first and dQ blocks after, so that dQ blocks fill the CUs the
 * dK/dV grid leaves idle; otherwise the two kernels in order.  Same
 * parameters, validation and errors as attn_bwd; results equal those of
 * attn_bwd_dkdv then attn_bwd_dq. */
hipError_t attn_bwd_dkdv_dq(const attn_bwd_params *p, hipStream_t stream);

/* Workspace bytes attn_bwd needs for this problem: two fp32 values per query
 * row and head (Delta_i and LSE_i * log2(e), written by attn_bwd_preprocess
 * and read by the other two steps), each array rounded up to 256 bytes,
 * then, in split mode, the fp32 partial sums (head_dim floats per copy, head
 * and row: dK and dV per key-side copy, dQ per query-side copy; rows are the
 * stacked tensor's rows, or batch * seqlen for a padded side), rounded up to
 * 256 bytes, and a 4-byte arrival counter per block of R rows of the dK/dV
 * and dQ grids (B H ceil(seqlen_k / R) + B H ceil(seqlen_q / R); R = 64 in
 * fp32, 128 in fp16 / bf16), rounded up to 256 bytes; 0 when the problem is
 * malformed.  A repacked call (see above)
 * needs, before those (sized for head dim Dp), padded copies of q, k, v, o,
 * dout, dq, dk and dv, each rounded up to 256 bytes.  Repacked, the three
 * step calls share the copies through the workspace: attn_bwd_preprocess
 * makes the input copies, attn_bwd_dkdv / attn_bwd_dq copy their outputs
 * back. */
uint64_t attn_bwd_workspace_size(const attn_bwd_params *p);

/* Host-only validation of a call, the same checks attn_fwd / attn_bwd make
 * first; no HIP call is made.  Returns hipSuccess or the error the call
 * would return before launching. */
hipError_t attn_fwd_check(const attn_fwd_params *p);
hipError_t attn_bwd_check(const attn_bwd_params *p);

/* ATTN_PARAMS_VERSION of the built library. */
uint32_t attn_params_version(void);

/* ------------------------------------------------------------ launch plans
 *
 * What a call would enqueue, for callers that label, profile or schedule its
 * work: the kernels in launch order, by function name (static strings owned
 * by the library, valid while it is loaded), with their workgroup counts and
 * sizes.  The plan is made by the same code that makes the launch choice of
 * the call, for the stream's device (its compute-unit count decides some
 * choices).  Host-only: nothing is enqueued and no device memory is read or
 * written.  The call's own validation runs first and its error is returned;
 * attn_bwd_plan does not look at the workspace, which decides nothing. */
#define ATTN_PLAN_MAX 8
typedef struct {
  const char *kernel[ATTN_PLAN_MAX]; /* kernel[i], i < count */
  uint32_t grid[ATTN_PLAN_MAX];      /* workgroups of launch i */
  uint32_t block[ATTN_PLAN_MAX];     /* threads per workgroup of launch i */
  int32_t count;                     /* launches; 0 for a problem with no rows */
  int32_t reserved;
} attn_plan;

/* Steps of the backward for attn_bwd_plan (bit mask, any non-empty subset):
 * attn_bwd is ATTN_BWD_ALL, attn_bwd_dkdv_dq is ATTN_BWD_DKDV | ATTN_BWD_DQ. */
#define ATTN_BWD_PREPROCESS 1u
#define ATTN_BWD_DKDV 2u
#define ATTN_BWD_DQ 4u
#define ATTN_BWD_ALL 7u

hipError_t attn_fwd_plan(const attn_fwd_params *p, hipStream_t stream, attn_plan *plan);
hipError_t attn_bwd_plan(const attn_bwd_params *p, uint32_t steps, hipStream_t stream, attn_plan *plan);

/* ------------------------------------------------- no-allocation backward
 *
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same work and results as attn_bwd (same kernels, bit for
 * bit; see the limit below), with the workspace taken from a static array of
 * ATTN_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs
 * on until the process ends.  p->workspace and p->workspace_bytes are
 * ignored.  Allocates nothing, on the host or the device.
 *  - Limit: a call whose split-mode partial sums would make its workspace
 *    (attn_bwd_workspace_size) exceed ATTN_NOALLOC_SCRATCH_BYTES runs
 *    without split mode (its results are then those of attn_bwd with
 *    ATTN_FLAG_NO_SPLIT); problems whose workspace exceeds the array even
 *    so, i.e. more than about two million (head, query row) pairs, return
 *    hipErrorOutOfMemory before enqueuing anything.
 *  - Every call on one device shares that device's array: calls that may
 *    overlap in time on one device (different streams, or other threads)
 *    race and must be ordered by the caller.  Nothing in it needs clearing
 *    by the caller: each call writes the part it reads before reading it
 *    (its preprocess kernel zeroes the split mode's arrival counters).
 *  - The array's device address is looked up on the first call on each
 *    device; that call must not be made under stream capture. */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
hipError_t attn_bwd_noalloc(const attn_bwd_params *p, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* ATTN_H */
