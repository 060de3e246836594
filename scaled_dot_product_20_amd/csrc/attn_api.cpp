// attn_api.cpp - the C ABI declared in include/attn.h: validation, argument
// marshalling into kernel argument blocks, and the device taken from the
// stream.  Nothing is allocated per call and nothing is printed.  The
// library's only state is written once per device and never changed after:
// the compute-unit count the launchers read (attn_launch.hpp), and the device
// address of the no-allocation backward's scratch array (below).
#include "attn.h"

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "attn_launch.hpp"

namespace {

using sdpa::Operand;

// ------------------------------------------------------ version 2 structs
//
// The params layout of version 2: attn_fwd_params without the version-3
// fields at its end, and attn_bwd_params embedding that shorter struct.
// Calls made with them are translated into version 3 (new fields zero).
struct FwdParamsV2 {
  uint32_t version, flags;
  int32_t dtype, layout, batch, heads, head_dim, seqlen_q, seqlen_k, window_left, window_right, diag;
  float scale;
  int32_t reserved0;
  int64_t total_q, total_k;
  const void *q, *k, *v;
  void* o;
  float* lse;
  const int32_t *cu_seqlens_q, *cu_seqlens_k;
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
  const int32_t *seqused_q, *seqused_k;
};
struct BwdParamsV2 {
  FwdParamsV2 fwd;
  const void* dout;
  void *dq, *dk, *dv;
  int64_t do_stride[3], dq_stride[3], dk_stride[3], dv_stride[3];
  void* workspace;
  uint64_t workspace_bytes;
};
static_assert(sizeof(FwdParamsV2) == offsetof(attn_fwd_params, varlen), "version 2 is a prefix of version 3");

// The version-3 view of a call's params (`tmp` holds a translated copy).
const attn_fwd_params* fwd_v3(const attn_fwd_params* p, attn_fwd_params* tmp) {
  if (!p || p->version != 2u) return p;
  std::memset(tmp, 0, sizeof(*tmp));
  std::memcpy(tmp, p, sizeof(FwdParamsV2));
  tmp->version = ATTN_PARAMS_VERSION;
  return tmp;
}
const attn_bwd_params* bwd_v3(const attn_bwd_params* p, attn_bwd_params* tmp) {
  if (!p || p->fwd.version != 2u) return p;
  const BwdParamsV2* o = reinterpret_cast<const BwdParamsV2*>(p);
  std::memset(tmp, 0, sizeof(*tmp));
  std::memcpy(&tmp->fwd, &o->fwd, sizeof(FwdParamsV2));
  tmp->fwd.version = ATTN_PARAMS_VERSION;
  tmp->dout = o->dout;
  tmp->dq = o->dq;
  tmp->dk = o->dk;
  tmp->dv = o->dv;
  std::memcpy(tmp->do_stride, o->do_stride, sizeof(o->do_stride));
  std::memcpy(tmp->dq_stride, o->dq_stride, sizeof(o->dq_stride));
  std::memcpy(tmp->dk_stride, o->dk_stride, sizeof(o->dk_stride));
  std::memcpy(tmp->dv_stride, o->dv_stride, sizeof(o->dv_stride));
  tmp->workspace = o->workspace;
  tmp->workspace_bytes = o->workspace_bytes;
  return tmp;
}

bool dtype_ok(int32_t d) { return d == ATTN_FP32 || d == ATTN_FP16 || d == ATTN_BF16; }
int64_t elem_bytes(int32_t d) { return d == ATTN_FP32 ? 4 : 2; }
bool head_dim_built(int32_t d) { return d == 32 || d == 48 || d == 64 || d == 80 || d == 96 || d == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ------------------------------------------------------ per-side addressing

// One side (Q or K) of a call: its mode byte (ATTN_SEQ_* bits) and arrays.
struct Side {
  uint32_t mode;
  const int32_t *cu, *len, *start;
  int32_t S;      // seqlen_q / seqlen_k
  int64_t total;  // stacked: rows of the tensor
  bool stacked() const { return (mode & ATTN_SEQ_STACKED) != 0; }
  uint32_t len_src() const { return (mode >> 1) & 3u; }
  uint32_t pos_src() const { return (mode >> 3) & 3u; }
};

Side side_of(const attn_fwd_params* p, bool q) {
  Side s{};
  s.cu = q ? p->cu_seqlens_q : p->cu_seqlens_k;
  s.len = q ? p->seqused_q : p->seqused_k;
  s.start = q ? p->seqstart_q : p->seqstart_k;
  s.S = q ? p->seqlen_q : p->seqlen_k;
  s.total = q ? p->total_q : p->total_k;
  if (p->layout == ATTN_BHSD)
    s.mode = s.len ? ATTN_SEQ_LEN_ARRAY : 0u;
  else if (p->layout == ATTN_THD)
    s.mode = ATTN_SEQ_STACKED | (s.len ? ATTN_SEQ_LEN_ARRAY : ATTN_SEQ_LEN_CUMSUM) | ATTN_SEQ_POS_CUMSUM;
  else
    s.mode = (p->varlen >> (q ? 0 : 8)) & 0xffu;
  return s;
}

// The mode byte and the arrays it names agree: an array is given exactly
// when the mode reads it (under ATTN_BHSD / ATTN_THD seqused stays optional,
// and the mode built above already follows it).
bool side_ok(const Side& s) {
  if (s.mode & ~0x1fu) return false;
  if (s.len_src() > 2 || s.pos_src() > 2) return false;
  if (!s.stacked() && s.pos_src() != 0) return false;
  const bool need_cu = s.len_src() == 1 || s.pos_src() == 1;
  if (need_cu != (s.cu != nullptr)) return false;
  if ((s.len_src() == 2) != (s.len != nullptr)) return false;
  if ((s.pos_src() == 2) != (s.start != nullptr)) return false;
  if (s.S < 0) return false;
  if (s.stacked() && (s.total < 0 || s.total > INT32_MAX)) return false;
  return true;
}

// Byte range [lo, hi) an operand can touch, for the overlap check.
struct Extent {
  uintptr_t lo, hi;
};

// Rows the operand holds per batch entry (padded) or in all (stacked).
int64_t side_rows(const Side& s) { return s.stacked() ? s.total : (int64_t)s.S; }

// A negative stride reaches below the base pointer: each axis adds
// (n - 1) * stride elements to the lower or the upper end.  A tensor with no
// elements touches nothing (its pointer may be NULL).
Extent extent_of(const void* ptr, const int64_t* stride, int64_t nb, int64_t nh, const Side& s, int64_t d,
                 int64_t esz) {
  const uintptr_t base = reinterpret_cast<uintptr_t>(ptr);
  const int64_t nrows = side_rows(s);
  if ((!s.stacked() && nb == 0) || nh == 0 || nrows == 0 || d == 0) return Extent{base, base};
  int64_t below = 0, above = d;  // elements; the last row's head_dim elements
  auto axis = [&](int64_t n, int64_t st) {
    if (n > 1) (st < 0 ? below : above) += (n - 1) * std::llabs(st);
  };
  if (!s.stacked()) axis(nb, stride[0]);
  axis(nh, stride[1]);
  axis(nrows, stride[2]);
  return Extent{base - (uintptr_t)(below * esz), base + (uintptr_t)(above * esz)};
}

bool overlap(Extent a, Extent b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool empty_side(const attn_fwd_params* p, const Side& s) {
  return s.stacked() ? s.total == 0 : (p->batch == 0 || s.S == 0);
}

bool strides_ok(const int64_t* stride, int64_t esz, bool stacked) {
  for (int i = stacked ? 1 : 0; i < 3; ++i)
    if ((stride[i] * esz) % 16 != 0) return false;
  return true;
}

// The 16-bit kernels copy tiles of up to 64 rows with 32-bit byte offsets
// from the tile's lowest row: 63 row strides plus one row must stay below
// 2^31 bytes.
bool tile_span_ok(const int64_t* stride, int64_t esz, int64_t d) {
  const int64_t rs = std::llabs(stride[2]);
  return rs <= ((int64_t)1 << 31) / 64 && (63 * rs + d) * esz < ((int64_t)1 << 31);
}

// ------------------------------------------------------ optional features

bool feat_on(const attn_fwd_params* p) { return p->bias || p->alibi_slopes || p->dropout_p != 0.f; }

// Bias / dbias element ranges: [batch, heads, seqlen_q, seqlen_k] with the
// given strides (0 broadcasts) and unit stride on the last axis.
Extent extent4(const void* ptr, const int64_t* stride, const attn_fwd_params* p, int64_t esz) {
  const uintptr_t base = reinterpret_cast<uintptr_t>(ptr);
  if (!ptr || p->batch == 0 || p->seqlen_q == 0 || p->seqlen_k == 0) return Extent{base, base};
  int64_t below = 0, above = p->seqlen_k;
  const int64_t n[3] = {p->batch, p->heads, p->seqlen_q};
  for (int t = 0; t < 3; ++t)
    if (n[t] > 1) (stride[t] < 0 ? below : above) += (n[t] - 1) * std::llabs(stride[t]);
  return Extent{base - (uintptr_t)(below * esz), base + (uintptr_t)(above * esz)};
}

hipError_t check_feat(const attn_fwd_params* p) {
  if (p->reserved2 != 0) return hipErrorInvalidValue;
  if (!(p->dropout_p >= 0.f && p->dropout_p < 1.f)) return hipErrorInvalidValue;  // also NaN
  if (p->bias && (reinterpret_cast<uintptr_t>(p->bias) % (uintptr_t)elem_bytes(p->dtype)) != 0)
    return hipErrorInvalidValue;
  if (p->alibi_slopes && (reinterpret_cast<uintptr_t>(p->alibi_slopes) & 3u) != 0) return hipErrorInvalidValue;
  return hipSuccess;
}

sdpa::FeatArgs feat_args(const attn_fwd_params* p) {
  sdpa::FeatArgs f{};
  f.bias = p->bias;
  if (p->bias) {
    f.bsb = p->bias_stride[0];
    f.bsh = p->bias_stride[1];
    f.bss = p->bias_stride[2];
  }
  f.alibi = p->alibi_slopes;
  if (p->dropout_p > 0.f) {
    const double t = std::floor((double)p->dropout_p * 4294967296.0);
    f.drop_thresh = (unsigned)std::min(t, 4294967295.0);
    f.drop_scale = (float)(1.0 / (1.0 - (double)p->dropout_p));
    f.seed_lo = (unsigned)p->philox_seed;
    f.seed_hi = (unsigned)(p->philox_seed >> 32);
    f.offset = p->philox_offset;
  }
  return f;
}

hipError_t check_problem(const attn_fwd_params* p) {
  if (!p) return hipErrorInvalidValue;
  if (p->version != ATTN_PARAMS_VERSION || p->reserved0 != 0 || p->reserved1 != 0) return hipErrorInvalidValue;
  if (!dtype_ok(p->dtype)) return hipErrorInvalidValue;
  if (p->layout != ATTN_BHSD && p->layout != ATTN_THD && p->layout != ATTN_VARLEN) return hipErrorInvalidValue;
  if (p->layout != ATTN_VARLEN && (p->varlen != 0 || p->seqstart_q || p->seqstart_k)) return hipErrorInvalidValue;
  if (p->layout == ATTN_VARLEN && (p->varlen >> 16) != 0) return hipErrorInvalidValue;
  if (p->diag != ATTN_TOP_LEFT && p->diag != ATTN_BOTTOM_RIGHT) return hipErrorInvalidValue;
  if (p->heads < 1 || p->head_dim < 1 || p->seqlen_q < 0 || p->seqlen_k < 0) return hipErrorInvalidValue;
  if (!std::isfinite(p->scale)) return hipErrorInvalidValue;
  const Side qs = side_of(p, true), ks = side_of(p, false);
  if (!side_ok(qs) || !side_ok(ks)) return hipErrorInvalidValue;
  if ((p->flags & ~(ATTN_FLAG_LSE_TH | ATTN_FLAG_NO_SPLIT)) != 0 || ((p->flags & ATTN_FLAG_LSE_TH) && !qs.stacked()))
    return hipErrorInvalidValue;
  if (p->batch < ((qs.stacked() || ks.stacked()) ? 1 : 0)) return hipErrorInvalidValue;
  // A pointer may be NULL only when its tensor has no elements.
  const bool no_q = empty_side(p, qs), no_k = empty_side(p, ks);
  if ((!p->q && !no_q) || (!p->o && !no_q) || (!p->lse && !no_q) || (!p->k && !no_k) ||
      (!p->v && !no_k))
    return hipErrorInvalidValue;
  const int64_t esz = elem_bytes(p->dtype);
  if (!aligned16(p->q) || !aligned16(p->k) || !aligned16(p->v) || !aligned16(p->o))
    return hipErrorInvalidValue;
  if (!strides_ok(p->q_stride, esz, qs.stacked()) || !strides_ok(p->k_stride, esz, ks.stacked()) ||
      !strides_ok(p->v_stride, esz, ks.stacked()) || !strides_ok(p->o_stride, esz, qs.stacked()))
    return hipErrorInvalidValue;
  if (check_feat(p) != hipSuccess) return hipErrorInvalidValue;
  if (!head_dim_built(p->head_dim)) return hipErrorNotSupported;
  if (p->dtype != ATTN_FP32 &&
      (!tile_span_ok(p->q_stride, esz, p->head_dim) || !tile_span_ok(p->k_stride, esz, p->head_dim) ||
       !tile_span_ok(p->v_stride, esz, p->head_dim)))
    return hipErrorNotSupported;
  return hipSuccess;
}

// fp32 entries of the LSE and of each workspace array: one per (head,
// query row) of the Q tensor.
int64_t lse_count(const attn_fwd_params* p) {
  return side_of(p, true).stacked() ? (int64_t)p->heads * p->total_q
                                    : (int64_t)p->batch * p->heads * p->seqlen_q;
}

Extent lse_extent(const attn_fwd_params* p) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p->lse);
  return Extent{lo, lo + (uintptr_t)(lse_count(p) * 4)};
}

// Workspace: Delta, then LSE * log2(e), each section rounded up to 256
// bytes.
uint64_t stat_section_bytes(const attn_fwd_params* p) { return ((uint64_t)lse_count(p) * 4 + 255) / 256 * 256; }
uint64_t delta_bytes(const attn_fwd_params* p) { return 2 * stat_section_bytes(p); }

// Split mode of the backward (the launch rules in attn_bwd.hip): taken for
// calls without optional features whose dK/dV or dQ grid (128 keys or
// queries per workgroup) has fewer than 64 workgroups, i.e. would leave at
// least three quarters of a 256-CU GPU idle.  Each grid is repeated to reach
// about 256 workgroups, at most 8 times and at most once per tile of the
// axis it splits; the fp32 partial sums are capped at 8 MiB (fewer copies,
// or no split, beyond that).  Depends on the call only, so the workspace
// size and the launch agree.
struct Split {
  int gkv = 1, gq = 1;
  int64_t rows_q = 0, rows_k = 0;
  uint64_t bytes = 0;  // 0: no split
};

Split split_of(const attn_bwd_params* p) {
  Split sp;
  const attn_fwd_params* f = &p->fwd;
  if (feat_on(f) || p->dbias || (f->flags & ATTN_FLAG_NO_SPLIT)) return sp;
  const Side qs = side_of(f, true), ks = side_of(f, false);
  const int64_t B = f->batch, H = f->heads, D = f->head_dim, Sq = f->seqlen_q, Sk = f->seqlen_k;
  const int64_t nkv = B * H * ((Sk + 127) / 128), nq = B * H * ((Sq + 127) / 128);
  if (nkv == 0 || nq == 0 || (nkv >= 64 && nq >= 64)) return sp;
  const int64_t tile = f->dtype == ATTN_FP32 ? 32 : 64;  // query tile of dK/dV, key tile of dQ
  auto groups = [](int64_t nblk, int64_t ntiles) {
    return (int)std::max<int64_t>(1, std::min<int64_t>({(256 + nblk - 1) / nblk, 8, ntiles}));
  };
  sp.gkv = groups(nkv, (Sq + tile - 1) / tile);
  sp.gq = groups(nq, (Sk + tile - 1) / tile);
  sp.rows_q = qs.stacked() ? f->total_q : B * Sq;
  sp.rows_k = ks.stacked() ? f->total_k : B * Sk;
  auto bytes = [&] { return (uint64_t)(4 * D * H * (2 * sp.gkv * sp.rows_k + sp.gq * sp.rows_q)); };
  constexpr uint64_t kCap = 8u << 20;
  while (bytes() > kCap && (sp.gkv > 1 || sp.gq > 1)) (sp.gkv >= sp.gq ? sp.gkv : sp.gq) -= 1;
  if (bytes() > kCap || (sp.gkv == 1 && sp.gq == 1)) return Split{};
  sp.bytes = (bytes() + 255) / 256 * 256;
  return sp;
}

// Workspace of a backward: Delta and LSE log2(e), then the split partials.
uint64_t bwd_ws_bytes(const attn_bwd_params* p) { return delta_bytes(&p->fwd) + split_of(p).bytes; }

sdpa::SideArgs side_args(const Side& s) {
  sdpa::SideArgs a{};
  a.mode = (int)s.mode;
  a.cu = s.cu;
  a.len = s.len;
  a.start = s.start;
  a.S = s.S;
  return a;
}

sdpa::ProblemArgs problem_args(const attn_fwd_params* p) {
  const Side qs = side_of(p, true), ks = side_of(p, false);
  sdpa::ProblemArgs a{};
  a.qs = side_args(qs);
  a.ks = side_args(ks);
  a.ragged = p->layout != ATTN_BHSD;
  a.B = p->batch;
  a.H = p->heads;
  a.Sq = p->seqlen_q;
  a.Sk = p->seqlen_k;
  a.wl = p->window_left;
  a.wr = p->window_right;
  a.diag = p->diag;
  a.scale = p->scale;
  a.scale_log2 = (float)((double)p->scale * 1.4426950408889634);
  if (qs.stacked()) {
    a.lse_sb = 0;
    a.lse_sh = p->total_q;
  } else {
    a.lse_sb = (int64_t)p->heads * p->seqlen_q;
    a.lse_sh = p->seqlen_q;
  }
  a.olse_sb = a.lse_sb;
  a.olse_sh = a.lse_sh;
  a.olse_ss = 1;
  if (p->flags & ATTN_FLAG_LSE_TH) {  // [total_q, heads]
    a.olse_sh = 1;
    a.olse_ss = p->heads;
  }
  a.total_q = qs.stacked() ? p->total_q : 0;
  return a;
}

Operand operand(const void* ptr, const int64_t* stride, bool stacked) {
  return Operand{ptr, stacked ? 0 : stride[0], stride[1], stride[2]};
}

Extent alibi_extent(const attn_fwd_params* p) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p->alibi_slopes);
  return Extent{lo, p->alibi_slopes ? lo + (uintptr_t)p->heads * 4 : lo};
}

hipError_t check_fwd(const attn_fwd_params* p) {
  hipError_t err = check_problem(p);
  if (err != hipSuccess) return err;
  const Side qs = side_of(p, true), ks = side_of(p, false);
  const int64_t esz = elem_bytes(p->dtype), B = p->batch, H = p->heads, D = p->head_dim;
  const Extent o = extent_of(p->o, p->o_stride, B, H, qs, D, esz);
  const Extent ins[3] = {extent_of(p->q, p->q_stride, B, H, qs, D, esz),
                         extent_of(p->k, p->k_stride, B, H, ks, D, esz),
                         extent_of(p->v, p->v_stride, B, H, ks, D, esz)};
  const Extent l = lse_extent(p);
  for (const Extent& in : ins)
    if (overlap(o, in) || overlap(l, in)) return hipErrorInvalidValue;
  if (overlap(o, l)) return hipErrorInvalidValue;
  const Extent fin[2] = {extent4(p->bias, p->bias_stride, p, esz), alibi_extent(p)};
  for (const Extent& in : fin)
    if (overlap(o, in) || overlap(l, in)) return hipErrorInvalidValue;
  return hipSuccess;
}

// The checks of attn_bwd_check; the workspace is checked only when `ws`
// (the plan query does not look at it, the no-allocation call brings its
// own).
hipError_t check_bwd(const attn_bwd_params* p, bool ws) {
  if (!p) return hipErrorInvalidValue;
  const attn_fwd_params* f = &p->fwd;
  hipError_t err = check_problem(f);
  if (err != hipSuccess) return err;
  const Side qs = side_of(f, true), ks = side_of(f, false);
  const bool no_q = empty_side(f, qs), no_k = empty_side(f, ks);
  if ((!p->dout && !no_q) || (!p->dq && !no_q) || (!p->dk && !no_k) || (!p->dv && !no_k))
    return hipErrorInvalidValue;
  if (ws && (!p->workspace || p->workspace_bytes < bwd_ws_bytes(p) ||
             (reinterpret_cast<uintptr_t>(p->workspace) & 255u) != 0))
    return hipErrorInvalidValue;
  const int64_t esz = elem_bytes(f->dtype);
  if (!aligned16(p->dout) || !aligned16(p->dq) || !aligned16(p->dk) || !aligned16(p->dv))
    return hipErrorInvalidValue;
  if (!strides_ok(p->do_stride, esz, qs.stacked()) || !strides_ok(p->dq_stride, esz, qs.stacked()) ||
      !strides_ok(p->dk_stride, esz, ks.stacked()) || !strides_ok(p->dv_stride, esz, ks.stacked()))
    return hipErrorInvalidValue;
  if (f->dtype != ATTN_FP32 && !tile_span_ok(p->do_stride, esz, f->head_dim)) return hipErrorNotSupported;
  if (p->dbias && (reinterpret_cast<uintptr_t>(p->dbias) & 3u) != 0) return hipErrorInvalidValue;
  const int64_t B = f->batch, H = f->heads, D = f->head_dim;
  const Extent outs[5] = {
      extent_of(p->dq, p->dq_stride, B, H, qs, D, esz), extent_of(p->dk, p->dk_stride, B, H, ks, D, esz),
      extent_of(p->dv, p->dv_stride, B, H, ks, D, esz),
      ws ? Extent{reinterpret_cast<uintptr_t>(p->workspace),
                  reinterpret_cast<uintptr_t>(p->workspace) + (uintptr_t)bwd_ws_bytes(p)}
         : Extent{0, 0},
      extent4(p->dbias, p->dbias_stride, f, 4)};
  const Extent ins[8] = {extent_of(f->q, f->q_stride, B, H, qs, D, esz),
                         extent_of(f->k, f->k_stride, B, H, ks, D, esz),
                         extent_of(f->v, f->v_stride, B, H, ks, D, esz),
                         extent_of(f->o, f->o_stride, B, H, qs, D, esz),
                         extent_of(p->dout, p->do_stride, B, H, qs, D, esz),
                         lse_extent(f),
                         extent4(f->bias, f->bias_stride, f, esz),
                         alibi_extent(f)};
  for (int i = 0; i < 5; ++i) {
    for (const Extent& in : ins)
      if (overlap(outs[i], in)) return hipErrorInvalidValue;
    for (int j = i + 1; j < 5; ++j)
      if (overlap(outs[i], outs[j])) return hipErrorInvalidValue;
  }
  return hipSuccess;
}

sdpa::FwdArgs fwd_args(const attn_fwd_params* p) {
  const bool qst = side_of(p, true).stacked(), kst = side_of(p, false).stacked();
  sdpa::FwdArgs a{};
  a.p = problem_args(p);
  a.q = operand(p->q, p->q_stride, qst);
  a.k = operand(p->k, p->k_stride, kst);
  a.v = operand(p->v, p->v_stride, kst);
  a.o = operand(p->o, p->o_stride, qst);
  a.lse = p->lse;
  a.f = feat_args(p);
  a.feat = feat_on(p);
  return a;
}

// Kernel arguments of a backward whose workspace (Delta, then LSE log2 e)
// starts at `ws`.
sdpa::BwdArgs bwd_args(const attn_bwd_params* p, void* ws) {
  const attn_fwd_params* f = &p->fwd;
  const bool qst = side_of(f, true).stacked(), kst = side_of(f, false).stacked();
  sdpa::BwdArgs a{};
  a.p = problem_args(f);
  a.q = operand(f->q, f->q_stride, qst);
  a.k = operand(f->k, f->k_stride, kst);
  a.v = operand(f->v, f->v_stride, kst);
  a.o = operand(f->o, f->o_stride, qst);
  a.dout = operand(p->dout, p->do_stride, qst);
  a.dq = operand(p->dq, p->dq_stride, qst);
  a.dk = operand(p->dk, p->dk_stride, kst);
  a.dv = operand(p->dv, p->dv_stride, kst);
  a.lse = f->lse;
  a.delta = static_cast<float*>(ws);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(ws) + stat_section_bytes(f));
  a.f = feat_args(f);
  a.f.dbias = p->dbias;
  if (p->dbias) {
    a.f.dsb = p->dbias_stride[0];
    a.f.dsh = p->dbias_stride[1];
    a.f.dss = p->dbias_stride[2];
  }
  a.feat = feat_on(f) || p->dbias != nullptr;
  a.split_kv = a.split_q = 1;
  const Split sp = split_of(p);
  if (sp.bytes) {
    // Integer arithmetic: the plan query passes no workspace.
    a.part = reinterpret_cast<float*>(reinterpret_cast<uintptr_t>(ws) + (uintptr_t)delta_bytes(f));
    a.rows_q = sp.rows_q;
    a.rows_k = sp.rows_k;
    a.split_kv = sp.gkv;
    a.split_q = sp.gq;
  }
  return a;
}

void plan_out(const sdpa::Plan& pl, attn_plan* out) {
  *out = attn_plan{};
  out->count = pl.n;
  for (int i = 0; i < pl.n; ++i) {
    out->kernel[i] = pl.e[i].name;
    out->grid[i] = pl.e[i].grid;
    out->block[i] = pl.e[i].block;
  }
}

}  // namespace

// ------------------------------------------------ no-allocation backward
//
// The workspace of attn_bwd_noalloc: one array per device, in the library's
// code object, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it names a stand-in, not device
// memory): the device address is looked up once per device, with that
// device current, and kept.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array.
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Runs `launch` with the stream's device current, restoring the caller's.
template <typename F>
hipError_t on_stream_device(hipStream_t stream, F launch) {
  int dev = -1, cur = -1;
  hipError_t err = hipStreamGetDevice(stream, &dev);
  if (err != hipSuccess) return err;
  err = hipGetDevice(&cur);
  if (err != hipSuccess) return err;
  if (dev != cur && (err = hipSetDevice(dev)) != hipSuccess) return err;
  const hipError_t lerr = launch();
  if (dev != cur) {
    err = hipSetDevice(cur);
    if (lerr == hipSuccess && err != hipSuccess) return err;
  }
  return lerr;
}

hipError_t bwd_stages(const attn_bwd_params* p, int stages, hipStream_t stream) {
  hipError_t err = check_bwd(p, true);
  if (err != hipSuccess) return err;
  const attn_fwd_params* f = &p->fwd;
  const sdpa::BwdArgs a = bwd_args(p, p->workspace);
  return on_stream_device(
      stream, [&] { return sdpa::launch_bwd(f->dtype, f->head_dim, a, stages, sdpa::Enqueue{stream}); });
}

}  // namespace

extern "C" {

uint32_t attn_params_version(void) { return ATTN_PARAMS_VERSION; }

hipError_t attn_fwd_check(const attn_fwd_params* p_in) {
  attn_fwd_params tmp;
  return check_fwd(fwd_v3(p_in, &tmp));
}

hipError_t attn_fwd(const attn_fwd_params* p_in, hipStream_t stream) {
  attn_fwd_params tmp;
  const attn_fwd_params* p = fwd_v3(p_in, &tmp);
  hipError_t err = check_fwd(p);
  if (err != hipSuccess) return err;
  const sdpa::FwdArgs a = fwd_args(p);
  return on_stream_device(stream, [&] { return sdpa::launch_fwd(p->dtype, p->head_dim, a, sdpa::Enqueue{stream}); });
}

hipError_t attn_fwd_plan(const attn_fwd_params* p_in, hipStream_t stream, attn_plan* plan) {
  if (!plan) return hipErrorInvalidValue;
  attn_fwd_params tmp;
  const attn_fwd_params* p = fwd_v3(p_in, &tmp);
  hipError_t err = check_fwd(p);
  if (err != hipSuccess) return err;
  const sdpa::FwdArgs a = fwd_args(p);
  sdpa::Plan pl{};
  err = on_stream_device(stream, [&] { return sdpa::launch_fwd(p->dtype, p->head_dim, a, sdpa::Record{&pl}); });
  if (err == hipSuccess) plan_out(pl, plan);
  return err;
}

uint64_t attn_bwd_workspace_size(const attn_bwd_params* p_in) {
  attn_bwd_params tmp;
  const attn_bwd_params* p = bwd_v3(p_in, &tmp);
  if (!p || check_problem(&p->fwd) != hipSuccess) return 0;
  return bwd_ws_bytes(p);
}

hipError_t attn_bwd_check(const attn_bwd_params* p_in) {
  attn_bwd_params tmp;
  return check_bwd(bwd_v3(p_in, &tmp), true);
}

hipError_t attn_bwd(const attn_bwd_params* p_in, hipStream_t stream) {
  attn_bwd_params tmp;
  return bwd_stages(bwd_v3(p_in, &tmp), sdpa::kStageAll, stream);
}

hipError_t attn_bwd_preprocess(const attn_bwd_params* p_in, hipStream_t stream) {
  attn_bwd_params tmp;
  return bwd_stages(bwd_v3(p_in, &tmp), sdpa::kStageDelta, stream);
}

hipError_t attn_bwd_dkdv(const attn_bwd_params* p_in, hipStream_t stream) {
  attn_bwd_params tmp;
  return bwd_stages(bwd_v3(p_in, &tmp), sdpa::kStageDkDv, stream);
}

hipError_t attn_bwd_dq(const attn_bwd_params* p_in, hipStream_t stream) {
  attn_bwd_params tmp;
  return bwd_stages(bwd_v3(p_in, &tmp), sdpa::kStageDq, stream);
}

hipError_t attn_bwd_dkdv_dq(const attn_bwd_params* p_in, hipStream_t stream) {
  attn_bwd_params tmp;
  return bwd_stages(bwd_v3(p_in, &tmp), sdpa::kStageDkDv | sdpa::kStageDq, stream);
}

hipError_t attn_bwd_plan(const attn_bwd_params* p_in, uint32_t steps, hipStream_t stream, attn_plan* plan) {
  if (!plan || steps == 0 || (steps & ~(uint32_t)ATTN_BWD_ALL) != 0) return hipErrorInvalidValue;
  attn_bwd_params tmp;
  const attn_bwd_params* p = bwd_v3(p_in, &tmp);
  hipError_t err = check_bwd(p, false);
  if (err != hipSuccess) return err;
  const attn_fwd_params* f = &p->fwd;
  const sdpa::BwdArgs a = bwd_args(p, nullptr);
  sdpa::Plan pl{};
  err = on_stream_device(
      stream, [&] { return sdpa::launch_bwd(f->dtype, f->head_dim, a, (int)steps, sdpa::Record{&pl}); });
  if (err == hipSuccess) plan_out(pl, plan);
  return err;
}

hipError_t attn_bwd_noalloc(const attn_bwd_params* p_in, hipStream_t stream) {
  attn_bwd_params tmp;
  const attn_bwd_params* p = bwd_v3(p_in, &tmp);
  hipError_t err = check_bwd(p, false);
  if (err != hipSuccess) return err;
  const attn_fwd_params* f = &p->fwd;
  if (bwd_ws_bytes(p) > (uint64_t)ATTN_NOALLOC_SCRATCH_BYTES) return hipErrorOutOfMemory;
  return on_stream_device(stream, [&] {
    void* ws = nullptr;
    const hipError_t serr = scratch_ptr(&ws);
    if (serr != hipSuccess) return serr;
    const sdpa::BwdArgs a = bwd_args(p, ws);
    return sdpa::launch_bwd(f->dtype, f->head_dim, a, sdpa::kStageAll, sdpa::Enqueue{stream});
  });
}

}  // extern "C"
