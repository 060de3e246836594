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
// Head dims with kernels built: 32 .. 128 for every dtype, 192 and 256 for
// fp16 / bf16 (whose accumulators and tiles fit there).
bool head_dim_built(int32_t d, int32_t dtype) {
  return d == 32 || d == 48 || d == 64 || d == 80 || d == 96 || d == 128 ||
         (dtype != ATTN_FP32 && (d == 192 || d == 256));
}
int max_dim(int32_t dtype) { return dtype == ATTN_FP32 ? 128 : 256; }

// Smallest built head dim >= d (d <= max_dim(dtype)).
int padded_dim(int d, int32_t dtype) {
  for (int b : {32, 48, 64, 80, 96, 128, 192, 256})
    if (d <= b && head_dim_built(b, dtype)) return b;
  return 0;
}

// Head dim of V, O, dO and dV.
int dim_v(const attn_fwd_params* p) { return p->head_dim_v ? p->head_dim_v : p->head_dim; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool elem_aligned(const void* p, int64_t esz) { return (reinterpret_cast<uintptr_t>(p) % (uintptr_t)esz) == 0; }

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
  if (p->heads < 1 || p->head_dim < 1 || p->head_dim_v < 0 || p->seqlen_q < 0 || p->seqlen_k < 0)
    return hipErrorInvalidValue;
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
  if (!elem_aligned(p->q, esz) || !elem_aligned(p->k, esz) || !elem_aligned(p->v, esz) ||
      !elem_aligned(p->o, esz))
    return hipErrorInvalidValue;
  if (check_feat(p) != hipSuccess) return hipErrorInvalidValue;
  if (p->head_dim > max_dim(p->dtype) || dim_v(p) > max_dim(p->dtype)) return hipErrorNotSupported;
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

// Split mode of the backward (the launch rules in attn_bwd_kernels.hpp): taken for
// calls without optional features whose dK/dV or dQ grid (128 keys or
// queries per workgroup) leaves most of the GPU idle:
//  - fewer than 64 workgroups (at fp16 / bf16 head dims 96 and 128, whose
//    unsplit dK/dV is the producer / consumer kernel the copies cannot use,
//    only up to 16 dK/dV workgroups: 1x4x1000x128 bf16 45 us unsplit
//    against 66 split);
//  - else, over axes of at least 1024 rows (2048 at head dims 96 and 128),
//    fewer than 200 workgroups (65 at head dims 96 and 128): 1x2x8192x64
//    bf16 161 against 320 us unsplit, fp16 1x4x4096x80 121 against 241,
//    fp32 1x8x2048x64 390 against 648, 1x12x2048x64 83 against 95, but
//    1x30x1024x64 (240 workgroups) 62.7 against 58.1 and 2x16x512x64 34.5
//    against 33.7; 1x2x4096x96 103 against 125, 1x4x2048x128 75 against 83,
//    but 1x4x4096x128 (128 workgroups) 201 against 166.
// Each grid is repeated to reach about 256 workgroups, at most 8 times and
// at most once per tile of the axis it splits; the fp32 partial sums are
// capped at 64 MiB (fewer copies, or no split, beyond that).  After the
// partials come the arrival counters, one 4-byte word per dK/dV and per dQ
// block of the finest grid the launch may pick.  Depends on the call only,
// so the workspace size and the launch agree.
struct Split {
  int gkv = 1, gq = 1;
  int64_t rows_q = 0, rows_k = 0;
  int64_t nkv = 0, nq = 0;  // counters: dK/dV and dQ blocks
  uint64_t part_bytes = 0;
  uint64_t bytes = 0;  // 0: no split
};

Split split_of(const attn_bwd_params* p) {
  Split sp;
  const attn_fwd_params* f = &p->fwd;
  if (feat_on(f) || p->dbias || (f->flags & ATTN_FLAG_NO_SPLIT)) return sp;
  const Side qs = side_of(f, true), ks = side_of(f, false);
  const int64_t B = f->batch, H = f->heads, D = f->head_dim, Sq = f->seqlen_q, Sk = f->seqlen_k;
  const int64_t nkv = B * H * ((Sk + 127) / 128), nq = B * H * ((Sq + 127) / 128);
  const bool pc = f->dtype != ATTN_FP32 && (D == 96 || D == 128);  // producer / consumer dK/dV unsplit
  const int64_t lim = pc ? 65 : 200, minlen = pc ? 2048 : 1024;
  if (nkv == 0 || nq == 0 || (nkv >= lim && nq >= lim)) return sp;
  const bool small = pc ? nkv <= 16 : (nkv < 64 || nq < 64);
  if (!small && (Sq < minlen || Sk < minlen)) return sp;
  const int64_t tile = f->dtype == ATTN_FP32 ? 32 : 64;  // query tile of dK/dV, key tile of dQ
  auto groups = [](int64_t nblk, int64_t ntiles) {
    return (int)std::max<int64_t>(1, std::min<int64_t>({(256 + nblk - 1) / nblk, 8, ntiles}));
  };
  sp.gkv = groups(nkv, (Sq + tile - 1) / tile);
  sp.gq = groups(nq, (Sk + tile - 1) / tile);
  sp.rows_q = qs.stacked() ? f->total_q : B * Sq;
  sp.rows_k = ks.stacked() ? f->total_k : B * Sk;
  auto bytes = [&] { return (uint64_t)(4 * D * H * (2 * sp.gkv * sp.rows_k + sp.gq * sp.rows_q)); };
  constexpr uint64_t kCap = 64u << 20;
  while (bytes() > kCap && (sp.gkv > 1 || sp.gq > 1)) (sp.gkv >= sp.gq ? sp.gkv : sp.gq) -= 1;
  if (bytes() > kCap || (sp.gkv == 1 && sp.gq == 1)) return Split{};
  // Counters per block of the finest split grid: 64 rows in fp32 (two-wave
  // workgroups), 128 in fp16 / bf16.
  const int64_t crow = f->dtype == ATTN_FP32 ? 64 : 128;
  sp.nkv = B * H * ((Sk + crow - 1) / crow);
  sp.nq = B * H * ((Sq + crow - 1) / crow);
  sp.part_bytes = (bytes() + 255) / 256 * 256;
  sp.bytes = sp.part_bytes + ((uint64_t)(4 * (sp.nkv + sp.nq)) + 255) / 256 * 256;
  return sp;
}

// Workspace of an in-place backward: Delta and LSE log2(e), then the split
// partials.
uint64_t inner_ws_bytes(const attn_bwd_params* p) { return delta_bytes(&p->fwd) + split_of(p).bytes; }

// ------------------------------------------------------------- repacking

// A call runs in place when its head dims are one built dim and every row
// it addresses is 16-byte aligned (and, for the 16-bit kernels' tile copies,
// within the 2 GiB span); any other call runs on zero-padded copies.
bool in_place_fwd(const attn_fwd_params* p) {
  if (!head_dim_built(p->head_dim, p->dtype) || dim_v(p) != p->head_dim) return false;
  const Side qs = side_of(p, true), ks = side_of(p, false);
  const int64_t esz = elem_bytes(p->dtype), D = p->head_dim;
  if (!aligned16(p->q) || !aligned16(p->k) || !aligned16(p->v) || !aligned16(p->o)) return false;
  if (!strides_ok(p->q_stride, esz, qs.stacked()) || !strides_ok(p->k_stride, esz, ks.stacked()) ||
      !strides_ok(p->v_stride, esz, ks.stacked()) || !strides_ok(p->o_stride, esz, qs.stacked()))
    return false;
  if (p->dtype != ATTN_FP32 && (!tile_span_ok(p->q_stride, esz, D) || !tile_span_ok(p->k_stride, esz, D) ||
                                !tile_span_ok(p->v_stride, esz, D)))
    return false;
  return true;
}

bool in_place_bwd(const attn_bwd_params* p) {
  const attn_fwd_params* f = &p->fwd;
  if (!in_place_fwd(f)) return false;
  const Side qs = side_of(f, true), ks = side_of(f, false);
  const int64_t esz = elem_bytes(f->dtype);
  if (!aligned16(p->dout) || !aligned16(p->dq) || !aligned16(p->dk) || !aligned16(p->dv)) return false;
  if (!strides_ok(p->do_stride, esz, qs.stacked()) || !strides_ok(p->dq_stride, esz, qs.stacked()) ||
      !strides_ok(p->dk_stride, esz, ks.stacked()) || !strides_ok(p->dv_stride, esz, ks.stacked()))
    return false;
  return f->dtype == ATTN_FP32 || tile_span_ok(p->do_stride, esz, f->head_dim);
}

// Padded copies of a repacked call in its workspace: q, k, v, o (and for
// the backward dout, dq, dk, dv), rows of Dp elements, each section
// rounded up to 256 bytes.
enum { kPQ, kPK, kPV, kPO, kPdO, kPdQ, kPdK, kPdV, kPN };
struct Pack {
  int Dp = 0;
  uint64_t off[kPN] = {};
  uint64_t bytes = 0;  // all sections of the call
};

Pack pack_of(const attn_fwd_params* f, bool bwd) {
  Pack pk;
  pk.Dp = padded_dim(std::max(f->head_dim, dim_v(f)), f->dtype);
  const Side qs = side_of(f, true), ks = side_of(f, false);
  const uint64_t esz = (uint64_t)elem_bytes(f->dtype), row = (uint64_t)f->heads * pk.Dp * esz;
  const uint64_t rq = (uint64_t)(qs.stacked() ? f->total_q : (int64_t)f->batch * f->seqlen_q);
  const uint64_t rk = (uint64_t)(ks.stacked() ? f->total_k : (int64_t)f->batch * f->seqlen_k);
  const uint64_t sq = (rq * row + 255) / 256 * 256, sk = (rk * row + 255) / 256 * 256;
  const bool q_side[kPN] = {true, false, false, true, true, true, false, false};
  for (int t = 0; t < (bwd ? kPN : kPdO); ++t) {
    pk.off[t] = pk.bytes;
    pk.bytes += q_side[t] ? sq : sk;
  }
  return pk;
}

// Strides of a padded copy: stacked [rows, heads, Dp], padded [batch,
// heads, seqlen, Dp].
void copy_strides(const Side& s, int H, int Dp, int64_t* st) {
  st[0] = s.stacked() ? 0 : (int64_t)H * s.S * Dp;
  st[1] = s.stacked() ? Dp : (int64_t)s.S * Dp;
  st[2] = s.stacked() ? (int64_t)H * Dp : Dp;
}

// The in-place call on the copies (ws: the workspace's address).
attn_fwd_params inner_fwd(const attn_fwd_params* p, uintptr_t ws, const Pack& pk) {
  attn_fwd_params in = *p;
  const Side qs = side_of(p, true), ks = side_of(p, false);
  in.head_dim = pk.Dp;
  in.head_dim_v = 0;
  in.q = reinterpret_cast<const void*>(ws + pk.off[kPQ]);
  in.k = reinterpret_cast<const void*>(ws + pk.off[kPK]);
  in.v = reinterpret_cast<const void*>(ws + pk.off[kPV]);
  in.o = reinterpret_cast<void*>(ws + pk.off[kPO]);
  copy_strides(qs, p->heads, pk.Dp, in.q_stride);
  copy_strides(ks, p->heads, pk.Dp, in.k_stride);
  copy_strides(ks, p->heads, pk.Dp, in.v_stride);
  copy_strides(qs, p->heads, pk.Dp, in.o_stride);
  // The rest of the caller's workspace, after the copies (the key-split
  // tail's, when large enough).
  in.workspace = ws ? reinterpret_cast<void*>(ws + pk.bytes) : nullptr;
  in.workspace_bytes = p->workspace_bytes > pk.bytes ? p->workspace_bytes - pk.bytes : 0;
  return in;
}

attn_bwd_params inner_bwd(const attn_bwd_params* p, uintptr_t ws, const Pack& pk) {
  attn_bwd_params in = *p;
  in.fwd = inner_fwd(&p->fwd, ws, pk);
  const Side qs = side_of(&p->fwd, true), ks = side_of(&p->fwd, false);
  in.dout = reinterpret_cast<const void*>(ws + pk.off[kPdO]);
  in.dq = reinterpret_cast<void*>(ws + pk.off[kPdQ]);
  in.dk = reinterpret_cast<void*>(ws + pk.off[kPdK]);
  in.dv = reinterpret_cast<void*>(ws + pk.off[kPdV]);
  copy_strides(qs, p->fwd.heads, pk.Dp, in.do_stride);
  copy_strides(qs, p->fwd.heads, pk.Dp, in.dq_stride);
  copy_strides(ks, p->fwd.heads, pk.Dp, in.dk_stride);
  copy_strides(ks, p->fwd.heads, pk.Dp, in.dv_stride);
  in.workspace = reinterpret_cast<void*>(ws + pk.bytes);
  in.workspace_bytes = p->workspace_bytes > pk.bytes ? p->workspace_bytes - pk.bytes : 0;
  return in;
}

// Key-split tail workspace of an in-place forward (the ping-pong launch in
// attn_fwd.hip): fp16 / bf16 at head dims up to 128 without optional
// features or ATTN_FLAG_NO_SPLIT, a band the ping-pong kernel takes (at
// least 1024 keys wide, or unbounded on a side) spanning at least two parts
// of ks_min_keys keys.  Sized for one full round of a 256-CU device, so it
// depends on the call only; whether the launch splits a tail depends on the
// device and the grid.
uint64_t ks_bytes(const attn_fwd_params* p) {
  if (p->dtype == ATTN_FP32 || p->head_dim > 128 || feat_on(p) || (p->flags & ATTN_FLAG_NO_SPLIT)) return 0;
  const bool inf = p->window_left == ATTN_WINDOW_INF || p->window_right == ATTN_WINDOW_INF;
  const int64_t width = (int64_t)p->window_left + p->window_right + 1;
  if (!inf && width < 1024) return 0;
  const int64_t kb = inf ? p->seqlen_k : std::min<int64_t>(p->seqlen_k, width + 255);
  return kb >= 2 * sdpa::ks_min_keys(p->head_dim) ? sdpa::ks_ws_bytes(p->head_dim) : 0;
}

// Workspace a forward needs: a repacked call's padded copies (0 in place).
uint64_t fwd_req_bytes(const attn_fwd_params* p) { return in_place_fwd(p) ? 0 : pack_of(p, false).bytes; }

// Workspace a forward can use: what it needs, then the key-split tail's
// (of the in-place call it runs).
uint64_t fwd_ws_bytes(const attn_fwd_params* p) {
  if (in_place_fwd(p)) return ks_bytes(p);
  const Pack pk = pack_of(p, false);
  const attn_fwd_params in = inner_fwd(p, 0, pk);
  return pk.bytes + ks_bytes(&in);
}

// Workspace bytes the forward uses of a caller's workspace: the key-split
// part only when all of it is there (and 256-byte aligned).
uint64_t fwd_used_bytes(const attn_fwd_params* p) {
  const uint64_t req = fwd_req_bytes(p), all = fwd_ws_bytes(p);
  const bool ok = p->workspace && (reinterpret_cast<uintptr_t>(p->workspace) & 255u) == 0 && p->workspace_bytes >= all;
  return ok ? all : req;
}

uint64_t bwd_ws_bytes(const attn_bwd_params* p) {
  if (in_place_bwd(p)) return inner_ws_bytes(p);
  const Pack pk = pack_of(&p->fwd, true);
  const attn_bwd_params in = inner_bwd(p, 0, pk);
  return pk.bytes + inner_ws_bytes(&in);
}

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

// The checks of attn_fwd_check; the workspace (of a repacked call) is
// checked only when `ws` (the plan query does not look at it).
hipError_t check_fwd(const attn_fwd_params* p, bool ws = true) {
  hipError_t err = check_problem(p);
  if (err != hipSuccess) return err;
  const Side qs = side_of(p, true), ks = side_of(p, false);
  const int64_t esz = elem_bytes(p->dtype), B = p->batch, H = p->heads, D = p->head_dim, DV = dim_v(p);
  const uint64_t req = ws ? fwd_req_bytes(p) : 0;
  if (req && (!p->workspace || p->workspace_bytes < req || (reinterpret_cast<uintptr_t>(p->workspace) & 255u)))
    return hipErrorInvalidValue;
  const uint64_t need = ws ? fwd_used_bytes(p) : 0;
  const uintptr_t w0 = reinterpret_cast<uintptr_t>(p->workspace);
  const Extent outs[3] = {extent_of(p->o, p->o_stride, B, H, qs, DV, esz), lse_extent(p),
                          need ? Extent{w0, w0 + (uintptr_t)need} : Extent{0, 0}};
  const Extent ins[5] = {extent_of(p->q, p->q_stride, B, H, qs, D, esz),
                         extent_of(p->k, p->k_stride, B, H, ks, D, esz),
                         extent_of(p->v, p->v_stride, B, H, ks, DV, esz), extent4(p->bias, p->bias_stride, p, esz),
                         alibi_extent(p)};
  for (int i = 0; i < 3; ++i) {
    for (const Extent& in : ins)
      if (overlap(outs[i], in)) return hipErrorInvalidValue;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return hipErrorInvalidValue;
  }
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
  if (!elem_aligned(p->dout, esz) || !elem_aligned(p->dq, esz) || !elem_aligned(p->dk, esz) ||
      !elem_aligned(p->dv, esz))
    return hipErrorInvalidValue;
  if (p->dbias && (reinterpret_cast<uintptr_t>(p->dbias) & 3u) != 0) return hipErrorInvalidValue;
  const int64_t B = f->batch, H = f->heads, D = f->head_dim, DV = dim_v(f);
  const Extent outs[5] = {
      extent_of(p->dq, p->dq_stride, B, H, qs, D, esz), extent_of(p->dk, p->dk_stride, B, H, ks, D, esz),
      extent_of(p->dv, p->dv_stride, B, H, ks, DV, esz),
      ws ? Extent{reinterpret_cast<uintptr_t>(p->workspace),
                  reinterpret_cast<uintptr_t>(p->workspace) + (uintptr_t)bwd_ws_bytes(p)}
         : Extent{0, 0},
      extent4(p->dbias, p->dbias_stride, f, 4)};
  const Extent ins[8] = {extent_of(f->q, f->q_stride, B, H, qs, D, esz),
                         extent_of(f->k, f->k_stride, B, H, ks, D, esz),
                         extent_of(f->v, f->v_stride, B, H, ks, DV, esz),
                         extent_of(f->o, f->o_stride, B, H, qs, DV, esz),
                         extent_of(p->dout, p->do_stride, B, H, qs, DV, esz),
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
  a.no_split = (p->flags & ATTN_FLAG_NO_SPLIT) ? 1 : 0;
  // The key-split tail's partials, when the caller's workspace holds them
  // (the launch may still not split: it depends on the grid).
  const uint64_t kb = ks_bytes(p);
  const uintptr_t ws = reinterpret_cast<uintptr_t>(p->workspace);
  if (kb && ws && (ws & 255u) == 0 && p->workspace_bytes >= kb) {
    a.ks_part = reinterpret_cast<float*>(ws);
    a.ks_units = (int)sdpa::ks_units(p->head_dim);
  }
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
    a.cnt_kv = reinterpret_cast<unsigned*>(reinterpret_cast<uintptr_t>(a.part) + (uintptr_t)sp.part_bytes);
    a.cnt_q = a.cnt_kv + sp.nkv;
    a.ncnt = sp.nkv + sp.nq;
  }
  return a;
}

// One repack launch: tensors (caller operand, copy operand, side, columns)
// in the given direction.
struct RepackList {
  sdpa::RepackArgs a{};
  void add(const void* caller, const int64_t* cs, const void* copy, const int64_t* ps, const Side& s, int side,
           int cols) {
    sdpa::RepackT& t = a.t[a.n++];
    const Operand user = operand(caller, cs, s.stacked()), pad = operand(copy, ps, s.stacked());
    t.src = a.out ? pad : user;
    t.dst = a.out ? user : pad;
    t.side = side;
    t.cols = cols;
  }
};

RepackList repack_list(const attn_fwd_params* p, int Dp, int out) {
  RepackList l;
  l.a.p = problem_args(p);
  l.a.out = out;
  l.a.pad = Dp;
  l.a.esz = (int)elem_bytes(p->dtype);
  return l;
}

// The forward of any call on executor ex: in place, or repacked through
// the workspace at ws (an address; the plan passes the caller's, maybe 0).
template <class Ex>
hipError_t run_fwd(const attn_fwd_params* p, uintptr_t ws, const Ex& ex) {
  if (in_place_fwd(p)) return sdpa::launch_fwd(p->dtype, p->head_dim, fwd_args(p), ex);
  const Pack pk = pack_of(p, false);
  const attn_fwd_params in = inner_fwd(p, ws, pk);
  const Side qs = side_of(p, true), ks = side_of(p, false);
  RepackList ci = repack_list(p, pk.Dp, 0);
  ci.add(p->q, p->q_stride, in.q, in.q_stride, qs, 0, p->head_dim);
  ci.add(p->k, p->k_stride, in.k, in.k_stride, ks, 1, p->head_dim);
  ci.add(p->v, p->v_stride, in.v, in.v_stride, ks, 1, dim_v(p));
  hipError_t err = sdpa::launch_repack(ci.a, ex);
  if (err == hipSuccess) err = sdpa::launch_fwd(in.dtype, in.head_dim, fwd_args(&in), ex);
  if (err != hipSuccess) return err;
  RepackList co = repack_list(p, pk.Dp, 1);
  co.add(p->o, p->o_stride, in.o, in.o_stride, qs, 0, dim_v(p));
  return sdpa::launch_repack(co.a, ex);
}

// The backward steps `stages` of any call (workspace at ws).  Repacked: the
// Delta step makes the input copies first; the dK/dV and dQ steps copy
// their outputs back after.
template <class Ex>
hipError_t run_bwd(const attn_bwd_params* p, uintptr_t ws, int stages, const Ex& ex) {
  const attn_fwd_params* f = &p->fwd;
  if (in_place_bwd(p))
    return sdpa::launch_bwd(f->dtype, f->head_dim, bwd_args(p, reinterpret_cast<void*>(ws)), stages, ex);
  const Pack pk = pack_of(f, true);
  const attn_bwd_params in = inner_bwd(p, ws, pk);
  const Side qs = side_of(f, true), ks = side_of(f, false);
  const int D = f->head_dim, DV = dim_v(f);
  hipError_t err = hipSuccess;
  if (stages & sdpa::kStageDelta) {
    RepackList ci = repack_list(f, pk.Dp, 0);
    ci.add(f->q, f->q_stride, in.fwd.q, in.fwd.q_stride, qs, 0, D);
    ci.add(f->k, f->k_stride, in.fwd.k, in.fwd.k_stride, ks, 1, D);
    ci.add(f->v, f->v_stride, in.fwd.v, in.fwd.v_stride, ks, 1, DV);
    ci.add(f->o, f->o_stride, in.fwd.o, in.fwd.o_stride, qs, 0, DV);
    ci.add(p->dout, p->do_stride, in.dout, in.do_stride, qs, 0, DV);
    err = sdpa::launch_repack(ci.a, ex);
  }
  if (err == hipSuccess) err = sdpa::launch_bwd(f->dtype, pk.Dp, bwd_args(&in, in.workspace), stages, ex);
  if (err != hipSuccess) return err;
  RepackList co = repack_list(f, pk.Dp, 1);
  if (stages & sdpa::kStageDq) co.add(p->dq, p->dq_stride, in.dq, in.dq_stride, qs, 0, D);
  if (stages & sdpa::kStageDkDv) {
    co.add(p->dk, p->dk_stride, in.dk, in.dk_stride, ks, 1, D);
    co.add(p->dv, p->dv_stride, in.dv, in.dv_stride, ks, 1, DV);
  }
  return sdpa::launch_repack(co.a, ex);
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
  const uintptr_t ws = reinterpret_cast<uintptr_t>(p->workspace);
  return on_stream_device(stream, [&] { return run_bwd(p, ws, stages, sdpa::Enqueue{stream}); });
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
  const uintptr_t ws = reinterpret_cast<uintptr_t>(p->workspace);
  return on_stream_device(stream, [&] { return run_fwd(p, ws, sdpa::Enqueue{stream}); });
}

uint64_t attn_fwd_workspace_size(const attn_fwd_params* p_in) {
  attn_fwd_params tmp;
  const attn_fwd_params* p = fwd_v3(p_in, &tmp);
  if (!p || check_problem(p) != hipSuccess) return 0;
  return fwd_ws_bytes(p);
}

hipError_t attn_fwd_plan(const attn_fwd_params* p_in, hipStream_t stream, attn_plan* plan) {
  if (!plan) return hipErrorInvalidValue;
  attn_fwd_params tmp;
  const attn_fwd_params* p = fwd_v3(p_in, &tmp);
  hipError_t err = check_fwd(p, false);
  if (err != hipSuccess) return err;
  const uintptr_t ws = reinterpret_cast<uintptr_t>(p->workspace);
  sdpa::Plan pl{};
  err = on_stream_device(stream, [&] { return run_fwd(p, ws, sdpa::Record{&pl}); });
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
  sdpa::Plan pl{};
  err = on_stream_device(stream, [&] { return run_bwd(p, 0, (int)steps, sdpa::Record{&pl}); });
  if (err == hipSuccess) plan_out(pl, plan);
  return err;
}

hipError_t attn_bwd_noalloc(const attn_bwd_params* p_in, hipStream_t stream) {
  attn_bwd_params tmp;
  const attn_bwd_params* p = bwd_v3(p_in, &tmp);
  hipError_t err = check_bwd(p, false);
  if (err != hipSuccess) return err;
  uint64_t need = bwd_ws_bytes(p);
  attn_bwd_params unsplit;
  if (need > (uint64_t)ATTN_NOALLOC_SCRATCH_BYTES && !(p->fwd.flags & ATTN_FLAG_NO_SPLIT)) {
    // The split mode's partials do not fit the array: the call without it.
    unsplit = *p;
    unsplit.fwd.flags |= ATTN_FLAG_NO_SPLIT;
    p = &unsplit;
    need = bwd_ws_bytes(p);
  }
  if (need > (uint64_t)ATTN_NOALLOC_SCRATCH_BYTES) return hipErrorOutOfMemory;
  return on_stream_device(stream, [&] {
    void* ws = nullptr;
    const hipError_t serr = scratch_ptr(&ws);
    if (serr != hipSuccess) return serr;
    attn_bwd_params q = *p;  // the scratch array as the workspace
    q.workspace = ws;
    q.workspace_bytes = need;
    return run_bwd(&q, reinterpret_cast<uintptr_t>(ws), sdpa::kStageAll, sdpa::Enqueue{stream});
  });
}

}  // extern "C"
