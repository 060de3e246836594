// attn_api.cpp - the C ABI declared in include/attn.h: validation, argument
// marshalling into kernel argument blocks, and the device taken from the
// stream.  Nothing is allocated per call and nothing is printed.  The
// library's only state is written once per device and never changed after:
// the compute-unit count the launchers read (attn_launch.hpp), and the device
// address of the no-allocation backward's scratch array (below).
#include "attn.h"

#include <cmath>
#include <cstdint>
#include <mutex>

#include "attn_launch.hpp"

namespace {

using sdpa::Operand;

bool dtype_ok(int32_t d) { return d == ATTN_FP32 || d == ATTN_FP16 || d == ATTN_BF16; }
int64_t elem_bytes(int32_t d) { return d == ATTN_FP32 ? 4 : 2; }
bool head_dim_built(int32_t d) { return d == 32 || d == 48 || d == 64 || d == 80 || d == 96 || d == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte range [lo, hi) an operand can touch, for the overlap check.
struct Extent {
  uintptr_t lo, hi;
};

// A negative stride reaches below the base pointer: each axis adds
// (n - 1) * stride elements to the lower or the upper end.  A tensor with no
// elements touches nothing (its pointer may be NULL).
Extent extent_of(const void* ptr, const int64_t* stride, int64_t nb, int64_t nh, int64_t nrows,
                 int64_t d, int64_t esz, bool packed) {
  const uintptr_t base = reinterpret_cast<uintptr_t>(ptr);
  if ((!packed && nb == 0) || nh == 0 || nrows == 0 || d == 0) return Extent{base, base};
  int64_t below = 0, above = d;  // elements; the last row's head_dim elements
  auto axis = [&](int64_t n, int64_t s) {
    if (n > 1) (s < 0 ? below : above) += (n - 1) * std::llabs(s);
  };
  if (!packed) axis(nb, stride[0]);
  axis(nh, stride[1]);
  axis(nrows, stride[2]);
  return Extent{base - (uintptr_t)(below * esz), base + (uintptr_t)(above * esz)};
}

bool overlap(Extent a, Extent b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool strides_ok(const int64_t* stride, int64_t esz, bool packed) {
  for (int i = packed ? 1 : 0; i < 3; ++i)
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

// Rows of the Q side / K side of the whole tensor.
int64_t q_rows(const attn_fwd_params* p) {
  return p->layout == ATTN_THD ? p->total_q : (int64_t)p->seqlen_q;
}
int64_t k_rows(const attn_fwd_params* p) {
  return p->layout == ATTN_THD ? p->total_k : (int64_t)p->seqlen_k;
}

hipError_t check_problem(const attn_fwd_params* p) {
  if (!p) return hipErrorInvalidValue;
  if (p->version != ATTN_PARAMS_VERSION || (p->flags & ~ATTN_FLAG_LSE_TH) != 0 || p->reserved0 != 0 ||
      ((p->flags & ATTN_FLAG_LSE_TH) && p->layout != ATTN_THD))
    return hipErrorInvalidValue;
  if (!dtype_ok(p->dtype)) return hipErrorInvalidValue;
  if (p->layout != ATTN_BHSD && p->layout != ATTN_THD) return hipErrorInvalidValue;
  if (p->diag != ATTN_TOP_LEFT && p->diag != ATTN_BOTTOM_RIGHT) return hipErrorInvalidValue;
  if (p->heads < 1 || p->head_dim < 1 || p->seqlen_q < 0 || p->seqlen_k < 0)
    return hipErrorInvalidValue;
  if (!std::isfinite(p->scale)) return hipErrorInvalidValue;
  if (p->layout == ATTN_BHSD) {
    if (p->batch < 0) return hipErrorInvalidValue;
    if (p->cu_seqlens_q || p->cu_seqlens_k) return hipErrorInvalidValue;
  } else {
    if (p->batch < 1) return hipErrorInvalidValue;
    if (!p->cu_seqlens_q || !p->cu_seqlens_k) return hipErrorInvalidValue;
    if (p->total_q < 0 || p->total_k < 0 || p->total_q > INT32_MAX || p->total_k > INT32_MAX)
      return hipErrorInvalidValue;
  }
  // A pointer may be NULL only when its tensor has no elements.
  const int64_t nb = p->layout == ATTN_THD ? 1 : p->batch;
  const bool no_q = nb == 0 || q_rows(p) == 0, no_k = nb == 0 || k_rows(p) == 0;
  if ((!p->q && !no_q) || (!p->o && !no_q) || (!p->lse && !no_q) || (!p->k && !no_k) ||
      (!p->v && !no_k))
    return hipErrorInvalidValue;
  const int64_t esz = elem_bytes(p->dtype);
  const bool packed = p->layout == ATTN_THD;
  if (!aligned16(p->q) || !aligned16(p->k) || !aligned16(p->v) || !aligned16(p->o))
    return hipErrorInvalidValue;
  if (!strides_ok(p->q_stride, esz, packed) || !strides_ok(p->k_stride, esz, packed) ||
      !strides_ok(p->v_stride, esz, packed) || !strides_ok(p->o_stride, esz, packed))
    return hipErrorInvalidValue;
  if (!head_dim_built(p->head_dim)) return hipErrorNotSupported;
  if (p->dtype != ATTN_FP32 &&
      (!tile_span_ok(p->q_stride, esz, p->head_dim) || !tile_span_ok(p->k_stride, esz, p->head_dim) ||
       !tile_span_ok(p->v_stride, esz, p->head_dim)))
    return hipErrorNotSupported;
  return hipSuccess;
}

Extent lse_extent(const attn_fwd_params* p) {
  const int64_t n = p->layout == ATTN_THD ? (int64_t)p->heads * p->total_q
                                          : (int64_t)p->batch * p->heads * p->seqlen_q;
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p->lse);
  return Extent{lo, lo + (uintptr_t)(n * 4)};
}

// Workspace: Delta, then LSE * log2(e), one fp32 per (head, query row)
// each, each section rounded up to 256 bytes.
uint64_t stat_section_bytes(const attn_fwd_params* p) {
  const int64_t n = p->layout == ATTN_THD ? (int64_t)p->heads * p->total_q
                                          : (int64_t)p->batch * p->heads * p->seqlen_q;
  return ((uint64_t)n * 4 + 255) / 256 * 256;
}
uint64_t delta_bytes(const attn_fwd_params* p) { return 2 * stat_section_bytes(p); }

sdpa::ProblemArgs problem_args(const attn_fwd_params* p) {
  sdpa::ProblemArgs a{};
  a.varlen = p->layout == ATTN_THD;
  a.cu_q = a.varlen ? p->cu_seqlens_q : nullptr;
  a.cu_k = a.varlen ? p->cu_seqlens_k : nullptr;
  a.B = p->batch;
  a.H = p->heads;
  a.Sq = p->seqlen_q;
  a.Sk = p->seqlen_k;
  a.wl = p->window_left;
  a.wr = p->window_right;
  a.diag = p->diag;
  a.scale = p->scale;
  a.scale_log2 = (float)((double)p->scale * 1.4426950408889634);
  if (a.varlen) {
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
  a.total_q = a.varlen ? p->total_q : 0;
  a.used_q = p->seqused_q;
  a.used_k = p->seqused_k;
  return a;
}

Operand operand(const void* ptr, const int64_t* stride, bool packed) {
  return Operand{ptr, packed ? 0 : stride[0], stride[1], stride[2]};
}

// The checks of attn_bwd_check; the workspace is checked only when `ws`
// (the plan query does not look at it).
hipError_t check_bwd(const attn_bwd_params* p, bool ws) {
  if (!p) return hipErrorInvalidValue;
  const attn_fwd_params* f = &p->fwd;
  hipError_t err = check_problem(f);
  if (err != hipSuccess) return err;
  const int64_t nb = f->layout == ATTN_THD ? 1 : f->batch;
  const bool no_q = nb == 0 || q_rows(f) == 0, no_k = nb == 0 || k_rows(f) == 0;
  if ((!p->dout && !no_q) || (!p->dq && !no_q) || (!p->dk && !no_k) || (!p->dv && !no_k))
    return hipErrorInvalidValue;
  if (ws && (!p->workspace || p->workspace_bytes < delta_bytes(f) ||
             (reinterpret_cast<uintptr_t>(p->workspace) & 255u) != 0))
    return hipErrorInvalidValue;
  const bool packed = f->layout == ATTN_THD;
  const int64_t esz = elem_bytes(f->dtype);
  if (!aligned16(p->dout) || !aligned16(p->dq) || !aligned16(p->dk) || !aligned16(p->dv))
    return hipErrorInvalidValue;
  if (!strides_ok(p->do_stride, esz, packed) || !strides_ok(p->dq_stride, esz, packed) ||
      !strides_ok(p->dk_stride, esz, packed) || !strides_ok(p->dv_stride, esz, packed))
    return hipErrorInvalidValue;
  if (f->dtype != ATTN_FP32 && !tile_span_ok(p->do_stride, esz, f->head_dim)) return hipErrorNotSupported;
  const int64_t B = packed ? 1 : f->batch, H = f->heads, D = f->head_dim;
  const Extent outs[4] = {
      extent_of(p->dq, p->dq_stride, B, H, q_rows(f), D, esz, packed),
      extent_of(p->dk, p->dk_stride, B, H, k_rows(f), D, esz, packed),
      extent_of(p->dv, p->dv_stride, B, H, k_rows(f), D, esz, packed),
      ws ? Extent{reinterpret_cast<uintptr_t>(p->workspace),
                  reinterpret_cast<uintptr_t>(p->workspace) + (uintptr_t)delta_bytes(f)}
         : Extent{0, 0}};
  const Extent ins[6] = {
      extent_of(f->q, f->q_stride, B, H, q_rows(f), D, esz, packed),
      extent_of(f->k, f->k_stride, B, H, k_rows(f), D, esz, packed),
      extent_of(f->v, f->v_stride, B, H, k_rows(f), D, esz, packed),
      extent_of(f->o, f->o_stride, B, H, q_rows(f), D, esz, packed),
      extent_of(p->dout, p->do_stride, B, H, q_rows(f), D, esz, packed),
      lse_extent(f)};
  for (int i = 0; i < 4; ++i) {
    for (const Extent& in : ins)
      if (overlap(outs[i], in)) return hipErrorInvalidValue;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return hipErrorInvalidValue;
  }
  return hipSuccess;
}

sdpa::FwdArgs fwd_args(const attn_fwd_params* p) {
  const bool packed = p->layout == ATTN_THD;
  sdpa::FwdArgs a{};
  a.p = problem_args(p);
  a.q = operand(p->q, p->q_stride, packed);
  a.k = operand(p->k, p->k_stride, packed);
  a.v = operand(p->v, p->v_stride, packed);
  a.o = operand(p->o, p->o_stride, packed);
  a.lse = p->lse;
  return a;
}

// Kernel arguments of a backward whose workspace (Delta, then LSE log2 e)
// starts at `ws`.
sdpa::BwdArgs bwd_args(const attn_bwd_params* p, void* ws) {
  const attn_fwd_params* f = &p->fwd;
  const bool packed = f->layout == ATTN_THD;
  sdpa::BwdArgs a{};
  a.p = problem_args(f);
  a.q = operand(f->q, f->q_stride, packed);
  a.k = operand(f->k, f->k_stride, packed);
  a.v = operand(f->v, f->v_stride, packed);
  a.o = operand(f->o, f->o_stride, packed);
  a.dout = operand(p->dout, p->do_stride, packed);
  a.dq = operand(p->dq, p->dq_stride, packed);
  a.dk = operand(p->dk, p->dk_stride, packed);
  a.dv = operand(p->dv, p->dv_stride, packed);
  a.lse = f->lse;
  a.delta = static_cast<float*>(ws);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(ws) + stat_section_bytes(f));
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

}  // namespace

extern "C" {

uint32_t attn_params_version(void) { return ATTN_PARAMS_VERSION; }

hipError_t attn_fwd_check(const attn_fwd_params* p) {
  hipError_t err = check_problem(p);
  if (err != hipSuccess) return err;
  const bool packed = p->layout == ATTN_THD;
  const int64_t esz = elem_bytes(p->dtype);
  const int64_t B = packed ? 1 : p->batch;
  const Extent o = extent_of(p->o, p->o_stride, B, p->heads, q_rows(p), p->head_dim, esz, packed);
  const Extent ins[3] = {
      extent_of(p->q, p->q_stride, B, p->heads, q_rows(p), p->head_dim, esz, packed),
      extent_of(p->k, p->k_stride, B, p->heads, k_rows(p), p->head_dim, esz, packed),
      extent_of(p->v, p->v_stride, B, p->heads, k_rows(p), p->head_dim, esz, packed)};
  const Extent l = lse_extent(p);
  for (const Extent& in : ins)
    if (overlap(o, in) || overlap(l, in)) return hipErrorInvalidValue;
  if (overlap(o, l)) return hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t attn_fwd(const attn_fwd_params* p, hipStream_t stream) {
  hipError_t err = attn_fwd_check(p);
  if (err != hipSuccess) return err;
  const sdpa::FwdArgs a = fwd_args(p);
  return on_stream_device(stream, [&] { return sdpa::launch_fwd(p->dtype, p->head_dim, a, sdpa::Enqueue{stream}); });
}

hipError_t attn_fwd_plan(const attn_fwd_params* p, hipStream_t stream, attn_plan* plan) {
  if (!plan) return hipErrorInvalidValue;
  hipError_t err = attn_fwd_check(p);
  if (err != hipSuccess) return err;
  const sdpa::FwdArgs a = fwd_args(p);
  sdpa::Plan pl{};
  err = on_stream_device(stream, [&] { return sdpa::launch_fwd(p->dtype, p->head_dim, a, sdpa::Record{&pl}); });
  if (err == hipSuccess) plan_out(pl, plan);
  return err;
}

uint64_t attn_bwd_workspace_size(const attn_bwd_params* p) {
  if (!p || check_problem(&p->fwd) != hipSuccess) return 0;
  return delta_bytes(&p->fwd);
}

hipError_t attn_bwd_check(const attn_bwd_params* p) { return check_bwd(p, true); }

}  // extern "C"

namespace {

hipError_t bwd_stages(const attn_bwd_params* p, int stages, hipStream_t stream) {
  hipError_t err = attn_bwd_check(p);
  if (err != hipSuccess) return err;
  const attn_fwd_params* f = &p->fwd;
  const sdpa::BwdArgs a = bwd_args(p, p->workspace);
  return on_stream_device(
      stream, [&] { return sdpa::launch_bwd(f->dtype, f->head_dim, a, stages, sdpa::Enqueue{stream}); });
}

}  // namespace

extern "C" {

hipError_t attn_bwd(const attn_bwd_params* p, hipStream_t stream) {
  return bwd_stages(p, sdpa::kStageAll, stream);
}

hipError_t attn_bwd_preprocess(const attn_bwd_params* p, hipStream_t stream) {
  return bwd_stages(p, sdpa::kStageDelta, stream);
}

hipError_t attn_bwd_dkdv(const attn_bwd_params* p, hipStream_t stream) {
  return bwd_stages(p, sdpa::kStageDkDv, stream);
}

hipError_t attn_bwd_dq(const attn_bwd_params* p, hipStream_t stream) {
  return bwd_stages(p, sdpa::kStageDq, stream);
}

hipError_t attn_bwd_dkdv_dq(const attn_bwd_params* p, hipStream_t stream) {
  return bwd_stages(p, sdpa::kStageDkDv | sdpa::kStageDq, stream);
}

hipError_t attn_bwd_plan(const attn_bwd_params* p, uint32_t steps, hipStream_t stream, attn_plan* plan) {
  if (!plan || steps == 0 || (steps & ~(uint32_t)ATTN_BWD_ALL) != 0) return hipErrorInvalidValue;
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

hipError_t attn_bwd_noalloc(const attn_bwd_params* p, hipStream_t stream) {
  hipError_t err = check_bwd(p, false);
  if (err != hipSuccess) return err;
  const attn_fwd_params* f = &p->fwd;
  if (delta_bytes(f) > (uint64_t)ATTN_NOALLOC_SCRATCH_BYTES) return hipErrorOutOfMemory;
  return on_stream_device(stream, [&] {
    void* ws = nullptr;
    const hipError_t serr = scratch_ptr(&ws);
    if (serr != hipSuccess) return serr;
    const sdpa::BwdArgs a = bwd_args(p, ws);
    return sdpa::launch_bwd(f->dtype, f->head_dim, a, sdpa::kStageAll, sdpa::Enqueue{stream});
  });
}

}  // extern "C"
