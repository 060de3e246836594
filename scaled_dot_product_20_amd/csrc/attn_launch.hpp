// attn_launch.hpp - kernel argument blocks and the launchers the C ABI calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

// Element strides of one operand: base + b*sb + h*sh + row*ss + d.  For the
// packed layout sb is 0 and `row` is the packed row (cu_seqlens[b] + i).
struct Operand {
  const void* ptr;
  long long sb, sh, ss;
};

struct ProblemArgs {
  const int* cu_q;   // packed layout only
  const int* cu_k;
  int varlen;
  int B, H;
  int Sq, Sk;        // dense: exact lengths; packed: maxima
  int wl, wr, diag;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  long long lse_sb, lse_sh;  // workspace (Delta, LSE log2 e): base + b*lse_sb + h*lse_sh + row
  long long olse_sb, olse_sh, olse_ss;  // the caller's LSE: + b*sb + h*sh + row*ss
  long long total_q;         // packed layout: rows of Q
  const int* used_q;         // optional: rows of sequence b in use (seqused_q)
  const int* used_k;
};

// Rows of sequence b: Q rows q0 .. q0+sq-1 and K rows k0 .. k0+sk-1 (packed:
// its cu_seqlens range; dense: all rows), cut to the used rows when the
// caller gives seqused arrays.  Every kernel computes on these rows only.
// (A template so that P may also sit in the kernel-argument segment.)
template <class PA>
__device__ __forceinline__ void seq_rows(PA& P, int b, long long& q0, int& sq, long long& k0, int& sk) {
  q0 = 0;
  k0 = 0;
  sq = P.Sq;
  sk = P.Sk;
  if (P.varlen) {
    q0 = P.cu_q[b];
    sq = P.cu_q[b + 1] - (int)q0;
    k0 = P.cu_k[b];
    sk = P.cu_k[b + 1] - (int)k0;
  }
  if (P.used_q) sq = max(0, min(sq, P.used_q[b]));
  if (P.used_k) sk = max(0, min(sk, P.used_k[b]));
}

struct FwdArgs {
  ProblemArgs p;
  Operand q, k, v, o;
  float* lse;
};

struct BwdArgs {
  ProblemArgs p;
  Operand q, k, v, o, dout, dq, dk, dv;
  const float* lse;
  float* delta;  // workspace: Delta_i = sum_d dO_id O_id (written by the preprocess)
  float* lse2;   // workspace: LSE_i * log2(e) (written by the preprocess)
};

// Steps of the backward, as a bit mask of `stages`; they run in this order.
constexpr int kStageDelta = 1, kStageDkDv = 2, kStageDq = 4, kStageAll = 7;

// A band unbounded on one side or at least 1024 keys wide.  Kernels with
// 256-row workgroups walk every key tile of their rows in lock step, so a
// narrower band goes to kernels with smaller workgroups, which visit fewer
// tiles outside each wave's band.
inline bool wide_window(const ProblemArgs& p) {
  constexpr int kInf = 2147483647;
  if (p.wl == kInf || p.wr == kInf) return true;
  return (long long)p.wl + (long long)p.wr + 1 >= 1024;
}

// Compute units of the current device (0 if unknown).  The library keeps
// one value per device, read from the runtime on first use and never changed
// after (racing first readers store the same value); the split forward tail
// and the fused dK/dV + dQ grid are chosen from it.
inline int device_cu_count() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    __atomic_store_n(&cache[dev], v, __ATOMIC_RELAXED);
  }
  return v;
}

// The launches of one call, as the C ABI's plan queries report them.
constexpr int kPlanMax = 4;
struct PlanEntry {
  const char* name;  // kernel function name (without template arguments)
  unsigned grid, block;
};
struct Plan {
  int n;
  PlanEntry e[kPlanMax];
};

// A launcher decides which kernels a call runs and hands each launch to an
// executor: Enqueue launches it on a stream, Record only lists it.  Both go
// through the same decision code, so a plan lists exactly what the call
// enqueues.  Kernel arguments are passed by value and referenced only for
// the duration of the launch call.
struct Enqueue {
  hipStream_t stream;
  template <class... A>
  hipError_t operator()(const void* fn, const char*, unsigned grid, unsigned block, A... args) const {
    void* ptrs[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(fn, dim3(grid), dim3(block), ptrs, 0, stream);
  }
};
struct Record {
  Plan* plan;
  template <class... A>
  hipError_t operator()(const void*, const char* name, unsigned grid, unsigned block, A...) const {
    if (plan->n >= kPlanMax) return hipErrorUnknown;
    plan->e[plan->n++] = PlanEntry{name, grid, block};
    return hipSuccess;
  }
};

// dtype codes follow the C ABI: 0 fp32, 1 fp16, 2 bf16.
hipError_t launch_fwd(int dtype, int head_dim, const FwdArgs& a, const Enqueue& ex);
hipError_t launch_fwd(int dtype, int head_dim, const FwdArgs& a, const Record& ex);
hipError_t launch_bwd(int dtype, int head_dim, const BwdArgs& a, int stages, const Enqueue& ex);
hipError_t launch_bwd(int dtype, int head_dim, const BwdArgs& a, int stages, const Record& ex);
// Rows past the used rows of every sequence (seqused_q for side 0, seqused_k
// for side 1): zeros in t0 and t1 (null pointers skipped) and, when lse is
// given, LSE = +inf.  Rows are row_bytes long (a multiple of 16).
template <class Ex>
hipError_t launch_pad_rows(const ProblemArgs& p, Operand t0, Operand t1, float* lse, int side, int row_bytes,
                           int esz, const Ex& ex);

}  // namespace sdpa
