// attn_launch.hpp - kernel argument blocks and the launchers the C ABI calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_feat.hpp"

namespace sdpa {

// Element strides of one operand: base + b*sb + h*sh + row*ss + d.  For the
// packed layout sb is 0 and `row` is the packed row (cu_seqlens[b] + i).
struct Operand {
  const void* ptr;
  long long sb, sh, ss;
};

// Addressing of one side (Q or K) of the problem: the mode byte of the C
// ABI (bit 0 stacked; bits 2:1 length source uniform / cumulative / array;
// bits 4:3 start source uniform / cumulative / array) and its arrays.
struct SideArgs {
  const int* cu;     // cumulative lengths [B+1] (length or start source 1)
  const int* len;    // lengths [B] (length source 2)
  const int* start;  // start rows [B] (start source 2)
  int mode;
  int S;             // uniform length and room; the largest length otherwise
};
constexpr int kSeqStacked = 1;
__host__ __device__ __forceinline__ int side_len_src(int mode) { return (mode >> 1) & 3; }
__host__ __device__ __forceinline__ int side_pos_src(int mode) { return (mode >> 3) & 3; }
// Whether a sequence of this side can have fewer rows than its room (the
// rows in between are written as masked rows).
__host__ __device__ __forceinline__ bool side_may_pad(int mode) {
  const int ls = side_len_src(mode), ps = side_pos_src(mode);
  if (!(mode & kSeqStacked) || ps == 0) return ls != 0;
  return ps == 1 && ls != 1;
}

// Rows of sequence b on one side: start row r0 (stacked tensors; 0 for a
// padded side, whose sequences start at b * stride[0]), length n, and room
// (rows the sequence owns; -1 when not known).  Lengths are clamped to
// [0, room], or to [0, S] when the room is not known.
struct SideRows {
  long long r0;
  int n, room;
};
template <class SA>
__device__ __forceinline__ SideRows side_rows(const SA& s, int b) {
  const int ls = side_len_src(s.mode), ps = side_pos_src(s.mode);
  SideRows r{0, s.S, s.S};
  if (s.mode & kSeqStacked) {
    if (ps == 0) {
      r.r0 = (long long)b * s.S;
    } else if (ps == 1) {
      r.r0 = s.cu[b];
      r.room = s.cu[b + 1] - s.cu[b];
    } else {
      r.r0 = s.start[b];
      r.room = -1;
    }
  }
  const int cap = r.room >= 0 ? r.room : s.S;
  int n = s.S;
  if (ls == 1) n = s.cu[b + 1] - s.cu[b];
  if (ls == 2) n = s.len[b];
  r.n = max(0, min(cap, n));
  return r;
}

struct ProblemArgs {
  SideArgs qs, ks;
  int ragged;        // sequences may differ in length: blocks run (sequence, head) fastest
  int B, H;
  int Sq, Sk;        // the sides' uniform lengths / rooms, else the largest lengths
  int wl, wr, diag;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  long long lse_sb, lse_sh;  // workspace (Delta, LSE log2 e): base + b*lse_sb + h*lse_sh + row
  long long olse_sb, olse_sh, olse_ss;  // the caller's LSE: + b*sb + h*sh + row*ss
  long long total_q;         // stacked Q side: rows of Q
};

// Rows of sequence b: Q rows q0 .. q0+sq-1 and K rows k0 .. k0+sk-1 (start
// rows in stacked tensors, 0 for padded sides) as the sides' modes resolve
// them.  Every kernel computes on these rows only.  (A template so that P
// may also sit in the kernel-argument segment.)
template <class PA>
__device__ __forceinline__ void seq_rows(PA& P, int b, long long& q0, int& sq, long long& k0, int& sk) {
  const SideRows q = side_rows(P.qs, b), k = side_rows(P.ks, b);
  q0 = q.r0;
  sq = q.n;
  k0 = k.r0;
  sk = k.n;
}

struct FwdArgs {
  ProblemArgs p;
  Operand q, k, v, o;
  float* lse;
  FeatArgs f;    // optional features (read by the FEAT kernels only)
  int feat;      // any feature present: the FEAT kernels run
  int no_split;  // the ping-pong grid alone, no key-split workgroups
  // Key-split tail of the 16-bit ping-pong forward (null ks_part: off).
  // The blocks of the grid's last, partly filled round run as np workgroups
  // each, workgroup s of a block over the s-th of np near-equal runs of its
  // key tiles; each stores its unnormalised (O^T, m, l) per wave and lane
  // into slot blockIdx.x of ks_part (ks_chunks(D) float4 per lane, chunk-
  // major, 8 waves x 64 lanes per slot), and a merge grid then combines each
  // block's np slots in slot order.  ks_units: slots ks_part holds.
  float* ks_part;
  int ks_units;
};

// Ping-pong forward workgroups per CU: two at head dims up to 64, where a
// wave fits in 128 registers; one otherwise.
__host__ __device__ constexpr int pp_wg_per_cu(int D) { return D <= 64 ? 2 : 1; }
// float4 chunks of one lane's key-split partial: O^T accumulators of
// ceil(D / 32) 32-column blocks (4 chunks each), then (m, l, 0, 0).
__host__ __device__ constexpr int ks_chunks(int D) { return 4 * ((D + 31) / 32) + 1; }
// Key-split workspace: one full round of slots on a 256-CU device.
constexpr long long kKsRoundCu = 256;
inline long long ks_units(int D) { return kKsRoundCu * pp_wg_per_cu(D); }
inline unsigned long long ks_ws_bytes(int D) { return (unsigned long long)ks_units(D) * 8 * 64 * ks_chunks(D) * 16; }
// Fewest keys of a block's band per key-split part: below this, the parts'
// start and end (Q rows, first tiles, partial stores of 8 x 64 x ks_chunks
// float4) outweigh the split (2x16x1024x64 bf16 in two parts of 512 keys:
// 28.3 against 31.8 us; 4x8x1024x128: 36.4 against 33.4 us).
__host__ __device__ constexpr long long ks_min_keys(int D) { return D <= 64 ? 512 : 1024; }

struct BwdArgs {
  ProblemArgs p;
  Operand q, k, v, o, dout, dq, dk, dv;
  const float* lse;
  float* delta;  // workspace: Delta_i = sum_d dO_id O_id (written by the preprocess)
  float* lse2;   // workspace: LSE_i * log2(e) (written by the preprocess)
  FeatArgs f;
  int feat;
  // Split mode (null part: off).  The dK/dV grid is repeated split_kv times,
  // copy g walking its g-th share of the query tiles, and the dQ grid
  // split_q times over the key tiles; each copy stores unscaled fp32 sums
  // into part, and the last copy of a block to finish adds them in copy
  // order.  Layout, in rows of head_dim floats: dK [split_kv][H][rows_k],
  // then dV likewise, then dQ [split_q][H][rows_q]; a row's index is its
  // storage row (stacked side) or b * seqlen + local row (padded side).
  // Arrival counters, one per block of the split grid (128 or 64 rows):
  // cnt_kv[(b H + h) nkb + kb] for the dK/dV blocks, cnt_q[(b H + h) nqb +
  // qb] for the dQ blocks (cnt_q past room for the finest dK/dV grid); the
  // preprocess zeroes all ncnt of them and the last arrival at a block
  // resets its counter.  Null: a reduction kernel sums the partials.
  float* part;
  long long rows_q, rows_k;
  int split_kv, split_q;
  unsigned* cnt_kv;
  unsigned* cnt_q;
  long long ncnt;
};

// Partial-sum row of local row i of sequence b on a side of the given mode
// and seqlen S whose sequence starts at storage row r0.
__host__ __device__ __forceinline__ long long part_row(int mode, int S, int b, long long r0, int i) {
  return (mode & kSeqStacked) ? r0 + i : (long long)b * S + i;
}

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
constexpr int kPlanMax = 8;
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
// One dtype's backward kernels (built in attn_bwd_<dtype>.hip).
hipError_t launch_bwd_f32(int head_dim, const BwdArgs& a, int stages, const Enqueue& ex);
hipError_t launch_bwd_f32(int head_dim, const BwdArgs& a, int stages, const Record& ex);
hipError_t launch_bwd_f16(int head_dim, const BwdArgs& a, int stages, const Enqueue& ex);
hipError_t launch_bwd_f16(int head_dim, const BwdArgs& a, int stages, const Record& ex);
hipError_t launch_bwd_bf16(int head_dim, const BwdArgs& a, int stages, const Enqueue& ex);
hipError_t launch_bwd_bf16(int head_dim, const BwdArgs& a, int stages, const Record& ex);
// Rows of each sequence's room past its length (side 0: Q, side 1: K): zeros
// in t0 and t1 (null pointers skipped) and, when lse is given, LSE = +inf.
// Rows are row_bytes long (a multiple of 16).  Launches nothing for a side
// whose lengths always fill their rooms.
template <class Ex>
hipError_t launch_pad_rows(const ProblemArgs& p, Operand t0, Operand t1, float* lse, int side, int row_bytes,
                           int esz, const Ex& ex);

// Copies between a caller's tensor and its zero-padded copy (repacked
// calls).  Inward (out = 0): each sequence's rows (its length) of src, cols
// columns, into dst with columns [cols, pad) zeroed.  Outward (out = 1):
// the first cols columns of each sequence's rows up to its room (the rows
// the kernels write: lengths, then masked padding rows) from the copy src
// back to the caller's dst.  Rows are addressed as the kernels address
// them (storage row r0 + i of sequence b), in both tensors.
struct RepackT {
  Operand src, dst;
  int side;  // 0: query rows, 1: key rows
  int cols;  // the caller's columns
};
constexpr int kRepackMax = 5;
struct RepackArgs {
  ProblemArgs p;
  RepackT t[kRepackMax];
  int n;    // tensors used
  int out;  // direction
  int pad;  // columns of the copies (<= 256)
  int esz;  // element size
};
template <class Ex>
hipError_t launch_repack(const RepackArgs& a, const Ex& ex);

}  // namespace sdpa
