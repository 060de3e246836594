// attn_bwd_kernels.hpp - fused attention backward for gfx950: the row-sum
// preprocess and the split dK/dV and dQ kernels (the "bwd_preprocess" and
// "triton_split" steps named in the AOTriton 0.14b release notes), and the
// launch rules, as templates.  attn_bwd_f32.hip, attn_bwd_f16.hip and
// attn_bwd_bf16.hip each build one dtype's kernels (in parallel);
// attn_bwd.hip dispatches on the dtype.
//
// With P recomputed from the forward's LSE (P_ij = exp(scale q_i.k_j -
// LSE_i) on visible pairs), Delta_i = sum_d dO_id O_id, dP = dO V^T and
// dS = P o (dP - Delta):
//   dV = P^T dO,  dK = scale dS^T Q   (per key block, kernel 2)
//   dQ = scale dS K                   (per query block, kernel 3)
// No floating-point atomics: every output element is summed by one lane in
// a fixed order, so results are run-to-run identical (the split mode's only
// atomics are integer arrival counts, which decide who sums, not the order).
#pragma once

#include <type_traits>
#include <utility>

#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace sdpa {

template <typename T>
__device__ __forceinline__ void store4b(T* p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  } else {
    typedef T t4 __attribute__((ext_vector_type(4)));
    t4 v;
    v[0] = (T)a; v[1] = (T)b; v[2] = (T)c; v[3] = (T)d;
    *reinterpret_cast<t4*>(p) = v;
  }
}

// ------------------------------------------------------------ split mode

// Copy sg of n takes the sg-th of n contiguous, nearly equal shares of the
// tiles (of T rows) that rows [lo, hi] touch, and narrows [lo, hi] to the
// rows of its share (lo > hi: no tile, when there are more copies than
// tiles or the range is empty).
__device__ __forceinline__ void split_rows(long long& lo, long long& hi, int T, int sg, int n) {
  if (n <= 1 || lo > hi) return;
  const long long t0 = lo / T, t1 = hi / T, per = (t1 - t0 + n) / n;
  const long long s0 = t0 + sg * per, s1 = min(t1, s0 + per - 1);
  if (s0 > s1) {
    hi = lo - 1;
    return;
  }
  lo = max(lo, s0 * T);
  hi = min(hi, s1 * T + T - 1);
}

// Unscaled fp32 dK and dV sums of this lane's key (partial-sum row prow of
// copy sg): the accumulator layout of the dK/dV kernels (lane half g holds
// columns 32 dt + 8 q4 + 4 g .. + 3).
template <int D>
__device__ __forceinline__ void store_partial_kv(float* part, long long rows_k, int split_kv, int H, int sg, int h,
                                                 long long prow, const f32x16* dk, const f32x16* dv, int g) {
  constexpr int DVT = (D + 31) / 32;
  float* pk = part + ((long long)(sg * H + h) * rows_k + prow) * D;
  float* pv = pk + (long long)split_kv * H * rows_k * D;
#pragma unroll
  for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * dt + 8 * q4 + 4 * g;
      if (d < D) {
        *reinterpret_cast<float4*>(pk + d) =
            make_float4(dk[dt][4 * q4], dk[dt][4 * q4 + 1], dk[dt][4 * q4 + 2], dk[dt][4 * q4 + 3]);
        *reinterpret_cast<float4*>(pv + d) =
            make_float4(dv[dt][4 * q4], dv[dt][4 * q4 + 1], dv[dt][4 * q4 + 2], dv[dt][4 * q4 + 3]);
      }
    }
}

// The same for dQ (part_q: the dQ section).
template <int D>
__device__ __forceinline__ void store_partial_q(float* part_q, long long rows_q, int H, int sg, int h, long long prow,
                                                const f32x16* dq, int g) {
  constexpr int DVT = (D + 31) / 32;
  float* pq = part_q + ((long long)(sg * H + h) * rows_q + prow) * D;
#pragma unroll
  for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * dt + 8 * q4 + 4 * g;
      if (d < D)
        *reinterpret_cast<float4*>(pq + d) =
            make_float4(dq[dt][4 * q4], dq[dt][4 * q4 + 1], dq[dt][4 * q4 + 2], dq[dt][4 * q4 + 3]);
    }
}

// The last copy's epilogue for one block: rows [lo, hi) of sequence b, head
// h (partial row part_row(mode, S, b, r0, i)) get the sum of their G partial
// rows in copy order (so the result does not depend on which copy is last),
// times sc, rounded into o0; with KV the second section (dV, one section of
// G H rows further on) goes unscaled into o1.  One workgroup reads all of
// it, so each thread keeps 32 float4 loads (U columns of every copy and
// section) in flight at once.
template <typename T, int D, int NT, bool KV, int G>
__device__ __forceinline__ void sum_partials_g(const float* part, long long rows, int H, int h, int mode, int S,
                                               int b, long long r0, int lo, int hi, T* o0, long long ss0, T* o1,
                                               long long ss1, float sc, int tid) {
  constexpr int V4 = D / 4, U = (KV ? 16 : 32) / G > 1 ? (KV ? 16 : 32) / G : 1;
  static_assert(D % 4 == 0, "row shape");
  const long long gstride = (long long)H * rows * D;
  const float* p1 = part + G * gstride;
  const int total = (hi - lo) * V4;
  for (int x0 = tid; x0 < total; x0 += U * NT) {
    float4 u[U][G], v[U][KV ? G : 1];
    long long off[U];
#pragma unroll
    for (int e = 0; e < U; ++e) {
      const int x = min(x0 + e * NT, total - 1);
      const int i = lo + x / V4, d = 4 * (x % V4);
      off[e] = ((long long)h * rows + part_row(mode, S, b, r0, i)) * D + d;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        u[e][g] = *reinterpret_cast<const float4*>(part + g * gstride + off[e]);
        if constexpr (KV) v[e][g] = *reinterpret_cast<const float4*>(p1 + g * gstride + off[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < U; ++e) {
      const int x = x0 + e * NT;
      if (x >= total) break;
      const int i = lo + x / V4, d = 4 * (x % V4);
      float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        s0.x += u[e][g].x; s0.y += u[e][g].y; s0.z += u[e][g].z; s0.w += u[e][g].w;
        if constexpr (KV) {
          s1.x += v[e][g].x; s1.y += v[e][g].y; s1.z += v[e][g].z; s1.w += v[e][g].w;
        }
      }
      store4b<T>(o0 + (long long)i * ss0 + d, s0.x * sc, s0.y * sc, s0.z * sc, s0.w * sc);
      if constexpr (KV) store4b<T>(o1 + (long long)i * ss1 + d, s1.x, s1.y, s1.z, s1.w);
    }
  }
}

// The same for n copies (2 <= n <= 8, the split rule's range).
template <typename T, int D, int NT, bool KV>
__device__ __forceinline__ void sum_partials(const float* part, long long rows, int H, int n, int h, int mode, int S,
                                             int b, long long r0, int lo, int hi, T* o0, long long ss0, T* o1,
                                             long long ss1, float sc, int tid) {
#define SDPA_SUM_CASE(G)                                                                                        \
  case G:                                                                                                       \
    sum_partials_g<T, D, NT, KV, G>(part, rows, H, h, mode, S, b, r0, lo, hi, o0, ss0, o1, ss1, sc, tid);       \
    break;
  switch (n) {
    SDPA_SUM_CASE(1)
    SDPA_SUM_CASE(2)
    SDPA_SUM_CASE(3)
    SDPA_SUM_CASE(4)
    SDPA_SUM_CASE(5)
    SDPA_SUM_CASE(6)
    SDPA_SUM_CASE(7)
    SDPA_SUM_CASE(8)
    default: break;
  }
#undef SDPA_SUM_CASE
}

template <typename T>
__device__ __forceinline__ float dot_chunk(uint4 x, uint4 y) {
  if constexpr (sizeof(T) == 4) {
    return __uint_as_float(x.x) * __uint_as_float(y.x) + __uint_as_float(x.y) * __uint_as_float(y.y) +
           __uint_as_float(x.z) * __uint_as_float(y.z) + __uint_as_float(x.w) * __uint_as_float(y.w);
  } else {
    typedef T t8 __attribute__((ext_vector_type(8)));
    t8 a = __builtin_bit_cast(t8, x), b = __builtin_bit_cast(t8, y);
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) s += (float)a[t] * (float)b[t];
    return s;
  }
}

// ------------------------------------------------------------ preprocess

// Delta_i = sum_d dO_id * O_id in fp32, one group of G lanes per row, each
// lane one 16-byte chunk; beside it LSE_i * log2(e), the form the 16-bit
// kernels use.  Rows are (b, h, i) for the dense layout and
// (packed row t, h) for the packed one.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(BwdArgs a, long long nrows) {
  constexpr int CE = 16 / (int)sizeof(T), CH = D / CE;
  constexpr int G = CH <= 8 ? 8 : (CH <= 16 ? 16 : 32);
  const ProblemArgs& P = a.p;
  for (long long x = (long long)blockIdx.x * 256 + threadIdx.x; x < a.ncnt; x += (long long)gridDim.x * 256)
    a.cnt_kv[x] = 0u;
  const long long row = (long long)blockIdx.x * (256 / G) + threadIdx.x / G;
  const int c = threadIdx.x % G;
  if (row >= nrows) return;  // whole groups leave together
  long long b, h, i;
  if (P.qs.mode & kSeqStacked) {
    i = row / P.H;  // stacked row
    h = row % P.H;
    b = 0;
  } else {
    const long long bh = row / P.Sq;
    i = row % P.Sq;
    h = bh % P.H;
    b = bh / P.H;
  }
  float s = 0.f;
  if (c < CH) {
    const T* op = (const T*)a.o.ptr + b * a.o.sb + h * a.o.sh + i * a.o.ss + c * CE;
    const T* dp = (const T*)a.dout.ptr + b * a.dout.sb + h * a.dout.sh + i * a.dout.ss + c * CE;
    s = dot_chunk<T>(*reinterpret_cast<const uint4*>(op), *reinterpret_cast<const uint4*>(dp));
  }
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, G);
  if (c == 0) {
    const long long idx = b * P.lse_sb + h * P.lse_sh + i;
    a.delta[idx] = s;
    a.lse2[idx] = a.lse[b * P.olse_sb + h * P.olse_sh + i * P.olse_ss] * kLog2e;  // +inf (empty row) stays +inf
  }
}

// ------------------------------------------------------------ dK / dV

// One workgroup = 32*NW keys of one (sequence, head), each wave 32 keys with
// its K and V rows held in registers; the workgroup walks the query tiles
// (BMQ rows) that can see its keys.  Per tile, Q and dO are staged both
// row-major (A operands of S = Q K^T and dP = dO V^T) and transposed (A
// operands of dK^T += Q^T dS and dV^T += dO^T P), with LSE and Delta.
// With FEAT the logits carry the bias / ALiBi terms and dropout multiplies
// P (in dV) and dP (in dS) by keep / (1 - p).
template <typename M, int D, int NW, int BMQ, bool FEAT, bool SPLIT>
__device__ __forceinline__ void dkdv_body(const BwdArgs& a, unsigned hw, unsigned nblk) {
  using T = typename M::elem;
  constexpr int NT = NW * 64, BNK = NW * 32, KPL = M::KPL;
  constexpr int DVT = (D + 31) / 32, DPAD = DVT * 32;
  constexpr int PAD = 16 / (int)sizeof(T);
  constexpr int RLD = D + PAD, TLD = BMQ + PAD;
  constexpr int MQ = BMQ / 32;
  constexpr int NS = D / (2 * KPL);
  constexpr int STAGE_T = 2 * BMQ * RLD + 2 * DPAD * TLD;
  __shared__ __attribute__((aligned(16))) T smem[2 * STAGE_T];
  __shared__ __attribute__((aligned(16))) float stats[2][2][BMQ];  // [buf][lse2, delta][row]

  const ProblemArgs& P = a.p;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int nbh = P.B * P.H;
  const int nsplit = SPLIT ? a.split_kv : 1;
  const int nkb = (int)(nblk / ((unsigned)nbh * nsplit));
  const int sg = (int)(hw / (unsigned)(nkb * nbh));  // split copy (0 without split)
  const GridPos gp = grid_pos((int)(hw % (unsigned)(nkb * nbh)), nkb * nbh, nkb, nbh, P.ragged);
  const int bh = gp.bh, h = bh % P.H, b = bh / P.H;
  const int kb = gp.i;

  long long q0, k0;
  int sq, sk;
  seq_rows(P, b, q0, sq, k0, sk);
  const int j0 = kb * BNK;
  if (j0 >= sk) return;
  const Window w = seq_window(P.wl, P.wr, P.diag, sq, sk);

  const T* qp = (const T*)a.q.ptr + b * a.q.sb + h * a.q.sh + q0 * a.q.ss;
  const T* kp = (const T*)a.k.ptr + b * a.k.sb + h * a.k.sh + k0 * a.k.ss;
  const T* vp = (const T*)a.v.ptr + b * a.v.sb + h * a.v.sh + k0 * a.v.ss;
  const T* dop = (const T*)a.dout.ptr + b * a.dout.sb + h * a.dout.sh + q0 * a.dout.ss;
  T* dkp = (T*)a.dk.ptr + b * a.dk.sb + h * a.dk.sh + k0 * a.dk.ss;
  T* dvp = (T*)a.dv.ptr + b * a.dv.sb + h * a.dv.sh + k0 * a.dv.ss;
  const float* lsep = a.lse + b * P.olse_sb + h * P.olse_sh + q0 * P.olse_ss;
  const float* delp = a.delta + b * P.lse_sb + h * P.lse_sh + q0;

  // Queries that can see the block's keys.
  const int jlast = min(j0 + BNK, sk) - 1;
  long long ilo = max(0LL, (long long)j0 - w.hi);
  long long ihi = min((long long)sq - 1, (long long)jlast - w.lo);
  if constexpr (SPLIT) split_rows(ilo, ihi, BMQ, sg, nsplit);
  const bool block_empty = w.lo > w.hi || ilo > ihi;

  const int jw0 = j0 + 32 * wave;
  const bool wave_live = jw0 < sk;
  const int kj = jw0 + r;  // this lane's key

  RowFrags<M, D> kf, vf;
  kf.load(kp + (long long)kj * a.k.ss, wave_live && kj < sk, g);
  vf.load(vp + (long long)kj * a.v.ss, wave_live && kj < sk, g);

  if constexpr (DPAD != D) {
    for (int x = tid; x < (DPAD - D) * TLD; x += NT)
#pragma unroll
      for (int bf = 0; bf < 2; ++bf)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          smem[bf * STAGE_T + 2 * BMQ * RLD + tt * DPAD * TLD + D * TLD + x] = (T)0.f;
  }

  f32x16 dk[DVT], dv[DVT];
#pragma unroll
  for (int dt = 0; dt < DVT; ++dt) {
    dk[dt] = zero16();
    dv[dt] = zero16();
  }

  if (!block_empty) {
    const int t0 = (int)(ilo / BMQ), t1 = (int)(ihi / BMQ);
    TileStage<T, BMQ, D, NT> qs, dos;
    float st_l = INFINITY, st_d = 0.f;  // this thread's LSE/Delta entry (tid < BMQ)
    auto load_tile = [&](int i0) {
      qs.load(qp + (long long)i0 * a.q.ss, a.q.ss, sq - i0, tid);
      dos.load(dop + (long long)i0 * a.dout.ss, a.dout.ss, sq - i0, tid);
      if (tid < BMQ) {
        const bool ok = i0 + tid < sq;
        st_l = ok ? lsep[(i0 + tid) * P.olse_ss] * kLog2e : INFINITY;
        st_d = ok ? delp[i0 + tid] : 0.f;
      }
    };
    auto store_tile = [&](int bf) {
      T* base = smem + bf * STAGE_T;
      qs.store_rows(base, RLD, tid);
      dos.store_rows(base + BMQ * RLD, RLD, tid);
      qs.store_transposed(base + 2 * BMQ * RLD, TLD, tid);
      dos.store_transposed(base + 2 * BMQ * RLD + DPAD * TLD, TLD, tid);
      if (tid < BMQ) {
        stats[bf][0][tid] = st_l;
        stats[bf][1][tid] = st_d;
      }
    };
    load_tile(t0 * BMQ);
    store_tile(0);
    __syncthreads();

    for (int t = t0; t <= t1; ++t) {
      const int bf = (t - t0) & 1;
      const int i0 = t * BMQ;
      if (t < t1) load_tile(i0 + BMQ);
      const T* Qs = smem + bf * STAGE_T;
      const T* dOs = Qs + BMQ * RLD;
      const T* Qt = Qs + 2 * BMQ * RLD;
      const T* dOt = Qt + DPAD * TLD;
      const int cls = wave_live ? classify(w, i0, BMQ, jw0, 32, sk) : kEmpty;
      if (cls != kEmpty) {
#pragma unroll
        for (int mq = 0; mq < MQ; ++mq) {
          // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys.
          f32x16 s = zero16(), dp = zero16();
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            const int off = (32 * mq + r) * RLD + 2 * KPL * st + KPL * g;
            s = M::mma(load_frag<M>(Qs + off), kf.f[st], s);
            dp = M::mma(load_frag<M>(dOs + off), vf.f[st], dp);
          }
          float p[16], ds[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int il = 32 * mq + acc_row(e, g);
            float x = s[e] * P.scale_log2;
            if constexpr (FEAT) x = __builtin_fmaf(s[e], P.scale_log2, extra_log2<T>(a.f, b, h, i0 + il, kj, sq, sk));
            float pe = __builtin_amdgcn_exp2f(x - stats[bf][0][il]);
            if (cls == kPartial) {
              const int diff = kj - (i0 + il);
              if (!(diff >= w.lo && diff <= w.hi && kj < sk)) pe = 0.f;
            }
            float pv = pe, dpe = dp[e];
            if constexpr (FEAT) {
              if (a.f.drop_thresh) {
                const bool kp = keep1(a.f, b, h, P.H, i0 + il, kj, P.Sq, P.Sk);
                pv = kp ? pe * a.f.drop_scale : 0.f;
                dpe = kp ? dp[e] * a.f.drop_scale : 0.f;
              }
            }
            p[e] = pv;
            ds[e] = pe * (dpe - stats[bf][1][il]);
          }
          // dV^T += dO^T P and dK^T += Q^T dS (scale applied at the end).
#pragma unroll
          for (int st = 0; st < 16 / KPL; ++st) {
            typename M::frag pf, dsf;
            M::pack(&p[KPL * st], pf);
            M::pack(&ds[KPL * st], dsf);
            const int pos = 32 * mq + perm_pos(KPL * st, g);
#pragma unroll
            for (int dt = 0; dt < DVT; ++dt) {
              dv[dt] = M::mma(load_frag<M>(dOt + (32 * dt + r) * TLD + pos), pf, dv[dt]);
              dk[dt] = M::mma(load_frag<M>(Qt + (32 * dt + r) * TLD + pos), dsf, dk[dt]);
            }
          }
        }
      }
      if (t < t1) store_tile(bf ^ 1);
      __syncthreads();
    }
  }

  if constexpr (SPLIT) {
    if (wave_live && kj < sk)
      store_partial_kv<D>(a.part, a.rows_k, a.split_kv, P.H, sg, h, part_row(P.ks.mode, P.Sk, b, k0, kj), dk, dv, g);
    if (a.cnt_kv != nullptr && last_arrival(a.cnt_kv + (long long)bh * nkb + kb, nsplit))
      sum_partials<T, D, NT, true>(a.part, a.rows_k, P.H, nsplit, h, P.ks.mode, P.Sk, b, k0, j0, jlast + 1, dkp,
                                   a.dk.ss, dvp, a.dv.ss, P.scale, tid);
  } else if (wave_live && kj < sk) {
    T* dkrow = dkp + (long long)kj * a.dk.ss;
    T* dvrow = dvp + (long long)kj * a.dv.ss;
    const float sc = P.scale;
#pragma unroll
    for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * dt + 8 * q4 + 4 * g;
        if (d < D) {
          store4b<T>(dkrow + d, dk[dt][4 * q4] * sc, dk[dt][4 * q4 + 1] * sc,
                     dk[dt][4 * q4 + 2] * sc, dk[dt][4 * q4 + 3] * sc);
          store4b<T>(dvrow + d, dv[dt][4 * q4], dv[dt][4 * q4 + 1], dv[dt][4 * q4 + 2],
                     dv[dt][4 * q4 + 3]);
        }
      }
  }
}

template <typename M, int D, int NW, int BMQ, bool FEAT = false, bool SPLIT = false>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dkdv_kernel(BwdArgs a) {
  dkdv_body<M, D, NW, BMQ, FEAT, SPLIT>(a, blockIdx.x, gridDim.x);
}

// ------------------------------------------------------------ dQ

// One workgroup = 32*NW queries, each wave 32 queries with its Q and dO rows,
// LSE and Delta in registers; the workgroup walks the key tiles its window
// can see, staging K (row-major and transposed) and V (row-major).
// With FEAT the logits carry the bias / ALiBi terms, dropout multiplies dP
// by keep / (1 - p), and with a dbias output every key tile is visited and
// dS is stored (zeros where masked).
template <typename M, int D, int NW, int BN, bool FEAT, bool SPLIT>
__device__ __forceinline__ void dq_body(const BwdArgs& a, unsigned hw, unsigned nblk) {
  using T = typename M::elem;
  constexpr int NT = NW * 64, BM = NW * 32, KPL = M::KPL;
  constexpr int DVT = (D + 31) / 32, DPAD = DVT * 32;
  constexpr int PAD = 16 / (int)sizeof(T);
  constexpr int RLD = D + PAD, TLD = BN + PAD;
  constexpr int KT = BN / 32;
  constexpr int NS = D / (2 * KPL);
  constexpr int STAGE = 2 * BN * RLD + DPAD * TLD;
  __shared__ __attribute__((aligned(16))) T smem[2 * STAGE];

  const ProblemArgs& P = a.p;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int nbh = P.B * P.H;
  const int nsplit = SPLIT ? a.split_q : 1;
  const int nq = (int)(nblk / ((unsigned)nbh * nsplit));
  const int sg = (int)(hw / (unsigned)(nq * nbh));  // split copy (0 without split)
  const GridPos gp = grid_pos((int)(hw % (unsigned)(nq * nbh)), nq * nbh, nq, nbh, P.ragged);
  const int bh = gp.bh, h = bh % P.H, b = bh / P.H;
  const int qb = nq - 1 - gp.i;

  long long q0, k0;
  int sq, sk;
  seq_rows(P, b, q0, sq, k0, sk);
  const int i0 = qb * BM;
  if (i0 >= sq) return;
  const Window w = seq_window(P.wl, P.wr, P.diag, sq, sk);

  const T* qp = (const T*)a.q.ptr + b * a.q.sb + h * a.q.sh + q0 * a.q.ss;
  const T* kp = (const T*)a.k.ptr + b * a.k.sb + h * a.k.sh + k0 * a.k.ss;
  const T* vp = (const T*)a.v.ptr + b * a.v.sb + h * a.v.sh + k0 * a.v.ss;
  const T* dop = (const T*)a.dout.ptr + b * a.dout.sb + h * a.dout.sh + q0 * a.dout.ss;
  T* dqp = (T*)a.dq.ptr + b * a.dq.sb + h * a.dq.sh + q0 * a.dq.ss;
  const float* lsep = a.lse + b * P.olse_sb + h * P.olse_sh + q0 * P.olse_ss;
  const float* delp = a.delta + b * P.lse_sb + h * P.lse_sh + q0;

  const bool all_tiles = FEAT && a.f.dbias != nullptr;
  const int ilast = min(i0 + BM, sq) - 1;
  long long jlo = max(0LL, (long long)i0 + w.lo);
  long long jhi = min((long long)sk - 1, (long long)ilast + w.hi);
  bool block_empty = w.lo > w.hi || jlo > jhi;
  if (all_tiles) {
    jlo = 0;
    jhi = (long long)sk - 1;
    block_empty = sk == 0;
  }
  if constexpr (SPLIT) {
    split_rows(jlo, jhi, BN, sg, nsplit);
    block_empty = block_empty || jlo > jhi;
  }

  const int iw0 = i0 + 32 * wave;
  const bool wave_live = iw0 < sq;
  const int qi = iw0 + r;
  const bool row_ok = wave_live && qi < sq;

  RowFrags<M, D> qf, dof;
  qf.load(qp + (long long)qi * a.q.ss, row_ok, g);
  dof.load(dop + (long long)qi * a.dout.ss, row_ok, g);
  const float lse2 = row_ok ? lsep[qi * P.olse_ss] * kLog2e : INFINITY;
  const float delta = row_ok ? delp[qi] : 0.f;

  if constexpr (DPAD != D) {
    for (int x = tid; x < (DPAD - D) * TLD; x += NT) {
      smem[2 * BN * RLD + D * TLD + x] = (T)0.f;
      smem[STAGE + 2 * BN * RLD + D * TLD + x] = (T)0.f;
    }
  }

  f32x16 dq[DVT];
#pragma unroll
  for (int dt = 0; dt < DVT; ++dt) dq[dt] = zero16();

  if (!block_empty) {
    const int t0 = (int)(jlo / BN), t1 = (int)(jhi / BN);
    TileStage<T, BN, D, NT> ks, vs;
    auto load_tile = [&](int j0) {
      ks.load(kp + (long long)j0 * a.k.ss, a.k.ss, sk - j0, tid);
      vs.load(vp + (long long)j0 * a.v.ss, a.v.ss, sk - j0, tid);
    };
    auto store_tile = [&](int bf) {
      T* base = smem + bf * STAGE;
      ks.store_rows(base, RLD, tid);
      vs.store_rows(base + BN * RLD, RLD, tid);
      ks.store_transposed(base + 2 * BN * RLD, TLD, tid);
    };
    load_tile(t0 * BN);
    store_tile(0);
    __syncthreads();

    for (int t = t0; t <= t1; ++t) {
      const int bf = (t - t0) & 1;
      const int j0 = t * BN;
      if (t < t1) load_tile(j0 + BN);
      const T* Ks = smem + bf * STAGE;
      const T* Vs = Ks + BN * RLD;
      const T* Kt = Ks + 2 * BN * RLD;
      int cls = wave_live ? classify(w, iw0, 32, j0, BN, sk) : kEmpty;
      if (all_tiles && wave_live && cls == kEmpty) cls = kPartial;  // its dS is stored: zeros
      if (cls != kEmpty) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          // S^T = K Q^T and dP^T = V dO^T for 32 keys x this wave's queries.
          f32x16 s = zero16(), dp = zero16();
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            const int off = (32 * kt + r) * RLD + 2 * KPL * st + KPL * g;
            s = M::mma(load_frag<M>(Ks + off), qf.f[st], s);
            dp = M::mma(load_frag<M>(Vs + off), dof.f[st], dp);
          }
          float ds[16];
          uint32_t keep = 0xffffu;
          if constexpr (FEAT) {
            if (a.f.drop_thresh) {
              keep = 0;
#pragma unroll
              for (int qd = 0; qd < 4; ++qd)
                keep |= keep4(a.f, b, h, P.H, qi, j0 + 32 * kt + 8 * qd + 4 * g, P.Sq, P.Sk) << (4 * qd);
            }
          }
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int j = j0 + 32 * kt + acc_row(e, g);
            float x = s[e] * P.scale_log2;
            if constexpr (FEAT) x = __builtin_fmaf(s[e], P.scale_log2, extra_log2<T>(a.f, b, h, qi, j, sq, sk));
            float pe = __builtin_amdgcn_exp2f(x - lse2);
            if (cls == kPartial) {
              const int diff = j - qi;
              if (!(diff >= w.lo && diff <= w.hi && j < sk)) pe = 0.f;
            }
            float dpe = dp[e];
            if constexpr (FEAT) {
              if (a.f.drop_thresh) dpe = ((keep >> e) & 1u) ? dp[e] * a.f.drop_scale : 0.f;
            }
            ds[e] = pe * (dpe - delta);
          }
          if constexpr (FEAT) {
            if (all_tiles && row_ok) {
              float* drow = a.f.dbias + b * a.f.dsb + h * a.f.dsh + (long long)qi * a.f.dss;
#pragma unroll
              for (int e = 0; e < 16; ++e) {
                const int j = j0 + 32 * kt + acc_row(e, g);
                if (j < sk) drow[j] = ds[e];
              }
            }
          }
          // dQ^T += K^T dS^T (scale applied at the end).
#pragma unroll
          for (int st = 0; st < 16 / KPL; ++st) {
            typename M::frag dsf;
            M::pack(&ds[KPL * st], dsf);
            const int pos = 32 * kt + perm_pos(KPL * st, g);
#pragma unroll
            for (int dt = 0; dt < DVT; ++dt)
              dq[dt] = M::mma(load_frag<M>(Kt + (32 * dt + r) * TLD + pos), dsf, dq[dt]);
          }
        }
      }
      if (t < t1) store_tile(bf ^ 1);
      __syncthreads();
    }
  }

  if constexpr (SPLIT) {
    float* const part_q = a.part + 2LL * a.split_kv * P.H * a.rows_k * D;
    if (row_ok) store_partial_q<D>(part_q, a.rows_q, P.H, sg, h, part_row(P.qs.mode, P.Sq, b, q0, qi), dq, g);
    if (a.cnt_q != nullptr && last_arrival(a.cnt_q + (long long)bh * nq + qb, nsplit))
      sum_partials<T, D, NT, false>(part_q, a.rows_q, P.H, nsplit, h, P.qs.mode, P.Sq, b, q0, i0, ilast + 1, dqp,
                                    a.dq.ss, nullptr, 0, P.scale, tid);
  } else if (row_ok) {
    T* dqrow = dqp + (long long)qi * a.dq.ss;
    const float sc = P.scale;
#pragma unroll
    for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * dt + 8 * q4 + 4 * g;
        if (d < D)
          store4b<T>(dqrow + d, dq[dt][4 * q4] * sc, dq[dt][4 * q4 + 1] * sc,
                     dq[dt][4 * q4 + 2] * sc, dq[dt][4 * q4 + 3] * sc);
      }
  }
}

template <typename M, int D, int NW, int BN, bool FEAT = false, bool SPLIT = false>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dq_kernel(BwdArgs a) {
  dq_body<M, D, NW, BN, FEAT, SPLIT>(a, blockIdx.x, gridDim.x);
}

// LDS of the 16-bit backward kernels that run 8-wave workgroups, and of the
// split grid: three stages of [Q | dO | LSE log2 e | Delta] (dK/dV) or
// [K | V] (dQ) and three fp16 P buffers.  They are named at namespace scope so that the kernel
// bodies refer to these objects directly: the compiler then knows every
// access is to LDS, and which stage array a direct load fills.  Sized for
// 64-row tiles of up to 128 columns of 16-bit elements.
constexpr int kBwdStageBytes = 2 * 64 * 128 * 2 + 4 * 64 * 4;
constexpr int kBwdXBytes = 4 * 2 * 2 * 64 * 16;
__shared__ __attribute__((aligned(1024))) char g_bwd_st0[kBwdStageBytes];
__shared__ __attribute__((aligned(1024))) char g_bwd_st1[kBwdStageBytes];
__shared__ __attribute__((aligned(1024))) char g_bwd_st2[kBwdStageBytes];
__shared__ __attribute__((aligned(16))) char g_bwd_x0[kBwdXBytes];
__shared__ __attribute__((aligned(16))) char g_bwd_x1[kBwdXBytes];
__shared__ __attribute__((aligned(16))) char g_bwd_x2[kBwdXBytes];

// ------------------------------------------------- 16-bit dK / dV kernel
//
// bf16 / fp16.  One workgroup = 32*NW keys of one (sequence, head); each
// wave keeps its 32 keys' K and V rows in registers (B operands).  Query
// tiles of BMQ rows of Q and dO are copied HBM -> LDS with direct loads into
// swizzled row-major tiles, two stages deep, with the tile's LSE (as log2)
// and Delta beside them; tile rows past the sequence repeat its last row
// (every loaded value is a finite input) and are masked out: the tile is
// treated as cut, and those rows' scores are set to -inf, so their P is
// exactly 0.  Per 32-query slice:
//   S = Q K^T and dP = dO V^T from 128-bit row reads of the Q and dO tiles;
//   P = 2^(c S - LSE log2(e)) with c = |scale| log2(e) (a negative scale is
//   moved into the K operand), dS = P o (dP - Delta);
//   dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T taken by
//   transposing reads of the same tiles.
// Each wave visits only the query tiles that can see its keys; tiles cut
// by the window or the sequence end have their scores set to -inf where
// masked.
template <typename M, int D, int BMQ>
struct Dkdv16 {
  using T = typename M::elem;
  using L = Swz<D>;
  using frag = typename M::frag;
  static constexpr int MQ = BMQ / 32, NS = D / 16, DVT = (D + 31) / 32;
  static constexpr int TILE = BMQ * L::PITCH;
  // Up to head_dim 128 (where it adds no spill): vf holds -V and the dP
  // accumulators start from the slice's Delta (element e is query row 32 mq
  // + 8 (e / 4) + 4 g + e % 4, the order of the Delta row in LDS), so they
  // end at Delta - dP and the dK sums are of -dS (the caller negates dK once
  // at the end); above, dS = P o (dP - Delta).
  static constexpr bool kFold = D <= 128;

  // One query tile against this wave's 32 keys, one 32-row slice at a time
  // (two waves per SIMD; one slice at a time keeps the registers low).
  static __device__ __forceinline__ void tile(const T* Qs, const T* dOs, const LdsOffsets<M, D>& lo, const float* lse2s,
                                              const float* dels, const RowFrags<M, D>& kf,
                                              const RowFrags<M, D>& vf, f32x16* dk, f32x16* dv, float c,
                                              bool masked, Window w, int i0, int kj, int sq, int g) {
#pragma unroll
    for (int mq = 0; mq < MQ; ++mq) {
      f32x16 s = zero16(), dp = zero16();
      if constexpr (kFold) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 dd = *reinterpret_cast<const float4*>(dels + 32 * mq + 8 * q4 + 4 * g);
          dp[4 * q4] = dd.x;
          dp[4 * q4 + 1] = dd.y;
          dp[4 * q4 + 2] = dd.z;
          dp[4 * q4 + 3] = dd.w;
        }
      }
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        s = M::mma(ld_row<M>(Qs + 32 * mq * L::PITCH, lo.row[st]), kf.f[st], s);
        dp = M::mma(ld_row<M>(dOs + 32 * mq * L::PITCH, lo.row[st]), vf.f[st], dp);
      }
      if (masked) {
        const long long ib = (long long)i0 + 32 * mq + 4 * g;
        mask_block(s, vis_bits((long long)kj - w.hi - ib, min((long long)kj - w.lo, (long long)sq - 1) - ib));
      }
      float p[16], ds[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 ll = *reinterpret_cast<const float4*>(lse2s + 32 * mq + 8 * q4 + 4 * g);
        const float lv[4] = {ll.x, ll.y, ll.z, ll.w};
        float dv4[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (!kFold) {
          const float4 dd = *reinterpret_cast<const float4*>(dels + 32 * mq + 8 * q4 + 4 * g);
          dv4[0] = dd.x;
          dv4[1] = dd.y;
          dv4[2] = dd.z;
          dv4[3] = dd.w;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = 4 * q4 + u;
          p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], c, -lv[u]));
          ds[e] = kFold ? p[e] * dp[e] : p[e] * (dp[e] - dv4[u]);
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        frag pf, dsf;
        M::pack(&p[8 * st], pf);
        M::pack(&ds[8 * st], dsf);
        const int rbase = (32 * mq + 16 * st) * L::PITCH;
#pragma unroll
        for (int dt = 0; dt < DVT; ++dt) {
          dv[dt] = M::mma(ld_tr<M>(dOs + rbase, lo.tra[dt], lo.trb[dt]), pf, dv[dt]);
          dk[dt] = M::mma(ld_tr<M>(Qs + rbase, lo.tra[dt], lo.trb[dt]), dsf, dk[dt]);
        }
      }
    }
  }
};

// The dK/dV tile with the optional features: logits x = c s + log2(e)
// (bias + alibi), P = 2^(x - LSE log2 e), and with dropout M = keep / (1 -
// p): dV^T += dO^T (P o M), dS = P o (M o dP - Delta).  Each lane holds one
// key, so every element needs its own dropout counter.
template <typename M, int D, int BMQ>
struct Dkdv16Feat {
  using F = Dkdv16<M, D, BMQ>;
  using T = typename M::elem;
  using L = Swz<D>;
  using frag = typename M::frag;
  static constexpr int MQ = F::MQ, NS = F::NS, DVT = F::DVT;

  static __device__ __forceinline__ void tile(const T* Qs, const T* dOs, const LdsOffsets<M, D>& lo, const float* lse2s,
                                              const float* dels, const RowFrags<M, D>& kf,
                                              const RowFrags<M, D>& vf, f32x16* dk, f32x16* dv, float c,
                                              bool masked, Window w, int i0, int kj, int sq, int sk, int g,
                                              const BwdArgs& a, int b, int h) {
    const FeatArgs& f = a.f;
#pragma unroll
    for (int mq = 0; mq < MQ; ++mq) {
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        s = M::mma(ld_row<M>(Qs + 32 * mq * L::PITCH, lo.row[st]), kf.f[st], s);
        dp = M::mma(ld_row<M>(dOs + 32 * mq * L::PITCH, lo.row[st]), vf.f[st], dp);
      }
      const int ib = i0 + 32 * mq;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        s[e] = __builtin_fmaf(s[e], c, extra_log2<T>(f, b, h, ib + acc_row(e, g), kj, sq, sk));
      if (masked) {
        const long long ibg = (long long)ib + 4 * g;
        mask_block(s, vis_bits((long long)kj - w.hi - ibg, min((long long)kj - w.lo, (long long)sq - 1) - ibg));
      }
      float p[16], ds[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int il = 32 * mq + acc_row(e, g);
        const float pe = __builtin_amdgcn_exp2f(s[e] - lse2s[il]);
        float mdp = dp[e], pm = pe;
        if (f.drop_thresh) {
          const bool kp = pe != 0.f && keep1(f, b, h, a.p.H, ib + acc_row(e, g), kj, a.p.Sq, a.p.Sk);
          mdp = kp ? dp[e] * f.drop_scale : 0.f;
          pm = kp ? pe * f.drop_scale : 0.f;
        }
        p[e] = pm;
        ds[e] = pe * (mdp - dels[il]);
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        frag pf, dsf;
        M::pack(&p[8 * st], pf);
        M::pack(&ds[8 * st], dsf);
        const int rbase = (32 * mq + 16 * st) * L::PITCH;
#pragma unroll
        for (int dt = 0; dt < DVT; ++dt) {
          dv[dt] = M::mma(ld_tr<M>(dOs + rbase, lo.tra[dt], lo.trb[dt]), pf, dv[dt]);
          dk[dt] = M::mma(ld_tr<M>(Qs + rbase, lo.tra[dt], lo.trb[dt]), dsf, dk[dt]);
        }
      }
    }
  }
};

// LDS of the 16-bit dK/dV workgroup: per stage its Q and dO tiles and the
// LSE log2(e) and Delta of its query rows.  Own arrays, one per stage and
// operand, so that the compiler can tell the tiles being read from those
// being filled by direct loads and does not wait for those loads before
// every read; with EXT the two namespace-scope stages, one array per stage
// (the split grid, whose dQ workgroups use the same two).
template <typename T, int TILE, int BMQ, bool EXT>
struct Dkdv16Lds {
  T* q[2];
  T* d[2];
  float* l[2];
  float* e[2];
  __device__ __forceinline__ Dkdv16Lds() {
    if constexpr (EXT) {
      static_assert(2 * TILE * (int)sizeof(T) + 2 * BMQ * 4 <= kBwdStageBytes, "tiles fit a stage");
      char* const st[2] = {g_bwd_st0, g_bwd_st1};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        q[u] = reinterpret_cast<T*>(st[u]);
        d[u] = q[u] + TILE;
        l[u] = reinterpret_cast<float*>(d[u] + TILE);
        e[u] = l[u] + BMQ;
      }
    } else {
      __shared__ __attribute__((aligned(1024))) T q_s0[TILE], q_s1[TILE];
      __shared__ __attribute__((aligned(1024))) T d_s0[TILE], d_s1[TILE];
      __shared__ __attribute__((aligned(16))) float l_s0[BMQ], l_s1[BMQ], e_s0[BMQ], e_s1[BMQ];
      q[0] = q_s0;
      q[1] = q_s1;
      d[0] = d_s0;
      d[1] = d_s1;
      l[0] = l_s0;
      l[1] = l_s1;
      e[0] = e_s0;
      e[1] = e_s1;
    }
  }
};

template <typename M, int D, int NW, int BMQ, bool FEAT, bool SPLIT, bool EXT = false>
__device__ __forceinline__ void dkdv16_body(const BwdArgs& a, unsigned hw, unsigned nblk) {
  using F = Dkdv16<M, D, BMQ>;
  using T = typename M::elem;
  using DL = DmaLane<T, D, BMQ, NW>;
  constexpr int NT = NW * 64, BNK = NW * 32, DVT = F::DVT;
  constexpr int RW = BMQ / NW;  // LSE / Delta rows each wave copies per tile
  static_assert(BMQ % NW == 0 && RW <= 64, "stats rows");
  const Dkdv16Lds<T, F::TILE, BMQ, EXT> lds;

  const ProblemArgs& P = a.p;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int nbh = P.B * P.H;
  const int nsplit = SPLIT ? a.split_kv : 1;
  const int nkb = (int)(nblk / ((unsigned)nbh * nsplit));
  const int sg = (int)(hw / (unsigned)(nkb * nbh));  // split copy (0 without split)
  const GridPos gp = grid_pos((int)(hw % (unsigned)(nkb * nbh)), nkb * nbh, nkb, nbh, P.ragged);
  const int bh = gp.bh, h = bh % P.H, b = bh / P.H;
  const int kb = gp.i;

  long long q0, k0;
  int sq, sk;
  seq_rows(P, b, q0, sq, k0, sk);
  const int j0 = kb * BNK;
  if (j0 >= sk) return;
  const Window w = seq_window(P.wl, P.wr, P.diag, sq, sk);

  const T* qp = (const T*)a.q.ptr + b * a.q.sb + h * a.q.sh + q0 * a.q.ss;
  const T* kp = (const T*)a.k.ptr + b * a.k.sb + h * a.k.sh + k0 * a.k.ss;
  const T* vp = (const T*)a.v.ptr + b * a.v.sb + h * a.v.sh + k0 * a.v.ss;
  const T* dop = (const T*)a.dout.ptr + b * a.dout.sb + h * a.dout.sh + q0 * a.dout.ss;
  T* dkp = (T*)a.dk.ptr + b * a.dk.sb + h * a.dk.sh + k0 * a.dk.ss;
  T* dvp = (T*)a.dv.ptr + b * a.dv.sb + h * a.dv.sh + k0 * a.dv.ss;
  const float* l2p = a.lse2 + b * P.lse_sb + h * P.lse_sh + q0;
  const float* delp = a.delta + b * P.lse_sb + h * P.lse_sh + q0;

  // Queries that can see the block's keys, and the tiles of this wave's keys.
  const int jlast = min(j0 + BNK, sk) - 1;
  long long ilo = max(0LL, (long long)j0 - w.hi);
  long long ihi = min((long long)sq - 1, (long long)jlast - w.lo);
  if constexpr (SPLIT) split_rows(ilo, ihi, BMQ, sg, nsplit);
  const bool block_empty = w.lo > w.hi || ilo > ihi;

  const int jw0 = j0 + 32 * wave;
  const bool wave_live = jw0 < sk;
  const int kj = jw0 + r;
  int tw0 = 0x7fffffff, tw1 = -1;
  if (wave_live && w.lo <= w.hi) {
    const long long a0 = max(0LL, (long long)jw0 - w.hi);
    const long long a1 = min((long long)sq - 1, (long long)min(jw0 + 31, sk - 1) - w.lo);
    if (a0 <= a1) {
      tw0 = (int)(a0 / BMQ);
      tw1 = (int)(a1 / BMQ);
    }
  }

  RowFrags<M, D> kf, vf;
  kf.load(kp + (long long)kj * a.k.ss, wave_live && kj < sk, g);
  vf.load(vp + (long long)kj * a.v.ss, wave_live && kj < sk, g);
  const float c = fmaxf(fabsf(P.scale_log2), 1e-30f);
  if (P.scale_log2 < 0.f) kf.negate();
  if constexpr (!FEAT && F::kFold) vf.negate();  // Dkdv16::tile takes -V (its dP starts from Delta)

  f32x16 dk[DVT], dv[DVT];
#pragma unroll
  for (int dt = 0; dt < DVT; ++dt) {
    dk[dt] = zero16();
    dv[dt] = zero16();
  }

  if (!block_empty) {
    LdsOffsets<M, D> lo;
    lo.init(lane);
    DL qd, dd;
    qd.init(a.q.ss, wave, lane);
    dd.init(a.dout.ss, wave, lane);
    T* const qs[2] = {lds.q[0], lds.q[1]};
    T* const ds_[2] = {lds.d[0], lds.d[1]};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      zero_unused_slots<T, D, BMQ, NT>(qs[u], tid);
      zero_unused_slots<T, D, BMQ, NT>(ds_[u], tid);
    }
    const int t0 = (int)(ilo / BMQ), t1 = (int)(ihi / BMQ);
    // One tile's loads, all direct to LDS: its Q and dO rows and, per wave,
    // RW rows of LSE log2(e) and Delta (rows past the sequence repeat its
    // last row and are masked).
    float* const ls[2] = {lds.l[0], lds.l[1]};
    float* const es[2] = {lds.e[0], lds.e[1]};
    auto issue = [&](int stage, int t) {
      const int i0 = t * BMQ;
      qd.issue(qs[stage], qp + (long long)i0 * a.q.ss, a.q.ss, sq - i0, wave, lane);
      dd.issue(ds_[stage], dop + (long long)i0 * a.dout.ss, a.dout.ss, sq - i0, wave, lane);
      if (lane < RW) {
        const int off = 4 * (min(i0 + wave * RW + lane, sq - 1) - i0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(l2p + i0), (lds_void*)(ls[stage] + wave * RW), 4, off, 0,
                                                 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(delp + i0), (lds_void*)(es[stage] + wave * RW), 4, off, 0,
                                                 0, 0);
      }
    };
    issue(0, t0);
    __syncthreads();
    // Step t: tile t sits in stage (t - t0) & 1; the loads of tile t+1 go
    // into the other stage during the step.
    auto step = [&](auto parity, int t) {
      constexpr int Pq = decltype(parity)::value;
      if (t + 1 <= t1) issue(Pq ^ 1, t + 1);
      if (tw0 <= t && t <= tw1) {
        const bool masked =
            classify(w, (long long)t * BMQ, BMQ, jw0, 32, sk) == kPartial || (t + 1) * BMQ > sq;
        if constexpr (FEAT)
          Dkdv16Feat<M, D, BMQ>::tile(qs[Pq], ds_[Pq], lo, ls[Pq], es[Pq], kf, vf, dk, dv, c, masked, w, t * BMQ, kj,
                                      sq, sk, g, a, b, h);
        else
          F::tile(qs[Pq], ds_[Pq], lo, ls[Pq], es[Pq], kf, vf, dk, dv, c, masked, w, t * BMQ, kj, sq, g);
      }
      __syncthreads();
    };
    for (int t = t0; t <= t1; t += 2) {
      step(std::integral_constant<int, 0>{}, t);
      if (t + 1 <= t1) step(std::integral_constant<int, 1>{}, t + 1);
    }
  }
  if constexpr (!FEAT && F::kFold) {
    // Dkdv16::tile summed -dS: dK's sign back, once.
#pragma unroll
    for (int dt = 0; dt < DVT; ++dt) dk[dt] = -dk[dt];
  }

  if constexpr (SPLIT) {
    if (wave_live && kj < sk)
      store_partial_kv<D>(a.part, a.rows_k, a.split_kv, P.H, sg, h, part_row(P.ks.mode, P.Sk, b, k0, kj), dk, dv, g);
    if (a.cnt_kv != nullptr && last_arrival(a.cnt_kv + (long long)bh * nkb + kb, nsplit))
      sum_partials<T, D, NT, true>(a.part, a.rows_k, P.H, nsplit, h, P.ks.mode, P.Sk, b, k0, j0, jlast + 1, dkp,
                                   a.dk.ss, dvp, a.dv.ss, P.scale, tid);
  } else if (wave_live && kj < sk) {
    T* dkrow = dkp + (long long)kj * a.dk.ss;
    T* dvrow = dvp + (long long)kj * a.dv.ss;
    const float sc = P.scale;
#pragma unroll
    for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * dt + 8 * q4 + 4 * g;
        if (d < D) {
          store4b<T>(dkrow + d, dk[dt][4 * q4] * sc, dk[dt][4 * q4 + 1] * sc,
                     dk[dt][4 * q4 + 2] * sc, dk[dt][4 * q4 + 3] * sc);
          store4b<T>(dvrow + d, dv[dt][4 * q4], dv[dt][4 * q4 + 1], dv[dt][4 * q4 + 2],
                     dv[dt][4 * q4 + 3]);
        }
      }
  }
}

template <typename M, int D, int NW, int BMQ, int WPE, bool FEAT = false, bool SPLIT = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void attn_bwd_dkdv16_kernel(BwdArgs a) {
  dkdv16_body<M, D, NW, BMQ, FEAT, SPLIT>(a, blockIdx.x, gridDim.x);
}

// ------------------------------------- 16-bit dK/dV, producer / consumer
//
// Eight waves for 128 keys.  Waves w and w+4 share a SIMD and own keys
// 32w .. 32w+31 of the block: w is the producer, w+4 the consumer.  For
// query tile t (64 rows), in one step between two barriers:
//   producer: S^T = K Q^T; P^T = 2^(c S^T - LSE log2 e), 0 where masked;
//             P^T to LDS in fp16; dV += P^T dO;
//   consumer: dS^T = P^T o (dP^T - Delta) for tile t-1 (its P^T from LDS,
//             dP^T kept from the previous step); dK += dS^T Q; then
//             dP^T = V dO^T of tile t.
// The consumer's vector work runs while the producer's S products run, the
// producer's softmax while the consumer's dK products run.  Q, dO, LSE
// log2(e) and Delta of tile t+1 are copied during step t (three stages: the
// consumer still reads tile t-1), P^T of each step gets its own of three
// buffers.  Each role needs only K or V and only dV or dK, so two waves fit
// in one SIMD's registers.

// The kernel's BwdArgs argument, read in place from the kernel-argument
// segment (a kernel whose first argument is BwdArgs).  Bodies shared by
// several kernels take it this way, so no private copy of the struct is made.
using KBwdArgs = const __attribute__((address_space(4))) BwdArgs;
__device__ __forceinline__ KBwdArgs& kernel_bwd_args() {
  return *(KBwdArgs*)__builtin_amdgcn_kernarg_segment_ptr();
}

// A private copy of the feature arguments (field by field: the implicit
// copy constructor does not take the kernel-argument address space).
__device__ __forceinline__ FeatArgs feat_args(KBwdArgs& a) {
  FeatArgs f;
  f.bias = a.f.bias;
  f.bsb = a.f.bsb;
  f.bsh = a.f.bsh;
  f.bss = a.f.bss;
  f.alibi = a.f.alibi;
  f.offset = a.f.offset;
  f.seed_lo = a.f.seed_lo;
  f.seed_hi = a.f.seed_hi;
  f.drop_thresh = a.f.drop_thresh;
  f.drop_scale = a.f.drop_scale;
  f.dbias = a.f.dbias;
  f.dsb = a.f.dsb;
  f.dsh = a.f.dsh;
  f.dss = a.f.dss;
  return f;
}

// Calls f(integral_constant<int, I>) for I = B .. E-1 in order.
template <int B, class Fn, int... Is>
__device__ __forceinline__ void static_for_impl(Fn&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, B + Is>{}), ...);
}
template <int B, int E, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  static_for_impl<B>(f, std::make_integer_sequence<int, E - B>{});
}

// Products B .. E-1 of a sequence, each with one LDS operand: load(i) reads
// product i's operand PD products ahead, prod(i, A) issues it, after(i) runs
// after it (vector work placed between products; after(B-1) runs once the
// first operands are requested, before the first product).
template <int B, int E, int PD, class Load, class Prod, class After>
__device__ __forceinline__ void mfma_stream(Load&& load, Prod&& prod, After&& after) {
  constexpr int D = PD < E - B ? PD : E - B;
  using frag = decltype(load(std::integral_constant<int, B>{}));
  frag buf[D];
  static_for<0, D>([&](auto i) __attribute__((always_inline)) { buf[i] = load(std::integral_constant<int, B + decltype(i)::value>{}); });
  after(std::integral_constant<int, B - 1>{});  // work placed before the first product
  static_for<B, E>([&](auto i) __attribute__((always_inline)) {
    constexpr int I = decltype(i)::value;
    const frag A = buf[(I - B) % D];
    if constexpr (I + D < E) buf[(I - B) % D] = load(std::integral_constant<int, I + D>{});
    prod(i, A);
    after(i);
  });
}

template <typename M, int D>
struct DkdvPC {
  using T = typename M::elem;
  using L = Swz<D>;
  using frag = typename M::frag;
  static constexpr int BMQ = 64, MQ = 2, NS = D / 16, DVT = (D + 31) / 32;
  static constexpr int TILE = BMQ * L::PITCH;              // elements of one Q or dO tile
  static constexpr int STAGE = 2 * TILE + 4 * BMQ * 4 / (int)sizeof(T);  // Q, dO, LSE log2 e, Delta
  static constexpr int XFR = 4 * MQ * 2 * 64;              // fp16 x8 fragments of one P buffer
  static_assert(STAGE * (int)sizeof(T) <= kBwdStageBytes && XFR * 16 <= kBwdXBytes, "LDS arrays");
  static constexpr int NA = MQ * NS, NB = MQ * 2 * DVT;    // row-read products, transposed-read products
  static constexpr int PD = 4;  // LDS operand reads ahead of the products

  // fp16 copy of 8 probabilities (exactly the MFMA fragment for fp16 input).
  static __device__ __forceinline__ f16x8 half8(const float* x, const frag& f) {
    if constexpr (std::is_same<T, _Float16>::value) {
      return f;
    } else {
      f16x8 h;
      MmaF16::pack(x, h);
      return h;
    }
  }
  // Operand of row-read product i (< NA): rows 32 (i / NS) .. +31, K step i % NS.
  static __device__ __forceinline__ frag row_op(const T* tile, const LdsOffsets<M, D>& lo, int i) {
    return ld_row<M>(tile + 32 * (i / NS) * L::PITCH, lo.row[i % NS]);
  }
  // Operand of transposed product j (< NB): rows 32 mq + 16 h .. +15 with
  // (mq, h, dt) = (j / (2 DVT), (j / DVT) % 2, j % DVT).
  static __device__ __forceinline__ frag tr_op(const T* tile, const LdsOffsets<M, D>& lo, int j) {
    const int dt = j % DVT;
    return ld_tr<M>(tile + (32 * (j / (2 * DVT)) + 16 * ((j / DVT) % 2)) * L::PITCH, lo.tra[dt], lo.trb[dt]);
  }

  // Producer: S, P (kept rounded for dV, stored in fp16 for the consumer), dV.
  static __device__ __forceinline__ void produce(const T* st, f16x8* xb, const LdsOffsets<M, D>& lo,
                                                 const RowFrags<M, D>& kf, f32x16* dv, float c, bool masked,
                                                 Window w, int i0, int kj, int sq, int kw, int lane, int g) {
    const T* Qs = st;
    const T* dOs = st + TILE;
    const float* l2 = reinterpret_cast<const float*>(st + 2 * TILE);
    f32x16 s[MQ];
    frag pf[MQ][2];
    // Slice MQ's probabilities: masked, 2^(c s - LSE log2 e), rounded for dV
    // and copied in fp16 for the consumer.
    auto softmax = [&](auto mqc) __attribute__((always_inline)) {
      constexpr int mq = decltype(mqc)::value;
      if (masked) {
        // Query i = ib + r(e) sees key kj iff kj - hi <= i <= min(kj - lo, sq - 1).
        const long long ib = (long long)i0 + 32 * mq + 4 * g;
        mask_block(s[mq], vis_bits((long long)kj - w.hi - ib, min((long long)kj - w.lo, (long long)sq - 1) - ib));
      }
      float p[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 ll = *reinterpret_cast<const float4*>(l2 + 32 * mq + 8 * q4 + 4 * g);
        const float lv[4] = {ll.x, ll.y, ll.z, ll.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          p[4 * q4 + u] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mq][4 * q4 + u], c, -lv[u]));
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        M::pack(&p[8 * h], pf[mq][h]);
        xb[((kw * MQ + mq) * 2 + h) * 64 + lane] = half8(&p[8 * h], pf[mq][h]);
      }
    };
    mfma_stream<0, NA + NB, PD>(
        [&](auto i) __attribute__((always_inline)) { return decltype(i)::value < NA ? row_op(Qs, lo, decltype(i)::value)
                                                     : tr_op(dOs, lo, decltype(i)::value - NA); },
        [&](auto i, const frag& A) __attribute__((always_inline)) {
          constexpr int I = decltype(i)::value;
          if constexpr (I < NA) {
            constexpr int mq = I / NS, k = I % NS;
            s[mq] = M::mma(A, kf.f[k], k == 0 ? zero16() : s[mq]);
          } else {
            constexpr int j = I - NA, dt = j % DVT;
            dv[dt] = M::mma(A, pf[j / (2 * DVT)][(j / DVT) % 2], dv[dt]);
          }
        },
        [&](auto i) __attribute__((always_inline)) {
          // Slice 0's softmax under slice 1's S products, slice 1's under
          // slice 0's dV products.
          static_assert(MQ == 2, "two slices");
          if constexpr (decltype(i)::value == NS - 1) softmax(std::integral_constant<int, 0>{});
          if constexpr (decltype(i)::value == NA - 1) softmax(std::integral_constant<int, 1>{});
        });
  }

  // Consumer: dS of the previous tile (stage sp, P buffer xb) and
  // dK += dS^T Q (when FIN), then dP^T = V dO^T of the current tile (stage
  // sc, when DP).  The consumer's V fragments are negated and its dP^T
  // accumulators start from the tile's Delta (element e of slice mq is row
  // 32 mq + 8 (e / 4) + 4 g + e % 4, the order of the Delta row in LDS), so
  // they hold Delta - dP and dS comes out negated (one multiply per
  // element); the dK epilogue scales by -scale.
  template <bool FIN, bool DP>
  static __device__ __forceinline__ void consume(const T* sp, const f16x8* xb, const T* sc,
                                                 const LdsOffsets<M, D>& lo, const RowFrags<M, D>& vf, f32x16* dp,
                                                 f32x16* dk, int kw, int lane, int g) {
    const T* Qp = sp;
    const T* dOs = sc + TILE;
    frag dsf[MQ][2];
    // -dS of slice MQ, rounded for dK.
    auto ds_slice = [&](auto mqc) __attribute__((always_inline)) {
      constexpr int mq = decltype(mqc)::value;
      const f16x8 h0 = xb[((kw * MQ + mq) * 2 + 0) * 64 + lane], h1 = xb[((kw * MQ + mq) * 2 + 1) * 64 + lane];
      float ds[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) ds[e] = (float)(e < 8 ? h0[e] : h1[e - 8]) * dp[mq][e];
      M::pack(&ds[0], dsf[mq][0]);
      M::pack(&ds[8], dsf[mq][1]);
    };
    if constexpr (DP) {
      const float* del = reinterpret_cast<const float*>(sc + 2 * TILE) + BMQ;
#pragma unroll
      for (int mq = 0; mq < MQ; ++mq)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 dd = *reinterpret_cast<const float4*>(del + 32 * mq + 8 * q4 + 4 * g);
          dp[mq][4 * q4] = dd.x;
          dp[mq][4 * q4 + 1] = dd.y;
          dp[mq][4 * q4 + 2] = dd.z;
          dp[mq][4 * q4 + 3] = dd.w;
        }
    }
    constexpr int B = FIN ? 0 : NB, E = DP ? NB + NA : NB;
    mfma_stream<B, E, PD>(
        [&](auto i) __attribute__((always_inline)) { return decltype(i)::value < NB ? tr_op(Qp, lo, decltype(i)::value)
                                                     : row_op(dOs, lo, decltype(i)::value - NB); },
        [&](auto i, const frag& A) __attribute__((always_inline)) {
          constexpr int I = decltype(i)::value;
          if constexpr (I < NB) {
            constexpr int dt = I % DVT;
            dk[dt] = M::mma(A, dsf[I / (2 * DVT)][(I / DVT) % 2], dk[dt]);
          } else {
            constexpr int j = I - NB, mq = j / NS, k = j % NS;
            dp[mq] = M::mma(A, vf.f[k], dp[mq]);
          }
        },
        [&](auto i) __attribute__((always_inline)) {
          // Slice 0's dS before the first dK product, slice 1's under slice
          // 0's dK products.
          if constexpr (FIN && decltype(i)::value == -1) ds_slice(std::integral_constant<int, 0>{});
          if constexpr (FIN && decltype(i)::value == 0) ds_slice(std::integral_constant<int, 1>{});
        });
  }
};

// The producer / consumer dK/dV workgroup's work: block hw of nblk, in the
// namespace-scope LDS stages and P buffers.
template <typename M, int D>
__device__ __forceinline__ void dkdv_pc_body(int hw, int nblk) {
  using F = DkdvPC<M, D>;
  using T = typename M::elem;
  using DL = DmaLane<T, D, F::BMQ, 4>;  // copies by the four producer waves
  constexpr int NT = 512, BMQ = F::BMQ, DVT = F::DVT, BNK = 128, RW = BMQ / 4;
  KBwdArgs& a = kernel_bwd_args();
  T* const st0 = reinterpret_cast<T*>(g_bwd_st0);
  T* const st1 = reinterpret_cast<T*>(g_bwd_st1);
  T* const st2 = reinterpret_cast<T*>(g_bwd_st2);
  f16x8* const x0 = reinterpret_cast<f16x8*>(g_bwd_x0);
  f16x8* const x1 = reinterpret_cast<f16x8*>(g_bwd_x1);
  f16x8* const x2 = reinterpret_cast<f16x8*>(g_bwd_x2);

  const auto& P = a.p;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const bool prod = wave < 4;
  const int kw = wave & 3;
  const int nkb = nblk / (P.B * P.H);
  const GridPos gp = grid_pos(hw, nblk, nkb, P.B * P.H, P.ragged);
  const int bh = gp.bh, h = bh % P.H, b = bh / P.H;
  const int kb = gp.i;

  long long q0, k0;
  int sq, sk;
  seq_rows(P, b, q0, sq, k0, sk);
  const int j0 = kb * BNK;
  if (j0 >= sk) return;
  const Window w = seq_window(P.wl, P.wr, P.diag, sq, sk);

  const T* qp = (const T*)a.q.ptr + b * a.q.sb + h * a.q.sh + q0 * a.q.ss;
  const T* kp = (const T*)a.k.ptr + b * a.k.sb + h * a.k.sh + k0 * a.k.ss;
  const T* vp = (const T*)a.v.ptr + b * a.v.sb + h * a.v.sh + k0 * a.v.ss;
  const T* dop = (const T*)a.dout.ptr + b * a.dout.sb + h * a.dout.sh + q0 * a.dout.ss;
  T* dkp = (T*)a.dk.ptr + b * a.dk.sb + h * a.dk.sh + k0 * a.dk.ss;
  T* dvp = (T*)a.dv.ptr + b * a.dv.sb + h * a.dv.sh + k0 * a.dv.ss;
  const float* l2p = a.lse2 + b * P.lse_sb + h * P.lse_sh + q0;
  const float* delp = a.delta + b * P.lse_sb + h * P.lse_sh + q0;

  const int jlast = min(j0 + BNK, sk) - 1;
  const long long ilo = max(0LL, (long long)j0 - w.hi);
  const long long ihi = min((long long)sq - 1, (long long)jlast - w.lo);
  const bool block_empty = w.lo > w.hi || ilo > ihi;

  const int jw0 = j0 + 32 * kw;
  const bool wave_live = jw0 < sk;
  const int kj = jw0 + r;
  int tw0 = 0x7fffffff, tw1 = -1;
  if (wave_live && w.lo <= w.hi) {
    const long long a0 = max(0LL, (long long)jw0 - w.hi);
    const long long a1 = min((long long)sq - 1, (long long)min(jw0 + 31, sk - 1) - w.lo);
    if (a0 <= a1) {
      tw0 = (int)(a0 / BMQ);
      tw1 = (int)(a1 / BMQ);
    }
  }

  // The producer holds its keys' K rows, the consumer their V rows.
  RowFrags<M, D> kv;
  kv.load(prod ? kp + (long long)kj * a.k.ss : vp + (long long)kj * a.v.ss, wave_live && kj < sk, g);
  const float c = fmaxf(fabsf(P.scale_log2), 1e-30f);
  if (prod ? P.scale_log2 < 0.f : true) kv.negate();  // consumers: -V (their dP^T starts from Delta)

  f32x16 acc[DVT];  // producer: dV, consumer: dK
#pragma unroll
  for (int dt = 0; dt < DVT; ++dt) acc[dt] = zero16();

  if (!block_empty) {
    LdsOffsets<M, D> lo;
    lo.init(lane);
    DL qd, dd;
    qd.init(a.q.ss, kw, lane);
    dd.init(a.dout.ss, kw, lane);
    // Stage and P buffer u, chosen at compile time so that every LDS access
    // names its own array.
    auto stg = [&](auto u) __attribute__((always_inline)) -> T* {
      constexpr int U = decltype(u)::value;
      return U == 0 ? st0 : (U == 1 ? st1 : st2);
    };
    auto xs = [&](auto u) __attribute__((always_inline)) -> f16x8* {
      constexpr int U = decltype(u)::value;
      return U == 0 ? x0 : (U == 1 ? x1 : x2);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    for (T* st : {st0, st1, st2}) {
      zero_unused_slots<T, D, BMQ, NT>(st, tid);
      zero_unused_slots<T, D, BMQ, NT>(st + F::TILE, tid);
    }
    const int t0 = (int)(ilo / BMQ), n = (int)(ihi / BMQ) - t0 + 1;
    // Tile copies, all direct to LDS (rows past the sequence repeat its last
    // row and are masked), issued by the producer waves only: they wait for
    // the consumer at every barrier, while copy instructions hold up the wave
    // that issues them, and the consumer's step is the longer one.  Every
    // producer wave copies RW rows of the statistics.
    auto issue = [&](T* dst, int t) __attribute__((always_inline)) {
      const int i0 = t * BMQ;
      qd.issue(dst, qp + (long long)i0 * a.q.ss, a.q.ss, sq - i0, kw, lane);
      dd.issue(dst + F::TILE, dop + (long long)i0 * a.dout.ss, a.dout.ss, sq - i0, kw, lane);
      if (lane < RW) {
        float* sts = reinterpret_cast<float*>(dst + 2 * F::TILE);
        const int off = 4 * (min(i0 + kw * RW + lane, sq - 1) - i0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(l2p + i0), (lds_void*)(sts + kw * RW), 4, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(delp + i0), (lds_void*)(sts + BMQ + kw * RW), 4, off, 0, 0,
                                                 0);
      }
    };
    // End of a step: this wave's copies and LDS traffic are complete
    // (explicit wait the compiler accounts for), then the workgroup barrier.
    auto barrier = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0x0070);
      asm volatile("s_barrier" ::: "memory");
    };
    auto mine = [&](int t) __attribute__((always_inline)) { return tw0 <= t && t <= tw1; };
    auto masked_at = [&](int t) __attribute__((always_inline)) {
      return classify(w, (long long)t * BMQ, BMQ, jw0, 32, sk) == kPartial || (t + 1) * BMQ > sq;
    };
    if (prod) issue(st0, t0);
    barrier();
    // Step it (tile t0+it in stage it % 3): copies of the next tile, this
    // role's work, barrier.  One loop per role, so that the consumer's dP^T
    // is not carried through the producer's code.
    auto run = [&](auto role) __attribute__((always_inline)) {
      constexpr bool PROD = decltype(role)::value;
      f32x16 dp[F::MQ];  // consumer: dP^T of the last tile
      auto step = [&](auto sc, int it) __attribute__((always_inline)) {
        constexpr int SI = decltype(sc)::value, SN = (SI + 1) % 3, SP = (SI + 2) % 3;
        using CI = std::integral_constant<int, SI>;
        using CN = std::integral_constant<int, SN>;
        using CP = std::integral_constant<int, SP>;
        const int t = t0 + it;
        if (PROD && it + 1 < n) issue(stg(CN{}), t + 1);
        if constexpr (PROD) {
          if (mine(t))
            F::produce(stg(CI{}), xs(CI{}), lo, kv, acc, c, masked_at(t), w, t * BMQ, kj, sq, kw, lane, g);
        } else {
          if (it >= 1 && mine(t - 1))
            F::template consume<true, false>(stg(CP{}), xs(CP{}), stg(CI{}), lo, kv, dp, acc, kw, lane, g);
          if (mine(t))
            F::template consume<false, true>(stg(CP{}), xs(CP{}), stg(CI{}), lo, kv, dp, acc, kw, lane, g);
        }
        barrier();
      };
      int it = 0;
      for (; it + 3 <= n; it += 3) {
        step(I0{}, it);
        step(I1{}, it + 1);
        step(I2{}, it + 2);
      }
      if (it < n) step(I0{}, it);
      if (it + 1 < n) step(I1{}, it + 1);
      // The consumer's dS / dK of the last tile.
      if constexpr (!PROD) {
        // No copy is in flight any more, so the stage can be picked at run time.
        if (mine(t0 + n - 1)) {
          const int sl = (n - 1) % 3;
          const T* sp = sl == 0 ? st0 : (sl == 1 ? st1 : st2);
          const f16x8* xp = sl == 0 ? x0 : (sl == 1 ? x1 : x2);
          F::template consume<true, false>(sp, xp, sp, lo, kv, dp, acc, kw, lane, g);
        }
      }
    };
    if (prod)
      run(std::true_type{});
    else
      run(std::false_type{});
  }

  if (wave_live && kj < sk) {
    T* row = prod ? dvp + (long long)kj * a.dv.ss : dkp + (long long)kj * a.dk.ss;
    const float sc = prod ? 1.f : -P.scale;  // the consumer's sums are of -dS
#pragma unroll
    for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * dt + 8 * q4 + 4 * g;
        if (d < D)
          store4b<T>(row + d, acc[dt][4 * q4] * sc, acc[dt][4 * q4 + 1] * sc, acc[dt][4 * q4 + 2] * sc,
                     acc[dt][4 * q4 + 3] * sc);
      }
  }
}

template <typename M, int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_dkdv16pc_kernel(BwdArgs) {
  dkdv_pc_body<M, D>(blockIdx.x, gridDim.x);
}

// ------------------------------------------------- 16-bit dQ kernel
//
// One workgroup = 32*NW queries; each wave keeps its 32 queries' Q and dO
// rows, LSE and Delta in registers and walks the key tiles its rows can
// see, K and V copied HBM -> LDS as in the forward.  Per 32-key slice:
// S^T = K Q^T and dP^T - Delta = V dO^T - Delta from row reads (the first
// product of dP^T accumulates onto a register block of -Delta: a lane's
// elements all belong to its query row, so the block is the same for every
// tile), dS^T = P^T o (dP^T - Delta), dQ^T += K^T dS^T with K^T taken by
// transposing reads.  Key rows past the
// sequence are copies of its last key and are masked out.
template <typename M, int D, int BN>
struct Dq16 {
  using T = typename M::elem;
  using L = Swz<D>;
  using frag = typename M::frag;
  static constexpr int KT = BN / 32, NS = D / 16, DVT = (D + 31) / 32;
  static constexpr int TILE = BN * L::PITCH;

  // One key tile (KT 32-key slices) against this wave's 32 queries.
  // Head_dim <= 80: one ordered stream of products with LDS operands read
  // ahead (S and dP of every slice, then dQ += dS K slice by slice; slice
  // kt's dS is computed under the next products once its S and dP are
  // complete).  Head_dim 128: slice by slice, which keeps both slices' S and
  // dP out of the registers at two waves per SIMD.
  static constexpr int NA = 2 * NS, NB = 2 * DVT;  // products per slice: S and dP, dQ
  static __device__ __forceinline__ void tile(const T* Ks, const T* Vs, const LdsOffsets<M, D>& lo,
                                              const RowFrags<M, D>& qf, const RowFrags<M, D>& dof, f32x16* dq,
                                              float c, float lse2, const f32x16& ndelta, bool masked, Window w,
                                              int j0, int qi, int sk, int g) {
    if constexpr (D > 80) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        f32x16 s = zero16(), dp = ndelta;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          s = M::mma(ld_row<M>(Ks + 32 * kt * L::PITCH, lo.row[st]), qf.f[st], s);
          dp = M::mma(ld_row<M>(Vs + 32 * kt * L::PITCH, lo.row[st]), dof.f[st], dp);
        }
        if (masked) {
          const long long jb = (long long)j0 + 32 * kt + 4 * g;
          mask_block(s, vis_bits((long long)qi + w.lo - jb, min((long long)qi + w.hi, (long long)sk - 1) - jb));
        }
        float ds[16];
#pragma unroll
        for (int e = 0; e < 16; ++e)
          ds[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], c, -lse2)) * dp[e];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          frag dsf;
          M::pack(&ds[8 * st], dsf);
          const int rbase = (32 * kt + 16 * st) * L::PITCH;
#pragma unroll
          for (int dt = 0; dt < DVT; ++dt)
            dq[dt] = M::mma(ld_tr<M>(Ks + rbase, lo.tra[dt], lo.trb[dt]), dsf, dq[dt]);
        }
      }
    } else {
    f32x16 s[KT], dp[KT];
    frag dsf[KT][2];
    auto ds_slice = [&](auto ktc) __attribute__((always_inline)) {
      constexpr int kt = decltype(ktc)::value;
      if (masked) {
        const long long jb = (long long)j0 + 32 * kt + 4 * g;
        mask_block(s[kt], vis_bits((long long)qi + w.lo - jb, min((long long)qi + w.hi, (long long)sk - 1) - jb));
      }
      float ds[16];
#pragma unroll
      for (int e = 0; e < 16; ++e)
        ds[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][e], c, -lse2)) * dp[kt][e];
      M::pack(&ds[0], dsf[kt][0]);
      M::pack(&ds[8], dsf[kt][1]);
    };
    mfma_stream<0, KT * (NA + NB), 4>(
        [&](auto i) __attribute__((always_inline)) {
          constexpr int I = decltype(i)::value;
          if constexpr (I < KT * NA) {
            constexpr int kt = I / NA, st = (I % NA) / 2;
            return ld_row<M>(((I & 1) ? Vs : Ks) + 32 * kt * L::PITCH, lo.row[st]);
          } else {
            constexpr int j = I - KT * NA, kt = j / NB, st = (j % NB) / DVT, dt = j % DVT;
            return ld_tr<M>(Ks + (32 * kt + 16 * st) * L::PITCH, lo.tra[dt], lo.trb[dt]);
          }
        },
        [&](auto i, const frag& A) __attribute__((always_inline)) {
          constexpr int I = decltype(i)::value;
          if constexpr (I < KT * NA) {
            constexpr int kt = I / NA, st = (I % NA) / 2;
            if constexpr (I & 1)
              dp[kt] = M::mma(A, dof.f[st], st == 0 ? ndelta : dp[kt]);
            else
              s[kt] = M::mma(A, qf.f[st], st == 0 ? zero16() : s[kt]);
          } else {
            constexpr int j = I - KT * NA, kt = j / NB, st = (j % NB) / DVT, dt = j % DVT;
            dq[dt] = M::mma(A, dsf[kt][st], dq[dt]);
          }
        },
        [&](auto i) __attribute__((always_inline)) {
          constexpr int I = decltype(i)::value;
          static_assert(KT == 2, "two slices");
          if constexpr (I == NA - 1) ds_slice(std::integral_constant<int, 0>{});
          if constexpr (I == KT * NA - 1) ds_slice(std::integral_constant<int, 1>{});
        });
    }
  }
};

// The dQ tile with the optional features: logits x = c s + log2(e)
// (bias + alibi), P = 2^(x - LSE log2 e), with dropout M = keep / (1 - p):
// dS = P o (M o dP - Delta), dQ^T += K^T dS^T; dS is also d loss / d logit,
// stored to dbias when asked for.  One counter serves the lane's four
// consecutive keys.
template <typename M, int D, int BN>
struct Dq16Feat {
  using F = Dq16<M, D, BN>;
  using T = typename M::elem;
  using L = Swz<D>;
  using frag = typename M::frag;
  static constexpr int KT = F::KT, NS = F::NS, DVT = F::DVT;

  static __device__ __forceinline__ void tile(const T* Ks, const T* Vs, const LdsOffsets<M, D>& lo,
                                              const RowFrags<M, D>& qf, const RowFrags<M, D>& dof, f32x16* dq,
                                              float c, float lse2, float delta, bool masked, Window w, int j0, int qi,
                                              int sq, int sk, int g, const FeatArgs& f, int b, int h, int H, int Sq,
                                              int Sk, bool row_ok) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        s = M::mma(ld_row<M>(Ks + 32 * kt * L::PITCH, lo.row[st]), qf.f[st], s);
        dp = M::mma(ld_row<M>(Vs + 32 * kt * L::PITCH, lo.row[st]), dof.f[st], dp);
      }
      const int jb = j0 + 32 * kt;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = __builtin_fmaf(s[e], c, extra_log2<T>(f, b, h, qi, jb + acc_row(e, g), sq, sk));
      if (masked) {
        const long long jbg = (long long)jb + 4 * g;
        mask_block(s, vis_bits((long long)qi + w.lo - jbg, min((long long)qi + w.hi, (long long)sk - 1) - jbg));
      }
      uint32_t keep = 0xffffu;
      if (f.drop_thresh) {
        keep = 0;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) keep |= keep4(f, b, h, H, qi, jb + 8 * qd + 4 * g, Sq, Sk) << (4 * qd);
      }
      float ds[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = __builtin_amdgcn_exp2f(s[e] - lse2);
        const float mdp = f.drop_thresh ? (((keep >> e) & 1u) ? dp[e] * f.drop_scale : 0.f) : dp[e];
        ds[e] = pe * (mdp - delta);
      }
      if (f.dbias && row_ok) {
        float* drow = f.dbias + b * f.dsb + h * f.dsh + (long long)qi * f.dss;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = jb + acc_row(e, g);
          if (j < sk) drow[j] = ds[e];
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        frag dsf;
        M::pack(&ds[8 * st], dsf);
        const int rbase = (32 * kt + 16 * st) * L::PITCH;
#pragma unroll
        for (int dt = 0; dt < DVT; ++dt) dq[dt] = M::mma(ld_tr<M>(Ks + rbase, lo.tra[dt], lo.trb[dt]), dsf, dq[dt]);
      }
    }
  }
};

// The dQ workgroup's work: block hw of nblk (the block's place in its own
// grid), K and V tiles of stage s in the first two namespace-scope LDS
// stages ([K | V] each).  With FEAT and a dbias output, every key tile of
// the sequence is visited (tiles the window leaves empty write their zeros).
template <typename M, int D, int NW, int BN, bool FEAT = false, bool SPLIT = false>
__device__ __forceinline__ void dq16_body(int hw, int nblk) {
  using F = Dq16<M, D, BN>;
  using T = typename M::elem;
  constexpr int NT = NW * 64, BM = NW * 32, DVT = F::DVT;
  static_assert(2 * F::TILE * (int)sizeof(T) <= kBwdStageBytes, "K and V tiles fit a stage");
  KBwdArgs& a = kernel_bwd_args();
  T* const k_s0 = reinterpret_cast<T*>(g_bwd_st0);
  T* const v_s0 = k_s0 + F::TILE;
  T* const k_s1 = reinterpret_cast<T*>(g_bwd_st1);
  T* const v_s1 = k_s1 + F::TILE;

  const auto& P = a.p;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int nbh = P.B * P.H;
  const int nsplit = SPLIT ? a.split_q : 1;
  const int nq = nblk / (nbh * nsplit);
  const int sg = hw / (nq * nbh);  // split copy (0 without split)
  const GridPos gp = grid_pos(hw % (nq * nbh), nq * nbh, nq, nbh, P.ragged);
  const int bh = gp.bh, h = bh % P.H, b = bh / P.H;
  const int qb = nq - 1 - gp.i;

  long long q0, k0;
  int sq, sk;
  seq_rows(P, b, q0, sq, k0, sk);
  const int i0 = qb * BM;
  if (i0 >= sq) return;
  const Window w = seq_window(P.wl, P.wr, P.diag, sq, sk);

  const T* qp = (const T*)a.q.ptr + b * a.q.sb + h * a.q.sh + q0 * a.q.ss;
  const T* kp = (const T*)a.k.ptr + b * a.k.sb + h * a.k.sh + k0 * a.k.ss;
  const T* vp = (const T*)a.v.ptr + b * a.v.sb + h * a.v.sh + k0 * a.v.ss;
  const T* dop = (const T*)a.dout.ptr + b * a.dout.sb + h * a.dout.sh + q0 * a.dout.ss;
  T* dqp = (T*)a.dq.ptr + b * a.dq.sb + h * a.dq.sh + q0 * a.dq.ss;
  const float* l2p = a.lse2 + b * P.lse_sb + h * P.lse_sh + q0;
  const float* delp = a.delta + b * P.lse_sb + h * P.lse_sh + q0;

  const bool all_tiles = FEAT && a.f.dbias != nullptr;
  const int ilast = min(i0 + BM, sq) - 1;
  long long jlo = max(0LL, (long long)i0 + w.lo);
  long long jhi = min((long long)sk - 1, (long long)ilast + w.hi);
  bool block_empty = w.lo > w.hi || jlo > jhi;
  if (all_tiles) {
    jlo = 0;
    jhi = (long long)sk - 1;
    block_empty = sk == 0;
  }
  if constexpr (SPLIT) {
    split_rows(jlo, jhi, BN, sg, nsplit);
    block_empty = block_empty || jlo > jhi;
  }

  const int iw0 = i0 + 32 * wave;
  const bool wave_live = iw0 < sq;
  const int qi = iw0 + r;
  const bool row_ok = wave_live && qi < sq;
  int tw0 = 0x7fffffff, tw1 = -1;
  if (wave_live && w.lo <= w.hi) {
    const long long a0 = max(0LL, (long long)iw0 + w.lo);
    const long long a1 = min((long long)sk - 1, (long long)min(iw0 + 31, sq - 1) + w.hi);
    if (a0 <= a1) {
      tw0 = (int)(a0 / BN);
      tw1 = (int)(a1 / BN);
    }
  }
  if (all_tiles && wave_live && sk > 0) {
    tw0 = 0;
    tw1 = (sk - 1) / BN;
  }

  RowFrags<M, D> qf, dof;
  qf.load(qp + (long long)qi * a.q.ss, row_ok, g);
  dof.load(dop + (long long)qi * a.dout.ss, row_ok, g);
  const float lse2 = row_ok ? l2p[qi] : INFINITY;
  const float delta = row_ok ? delp[qi] : 0.f;
  const float c = fmaxf(fabsf(P.scale_log2), 1e-30f);
  if (P.scale_log2 < 0.f) qf.negate();
  f32x16 ndelta;  // the first dP product's accumulator input (FEAT: unused)
#pragma unroll
  for (int e = 0; e < 16; ++e) ndelta[e] = -delta;

  f32x16 dq[DVT];
#pragma unroll
  for (int dt = 0; dt < DVT; ++dt) dq[dt] = zero16();

  if (!block_empty) {
    LdsOffsets<M, D> lo;
    lo.init(lane);
    DmaLane<T, D, BN, NW> kd, vd;
    kd.init(a.k.ss, wave, lane);
    vd.init(a.v.ss, wave, lane);
    zero_unused_slots<T, D, BN, NT>(k_s0, tid);
    zero_unused_slots<T, D, BN, NT>(k_s1, tid);
    zero_unused_slots<T, D, BN, NT>(v_s0, tid);
    zero_unused_slots<T, D, BN, NT>(v_s1, tid);
    const int t0 = (int)(jlo / BN), t1 = (int)(jhi / BN);
    auto dma = [&](T* kb, T* vb, int t) __attribute__((always_inline)) {
      kd.issue(kb, kp + (long long)t * BN * a.k.ss, a.k.ss, sk - t * BN, wave, lane);
      vd.issue(vb, vp + (long long)t * BN * a.v.ss, a.v.ss, sk - t * BN, wave, lane);
    };
    dma(k_s0, v_s0, t0);
    __syncthreads();
    auto step = [&](auto parity, int t) __attribute__((always_inline)) {
      constexpr int Pq = decltype(parity)::value;
      if (t + 1 <= t1) dma(Pq ? k_s0 : k_s1, Pq ? v_s0 : v_s1, t + 1);
      if (tw0 <= t && t <= tw1) {
        if constexpr (FEAT) {
          const FeatArgs f = feat_args(a);
          const bool masked = classify(w, iw0, 32, (long long)t * BN, BN, sk) != kFull;
          Dq16Feat<M, D, BN>::tile(Pq ? k_s1 : k_s0, Pq ? v_s1 : v_s0, lo, qf, dof, dq, c, lse2, delta, masked, w,
                                   t * BN, qi, sq, sk, g, f, b, h, P.H, P.Sq, P.Sk, row_ok);
        } else {
          const bool masked = classify(w, iw0, 32, (long long)t * BN, BN, sk) == kPartial;
          F::tile(Pq ? k_s1 : k_s0, Pq ? v_s1 : v_s0, lo, qf, dof, dq, c, lse2, ndelta, masked, w, t * BN, qi, sk,
                  g);
        }
      }
      __syncthreads();
    };
    for (int t = t0; t <= t1; t += 2) {
      step(std::integral_constant<int, 0>{}, t);
      if (t + 1 <= t1) step(std::integral_constant<int, 1>{}, t + 1);
    }
  }

  if constexpr (SPLIT) {
    float* const part_q = a.part + 2LL * a.split_kv * P.H * a.rows_k * D;
    if (row_ok) store_partial_q<D>(part_q, a.rows_q, P.H, sg, h, part_row(P.qs.mode, P.Sq, b, q0, qi), dq, g);
    if (a.cnt_q != nullptr && last_arrival(a.cnt_q + (long long)bh * nq + qb, nsplit))
      sum_partials<T, D, NT, false>(part_q, a.rows_q, P.H, nsplit, h, P.qs.mode, P.Sq, b, q0, i0, ilast + 1, dqp,
                                    a.dq.ss, nullptr, 0, P.scale, tid);
  } else if (row_ok) {
    T* dqrow = dqp + (long long)qi * a.dq.ss;
    const float sc = P.scale;
#pragma unroll
    for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * dt + 8 * q4 + 4 * g;
        if (d < D)
          store4b<T>(dqrow + d, dq[dt][4 * q4] * sc, dq[dt][4 * q4 + 1] * sc,
                     dq[dt][4 * q4 + 2] * sc, dq[dt][4 * q4 + 3] * sc);
      }
  }
}

template <typename M, int D, int NW, int BN, int WPE, bool FEAT = false, bool SPLIT = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void attn_bwd_dq16_kernel(BwdArgs) {
  dq16_body<M, D, NW, BN, FEAT, SPLIT>(blockIdx.x, gridDim.x);
}

// ------------------------------------------ 16-bit dK/dV + dQ in one grid
//
// Blocks [0, nkv) are producer / consumer dK/dV workgroups, the rest dQ
// workgroups of 256 query rows (8 waves).  Both kinds need 8 waves and at
// most the dK/dV LDS, so each CU holds one of either; with the longer dK/dV
// blocks dispatched first, dQ blocks fill the CUs the last dK/dV round
// leaves idle, and the dQ grid's own partial last round shrinks to a tail of
// short blocks.  dQ's K / V stages live in the first two dK/dV stages.
template <typename M, int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_fused16_kernel(BwdArgs,
                                                                                                        int nkv) {
  const int hw = (int)blockIdx.x;
  if (hw < nkv)
    dkdv_pc_body<M, D>(hw, nkv);
  else
    dq16_body<M, D, 8, 64>(hw - nkv, (int)gridDim.x - nkv);
}

// ------------------------------------------------ split mode, one grid
//
// Blocks [0, nkv) are split dK/dV copies, the rest split dQ copies: the two
// run side by side rather than one grid after the other.  Split mode is for
// calls whose grids leave most of the GPU idle, where a kernel takes about
// as long as its longest workgroup.
template <typename M, int D, int NW_KV, int BMQ, int NW_Q, int BN, int WPE>
__global__ __launch_bounds__(NW_KV * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void attn_bwd_split16_kernel(
    BwdArgs a, int nkv) {
  static_assert(NW_KV == NW_Q, "one workgroup size");
  const int hw = (int)blockIdx.x;
  if (hw < nkv)
    dkdv16_body<M, D, NW_KV, BMQ, false, true, true>(a, (unsigned)hw, (unsigned)nkv);
  else
    dq16_body<M, D, NW_Q, BN, false, true>(hw - nkv, (int)gridDim.x - nkv);
}

// The same for fp32.
template <typename M, int D, int NW_KV, int BMQ, int NW_Q, int BN>
__global__ __launch_bounds__(NW_KV * 64) void attn_bwd_split_kernel(BwdArgs a, int nkv) {
  static_assert(NW_KV == NW_Q, "one workgroup size");
  const unsigned hw = blockIdx.x;
  if (hw < (unsigned)nkv)
    dkdv_body<M, D, NW_KV, BMQ, false, true>(a, hw, (unsigned)nkv);
  else
    dq_body<M, D, NW_Q, BN, false, true>(a, hw - (unsigned)nkv, gridDim.x - (unsigned)nkv);
}

// ------------------------------------------------------------ split reduce

// Split-mode epilogue as its own grid, where the partials are too large for
// one workgroup per block to sum them fast: one workgroup per (side,
// sequence, head, row slice); each row of a sequence's length gets the sum
// of its partial rows in copy order, times the scale for dQ and dK, rounded
// to the output type.  sides: 1 Q (dQ), 2 K (dK, dV), 3 both; the grid is
// nsides * B * H * slices, Q side first.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_reduce_kernel(BwdArgs a, int sides, int slices) {
  constexpr int V4 = D / 4, RPP = 256 / V4;  // float4 columns per row, rows per pass
  static_assert(D % 4 == 0 && RPP >= 1, "row shape");
  const int tid = threadIdx.x, ri = tid / V4, d = 4 * (tid % V4);
  if (ri >= RPP) return;  // threads past the last whole row of a pass
  const ProblemArgs& P = a.p;
  const int nbh = P.B * P.H;
  int blk = (int)blockIdx.x;
  const int sl = blk % slices;
  blk /= slices;
  const int bh = blk % nbh;
  const int side = (sides == 3) ? blk / nbh : (sides == 2 ? 1 : 0);  // 0: Q, 1: K
  const int h = bh % P.H, b = bh / P.H;
  const SideArgs& S = side ? P.ks : P.qs;
  const SideRows r = side_rows(S, b);
  const long long rows = side ? a.rows_k : a.rows_q;
  const int groups = side ? a.split_kv : a.split_q;
  const float* p0 = side ? a.part : a.part + 2LL * a.split_kv * P.H * a.rows_k * D;  // dK or dQ
  const float* p1 = a.part + (long long)a.split_kv * P.H * a.rows_k * D;             // dV
  const long long gstride = (long long)P.H * rows * D;
  const Operand o0 = side ? a.dk : a.dq;
  const float sc = P.scale;
  for (long long i = (long long)sl * RPP + ri; i < r.n; i += (long long)slices * RPP) {
    float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
    const long long off = ((long long)h * rows + part_row(S.mode, S.S, b, r.r0, (int)i)) * D + d;
    for (int g = 0; g < groups; ++g) {
      const float4 x = *reinterpret_cast<const float4*>(p0 + g * gstride + off);
      s0.x += x.x; s0.y += x.y; s0.z += x.z; s0.w += x.w;
      if (side) {
        const float4 y = *reinterpret_cast<const float4*>(p1 + g * gstride + off);
        s1.x += y.x; s1.y += y.y; s1.z += y.z; s1.w += y.w;
      }
    }
    const long long row = r.r0 + i;
    store4b<T>((T*)o0.ptr + b * o0.sb + h * o0.sh + row * o0.ss + d, s0.x * sc, s0.y * sc, s0.z * sc, s0.w * sc);
    if (side)
      store4b<T>((T*)a.dv.ptr + b * a.dv.sb + h * a.dv.sh + row * a.dv.ss + d, s1.x, s1.y, s1.z, s1.w);
  }
}

// ------------------------------------------------------------ launch

// Workgroup shapes.  16-bit: dK/dV 4 waves (128 keys) over 64-row query
// tiles (32 at head_dim 80) at two waves per SIMD for head_dim <= 80,
// producer / consumer pairs
// (8 waves, 128 keys) at head_dim 128; dQ 4 waves (128 queries) over 64-key
// tiles, two per SIMD.  fp32 (register-staged kernels): 4 waves each, tiles
// of 32 to fit LDS.
template <typename M, int D>
struct BwdShape {
  static constexpr bool k16 = sizeof(typename M::elem) == 2;
  // Query tiles of 32 rows at head_dim 80: the 64-row tile's slices spilled
  // registers at two waves per SIMD (1x32x4096x80 bf16 backward 777 ->
  // 753 us; the (256, 0) window at 2048 rows 216 -> 198 us).  At 64 the
  // 64-row tile stays faster (BERT-like 1119 against 1153 us).
  static constexpr int NW_KV = 4, BMQ = k16 ? (D == 80 ? 32 : 64) : 32;
  // dQ key tiles: 32 keys above head_dim 128 (K and V tiles of 64 keys would
  // not fit a stage).
  static constexpr int NW_Q = 4, BN = k16 ? (D > 128 ? 32 : 64) : 32;
  // dK/dV by producer / consumer wave pairs (128 keys per workgroup, as NW_KV).
  static constexpr bool PC = k16 && D > 80 && D <= 128;
  // Waves per SIMD the registers allow: dK/dV (plain kernel) and dQ.
  static constexpr int WPE_KV = D > 80 ? 1 : 2, WPE_Q = D > 128 ? 1 : 2;
};

template <typename M, int D, class Ex>
static hipError_t launch_bwd_t(const BwdArgs& a, int stages, const Ex& ex) {
  using T = typename M::elem;
  using S = BwdShape<M, D>;
  constexpr int NW_KV = S::NW_KV, BMQ = S::BMQ, NW_Q = S::NW_Q, BN = S::BN;
  hipError_t err;
  // 1. Delta.
  if (stages & kStageDelta) {
    const long long nrows =
        (a.p.qs.mode & kSeqStacked) ? a.p.total_q * a.p.H : (long long)a.p.B * a.p.H * a.p.Sq;
    constexpr int CE = 16 / (int)sizeof(T), CH = D / CE;
    constexpr int G = CH <= 8 ? 8 : (CH <= 16 ? 16 : 32);
    long long nblk = (nrows + (256 / G) - 1) / (256 / G);
    if (a.ncnt > 0 && nblk < 1) nblk = 1;  // it also zeroes the split counters
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    if (nblk > 0) {
      err = ex(reinterpret_cast<const void*>(&attn_bwd_pre_kernel<T, D>), "attn_bwd_pre_kernel", (unsigned)nblk,
               256u, a, nrows);
      if (err != hipSuccess) return err;
    }
  }
  // Split mode (the call's grids would leave most of the GPU idle): split
  // copies of the dK/dV and dQ grids, both in one launch where the two
  // kinds' LDS fits one workgroup.  In fp32, whose products are slow enough
  // that the copies' partials are small next to their work, the last copy
  // of each block sums them, and workgroups of 64 rows (two waves) spread
  // the copies over twice the CUs whenever that grid fits the device at one
  // workgroup per CU; in fp16 / bf16 a reduction grid sums the partials,
  // spread over the whole GPU.
  if (a.part) {
    if (a.split_kv < 1 || a.split_kv > 8 || a.split_q < 1 || a.split_q > 8) return hipErrorInvalidValue;
    constexpr bool kLastCopySums = !S::k16;
    BwdArgs sa = a;
    if (!kLastCopySums) sa.cnt_kv = sa.cnt_q = nullptr;
    auto grids = [&](int nw, long long& nkv, long long& nq) {
      nkv = (stages & kStageDkDv) ? (a.p.Sk + nw * 32 - 1) / (nw * 32) * a.p.H * a.p.B * a.split_kv : 0;
      nq = (stages & kStageDq) ? (a.p.Sq + nw * 32 - 1) / (nw * 32) * a.p.H * a.p.B * a.split_q : 0;
    };
    long long nkv, nq;
    grids(NW_KV, nkv, nq);
    bool two = false;
    if constexpr (!S::k16) {
      long long nkv2, nq2;
      grids(2, nkv2, nq2);
      const long long cus = device_cu_count();
      two = cus > 0 && nkv2 + nq2 <= cus;
      if (two) {
        nkv = nkv2;
        nq = nq2;
      }
    }
    if (nkv + nq > 0x7fffffffLL) return hipErrorInvalidValue;
    // The copies with SNW waves per workgroup.
    auto copies = [&](auto snw) -> hipError_t {
      constexpr int SNW = decltype(snw)::value;
      hipError_t e = hipSuccess;
      bool one = false;
      if constexpr (S::k16 ? D <= 128 : D <= 64) one = nkv > 0 && nq > 0;
      if (one) {
        if constexpr (S::k16 ? D <= 128 : D <= 64) {
          if constexpr (S::k16)
            return ex(reinterpret_cast<const void*>(&attn_bwd_split16_kernel<M, D, SNW, BMQ, SNW, BN, S::WPE_KV>),
                      "attn_bwd_split16_kernel", (unsigned)(nkv + nq), (unsigned)(SNW * 64), sa, (int)nkv);
          else
            return ex(reinterpret_cast<const void*>(&attn_bwd_split_kernel<M, D, SNW, BMQ, SNW, BN>),
                      "attn_bwd_split_kernel", (unsigned)(nkv + nq), (unsigned)(SNW * 64), sa, (int)nkv);
        }
      }
      if (nkv > 0) {
        if constexpr (S::k16)
          e = ex(reinterpret_cast<const void*>(&attn_bwd_dkdv16_kernel<M, D, SNW, BMQ, S::WPE_KV, false, true>),
                 "attn_bwd_dkdv16_kernel", (unsigned)nkv, (unsigned)(SNW * 64), sa);
        else
          e = ex(reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<M, D, SNW, BMQ, false, true>),
                 "attn_bwd_dkdv_kernel", (unsigned)nkv, (unsigned)(SNW * 64), sa);
        if (e != hipSuccess) return e;
      }
      if (nq > 0) {
        if constexpr (S::k16)
          e = ex(reinterpret_cast<const void*>(&attn_bwd_dq16_kernel<M, D, SNW, BN, S::WPE_Q, false, true>),
                 "attn_bwd_dq16_kernel", (unsigned)nq, (unsigned)(SNW * 64), sa);
        else
          e = ex(reinterpret_cast<const void*>(&attn_bwd_dq_kernel<M, D, SNW, BN, false, true>),
                 "attn_bwd_dq_kernel", (unsigned)nq, (unsigned)(SNW * 64), sa);
      }
      return e;
    };
    static_assert(NW_KV == NW_Q, "split copies share one workgroup size");
    if constexpr (!S::k16)
      err = two ? copies(std::integral_constant<int, 2>{}) : copies(std::integral_constant<int, NW_KV>{});
    else
      err = copies(std::integral_constant<int, NW_KV>{});
    if (err != hipSuccess) return err;
    const int sides = (nq > 0 ? 1 : 0) | (nkv > 0 ? 2 : 0);
    if (!kLastCopySums && sides) {
      constexpr int RPP = 256 / (D / 4);
      const int rows = sides == 1 ? a.p.Sq : (sides == 2 ? a.p.Sk : max(a.p.Sq, a.p.Sk));
      const int slices = max(1, min(64, (rows + RPP - 1) / RPP));
      const long long nblk = (long long)(sides == 3 ? 2 : 1) * a.p.B * a.p.H * slices;
      if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
      if (nblk > 0)
        return ex(reinterpret_cast<const void*>(&attn_bwd_reduce_kernel<T, D>), "attn_bwd_reduce_kernel",
                  (unsigned)nblk, 256u, a, sides, slices);
    }
    return hipSuccess;
  }
  // Bias, ALiBi, dropout or dbias: the kernels built with them (16-bit dK/dV
  // one wave per SIMD above head_dim 64, where their registers do not fit
  // two), never the fused or producer / consumer ones.
  if (a.feat) {
    if (stages & kStageDkDv) {
      const long long nblk = (a.p.Sk + NW_KV * 32 - 1) / (NW_KV * 32) * a.p.H * a.p.B;
      if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
      if (nblk > 0) {
        if constexpr (S::k16)
          err = ex(reinterpret_cast<const void*>(&attn_bwd_dkdv16_kernel<M, D, NW_KV, BMQ, (D > 64 ? 1 : 2), true>),
                   "attn_bwd_dkdv16_kernel", (unsigned)nblk, (unsigned)(NW_KV * 64), a);
        else
          err = ex(reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<M, D, NW_KV, BMQ, true>),
                   "attn_bwd_dkdv_kernel", (unsigned)nblk, (unsigned)(NW_KV * 64), a);
        if (err != hipSuccess) return err;
      }
    }
    if (stages & kStageDq) {
      const long long nblk = (a.p.Sq + NW_Q * 32 - 1) / (NW_Q * 32) * a.p.H * a.p.B;
      if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
      if (nblk > 0) {
        if constexpr (S::k16)
          err = ex(reinterpret_cast<const void*>(&attn_bwd_dq16_kernel<M, D, NW_Q, BN, (D > 80 ? 1 : 2), true>),
                   "attn_bwd_dq16_kernel", (unsigned)nblk, (unsigned)(NW_Q * 64), a);
        else
          err = ex(reinterpret_cast<const void*>(&attn_bwd_dq_kernel<M, D, NW_Q, BN, true>), "attn_bwd_dq_kernel",
                   (unsigned)nblk, (unsigned)(NW_Q * 64), a);
        if (err != hipSuccess) return err;
      }
    }
    return hipSuccess;
  }
  // 2 + 3 in one grid where the build has the fused kernel and it pays: a
  // wide band (its dQ workgroups are 256 rows) and a separate dQ grid whose
  // last round would be at most a quarter full (2 workgroups of 128 rows per
  // CU).  At half full the filled tail no longer makes up for the 256-row
  // dQ workgroups (1x32x15300x128: 12.47 ms fused against 11.70 ms).
  if constexpr (S::PC) {
    const long long ndq4 = (a.p.Sq + NW_Q * 32 - 1) / (NW_Q * 32) * a.p.H * a.p.B;
    const long long slots = 2LL * device_cu_count();
    const long long tail = slots > 0 ? ndq4 % slots : 0;
    if ((stages & kStageDkDv) && (stages & kStageDq) && wide_window(a.p) && tail > 0 && 4 * tail <= slots) {
      const long long nkv = (a.p.Sk + 127) / 128 * a.p.H * a.p.B;
      const long long ndq = (a.p.Sq + 255) / 256 * a.p.H * a.p.B;
      if (nkv + ndq > 0x7fffffffLL) return hipErrorInvalidValue;
      if (nkv > 0 && ndq > 0)  // otherwise the separate kernels below write the zeros
        return ex(reinterpret_cast<const void*>(&attn_bwd_fused16_kernel<M, D>), "attn_bwd_fused16_kernel",
                  (unsigned)(nkv + ndq), 512u, a, (int)nkv);
    }
  }
  // 2. dK, dV.
  if (stages & kStageDkDv) {
    const long long nkb = (a.p.Sk + NW_KV * 32 - 1) / (NW_KV * 32);
    const long long nblk = nkb * a.p.H * a.p.B;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    if (nblk > 0) {
      if constexpr (S::PC)
        err = ex(reinterpret_cast<const void*>(&attn_bwd_dkdv16pc_kernel<M, D>), "attn_bwd_dkdv16pc_kernel",
                 (unsigned)nblk, 512u, a);
      else if constexpr (S::k16)
        err = ex(reinterpret_cast<const void*>(&attn_bwd_dkdv16_kernel<M, D, NW_KV, BMQ, S::WPE_KV>),
                 "attn_bwd_dkdv16_kernel", (unsigned)nblk, (unsigned)(NW_KV * 64), a);
      else
        err = ex(reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<M, D, NW_KV, BMQ>), "attn_bwd_dkdv_kernel",
                 (unsigned)nblk, (unsigned)(NW_KV * 64), a);
      if (err != hipSuccess) return err;
    }
  }
  // 3. dQ.
  if (stages & kStageDq) {
    const long long nq = (a.p.Sq + NW_Q * 32 - 1) / (NW_Q * 32);
    const long long nblk = nq * a.p.H * a.p.B;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    if (nblk > 0) {
      if constexpr (S::k16)
        err = ex(reinterpret_cast<const void*>(&attn_bwd_dq16_kernel<M, D, NW_Q, BN, S::WPE_Q>),
                 "attn_bwd_dq16_kernel", (unsigned)nblk, (unsigned)(NW_Q * 64), a);
      else
        err = ex(reinterpret_cast<const void*>(&attn_bwd_dq_kernel<M, D, NW_Q, BN>), "attn_bwd_dq_kernel",
                 (unsigned)nblk, (unsigned)(NW_Q * 64), a);
      if (err != hipSuccess) return err;
    }
  }
  return hipSuccess;
}

template <typename M, class Ex>
static hipError_t launch_bwd_d(int head_dim, const BwdArgs& a, int stages, const Ex& ex) {
  switch (head_dim) {
    case 32: return launch_bwd_t<M, 32>(a, stages, ex);
    case 48: return launch_bwd_t<M, 48>(a, stages, ex);
    case 64: return launch_bwd_t<M, 64>(a, stages, ex);
    case 80: return launch_bwd_t<M, 80>(a, stages, ex);
    case 96: return launch_bwd_t<M, 96>(a, stages, ex);
    case 128: return launch_bwd_t<M, 128>(a, stages, ex);
    case 192:
      if constexpr (sizeof(typename M::elem) == 2) return launch_bwd_t<M, 192>(a, stages, ex);
      return hipErrorNotSupported;
    case 256:
      if constexpr (sizeof(typename M::elem) == 2) return launch_bwd_t<M, 256>(a, stages, ex);
      return hipErrorNotSupported;
    default: return hipErrorNotSupported;
  }
}

}  // namespace sdpa
