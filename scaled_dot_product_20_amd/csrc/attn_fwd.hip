// attn_fwd.hip - fused attention forward for gfx950.
//
// One workgroup = NW waves = one block of 32*NW query rows of one (sequence,
// head); each wave owns 32 query rows.  The workgroup walks the key tiles
// its window can see (FlashAttention, the kernel family of the AOTriton
// README, "Kernel Support"); tiles outside the window of a wave's rows are
// skipped and only tiles cut by the window edge, the diagonal or the ragged
// end of the sequence are masked element by element (generalized sliding
// window of the AOTriton 0.10b release notes; diagonal choice of the 0.15b
// notes, "Bottom-Right Aligned Sliding Windows").
//
// Per key tile of BN keys:
//   K and V are copied HBM -> LDS with direct loads into swizzled row-major
//     tiles (two stages in the narrow-band kernel, three in the ping-pong
//     kernel), the next tiles' copies in flight during this tile;
//   S^T = K Q^T on the matrix cores (Q fragments stay in registers);
//   online softmax in the log2 domain: x = c*s with c = |scale|*log2(e)
//     (a negative scale is moved into Q, so c >= 0 and max_j x_j is
//     c * max_j s_j), p = 2^(x - m) in one FMA and one exp;
//   the reference max m of a row is only raised when the tile's max exceeds
//     it by more than kRescaleSlack (so p <= 2^kRescaleSlack); O and l are
//     rescaled only then, and skipped when no row of the wave moved (the
//     ping-pong kernel computes the tile's max only when a lane's sum of p
//     against the current m passes 2^kRescaleSlack, or the row has no m);
//   P is rounded to the working type (round to nearest even, the fix in the
//     AOTriton 0.15b notes) and O^T += V^T P^T on the matrix cores.
// Epilogue: O = acc / l, LSE = ln(2) * (m + log2 l); rows with no visible key
// get O = 0 and LSE = +inf.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace sdpa {

// Largest log2 growth of a row max absorbed without rescaling.
constexpr float kRescaleSlack = 8.f;
constexpr float kRescaleBound = 256.f;  // 2^kRescaleSlack

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  } else {
    typedef T t4 __attribute__((ext_vector_type(4)));
    t4 v;
    v[0] = (T)a; v[1] = (T)b; v[2] = (T)c; v[3] = (T)d;
    *reinterpret_cast<t4*>(p) = v;
  }
}

template <typename M, int D, int NW, int BN, bool FEAT = false>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(FwdArgs a) {
  using T = typename M::elem;
  constexpr int NT = NW * 64, BM = NW * 32, KPL = M::KPL;
  constexpr int DVT = (D + 31) / 32, DPAD = DVT * 32;
  constexpr int PAD = 16 / (int)sizeof(T);
  constexpr int KLD = D + PAD, VLD = BN + PAD;
  constexpr int KT = BN / 32;
  constexpr int NS = D / (2 * KPL);
  constexpr int STAGE = BN * KLD + DPAD * VLD;
  __shared__ __attribute__((aligned(16))) T smem[2 * STAGE];

  const ProblemArgs& P = a.p;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int nq = (int)(gridDim.x / (P.B * P.H));
  const GridPos gp = grid_pos(blockIdx.x, gridDim.x, nq, P.B * P.H, P.ragged);
  const int bh = gp.bh, h = bh % P.H, b = bh / P.H;
  const int qb = nq - 1 - gp.i;  // longest rows (under causal) first

  long long q0, k0;
  int sq, sk;
  seq_rows(P, b, q0, sq, k0, sk);
  const int i0 = qb * BM;
  if (i0 >= sq) return;
  const Window w = seq_window(P.wl, P.wr, P.diag, sq, sk);

  const T* qp = (const T*)a.q.ptr + b * a.q.sb + h * a.q.sh + q0 * a.q.ss;
  const T* kp = (const T*)a.k.ptr + b * a.k.sb + h * a.k.sh + k0 * a.k.ss;
  const T* vp = (const T*)a.v.ptr + b * a.v.sb + h * a.v.sh + k0 * a.v.ss;
  T* op = (T*)a.o.ptr + b * a.o.sb + h * a.o.sh + q0 * a.o.ss;
  float* lp = a.lse + b * P.olse_sb + h * P.olse_sh + q0 * P.olse_ss;

  // Keys the block can see.
  const int ilast = min(i0 + BM, sq) - 1;
  const long long jlo = max(0LL, (long long)i0 + w.lo);
  const long long jhi = min((long long)sk - 1, (long long)ilast + w.hi);
  const bool block_empty = w.lo > w.hi || jlo > jhi;

  const int iw0 = i0 + 32 * wave;
  const bool wave_live = iw0 < sq;
  const int qi = iw0 + r;  // this lane's query row

  RowFrags<M, D> qf;
  qf.load(qp + (long long)qi * a.q.ss, wave_live && qi < sq, g);
  const float c = fabsf(P.scale_log2);
  if (P.scale_log2 < 0.f) qf.negate();

  if constexpr (DPAD != D) {  // padding rows of the transposed V tile
    for (int x = tid; x < (DPAD - D) * VLD; x += NT) {
      smem[BN * KLD + D * VLD + x] = (T)0.f;
      smem[STAGE + BN * KLD + D * VLD + x] = (T)0.f;
    }
  }

  float m = -INFINITY, l = 0.f;
  f32x16 acc[DVT];
#pragma unroll
  for (int dt = 0; dt < DVT; ++dt) acc[dt] = zero16();

  if (!block_empty) {
    const int t0 = (int)(jlo / BN), t1 = (int)(jhi / BN);
    TileStage<T, BN, D, NT> ks, vs;
    {
      const int j0 = t0 * BN;
      ks.load(kp + (long long)j0 * a.k.ss, a.k.ss, sk - j0, tid);
      vs.load(vp + (long long)j0 * a.v.ss, a.v.ss, sk - j0, tid);
      ks.store_rows(smem, KLD, tid);
      vs.store_transposed(smem + BN * KLD, VLD, tid);
    }
    __syncthreads();

    for (int t = t0; t <= t1; ++t) {
      const int buf = (t - t0) & 1;
      const int j0 = t * BN;
      if (t < t1) {
        const int jn = j0 + BN;
        ks.load(kp + (long long)jn * a.k.ss, a.k.ss, sk - jn, tid);
        vs.load(vp + (long long)jn * a.v.ss, a.v.ss, sk - jn, tid);
      }
      const T* Ks = smem + buf * STAGE;
      const T* Vt = Ks + BN * KLD;
      const int cls = wave_live ? classify(w, iw0, 32, j0, BN, sk) : kEmpty;
      if (cls != kEmpty) {
        // S^T = K Q^T, 32 keys per sub-tile.
        f32x16 s[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          s[kt] = zero16();
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            const auto A = load_frag<M>(Ks + (32 * kt + r) * KLD + 2 * KPL * st + KPL * g);
            s[kt] = M::mma(A, qf.f[st], s[kt]);
          }
        }
        const bool partial = cls == kPartial;
        float cc = c;
        uint32_t keep[KT];
        if constexpr (FEAT) {
          // Logits in the log2 domain with the additive terms, and the
          // dropout bits of every element (4 consecutive keys per counter).
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            const int jb = j0 + 32 * kt;
#pragma unroll
            for (int e = 0; e < 16; ++e)
              s[kt][e] = __builtin_fmaf(s[kt][e], c, extra_log2<T>(a.f, b, h, qi, jb + acc_row(e, g), sq, sk));
            keep[kt] = 0xffffu;
            if (a.f.drop_thresh) {
              keep[kt] = 0;
#pragma unroll
              for (int qd = 0; qd < 4; ++qd)
                keep[kt] |= keep4(a.f, b, h, P.H, qi, jb + 8 * qd + 4 * g, P.Sq, P.Sk) << (4 * qd);
            }
          }
          cc = 1.f;
        }
        if (partial) {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int j = j0 + 32 * kt + acc_row(e, g);
              const int diff = j - qi;
              if (!(diff >= w.lo && diff <= w.hi && j < sk)) s[kt][e] = -INFINITY;
            }
        }
        float smax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) smax = fmaxf(smax, s[kt][e]);
        smax = halves_max(smax);
        // Max of x = c*s over the row's visible keys of this tile.
        const float mx = smax == -INFINITY ? -INFINITY : smax * cc;
        const bool raise = mx > m + kRescaleSlack;  // also when m is still -inf
        if (__builtin_amdgcn_ballot_w64(raise)) {
          const float alpha = raise ? __builtin_amdgcn_exp2f(m - mx) : 1.f;
          if (raise) m = mx;
          l *= alpha;
#pragma unroll
          for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[dt][e] *= alpha;
        }
        // A row with no visible key so far keeps m = -inf; its p must be 0.
        const float nm = m == -INFINITY ? 0.f : -m;
        float x[KT][16];
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][e], cc, nm));
            if ((partial || FEAT) && s[kt][e] == -INFINITY) pe = 0.f;
            ls += pe;
            if constexpr (FEAT) pe = ((keep[kt] >> e) & 1u) ? pe : 0.f;
            x[kt][e] = pe;
          }
        l += ls;
        // O^T += V^T P^T
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int st = 0; st < 16 / KPL; ++st) {
            typename M::frag pf;
            M::pack(&x[kt][KPL * st], pf);
            const int pos = 32 * kt + perm_pos(KPL * st, g);
#pragma unroll
            for (int dt = 0; dt < DVT; ++dt) {
              const auto A = load_frag<M>(Vt + (32 * dt + r) * VLD + pos);
              acc[dt] = M::mma(A, pf, acc[dt]);
            }
          }
      }
      if (t < t1) {
        T* nb = smem + (buf ^ 1) * STAGE;
        ks.store_rows(nb, KLD, tid);
        vs.store_transposed(nb + BN * KLD, VLD, tid);
      }
      __syncthreads();
    }
  }

  if (wave_live) {
    const float lt = halves_sum(l);
    if (qi < sq) {
      const float inv = lt > 0.f ? (FEAT && a.f.drop_thresh ? a.f.drop_scale : 1.f) / lt : 0.f;
      T* orow = op + (long long)qi * a.o.ss;
#pragma unroll
      for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = 32 * dt + 8 * q4 + 4 * g;
          if (d < D)
            store4<T>(orow + d, acc[dt][4 * q4] * inv, acc[dt][4 * q4 + 1] * inv,
                      acc[dt][4 * q4 + 2] * inv, acc[dt][4 * q4 + 3] * inv);
        }
      if (g == 0) lp[qi * P.olse_ss] = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : INFINITY;
    }
  }
}

// fp32 forward of small grids: one workgroup = 64 query rows (two 32-row
// groups) x two key halves.  Waves 0-1 take the rows over the first half of
// the block's key tiles, waves 2-3 over the second half, each half staging
// its own tiles (both halves step together, one barrier per step); at the
// end the second half's (O^T, m, l) pass through LDS and the first half's
// waves merge them: m = max(m0, m1), O = 2^(m0-m) O0 + 2^(m1-m) O1, l
// likewise.  Each wave's chain of fp32 products covers half the keys.
template <typename M, int D, int BN>
__global__ __launch_bounds__(256) void attn_fwd_ks_kernel(FwdArgs a) {
  using T = typename M::elem;
  constexpr int HT = 128, BM = 64, KPL = M::KPL;  // threads per key half, rows per workgroup
  constexpr int DVT = (D + 31) / 32, DPAD = DVT * 32;
  constexpr int PAD = 16 / (int)sizeof(T);
  constexpr int KLD = D + PAD, VLD = BN + PAD;
  constexpr int KT = BN / 32;
  constexpr int NS = D / (2 * KPL);
  constexpr int STAGE = BN * KLD + DPAD * VLD;
  static_assert(2 * (DVT * 16 * 64 + 128) <= 2 * STAGE, "merge area fits the first half's stages");
  __shared__ __attribute__((aligned(16))) T smem[4 * STAGE];  // [key half][stage]

  const ProblemArgs& P = a.p;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int rg = wave & 1, kh = wave >> 1, htid = tid & (HT - 1);
  const int nq = (int)(gridDim.x / (P.B * P.H));
  const GridPos gp = grid_pos(blockIdx.x, gridDim.x, nq, P.B * P.H, P.ragged);
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
  T* op = (T*)a.o.ptr + b * a.o.sb + h * a.o.sh + q0 * a.o.ss;
  float* lp = a.lse + b * P.olse_sb + h * P.olse_sh + q0 * P.olse_ss;

  const int ilast = min(i0 + BM, sq) - 1;
  const long long jlo = max(0LL, (long long)i0 + w.lo);
  const long long jhi = min((long long)sk - 1, (long long)ilast + w.hi);
  const bool block_empty = w.lo > w.hi || jlo > jhi;

  const int iw0 = i0 + 32 * rg;
  const bool wave_live = iw0 < sq;
  const int qi = iw0 + r;

  RowFrags<M, D> qf;
  qf.load(qp + (long long)qi * a.q.ss, wave_live && qi < sq, g);
  const float c = fabsf(P.scale_log2);
  if (P.scale_log2 < 0.f) qf.negate();

  T* const hs = smem + kh * 2 * STAGE;  // this half's two stages
  if constexpr (DPAD != D) {  // padding rows of the transposed V tiles
    for (int x = htid; x < (DPAD - D) * VLD; x += HT) {
      hs[BN * KLD + D * VLD + x] = (T)0.f;
      hs[STAGE + BN * KLD + D * VLD + x] = (T)0.f;
    }
  }

  float m = -INFINITY, l = 0.f;
  f32x16 acc[DVT];
#pragma unroll
  for (int dt = 0; dt < DVT; ++dt) acc[dt] = zero16();

  if (!block_empty) {
    const int t0 = (int)(jlo / BN), n = (int)(jhi / BN) - t0 + 1, n0 = (n + 1) / 2;
    const int tb = kh ? t0 + n0 : t0, cnt = kh ? n - n0 : n0;  // this half's tiles
    TileStage<T, BN, D, HT> ks, vs;
    if (cnt > 0) {
      const int j0 = tb * BN;
      ks.load(kp + (long long)j0 * a.k.ss, a.k.ss, sk - j0, htid);
      vs.load(vp + (long long)j0 * a.v.ss, a.v.ss, sk - j0, htid);
      ks.store_rows(hs, KLD, htid);
      vs.store_transposed(hs + BN * KLD, VLD, htid);
    }
    __syncthreads();
    for (int st = 0; st < n0; ++st) {  // both halves step together
      const int buf = st & 1, t = tb + st, j0 = t * BN;
      if (st + 1 < cnt) {
        const int jn = j0 + BN;
        ks.load(kp + (long long)jn * a.k.ss, a.k.ss, sk - jn, htid);
        vs.load(vp + (long long)jn * a.v.ss, a.v.ss, sk - jn, htid);
      }
      const T* Ks = hs + buf * STAGE;
      const T* Vt = Ks + BN * KLD;
      const int cls = (wave_live && st < cnt) ? classify(w, iw0, 32, j0, BN, sk) : kEmpty;
      if (cls != kEmpty) {
        // S^T = K Q^T, 32 keys per sub-tile.
        f32x16 s[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          s[kt] = zero16();
#pragma unroll
          for (int ss = 0; ss < NS; ++ss) {
            const auto A = load_frag<M>(Ks + (32 * kt + r) * KLD + 2 * KPL * ss + KPL * g);
            s[kt] = M::mma(A, qf.f[ss], s[kt]);
          }
        }
        const bool partial = cls == kPartial;
        if (partial) {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int j = j0 + 32 * kt + acc_row(e, g);
              const int diff = j - qi;
              if (!(diff >= w.lo && diff <= w.hi && j < sk)) s[kt][e] = -INFINITY;
            }
        }
        float smax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) smax = fmaxf(smax, s[kt][e]);
        smax = halves_max(smax);
        const float mx = smax == -INFINITY ? -INFINITY : smax * c;
        const bool raise = mx > m + kRescaleSlack;  // also when m is still -inf
        if (__builtin_amdgcn_ballot_w64(raise)) {
          const float alpha = raise ? __builtin_amdgcn_exp2f(m - mx) : 1.f;
          if (raise) m = mx;
          l *= alpha;
#pragma unroll
          for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[dt][e] *= alpha;
        }
        const float nm = m == -INFINITY ? 0.f : -m;
        float x[KT][16];
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][e], c, nm));
            if (partial && s[kt][e] == -INFINITY) pe = 0.f;
            ls += pe;
            x[kt][e] = pe;
          }
        l += ls;
        // O^T += V^T P^T
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int ss = 0; ss < 16 / KPL; ++ss) {
            typename M::frag pf;
            M::pack(&x[kt][KPL * ss], pf);
            const int pos = 32 * kt + perm_pos(KPL * ss, g);
#pragma unroll
            for (int dt = 0; dt < DVT; ++dt) {
              const auto A = load_frag<M>(Vt + (32 * dt + r) * VLD + pos);
              acc[dt] = M::mma(A, pf, acc[dt]);
            }
          }
      }
      if (st + 1 < cnt) {
        T* nb = hs + (buf ^ 1) * STAGE;
        ks.store_rows(nb, KLD, htid);
        vs.store_transposed(nb + BN * KLD, VLD, htid);
      }
      __syncthreads();
    }
  }

  // Merge: the second half's waves leave O^T, m, l in the first half's
  // stages (free after the last barrier); the first half's waves combine.
  float* part = reinterpret_cast<float*>(smem) + rg * (DVT * 16 * 64 + 128);
  float* stat = part + DVT * 16 * 64;
  if (kh == 1) {
#pragma unroll
    for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4*>(part + ((dt * 4 + q4) * 64 + lane) * 4) =
            make_float4(acc[dt][4 * q4], acc[dt][4 * q4 + 1], acc[dt][4 * q4 + 2], acc[dt][4 * q4 + 3]);
    stat[lane] = m;
    stat[64 + lane] = l;
  }
  __syncthreads();
  if (kh == 1 || !wave_live) return;
  const float m1 = stat[lane], l1 = stat[64 + lane];
  const float mm = fmaxf(m, m1);
  const float a0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mm);
  const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
  const float lt = halves_sum(l * a0 + l1 * a1);
  if (qi < sq) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    T* orow = op + (long long)qi * a.o.ss;
#pragma unroll
    for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * dt + 8 * q4 + 4 * g;
        const float4 o1 = *reinterpret_cast<const float4*>(part + ((dt * 4 + q4) * 64 + lane) * 4);
        if (d < D)
          store4<T>(orow + d, (acc[dt][4 * q4] * a0 + o1.x * a1) * inv, (acc[dt][4 * q4 + 1] * a0 + o1.y * a1) * inv,
                    (acc[dt][4 * q4 + 2] * a0 + o1.z * a1) * inv, (acc[dt][4 * q4 + 3] * a0 + o1.w * a1) * inv);
      }
    if (g == 0) lp[qi * P.olse_ss] = lt > 0.f ? (mm + __builtin_amdgcn_logf(lt)) * kLn2 : INFINITY;
  }
}

// ------------------------------------------------------ 16-bit kernel
//
// The bf16 / fp16 forward.  K and V tiles are copied HBM -> LDS with direct
// loads into swizzled row-major tiles, two stages deep (the next tile's copy
// in flight while this one is used); K feeds S^T = K Q^T through 128-bit
// row reads and V feeds O^T += V^T P^T through transposing reads, so the
// waves never rearrange a tile.  Each wave owns RB blocks of 32 query rows:
// every K or V operand read from LDS feeds RB products, and the RB blocks'
// independent chains keep the matrix cores busy while the vector units work
// on another block's probabilities.  Each wave only visits the tiles its own
// rows can see (a contiguous range under a band window); tiles cut by the
// window, the diagonal or the ragged end are masked after their scores are
// computed.
template <typename M, int D, int BN, int RB>
struct Fwd16 {
  using T = typename M::elem;
  using L = Swz<D>;
  using frag = typename M::frag;
  static constexpr int KT = BN / 32, NS = D / 16, DVT = (D + 31) / 32;
  static constexpr int TILE = BN * L::PITCH;

  // s[rb][kt] = (K Q^T) of one tile (K: the swizzled LDS tile) for every
  // row block.
  static __device__ __forceinline__ void scores(const T* K, const LdsOffsets<M, D>& lo,
                                                const RowFrags<M, D>* qf, f32x16 (*s)[KT]) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s[rb][kt] = zero16();
    // K step outermost: consecutive products go to different accumulators.
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const frag A = ld_row<M>(K + 32 * kt * L::PITCH, lo.row[st]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[rb][kt] = M::mma(A, qf[rb].f[st], s[rb][kt]);
      }
  }

  // Masks one row block's scores of a tile cut by the window or the
  // sequence end: key j = jb + r(e) is visible iff qi + lo <= j <= min(qi +
  // hi, sk - 1).  c >= 1e-30, so a masked score (-inf) always maps to -inf
  // and then to p = 0.
  static __device__ __forceinline__ void mask(f32x16* s, Window w, int j0, int qi, int sk, int g) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const long long jb = (long long)j0 + 32 * kt + 4 * g;
      mask_block(s[kt], vis_bits((long long)qi + w.lo - jb, min((long long)qi + w.hi, (long long)sk - 1) - jb));
    }
  }

  // mask (when `masked`), then raise.
  static __device__ __forceinline__ void finalize(f32x16* s, bool masked, Window w, int j0, int qi, int sk,
                                                  float c, float& m, float& l, f32x16* acc, int g) {
    if (masked) mask(s, w, j0, qi, sk, g);
    raise(s, c, m, l, acc);
  }

  // Raises the row's reference max m when the tile's max exceeds it by more
  // than `slack`, rescaling l and O.  Wave-level (the row max is exchanged
  // between the half-waves).
  static __device__ __forceinline__ void raise(const f32x16* s, float c, float& m, float& l, f32x16* acc,
                                               float slack = kRescaleSlack) {
    float smax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) smax = fmaxf(smax, s[kt][e]);
    const float mx = halves_max(smax) * c;
    const bool raise = mx > m + slack;  // also when m is still -inf
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float alpha = raise ? __builtin_amdgcn_exp2f(m - mx) : 1.f;
      if (raise) m = mx;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[dt][e] *= alpha;
    }
  }

  // P = 2^(c s - m), rounded to the working type, and O^T += V^T P^T, for
  // every row block.  With DROP, element e of block (rb, kt) enters the row
  // sum and then the product only when bit e of keep[rb][kt] is set.
  template <bool DROP = false>
  static __device__ __forceinline__ void softmax_pv(const T* V, const LdsOffsets<M, D>& lo,
                                                    const f32x16 (*s)[KT], f32x16 (*acc)[DVT], const float* m,
                                                    float c, float* l, const uint32_t (*keep)[KT] = nullptr) {
    float nm[RB], ls[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      nm[rb] = m[rb] == -INFINITY ? 0.f : -m[rb];  // nothing visible yet: p = 0
      ls[rb] = 0.f;
    }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      frag pf[RB][2];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float x[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][kt][e], c, nm[rb]));
          ls[rb] += x[e];
          if constexpr (DROP) x[e] = ((keep[rb][kt] >> e) & 1u) ? x[e] : 0.f;
        }
        M::pack(&x[0], pf[rb][0]);
        M::pack(&x[8], pf[rb][1]);
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const T* vb = V + (32 * kt + 16 * st) * L::PITCH;
#pragma unroll
        for (int dt = 0; dt < DVT; ++dt) {
          const frag A = ld_tr<M>(vb, lo.tra[dt], lo.trb[dt]);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) acc[rb][dt] = M::mma(A, pf[rb][st], acc[rb][dt]);
        }
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) l[rb] += ls[rb];
  }
};

template <typename M, int D, int NW, int BN, int RB, int WPE, bool FEAT = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void attn_fwd16_kernel(FwdArgs a) {
  using F = Fwd16<M, D, BN, RB>;
  using T = typename M::elem;
  constexpr int NT = NW * 64, WR = 32 * RB, BM = NW * WR, KT = F::KT, DVT = F::DVT;
  // One LDS array per stage and operand, so that the compiler can tell the
  // tile being read from the tile being filled by direct loads and does not
  // wait for those loads before every read.
  __shared__ __attribute__((aligned(1024))) T k_s0[F::TILE], k_s1[F::TILE], v_s0[F::TILE], v_s1[F::TILE];

  const ProblemArgs& P = a.p;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int nq = (int)(gridDim.x / (P.B * P.H));
  const GridPos gp = grid_pos(blockIdx.x, gridDim.x, nq, P.B * P.H, P.ragged);
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
  T* op = (T*)a.o.ptr + b * a.o.sb + h * a.o.sh + q0 * a.o.ss;
  float* lp = a.lse + b * P.olse_sb + h * P.olse_sh + q0 * P.olse_ss;

  // Keys the block can see, and the tiles of this wave's rows.
  const int ilast = min(i0 + BM, sq) - 1;
  const long long jlo = max(0LL, (long long)i0 + w.lo);
  const long long jhi = min((long long)sk - 1, (long long)ilast + w.hi);
  const bool block_empty = w.lo > w.hi || jlo > jhi;

  const int iw0 = i0 + WR * wave;
  const bool wave_live = iw0 < sq;
  int tw0 = 0x7fffffff, tw1 = -1;
  if (wave_live && w.lo <= w.hi) {
    const long long a0 = max(0LL, (long long)iw0 + w.lo);
    const long long a1 = min((long long)sk - 1, (long long)min(iw0 + WR - 1, sq - 1) + w.hi);
    if (a0 <= a1) {
      tw0 = (int)(a0 / BN);
      tw1 = (int)(a1 / BN);
    }
  }
  // Tiles the window leaves whole for all of the wave's rows (and inside the
  // sequence): no masking there.
  const TileRange full = tiles_starting_in((long long)iw0 + WR - 1 + w.lo,
                                           min((long long)iw0 + w.hi, (long long)sk - 1) - BN + 1, BN);

  const float c = fmaxf(fabsf(P.scale_log2), 1e-30f);
  RowFrags<M, D> qf[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int qi = iw0 + 32 * rb + r;
    qf[rb].load(qp + (long long)qi * a.q.ss, wave_live && qi < sq, g);
    if (P.scale_log2 < 0.f) qf[rb].negate();
  }

  float m[RB], l[RB];
  f32x16 acc[RB][DVT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DVT; ++dt) acc[rb][dt] = zero16();
  }

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
    auto dma = [&](T* kb, T* vb, int t) {
      kd.issue(kb, kp + (long long)t * BN * a.k.ss, a.k.ss, sk - t * BN, wave, lane);
      vd.issue(vb, vp + (long long)t * BN * a.v.ss, a.v.ss, sk - t * BN, wave, lane);
    };
    // Step t: K_t and V_t sit in stage P = (t - t0) & 1; the copies of K_{t+1}
    // and V_{t+1} into stage P^1 fly during the step.
    dma(k_s0, v_s0, t0);
    __syncthreads();
    auto step = [&](auto parity, int t) {
      constexpr int Pq = decltype(parity)::value;
      T* kc = Pq ? k_s1 : k_s0;
      T* vc = Pq ? v_s1 : v_s0;
      if (t + 1 <= t1) dma(Pq ? k_s0 : k_s1, Pq ? v_s0 : v_s1, t + 1);
      if (tw0 <= t && t <= tw1) {
        f32x16 s[RB][KT];
        F::scores(kc, lo, qf, s);
        const bool masked = t < full.t0 || t > full.t1;
        float cc = c;
        uint32_t keep[RB][KT];
        if constexpr (FEAT) {
          // Logits in the log2 domain with the additive terms, and the
          // dropout bits of every element (4 consecutive keys per counter).
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
              const int qi = iw0 + 32 * rb + r, jb = t * BN + 32 * kt;
              keep[rb][kt] = 0xffffu;
#pragma unroll
              for (int e = 0; e < 16; ++e)
                s[rb][kt][e] = __builtin_fmaf(s[rb][kt][e], c, extra_log2<T>(a.f, b, h, qi, jb + acc_row(e, g), sq, sk));
              if (a.f.drop_thresh) {
                keep[rb][kt] = 0;
#pragma unroll
                for (int qd = 0; qd < 4; ++qd)
                  keep[rb][kt] |= keep4(a.f, b, h, P.H, qi, jb + 8 * qd + 4 * g, P.Sq, P.Sk) << (4 * qd);
              }
            }
          cc = 1.f;
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int rb0 = iw0 + 32 * rb;
          F::finalize(s[rb], masked, w, t * BN, rb0 + r, sk, cc, m[rb], l[rb], acc[rb], g);
        }
        if (FEAT && a.f.drop_thresh)
          F::template softmax_pv<true>(vc, lo, s, acc, m, cc, l, keep);
        else
          F::softmax_pv(vc, lo, s, acc, m, cc, l);
      }
      __syncthreads();
    };
    for (int t = t0; t <= t1; t += 2) {
      step(std::integral_constant<int, 0>{}, t);
      if (t + 1 <= t1) step(std::integral_constant<int, 1>{}, t + 1);
    }
  }

  if (wave_live) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int qi = iw0 + 32 * rb + r;
      const float lt = halves_sum(l[rb]);
      if (qi < sq) {
        const float inv = lt > 0.f ? (FEAT && a.f.drop_thresh ? a.f.drop_scale : 1.f) / lt : 0.f;
        T* orow = op + (long long)qi * a.o.ss;
#pragma unroll
        for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int d = 32 * dt + 8 * q4 + 4 * g;
            if (d < D)
              store4<T>(orow + d, acc[rb][dt][4 * q4] * inv, acc[rb][dt][4 * q4 + 1] * inv,
                        acc[rb][dt][4 * q4 + 2] * inv, acc[rb][dt][4 * q4 + 3] * inv);
          }
        if (g == 0) lp[qi * P.olse_ss] = lt > 0.f ? (m[rb] + __builtin_amdgcn_logf(lt)) * kLn2 : INFINITY;
      }
    }
  }
}

// ------------------------------------------------ 16-bit ping-pong kernel
//
// Eight waves, 32 query rows each, in two groups of four; waves w and w+4
// share a SIMD.  Per key tile k a wave runs a matrix block M_k
// (O^T += V^T P^T of tile k-1, then S^T = K Q^T of tile k) and a vector
// block V_k (mask, row max, rescale, exp and rounding of P).  Group B runs
// one block behind group A and a workgroup barrier closes every block, so on
// each SIMD one wave keeps the matrix cores busy while the other works on
// the vector units.  Group A copies the K tiles (K_{k+2} during V_k, K_0
// and K_1 up front), group B the V tiles (V_{k+2} during V_k, V_0 and V_1
// up front), three stages each: a copy has about three blocks to land, each
// phase issues the copies of one tile, and each group waits only for the
// tile its next block reads (a partial vmcnt) at the barrier one block
// before its first reader.
template <typename M, int D, int BN>
struct FwdPP {
  using F = Fwd16<M, D, BN, 1>;
  using T = typename M::elem;
  using frag = typename M::frag;
  static constexpr int KT = F::KT, DVT = F::DVT;
  using Dma = DmaLane<T, D, BN, 4>;

  // K stages 0-2 then V stages 0-2 in one LDS array.  Operand reads address
  // a stage through an immediate offset from the array start (at most 64
  // KiB), so the V reads take lane offsets biased by 3 tiles (VOff).
  struct Ctx {
    T* ks[3];
    T* vs[3];
    const T* kp;
    const T* vp;
    long long kss, vss;
    int t0, nt, tw0, tw1, sk, qi, gw, lane, g;
    TileRange full;
    Window w;
    float c;
  };

  static constexpr int NPV = KT * 2 * DVT, NSC = KT * F::NS;
  static constexpr int NSTG = 3;  // K and V stages
  static constexpr int prev(int ks) { return (ks + NSTG - 1) % NSTG; }
  // Transposing-read offsets of the V tiles, biased by NSTG tiles (the V
  // region) and hidden from constant folding, so that a read of V stage p
  // is ks[p] + an immediate.
  struct VOff {
    int a[DVT], b[DVT];
    __device__ __forceinline__ void init(const LdsOffsets<M, D>& lo) {
#pragma unroll
      for (int dt = 0; dt < DVT; ++dt) {
        a[dt] = lo.tra[dt] + NSTG * F::TILE;
        b[dt] = lo.trb[dt] + NSTG * F::TILE;
        asm volatile("" : "+v"(a[dt]), "+v"(b[dt]));
      }
    }
  };
  template <int KS, int B, int E>
  struct Steps {
    static constexpr int PD = 4 < E - B ? 4 : E - B;  // LDS operand reads ahead of the products
    static constexpr int reads(int i) { return i < NPV ? 2 : 1; }  // LDS instructions of step i
    const Ctx& x;
    const LdsOffsets<M, D>& lo;
    const VOff& vo;
    const RowFrags<M, D>& qf;
    frag (*pf)[2];
    f32x16* acc;
    f32x16* s;
    frag buf[PD];

    __device__ __forceinline__ frag load(int i) const {
      if (i < NPV) {
        const int kt = i / (2 * DVT), st = (i / DVT) % 2, dt = i % DVT;
        return ld_tr<M>(x.ks[prev(KS)] + (32 * kt + 16 * st) * F::L::PITCH, vo.a[dt], vo.b[dt]);
      }
      const int j = i - NPV, kt = j % KT, st = j / KT;  // two accumulators in turn
      return ld_row<M>(x.ks[KS] + 32 * kt * F::L::PITCH, lo.row[st]);
    }
    template <int I>
    __device__ __forceinline__ void step() {
      const frag A = buf[(I - B) % PD];
      if constexpr (I + PD < E) buf[(I - B) % PD] = load(I + PD);
      if constexpr (I < NPV) {
        constexpr int kt = I / (2 * DVT), st = (I / DVT) % 2, dt = I % DVT;
        acc[dt] = M::mma(A, pf[kt][st], acc[dt]);
      } else {
        constexpr int j = I - NPV, kt = j % KT, st = j / KT;
        s[kt] = M::mma(A, qf.f[st], st == 0 ? zero16() : s[kt]);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (I + PD < E) __builtin_amdgcn_sched_group_barrier(0x100, reads(I + PD), 0);
    }
    template <int... Is>
    __device__ __forceinline__ void all(std::integer_sequence<int, Is...>) {
      (step<B + Is>(), ...);
    }
    __device__ __forceinline__ void run() {
#pragma unroll
      for (int i = 0; i < PD; ++i) buf[i] = load(B + i);
      constexpr int PRO = (B + PD <= NPV ? 2 * PD : (B >= NPV ? PD : 2 * (NPV - B) + (B + PD - NPV)));
      __builtin_amdgcn_sched_group_barrier(0x100, PRO, 0);
      all(std::make_integer_sequence<int, E - B>{});
    }
  };
  // Matrix steps i in [B, E) of one block: steps below NPV are
  // O^T += V^T P^T (V of the previous tile, stage prev(KS)), the rest
  // S^T = K Q^T (K stage KS).  The LDS operands run PD steps ahead of the
  // MFMAs.
  template <int KS, int B, int E>
  static __device__ __forceinline__ void mma_steps(const Ctx& x, const LdsOffsets<M, D>& lo, const VOff& vo,
                                                   const RowFrags<M, D>& qf, frag (*pf)[2], f32x16* acc, f32x16* s) {
    Steps<KS, B, E> st{x, lo, vo, qf, pf, acc, s, {}};
    st.run();
  }

  template <int GRP>
  static __device__ __forceinline__ void run(const Ctx& x, const LdsOffsets<M, D>& lo, const VOff& vo,
                                             const Dma& dma, const RowFrags<M, D>* qf, float& m, float& l,
                                             f32x16* acc) {
    f32x16 s[1][KT];
    frag pf[KT][2];
    auto mine = [&](int kk) { return x.tw0 <= x.t0 + kk && x.t0 + kk <= x.tw1; };
    auto copy = [&](T* dst, const T* base, long long ss, int kk) {
      const int j0 = (x.t0 + kk) * BN;
      dma.issue(dst, base + (long long)j0 * ss, ss, x.sk - j0, x.gw, x.lane);
    };
    // Barrier closing a block.  With `vm` it first waits for this wave's
    // copies except the newest tile's, or for all of them when `all` (no
    // newer tile was issued): an explicit s_waitcnt (vmcnt(N) lgkmcnt(0);
    // copies complete in order) that the compiler keeps and accounts for;
    // the asm barrier keeps memory accesses on their side of it.
    auto barrier = [&](auto vm, bool all) {
      if constexpr (decltype(vm)::value) {
        if (all)
          __builtin_amdgcn_s_waitcnt(0x0070);
        else
          __builtin_amdgcn_s_waitcnt(0x0070 | Dma::PER);
        asm volatile("s_barrier" ::: "memory");
      } else {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
    };
    auto mblock = [&](auto kst, int kk) {
      constexpr int KS = decltype(kst)::value;
      const bool pv = kk >= 1 && mine(kk - 1), sc = kk < x.nt && mine(kk);
      if (pv) mma_steps<KS, 0, NPV>(x, lo, vo, qf[0], pf, acc, s[0]);
      if (sc) mma_steps<KS, NPV, NPV + NSC>(x, lo, vo, qf[0], pf, acc, s[0]);
      // Group B: V_kk, read by the next block of group A, must have landed.
      // M_nt (the last tile's P.V only) closes with group B's last vector
      // block, so only group A meets a barrier there.
      if (GRP == 0 || kk < x.nt) barrier(std::integral_constant<bool, GRP == 1>{}, kk + 1 >= x.nt);
    };
    auto vblock = [&](auto kst, int kk) {
      constexpr int KS = decltype(kst)::value;
      // Copies of tile kk+2: K by group A here (while group B runs M_kk), V
      // by group B here (while group A runs M_kk+1), so each phase issues
      // one tile of copies, from the waves that run vector work.
      if (kk + 2 < x.nt) {
        if constexpr (GRP == 0)
          copy(x.ks[(KS + 2) % NSTG], x.kp, x.kss, kk + 2);
        else
          copy(x.vs[(KS + 2) % NSTG], x.vp, x.vss, kk + 2);
      }
      if (mine(kk)) {
        const int t = x.t0 + kk;
        if (t < x.full.t0 || t > x.full.t1) F::mask(s[0], x.w, t * BN, x.qi, x.sk, x.g);
        // P = 2^(c s - m) against the current reference max, packed, and
        // this lane's share of the row sum.
        auto probs = [&]() __attribute__((always_inline)) {
          const float nm = m == -INFINITY ? 0.f : -m;
          float sum = 0.f;
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            float e2[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              e2[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[0][kt][e], x.c, nm));
              sum += e2[e];
            }
            M::pack(&e2[0], pf[kt][0]);
            M::pack(&e2[8], pf[kt][1]);
          }
          return sum;
        };
        float ls = probs();
        // Each P of a lane is at most the lane's sum, so a sum within
        // 2^kRescaleSlack keeps every P there without the tile's max.  A row
        // with no reference max yet, or a larger (or non-finite) sum, takes
        // the max first, raises m to it (no slack: the next tiles of such a
        // row start from its new max) and computes the P again.
        if (__builtin_amdgcn_ballot_w64(m == -INFINITY || !(ls <= kRescaleBound))) {
          F::raise(s[0], x.c, m, l, acc, 0.f);
          ls = probs();
        }
        l += ls;
      }
      // Group A: K_{kk+1}, read by its next block, must have landed.
      barrier(std::integral_constant<bool, GRP == 0>{}, kk + 2 >= x.nt);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    if constexpr (GRP == 1) {
      copy(x.vs[0], x.vp, x.vss, 0);
      if (x.nt > 1) copy(x.vs[1], x.vp, x.vss, 1);
      barrier(std::false_type{}, true);
    }
    // Tiles 0 .. nt-1, then M_nt: O^T += V^T P^T of the last tile.
    for (int kk = 0;; kk += 3) {
      mblock(I0{}, kk);
      if (kk >= x.nt) break;
      vblock(I0{}, kk);
      mblock(I1{}, kk + 1);
      if (kk + 1 >= x.nt) break;
      vblock(I1{}, kk + 1);
      mblock(I2{}, kk + 2);
      if (kk + 2 >= x.nt) break;
      vblock(I2{}, kk + 2);
    }
  }
};

// Workgroups of the ping-pong kernel per CU (pp_wg_per_cu): two at
// head_dim 64, where a wave fits in 128 registers, so one workgroup's start
// (Q rows, first tiles) and end (O rows) overlap the other's steady state
// (192x16x512x64 fp16: 0.427 -> 0.374 ms); one otherwise.
template <int D>
constexpr int pp_per_cu() { return pp_wg_per_cu(D); }

// One 256-row block (bh, qb) of the ping-pong kernel.  With KS the
// workgroup is part `part` of `np` over the block's key tiles and stores
// its partial into slot `slot` of the key-split partials instead of O and
// LSE.
template <typename M, int D, int BN, bool KS>
__device__ __forceinline__ void fwd16pp_block(const FwdArgs& a, typename M::elem* kv_s, int bh, int qb, int part,
                                              int np, int slot) {
  using PP = FwdPP<M, D, BN>;
  using F = typename PP::F;
  using T = typename M::elem;
  constexpr int BM = 256, DVT = F::DVT;

  const ProblemArgs& P = a.p;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int h = bh % P.H, b = bh / P.H;

  long long q0, k0;
  int sq, sk;
  seq_rows(P, b, q0, sq, k0, sk);
  const int i0 = qb * BM;
  if (i0 >= sq) return;  // every part of the block (and its merge) returns here
  const Window w = seq_window(P.wl, P.wr, P.diag, sq, sk);

  const T* qp = (const T*)a.q.ptr + b * a.q.sb + h * a.q.sh + q0 * a.q.ss;
  T* op = (T*)a.o.ptr + b * a.o.sb + h * a.o.sh + q0 * a.o.ss;
  float* lp = a.lse + b * P.olse_sb + h * P.olse_sh + q0 * P.olse_ss;

  const int ilast = min(i0 + BM, sq) - 1;
  const long long jlo = max(0LL, (long long)i0 + w.lo);
  const long long jhi = min((long long)sk - 1, (long long)ilast + w.hi);
  const bool block_empty = w.lo > w.hi || jlo > jhi;

  const int iw0 = i0 + 32 * wave;
  const bool wave_live = iw0 < sq;
  const int qi = iw0 + r;

  typename PP::Ctx x;
  x.tw0 = 0x7fffffff;
  x.tw1 = -1;
  if (wave_live && w.lo <= w.hi) {
    const long long a0 = max(0LL, (long long)iw0 + w.lo);
    const long long a1 = min((long long)sk - 1, (long long)min(iw0 + 31, sq - 1) + w.hi);
    if (a0 <= a1) {
      x.tw0 = (int)(a0 / BN);
      x.tw1 = (int)(a1 / BN);
    }
  }
  x.full = tiles_starting_in((long long)iw0 + 31 + w.lo, min((long long)iw0 + w.hi, (long long)sk - 1) - BN + 1, BN);
  x.c = fmaxf(fabsf(P.scale_log2), 1e-30f);
  x.w = w;
  x.sk = sk;
  x.qi = qi;
  x.lane = lane;
  x.g = g;
  x.gw = wave & 3;

  RowFrags<M, D> qf[1];
  qf[0].load(qp + (long long)qi * a.q.ss, wave_live && qi < sq, g);
  if (P.scale_log2 < 0.f) qf[0].negate();

  float m = -INFINITY, l = 0.f;
  f32x16 acc[DVT];
#pragma unroll
  for (int dt = 0; dt < DVT; ++dt) acc[dt] = zero16();

  x.t0 = (int)(jlo / BN);
  x.nt = block_empty ? 0 : (int)(jhi / BN) - x.t0 + 1;
  if constexpr (KS) {
    // Part `part` takes tiles [nt part / np, nt (part + 1) / np) of the block's.
    const int s0 = (int)((long long)x.nt * part / np), s1 = (int)((long long)x.nt * (part + 1) / np);
    x.t0 += s0;
    x.nt = s1 - s0;
  }
  if (x.nt > 0) {
    LdsOffsets<M, D> lo;
    lo.init(lane);
    typename PP::Dma dma;
    const bool grp_b = wave >= 4;
    dma.init(grp_b ? a.v.ss : a.k.ss, x.gw, lane);
#pragma unroll
    for (int i = 0; i < PP::NSTG; ++i) {
      x.ks[i] = kv_s + i * F::TILE;
      x.vs[i] = kv_s + (PP::NSTG + i) * F::TILE;
      zero_unused_slots<T, D, BN, 512>(x.ks[i], tid);
      zero_unused_slots<T, D, BN, 512>(x.vs[i], tid);
    }
    typename PP::VOff vo;
    vo.init(lo);
    x.kp = (const T*)a.k.ptr + b * a.k.sb + h * a.k.sh + k0 * a.k.ss;
    x.vp = (const T*)a.v.ptr + b * a.v.sb + h * a.v.sh + k0 * a.v.ss;
    x.kss = a.k.ss;
    x.vss = a.v.ss;
    if (!grp_b) {
      // K_0 and K_1 up front; this wave's part of K_0 lands before the barrier.
      dma.issue(x.ks[0], x.kp + (long long)x.t0 * BN * a.k.ss, a.k.ss, sk - x.t0 * BN, x.gw, lane);
      if (x.nt > 1) {
        dma.issue(x.ks[1], x.kp + (long long)(x.t0 + 1) * BN * a.k.ss, a.k.ss, sk - (x.t0 + 1) * BN, x.gw, lane);
        __builtin_amdgcn_s_waitcnt(0x0070 | PP::Dma::PER);
      } else {
        __builtin_amdgcn_s_waitcnt(0x0070);
      }
    }
    __syncthreads();
    if (grp_b)
      PP::template run<1>(x, lo, vo, dma, qf, m, l, acc);
    else
      PP::template run<0>(x, lo, vo, dma, qf, m, l, acc);
  }

  if constexpr (KS) {
    // This part's unnormalised (O^T, m, l) per lane (l: the lane's half of
    // the row sum); the merge kernel combines the block's parts.
    constexpr int NC = ks_chunks(D);
    float4* pw = reinterpret_cast<float4*>(a.ks_part) + ((long long)slot * 8 + wave) * NC * 64 + lane;
#pragma unroll
    for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        pw[(4 * dt + q4) * 64] = make_float4(acc[dt][4 * q4], acc[dt][4 * q4 + 1], acc[dt][4 * q4 + 2],
                                             acc[dt][4 * q4 + 3]);
    pw[(NC - 1) * 64] = make_float4(m, l, 0.f, 0.f);
    return;
  }

  if (wave_live) {
    const float lt = halves_sum(l);
    if (qi < sq) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      T* orow = op + (long long)qi * a.o.ss;
#pragma unroll
      for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = 32 * dt + 8 * q4 + 4 * g;
          if (d < D)
            store4<T>(orow + d, acc[dt][4 * q4] * inv, acc[dt][4 * q4 + 1] * inv, acc[dt][4 * q4 + 2] * inv,
                      acc[dt][4 * q4 + 3] * inv);
        }
      if (g == 0) lp[qi * P.olse_ss] = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : INFINITY;
    }
  }
}

// The ping-pong grid: logical blocks [0, gridDim.x) of nq 256-row blocks per
// (batch, head), in grid_pos order; the rest, if any, go to a tail kernel.
template <typename M, int D, int BN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2 * pp_per_cu<D>(), 2 * pp_per_cu<D>()))) void
attn_fwd16pp_kernel(FwdArgs a, int nq) {
  using PP = FwdPP<M, D, BN>;
  using T = typename M::elem;
  __shared__ __attribute__((aligned(1024))) T kv_s[2 * PP::NSTG * PP::F::TILE];
  const GridPos gp = grid_pos(blockIdx.x, gridDim.x, nq, a.p.B * a.p.H, a.p.ragged);
  fwd16pp_block<M, D, BN, false>(a, kv_s, gp.bh, nq - 1 - gp.i, 0, 1, 0);
}

// (batch, head) and block index along the sequence of logical block L of a
// grid of nq blocks per (batch, head), in grid_pos's logical order.
__device__ __forceinline__ GridPos logical_pos(const ProblemArgs& P, int L, int nq) {
  const int nbh = P.B * P.H;
  return P.ragged ? GridPos{L % nbh, L / nbh} : GridPos{L / nq, L % nq};
}

// The key-split tail: np workgroups per logical block lbase + blockIdx.x /
// np (the blocks after the ping-pong grid's, in the same order), part
// blockIdx.x % np of its key tiles, into partial slot blockIdx.x.
template <typename M, int D, int BN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2 * pp_per_cu<D>(), 2 * pp_per_cu<D>()))) void
attn_fwd16ppks_kernel(FwdArgs a, int nq, int lbase, int np) {
  using PP = FwdPP<M, D, BN>;
  using T = typename M::elem;
  __shared__ __attribute__((aligned(1024))) T kv_s[2 * PP::NSTG * PP::F::TILE];
  const GridPos gp = logical_pos(a.p, lbase + (int)blockIdx.x / np, nq);
  fwd16pp_block<M, D, BN, true>(a, kv_s, gp.bh, nq - 1 - gp.i, (int)blockIdx.x % np, np, (int)blockIdx.x);
}

// The key-split tail's merge: one wave per workgroup, for rows 32 w .. 32 w
// + 31 (wave w's) and columns 32 c .. 32 c + 31 of tail block blockIdx.x /
// (8 C) (C = ceil(D / 32) column blocks), which combines the block's np
// slots in slot order, m = max_s m_s, O^T = sum_s 2^(m_s - m) O_s^T, l
// likewise, and writes O = O^T / l (and, for c = 0, LSE) as the ping-pong
// epilogue does.  Each part's loads are issued before the previous part's
// products.  The kernel boundary orders the tail grid's stores before
// these loads.
template <typename M, int D>
__global__ __launch_bounds__(64) void attn_fwd16ksmerge_kernel(FwdArgs a, int nq, int lbase, int np) {
  using T = typename M::elem;
  constexpr int DVT = (D + 31) / 32, NC = ks_chunks(D);
  const ProblemArgs& P = a.p;
  const int bid = (int)blockIdx.x, dt = bid % DVT, wave = (bid / DVT) % 8, tb = bid / (8 * DVT);
  const int lane = threadIdx.x, r = lane & 31, g = lane >> 5;
  const GridPos gp = logical_pos(P, lbase + tb, nq);
  const int h = gp.bh % P.H, b = gp.bh / P.H, qb = nq - 1 - gp.i;
  long long q0, k0;
  int sq, sk;
  seq_rows(P, b, q0, sq, k0, sk);
  const int iw0 = qb * 256 + 32 * wave, qi = iw0 + r;
  if (iw0 >= sq) return;  // whole wave: no partial was stored for these rows' block, or they are past the end
  const long long SLOT = 8LL * NC * 64;
  const float4* pb = reinterpret_cast<const float4*>(a.ks_part) + ((long long)tb * np * 8 + wave) * NC * 64 + lane;
  float mx = -INFINITY;
  for (int s = 0; s < np; ++s) mx = fmaxf(mx, pb[s * SLOT + (NC - 1) * 64].x);
  // Chunks 4 dt .. 4 dt + 3 (this column block) and NC - 1 (m, l) of a slot.
  auto load = [&](int s, float4* c) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) c[q4] = pb[s * SLOT + (4 * dt + q4) * 64];
    c[4] = pb[s * SLOT + (NC - 1) * 64];
  };
  float4 cur[5], nxt[5];
  load(0, cur);
  float l = 0.f;
  float4 o[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) o[q4] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < np; ++s) {
    if (s + 1 < np) load(s + 1, nxt);
    const float f = cur[4].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(cur[4].x - mx);
    l = __builtin_fmaf(f, cur[4].y, l);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      o[q4].x = __builtin_fmaf(f, cur[q4].x, o[q4].x);
      o[q4].y = __builtin_fmaf(f, cur[q4].y, o[q4].y);
      o[q4].z = __builtin_fmaf(f, cur[q4].z, o[q4].z);
      o[q4].w = __builtin_fmaf(f, cur[q4].w, o[q4].w);
    }
    if (s + 1 < np)
#pragma unroll
      for (int q4 = 0; q4 < 5; ++q4) cur[q4] = nxt[q4];
  }
  const float lt = halves_sum(l);
  if (qi >= sq) return;
  T* orow = (T*)a.o.ptr + b * a.o.sb + h * a.o.sh + (q0 + qi) * a.o.ss;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int d = 32 * dt + 8 * q4 + 4 * g;
    if (d < D) store4<T>(orow + d, o[q4].x * inv, o[q4].y * inv, o[q4].z * inv, o[q4].w * inv);
  }
  float* lp = a.lse + b * P.olse_sb + h * P.olse_sh + q0 * P.olse_ss;
  if (dt == 0 && g == 0) lp[qi * P.olse_ss] = lt > 0.f ? (mx + __builtin_amdgcn_logf(lt)) * kLn2 : INFINITY;
}

// -------------------------------------------- 16-bit forward, grid tail
//
// The rows of the ping-pong grid's last, partly filled round: each 256-row
// block becomes four workgroups of 64 rows, and each workgroup splits its
// key tiles into two halves.  Waves 0-1 take rows 0-31 / 32-63 over the
// first half, waves 2-3 the same rows over the second half, each half with
// its own two-stage K/V tiles; at the end the second half's (O^T, m, l)
// pass through LDS and the first half's waves merge them:
//   m = max(m0, m1), O^T = 2^(m0-m) O0^T + 2^(m1-m) O1^T, l likewise.
// Four times as many workgroups with half the keys each spread the tail
// over every CU, one wave per SIMD.
template <typename M, int D>
struct FwdSplit {
  using F = Fwd16<M, D, 64, 1>;
  using T = typename M::elem;
  static constexpr int BN = 64, DVT = F::DVT;
};

template <typename M, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_fwd16split_kernel(FwdArgs a,
                                                                                                      int nq,
                                                                                                      int lbase) {
  using F = typename FwdSplit<M, D>::F;
  using T = typename M::elem;
  constexpr int BN = 64, NT = 256, DVT = F::DVT, KT = F::KT;
  // Key half 0 and key half 1, two stages of K and V each.
  __shared__ __attribute__((aligned(1024))) T k00[F::TILE], k01[F::TILE], v00[F::TILE], v01[F::TILE];
  __shared__ __attribute__((aligned(1024))) T k10[F::TILE], k11[F::TILE], v10[F::TILE], v11[F::TILE];

  const ProblemArgs& P = a.p;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int rg = wave & 1, kh = wave >> 1;                     // row group, key half
  const int L = lbase + (int)blockIdx.x / 4, sub = (int)blockIdx.x % 4;
  // Logical block L of the whole grid, in the order grid_pos gives the
  // ping-pong kernel's blocks (which cover L < lbase).
  const int nbh = P.B * P.H;
  const int bh = P.ragged ? L % nbh : L / nq, h = bh % P.H, b = bh / P.H;
  const int qb = nq - 1 - (P.ragged ? L / nbh : L % nq);

  long long q0, k0;
  int sq, sk;
  seq_rows(P, b, q0, sq, k0, sk);
  const int i0 = qb * 256 + 64 * sub;
  if (i0 >= sq) return;
  const Window w = seq_window(P.wl, P.wr, P.diag, sq, sk);

  const T* qp = (const T*)a.q.ptr + b * a.q.sb + h * a.q.sh + q0 * a.q.ss;
  const T* kp = (const T*)a.k.ptr + b * a.k.sb + h * a.k.sh + k0 * a.k.ss;
  const T* vp = (const T*)a.v.ptr + b * a.v.sb + h * a.v.sh + k0 * a.v.ss;
  T* op = (T*)a.o.ptr + b * a.o.sb + h * a.o.sh + q0 * a.o.ss;
  float* lp = a.lse + b * P.olse_sb + h * P.olse_sh + q0 * P.olse_ss;

  const int ilast = min(i0 + 64, sq) - 1;
  const long long jlo = max(0LL, (long long)i0 + w.lo);
  const long long jhi = min((long long)sk - 1, (long long)ilast + w.hi);
  const bool block_empty = w.lo > w.hi || jlo > jhi;

  const int iw0 = i0 + 32 * rg;
  const bool wave_live = iw0 < sq;
  const int qi = iw0 + r;
  int tw0 = 0x7fffffff, tw1 = -1;
  if (wave_live && w.lo <= w.hi) {
    const long long a0 = max(0LL, (long long)iw0 + w.lo);
    const long long a1 = min((long long)sk - 1, (long long)min(iw0 + 31, sq - 1) + w.hi);
    if (a0 <= a1) {
      tw0 = (int)(a0 / BN);
      tw1 = (int)(a1 / BN);
    }
  }
  const TileRange full = tiles_starting_in((long long)iw0 + 31 + w.lo,
                                           min((long long)iw0 + w.hi, (long long)sk - 1) - BN + 1, BN);
  const float c = fmaxf(fabsf(P.scale_log2), 1e-30f);
  RowFrags<M, D> qf[1];
  qf[0].load(qp + (long long)qi * a.q.ss, wave_live && qi < sq, g);
  if (P.scale_log2 < 0.f) qf[0].negate();

  float m[1] = {-INFINITY}, l[1] = {0.f};
  f32x16 acc[1][DVT];
#pragma unroll
  for (int dt = 0; dt < DVT; ++dt) acc[0][dt] = zero16();

  // Barrier that also waits for this wave's direct loads (explicit wait the
  // compiler accounts for).
  auto barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0070);
    asm volatile("s_barrier" ::: "memory");
  };
  const int t0 = (int)(jlo / BN), n = block_empty ? 0 : (int)(jhi / BN) - t0 + 1, n0 = (n + 1) / 2;
  if (!block_empty) {
    LdsOffsets<M, D> lo;
    lo.init(lane);
    DmaLane<T, D, BN, 2> kd, vd;
    kd.init(a.k.ss, rg, lane);
    vd.init(a.v.ss, rg, lane);
    for (T* t : {k00, k01, v00, v01, k10, k11, v10, v11}) zero_unused_slots<T, D, BN, NT>(t, tid);
    // Key half HALF: tiles [tb, tb + cnt), both halves stepping together for
    // n0 steps (half 1 has n0 or n0 - 1 tiles).
    auto run = [&](T* ka, T* kb, T* va, T* vb, int tb, int cnt) {
      auto dma = [&](T* kdst, T* vdst, int t) {
        kd.issue(kdst, kp + (long long)t * BN * a.k.ss, a.k.ss, sk - t * BN, rg, lane);
        vd.issue(vdst, vp + (long long)t * BN * a.v.ss, a.v.ss, sk - t * BN, rg, lane);
      };
      if (cnt > 0) dma(ka, va, tb);
      barrier();
      auto step = [&](auto parity, int st) {
        constexpr int Pq = decltype(parity)::value;
        if (st + 1 < cnt) dma(Pq ? ka : kb, Pq ? va : vb, tb + st + 1);
        const int t = tb + st;
        if (st < cnt && tw0 <= t && t <= tw1) {
          f32x16 sc[1][KT];
          F::scores(Pq ? kb : ka, lo, qf, sc);
          F::finalize(sc[0], t < full.t0 || t > full.t1, w, t * BN, qi, sk, c, m[0], l[0], acc[0], g);
          F::softmax_pv(Pq ? vb : va, lo, sc, acc, m, c, l);
        }
        barrier();
      };
      for (int st = 0; st < n0; st += 2) {
        step(std::integral_constant<int, 0>{}, st);
        if (st + 1 < n0) step(std::integral_constant<int, 1>{}, st + 1);
      }
    };
    if (kh == 0)
      run(k00, k01, v00, v01, t0, n0);
    else
      run(k10, k11, v10, v11, t0 + n0, n - n0);
  }

  // Merge: the second half's waves leave O^T, m, l in LDS (half 1's K tiles
  // hold one wave's O^T each, its V tile the row statistics); the first
  // half's waves combine and write.
  float* part = reinterpret_cast<float*>(rg == 0 ? k10 : k11);
  float* stat = reinterpret_cast<float*>(v10) + rg * 128;
  if (kh == 1) {
#pragma unroll
    for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4*>(part + ((dt * 4 + q4) * 64 + lane) * 4) =
            make_float4(acc[0][dt][4 * q4], acc[0][dt][4 * q4 + 1], acc[0][dt][4 * q4 + 2], acc[0][dt][4 * q4 + 3]);
    stat[lane] = m[0];
    stat[64 + lane] = l[0];
  }
  barrier();
  if (kh == 1 || !wave_live) return;
  const float m1 = stat[lane], l1 = stat[64 + lane];
  const float mm = fmaxf(m[0], m1);
  const float a0 = m[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[0] - mm);
  const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
  const float lt = halves_sum(l[0] * a0 + l1 * a1);
  if (qi < sq) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    T* orow = op + (long long)qi * a.o.ss;
#pragma unroll
    for (int dt = 0; dt < DVT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * dt + 8 * q4 + 4 * g;
        const float4 o1 = *reinterpret_cast<const float4*>(part + ((dt * 4 + q4) * 64 + lane) * 4);
        if (d < D)
          store4<T>(orow + d, (acc[0][dt][4 * q4] * a0 + o1.x * a1) * inv,
                    (acc[0][dt][4 * q4 + 1] * a0 + o1.y * a1) * inv, (acc[0][dt][4 * q4 + 2] * a0 + o1.z * a1) * inv,
                    (acc[0][dt][4 * q4 + 3] * a0 + o1.w * a1) * inv);
      }
    if (g == 0) lp[qi * P.olse_ss] = lt > 0.f ? (mm + __builtin_amdgcn_logf(lt)) * kLn2 : INFINITY;
  }
}

// Workgroup shapes.  fp32 (register-staged kernel, tiles twice as large):
// 4 waves, 64-key tiles.  16-bit, 64-key tiles, one 32-row block per wave,
// two waves per SIMD: the ping-pong kernel (8 waves) for wide bands; for
// narrower ones 4 waves (128-row blocks: under a band the finer blocks
// visit fewer keys; 8x16x2048x64 bf16 with a (256, 0) window 53.8 against
// 66.3 us at 8 waves, 8x16x2048x80 63.2 against 75.6 us).
template <typename M, int D>
struct FwdShape {
  static constexpr bool k16 = sizeof(typename M::elem) == 2;
  static constexpr bool PP = k16 && D <= 128;  // ping-pong kernel built (8 waves, 256 rows)
  static constexpr int RB = 1;
  static constexpr int NW = 4;
  static constexpr int BN = 64;
  static constexpr int WPE = D > 128 ? 1 : 2;  // waves per SIMD the registers allow
};

template <typename M, int D, class Ex>
static hipError_t launch_fwd_t(const FwdArgs& a, const Ex& ex) {
  using S = FwdShape<M, D>;
  constexpr int BN = S::BN;
  if (a.feat) {
    // Bias, ALiBi or dropout: the narrow kernel built with them (one wave
    // per SIMD above head_dim 80, where their registers do not fit two).
    const long long nq = (a.p.Sq + S::NW * 32 - 1) / (S::NW * 32);
    const long long nblk = nq * a.p.H * a.p.B;
    if (nblk == 0) return hipSuccess;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    if constexpr (S::k16)
      return ex(reinterpret_cast<const void*>(&attn_fwd16_kernel<M, D, S::NW, BN, 1, (D > 80 ? 1 : 2), true>),
                "attn_fwd16_kernel", (unsigned)nblk, (unsigned)(S::NW * 64), a);
    else
      return ex(reinterpret_cast<const void*>(&attn_fwd_kernel<M, D, S::NW, BN, true>), "attn_fwd_kernel",
                (unsigned)nblk, (unsigned)(S::NW * 64), a);
  }
  const bool pp = S::PP && wide_window(a.p);
  const int nw = pp ? 8 : S::NW, bm = nw * 32 * (pp ? 1 : S::RB);
  const long long nq = (a.p.Sq + bm - 1) / bm;
  const long long nblk = nq * a.p.H * a.p.B;
  if (nblk == 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  if constexpr (S::k16) {
    if constexpr (S::PP) if (pp) {
      // Full rounds of 256-row workgroups (pp_per_cu per CU) on the
      // ping-pong kernel.  A grid of at most a quarter as many blocks as CUs
      // goes to the split kernel whole: four workgroups per block, each over
      // half the keys, still fit one round (1x2x512x64: 8.9 against 15.7
      // us; 1x8x2048x128: 40.4 against 51.3 us), where a grid of half the
      // CUs would take two (4x8x1024x128: 46.8 against 33.0 us).
      long long nmain = nblk;
      const long long cu = device_cu_count(), cus = cu * pp_per_cu<D>();
      const int nqi = (int)nq;
      // Key tiles of 32 at head_dim <= 64: four waves per SIMD leave 128
      // registers, which the 64-key tile's scores overran (spilled to
      // scratch in the loop); the halved tile fits (BERT-like 192x16x512x64
      // bf16: 380 against 404 us).
      constexpr int PBN = D <= 64 ? 32 : BN;
      hipError_t err = hipSuccess;
      if (!a.no_split && cu > 0 && a.ks_part != nullptr) {
        // With a key-split workspace, the r blocks of a partly filled last
        // round (the whole grid when it has fewer blocks than a round) run
        // as np = min(8, cus / r) ping-pong workgroups each, every part over
        // at least ks_min_keys(D) keys of the block's band, so the tail
        // fills the round (1x32x6630x128: 64 tail blocks as 256 parts).  A
        // grid of at most a quarter as many blocks as CUs takes this only
        // when its parts cover every CU; else the split kernel below, whose
        // 64-row workgroups spread a small grid further (1x2x2048x64: 22.0
        // against 23.4 us; but 1x2x8192x128: 77 against 132 us, 1x1x16384x128:
        // 133 against 255 us, 1x4x4096x128: 48.8 against 69.7 us).
        const long long r = nblk % cus, nm = nblk - r;
        long long kb = a.p.Sk;
        if (a.p.wl != kWindowInf && a.p.wr != kWindowInf) kb = std::min(kb, (long long)a.p.wl + a.p.wr + 256);
        const long long np = r > 0 ? std::min(std::min(8LL, cus / r), kb / ks_min_keys(D)) : 0;
        if (np >= 2 && r * np <= a.ks_units && (4 * nblk > cu || r * np >= cu)) {
          if (nm > 0)
            err = ex(reinterpret_cast<const void*>(&attn_fwd16pp_kernel<M, D, PBN>), "attn_fwd16pp_kernel",
                     (unsigned)nm, 512u, a, nqi);
          if (err == hipSuccess)
            err = ex(reinterpret_cast<const void*>(&attn_fwd16ppks_kernel<M, D, PBN>), "attn_fwd16ppks_kernel",
                     (unsigned)(r * np), 512u, a, nqi, (int)nm, (int)np);
          if (err != hipSuccess) return err;
          return ex(reinterpret_cast<const void*>(&attn_fwd16ksmerge_kernel<M, D>), "attn_fwd16ksmerge_kernel",
                    (unsigned)(8 * ((D + 31) / 32) * r), 64u, a, nqi, (int)nm, (int)np);
        }
      }
      // Without it: with at most three full rounds, a last round at most a
      // quarter full goes to the split tail kernel, which then fills every
      // CU once (1x32x6630x128: 0.717 ms against 0.743 ms).  With more
      // rounds, or a fuller last round, the tail's share is too small to pay
      // for the split kernel's one wave per SIMD (1x32x15300x128: 3.63
      // against 3.46).
      if (!a.no_split) {
        if (cus > 0 && nblk >= cus && nblk < 4 * cus && 4 * (nblk % cus) <= cus)
          nmain = nblk - nblk % cus;
        else if (cu > 0 && 4 * nblk <= cu)
          nmain = 0;
      }
      if (nmain > 0)
        err = ex(reinterpret_cast<const void*>(&attn_fwd16pp_kernel<M, D, PBN>), "attn_fwd16pp_kernel",
                 (unsigned)nmain, 512u, a, nqi);
      if (err != hipSuccess || nmain == nblk) return err;
      return ex(reinterpret_cast<const void*>(&attn_fwd16split_kernel<M, D>), "attn_fwd16split_kernel",
                (unsigned)(4 * (nblk - nmain)), 256u, a, nqi, (int)nmain);
    }
    return ex(reinterpret_cast<const void*>(&attn_fwd16_kernel<M, D, S::NW, BN, S::RB, S::WPE>),
              "attn_fwd16_kernel", (unsigned)nblk, (unsigned)(nw * 64), a);
  } else {
    // Small grids at head_dim <= 64 (where two halves' stages fit LDS): 64-
    // row workgroups over two key halves, when at most half as many as CUs.
    if constexpr (D <= 64) {
      const long long nks = (a.p.Sq + 63) / 64 * a.p.H * a.p.B, cu = device_cu_count();
      if (!a.no_split && cu > 0 && 2 * nks <= cu)
        return ex(reinterpret_cast<const void*>(&attn_fwd_ks_kernel<M, D, BN>), "attn_fwd_ks_kernel",
                  (unsigned)nks, 256u, a);
    }
    return ex(reinterpret_cast<const void*>(&attn_fwd_kernel<M, D, S::NW, BN>), "attn_fwd_kernel", (unsigned)nblk,
              (unsigned)(nw * 64), a);
  }
}

template <typename M, class Ex>
static hipError_t launch_fwd_d(int head_dim, const FwdArgs& a, const Ex& ex) {
  switch (head_dim) {
    case 32: return launch_fwd_t<M, 32>(a, ex);
    case 48: return launch_fwd_t<M, 48>(a, ex);
    case 64: return launch_fwd_t<M, 64>(a, ex);
    case 80: return launch_fwd_t<M, 80>(a, ex);
    case 96: return launch_fwd_t<M, 96>(a, ex);
    case 128: return launch_fwd_t<M, 128>(a, ex);
    case 192:
      if constexpr (sizeof(typename M::elem) == 2) return launch_fwd_t<M, 192>(a, ex);
      return hipErrorNotSupported;
    case 256:
      if constexpr (sizeof(typename M::elem) == 2) return launch_fwd_t<M, 256>(a, ex);
      return hipErrorNotSupported;
    default: return hipErrorNotSupported;
  }
}

// ------------------------------------------------ rows past the used ones
//
// Rows of a sequence's room past its length (lengths from seqused arrays,
// or cumulative lengths inside uniform rooms) take part in no attention:
// they are written as fully masked rows (zeros, LSE +inf).  One workgroup
// per (sequence, head); 16-byte stores.
struct PadArgs {
  ProblemArgs p;
  Operand t[2];  // tensors whose padding rows are zeroed (null: none)
  float* lse;    // LSE rows set to +inf (query side of the forward), or null
  int side;      // 0: query rows, 1: key rows
  int chunks;    // 16-byte chunks per row
  int esz;       // element size of t
};

__global__ __launch_bounds__(256) void attn_pad_rows_kernel(PadArgs a) {
  const ProblemArgs& P = a.p;
  const int h = (int)(blockIdx.x % P.H), b = (int)(blockIdx.x / P.H);
  const SideRows r = side_rows(a.side ? P.ks : P.qs, b);
  if (r.room < 0) return;
  const long long work = (long long)(r.room - r.n) * a.chunks;
  for (long long x = threadIdx.x; x < work; x += 256) {
    const long long row = r.r0 + r.n + x / a.chunks;
    const int c = (int)(x % a.chunks);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (a.t[i].ptr) {
        char* p = (char*)a.t[i].ptr + (b * a.t[i].sb + h * a.t[i].sh + row * a.t[i].ss) * a.esz + 16 * c;
        *reinterpret_cast<uint4*>(p) = make_uint4(0, 0, 0, 0);
      }
  }
  if (a.lse)
    for (int x = threadIdx.x; x < r.room - r.n; x += 256)
      a.lse[b * P.olse_sb + h * P.olse_sh + (r.r0 + r.n + x) * P.olse_ss] = INFINITY;
}

template <class Ex>
hipError_t launch_pad_rows(const ProblemArgs& p, Operand t0, Operand t1, float* lse, int side, int row_bytes,
                           int esz, const Ex& ex) {
  if (!side_may_pad(side ? p.ks.mode : p.qs.mode)) return hipSuccess;
  const long long nblk = (long long)p.B * p.H;
  if (nblk == 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  PadArgs a{};
  a.p = p;
  a.t[0] = t0;
  a.t[1] = t1;
  a.lse = lse;
  a.side = side;
  a.chunks = row_bytes / 16;
  a.esz = esz;
  return ex(reinterpret_cast<const void*>(&attn_pad_rows_kernel), "attn_pad_rows_kernel", (unsigned)nblk, 256u, a);
}
template hipError_t launch_pad_rows<Enqueue>(const ProblemArgs&, Operand, Operand, float*, int, int, int,
                                             const Enqueue&);
template hipError_t launch_pad_rows<Record>(const ProblemArgs&, Operand, Operand, float*, int, int, int,
                                            const Record&);

// One workgroup per (sequence, head) and slice of its rows; half a
// workgroup per row (128 columns per pass), element by element, so rows of
// any alignment and width are copied.
__global__ __launch_bounds__(256) void attn_repack_kernel(RepackArgs a, int slices) {
  const ProblemArgs& P = a.p;
  const int sl = (int)(blockIdx.x % (unsigned)slices), bh = (int)(blockIdx.x / (unsigned)slices);
  const int h = bh % P.H, b = bh / P.H;
  const int half = threadIdx.x >> 7, col = threadIdx.x & 127;
#pragma unroll
  for (int t = 0; t < kRepackMax; ++t) {
    if (t >= a.n) break;
    const RepackT x = a.t[t];
    const SideRows r = side_rows(x.side ? P.ks : P.qs, b);
    const long long rows = a.out ? (r.room > r.n ? r.room : r.n) : r.n;
    const int w = a.out ? x.cols : a.pad;  // columns written
    for (long long i = 2LL * sl + half; i < rows; i += 2LL * slices) {
      const long long row = r.r0 + i;
      for (int c = col; c < w; c += 128) {
        const long long so = b * x.src.sb + h * x.src.sh + row * x.src.ss + c;
        const long long d = b * x.dst.sb + h * x.dst.sh + row * x.dst.ss + c;
        const bool have = a.out || c < x.cols;
        if (a.esz == 2) {
          const uint16_t v = have ? ((const uint16_t*)x.src.ptr)[so] : (uint16_t)0;
          ((uint16_t*)x.dst.ptr)[d] = v;
        } else {
          const uint32_t v = have ? ((const uint32_t*)x.src.ptr)[so] : 0u;
          ((uint32_t*)x.dst.ptr)[d] = v;
        }
      }
    }
  }
}

template <class Ex>
hipError_t launch_repack(const RepackArgs& a, const Ex& ex) {
  if (a.n == 0 || a.pad > 256) return a.n == 0 ? hipSuccess : hipErrorInvalidValue;
  const long long nbh = (long long)a.p.B * a.p.H;
  if (nbh == 0) return hipSuccess;
  const int rows = a.p.Sq > a.p.Sk ? a.p.Sq : a.p.Sk;
  const int slices = rows < 2 ? 1 : (rows / 2 < 64 ? rows / 2 : 64);
  if (nbh * slices > 0x7fffffffLL) return hipErrorInvalidValue;
  return ex(reinterpret_cast<const void*>(&attn_repack_kernel), "attn_repack_kernel", (unsigned)(nbh * slices), 256u,
            a, slices);
}
template hipError_t launch_repack<Enqueue>(const RepackArgs&, const Enqueue&);
template hipError_t launch_repack<Record>(const RepackArgs&, const Record&);

template <class Ex>
static hipError_t launch_fwd_any(int dtype, int head_dim, const FwdArgs& a, const Ex& ex) {
  hipError_t err;
  switch (dtype) {
    case 0: err = launch_fwd_d<MmaF32>(head_dim, a, ex); break;
    case 1: err = launch_fwd_d<MmaF16>(head_dim, a, ex); break;
    case 2: err = launch_fwd_d<MmaBF16>(head_dim, a, ex); break;
    default: return hipErrorNotSupported;
  }
  if (err != hipSuccess) return err;
  const int esz = dtype == 0 ? 4 : 2;
  return launch_pad_rows(a.p, a.o, Operand{}, a.lse, 0, head_dim * esz, esz, ex);
}

hipError_t launch_fwd(int dtype, int head_dim, const FwdArgs& a, const Enqueue& ex) {
  return launch_fwd_any(dtype, head_dim, a, ex);
}
hipError_t launch_fwd(int dtype, int head_dim, const FwdArgs& a, const Record& ex) {
  return launch_fwd_any(dtype, head_dim, a, ex);
}

}  // namespace sdpa
