// attn_device.hpp - gfx950 device building blocks shared by the forward and
// backward kernels: MFMA operand types, register fragments, LDS tile staging,
// the window predicate and the XCD-aware block order.
//
// Matrix-core convention (CDNA 32x32xK MFMA, 64-wide wavefront).  For lane
// l let r = l % 32 and g = l / 32.  An A operand (M x K) holds A[r][KPL*g +
// t], t < KPL; a B operand (K x N) holds B[KPL*g + t][r]; the 32x32 fp32
// accumulator holds C[8*(e/4) + 4*g + e%4][r] in element e < 16.  KPL is 8
// for bf16/fp16 (v_mfma_f32_32x32x16_{bf16,f16}) and 1 for fp32
// (v_mfma_f32_32x32x2_f32).
//
// The kernels compute transposed products (S^T = K Q^T, O^T = V^T P^T, ...)
// so that each lane owns one query (or key) column of every accumulator:
// row statistics are then in-lane except for one exchange between the two
// half-waves, and an accumulator can be fed straight back as the B operand
// of the next product.  The K index order of such a B operand is the
// accumulator's row order; the matching A operand is read from an LDS tile
// stored transposed with the row index permuted by `perm16` below, which
// makes the KPL values one lane needs contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kWindowInf = 2147483647;
constexpr int kBig = 2147483647;  // |j - i| never exceeds this
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- MFMA types

struct MmaBF16 {
  using elem = __bf16;
  using frag = bf16x8;
  static constexpr int KPL = 8;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void pack(const float* x, frag& f) {
#pragma unroll
    for (int t = 0; t < 8; ++t) f[t] = (__bf16)x[t];  // RNE
  }
};

struct MmaF16 {
  using elem = _Float16;
  using frag = f16x8;
  static constexpr int KPL = 8;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void pack(const float* x, frag& f) {
#pragma unroll
    for (int t = 0; t < 8; ++t) f[t] = (_Float16)x[t];  // RNE
  }
};

struct MmaF32 {
  using elem = float;
  using frag = float;
  static constexpr int KPL = 1;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void pack(const float* x, frag& f) { f = x[0]; }
};

template <typename M>
__device__ __forceinline__ typename M::frag load_frag(const typename M::elem* p) {
  return *reinterpret_cast<const typename M::frag*>(p);
}

// Exact negation of every element of a fragment (flips the sign bits).
template <typename F>
__device__ __forceinline__ F negate_frag(F f) {
  if constexpr (sizeof(F) == 4) {
    return __builtin_bit_cast(F, __builtin_bit_cast(uint32_t, f) ^ 0x80000000u);
  } else {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(F, __builtin_bit_cast(u4, f) ^ 0x80008000u);
  }
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.f;
  return z;
}

// Row of accumulator element e for half-wave g.
__host__ __device__ __forceinline__ int acc_row(int e, int g) { return 8 * (e >> 2) + 4 * g + (e & 3); }

// Position, inside a 32-row block of a transposed LDS tile, of the row held
// by accumulator element e of half-wave g: the A-operand side of a product
// whose B operand is that accumulator.
__host__ __device__ __forceinline__ int perm_pos(int e, int g) { return 16 * (e >> 3) + 8 * g + (e & 7); }

// Same map written on the row index: swaps bits 2 and 3.
__host__ __device__ constexpr int perm16(int row) {
  return (row & ~12) | ((row & 4) << 1) | ((row & 8) >> 1);
}

// Sum / max of a value over the two half-waves (lanes r and r + 32).
__device__ __forceinline__ float halves_max(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Arrival of a workgroup that has stored its partial results for a block
// shared by n workgroups.  Every wave first waits until its own stores have
// completed (are in its XCD's L2; a workgroup barrier alone does not wait
// for other waves' global stores), then, after a barrier, lane 0 counts the
// workgroup in with one agent-scope release / acquire add, whose release
// writes the L2 back for the other XCDs: the fence work is paid once per
// workgroup, not per wave.  The workgroup that brings the count to n resets
// the counter (for the next call on the buffer), acquires the others'
// stores and returns true: it combines the partials.  No workgroup waits
// for another, so the grid drains in any schedule.
__device__ __forceinline__ bool last_arrival(unsigned* cnt, int n) {
  __shared__ int s_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev + 1u == (unsigned)n;
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last ? 1 : 0;
  }
  __syncthreads();
  const bool last = s_last != 0;
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return last;
}

// ------------------------------------------------------------------- window

// Bounds lo <= j - i <= hi of one sequence (0-based local indices), clamped
// to the int32 range, where |j - i| always lies.
struct Window {
  int lo, hi;
};

__host__ __device__ __forceinline__ Window seq_window(int wl, int wr, int diag, int sq, int sk) {
  const bool left_inf = wl == kWindowInf, right_inf = wr == kWindowInf;
  long long L = wl, R = wr;
  if (diag == 1 && !left_inf && !right_inf) {
    const long long d = (long long)sk - sq;
    L -= d;
    R += d;
  }
  long long lo = left_inf ? -(long long)kBig : -L;
  long long hi = right_inf ? (long long)kBig : R;
  lo = lo < -(long long)kBig ? -(long long)kBig : (lo > kBig ? kBig : lo);
  hi = hi < -(long long)kBig ? -(long long)kBig : (hi > kBig ? kBig : hi);
  return Window{(int)lo, (int)hi};
}

enum TileClass { kEmpty = 0, kPartial = 1, kFull = 2 };

// Class of the rectangle rows [i0, i0+nr) x cols [j0, j0+nc) of the
// visibility matrix; cols at or beyond `sk` count as masked.
__host__ __device__ __forceinline__ int classify(Window w, long long i0, int nr, long long j0, int nc,
                                        long long sk) {
  const long long dmin = j0 - (i0 + nr - 1), dmax = j0 + nc - 1 - i0;
  if (dmax < w.lo || dmin > w.hi || j0 >= sk || w.lo > w.hi) return kEmpty;
  if (dmin >= w.lo && dmax <= w.hi && j0 + nc <= sk) return kFull;
  return kPartial;
}

// --------------------------------------------------------------- grid order

// Blocks are dealt round-robin to the 8 XCDs; remap the hardware block id so
// that each XCD receives one contiguous range of logical blocks (the blocks
// of the same heads share K/V in that XCD's L2).
__host__ __device__ __forceinline__ int xcd_remap(int hw, int n) {
  const int x = hw & 7, local = hw >> 3;
  const int per = n >> 3, rem = n & 7;
  return x * per + (x < rem ? x : rem) + local;
}

// Position of hardware block hw in a grid of n = nseq * nbh workgroups:
// (sequence-head index bh, block index i along the sequence).  Dense
// problems: xcd_remap hands each XCD a contiguous range, so the blocks of
// one head share its K/V in that XCD's L2.  Sequences of different
// lengths (`ragged`): bh runs fastest, so each XCD (hardware blocks are dealt to the
// XCDs round-robin) gets the same heads of every sequence at every position
// along it.  A contiguous range would give whole sequences to one XCD (24
// sequences of 64..2048 rows, 128-row blocks: the busiest XCD had 1.43x the
// mean work while others idled).
struct GridPos {
  int bh, i;
};
__host__ __device__ __forceinline__ GridPos grid_pos(int hw, int n, int nseq, int nbh, bool ragged) {
  if (ragged) return GridPos{hw % nbh, hw / nbh};
  const int blk = xcd_remap(hw, n);
  return GridPos{blk / nseq, blk % nseq};
}

// ---------------------------------------------------------- global -> LDS

// A ROWS x D tile of T staged through registers by NT threads.  Each work
// unit is four consecutive rows x one 16-byte column chunk, so the tile can
// be written to LDS both row-major and transposed (4 rows become 4
// consecutive positions of a transposed row).
template <typename T, int ROWS, int D, int NT>
struct TileStage {
  static constexpr int CE = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  static constexpr int CH = D / CE;              // chunks per row
  static constexpr int UNITS = (ROWS / 4) * CH;
  static constexpr int U = (UNITS + NT - 1) / NT;
  static_assert(D % CE == 0, "head_dim must be a multiple of 16 bytes");
  static_assert(ROWS % 16 == 0, "tile rows must be a multiple of 16");
  uint4 buf[U][4];

  // Rows at or beyond `nvalid` are zero-filled.
  __device__ __forceinline__ void load(const T* __restrict__ base, long long row_stride,
                                       int nvalid, int tid) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int unit = tid + u * NT;
      if (UNITS % NT == 0 || unit < UNITS) {
        const int rg = unit / CH, c = unit % CH;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 4 * rg + r;
          if (row < nvalid)
            buf[u][r] = *reinterpret_cast<const uint4*>(base + row * row_stride + c * CE);
          else
            buf[u][r] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  }

  // lds[row * ld + d]
  __device__ __forceinline__ void store_rows(T* lds, int ld, int tid) const {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int unit = tid + u * NT;
      if (UNITS % NT == 0 || unit < UNITS) {
        const int rg = unit / CH, c = unit % CH;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<uint4*>(lds + (4 * rg + r) * ld + c * CE) = buf[u][r];
      }
    }
  }

  // ldsT[d * ldT + perm16(row)], rows permuted within each 16-row group.
  __device__ __forceinline__ void store_transposed(T* ldsT, int ldT, int tid) const {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int unit = tid + u * NT;
      if (UNITS % NT == 0 || unit < UNITS) {
        const int rg = unit / CH, c = unit % CH;
        const int p0 = perm16(4 * rg);
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int w = e >> 1, sh = (e & 1) * 16;
            auto word = [&](int r) {
              const uint4& b = buf[u][r];
              const uint32_t x = w == 0 ? b.x : (w == 1 ? b.y : (w == 2 ? b.z : b.w));
              return (x >> sh) & 0xffffu;
            };
            uint2 out;
            out.x = word(0) | (word(1) << 16);
            out.y = word(2) | (word(3) << 16);
            *reinterpret_cast<uint2*>(ldsT + (c * 8 + e) * ldT + p0) = out;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            auto word = [&](int r) {
              const uint4& b = buf[u][r];
              return e == 0 ? b.x : (e == 1 ? b.y : (e == 2 ? b.z : b.w));
            };
            *reinterpret_cast<uint4*>(ldsT + (c * 4 + e) * ldT + p0) =
                make_uint4(word(0), word(1), word(2), word(3));
          }
        }
      }
    }
  }
};

// B-operand fragments of 32 rows held in registers for a whole kernel: lane
// (r, g) holds row r, columns 2*KPL*s + KPL*g .. +KPL-1 of every K step s.
template <typename M, int DK>
struct RowFrags {
  static constexpr int NS = DK / (2 * M::KPL);
  typename M::frag f[NS];
  __device__ __forceinline__ void load(const typename M::elem* __restrict__ row_ptr, bool valid,
                                       int g) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (valid)
        f[s] = load_frag<M>(row_ptr + 2 * M::KPL * s + M::KPL * g);
      else
        f[s] = typename M::frag{};
    }
  }
  __device__ __forceinline__ void negate() {
#pragma unroll
    for (int s = 0; s < NS; ++s) f[s] = negate_frag(f[s]);
  }
};

}  // namespace sdpa

namespace sdpa {

// ------------------------------------------- swizzled 16-bit LDS tiles

// A tile of 16-bit rows kept row-major in LDS, each row in 16-byte chunks.
// Chunk c of row r sits at chunk slot c ^ sigma(r) of that row, so that
//  - a 128-bit read of one chunk by 16 consecutive rows (an MFMA operand
//    read straight from rows), and
//  - a 64-bit transposing read of 4 consecutive rows (aligned to 4) x 4
//    consecutive chunks (aligned to 4) by 32 lanes (an operand read across
//    rows, see tr_frag)
// both touch every bank once.  Rows are 8 chunk slots (head_dim up to 64) or
// 16 (head_dim 80 to 128); a head_dim below the slot count (32, 48, 80, 96)
// leaves slots unused.
template <int D>
struct Swz {
  static constexpr int CH = D / 8;                                   // chunks holding data
  static constexpr int SLOTS = D <= 64 ? 8 : (D <= 128 ? 16 : 32);  // chunk slots per row
  static constexpr int PITCH = SLOTS * 8;                            // elements per row
  static_assert(D % 16 == 0 && D <= 256, "head_dim must be a multiple of 16, at most 256");
  // Rows of 32 slots (512 bytes) start on the same bank as rows of 16; the
  // same 16 XOR patterns spread a column over every bank.
  __host__ __device__ static constexpr int sigma(int r) {
    return SLOTS >= 16 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
  // Element offset of chunk c of row r.
  __host__ __device__ static constexpr int off(int r, int c) { return r * PITCH + ((c ^ sigma(r)) << 3); }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Zeroes the chunk slots of a tile that DmaLane never writes (head_dim 80).
template <typename T, int D, int ROWS, int NT>
__device__ __forceinline__ void zero_unused_slots(T* lds, int tid) {
  using L = Swz<D>;
  if constexpr (L::CH < L::SLOTS) {
    constexpr int PER_ROW = L::SLOTS - L::CH;
    for (int x = tid; x < ROWS * PER_ROW; x += NT) {
      const int row = x / PER_ROW, c = L::CH + x % PER_ROW;
      *reinterpret_cast<uint4*>(lds + L::off(row, c)) = make_uint4(0, 0, 0, 0);
    }
  }
}

// A operand (32 x 16) read straight from rows row0 .. row0+31 of a swizzled
// tile, K step st: lane (r, g) gets chunk 2*st + g of row row0 + r.
template <typename M, int D>
__device__ __forceinline__ typename M::frag row_frag(const typename M::elem* lds, int row0, int st, int r, int g) {
  return *reinterpret_cast<const typename M::frag*>(lds + Swz<D>::off(row0 + r, 2 * st + g));
}

// A operand (32 columns x 16 rows of the tile, i.e. the transpose of a
// 16 x 32 block) read with two transposing loads: lane (r, g) gets column
// 32*dt + r of rows ra + 4*g + {0..3} (elements 0..3) and rb + 4*g + {0..3}
// (elements 4..7); ra and rb are multiples of 8.  Within each 16-lane group
// the transposing load hands lane j the j-th column of the 4 rows x 16
// columns the group's lanes address, 4 consecutive elements per lane.
template <typename M, int D>
__device__ __forceinline__ typename M::frag tr_frag(const typename M::elem* lds, int ra, int rb, int dt, int lane) {
  using L = Swz<D>;
  const int s = lane & 15, grp = lane >> 4, g = lane >> 5;
  const int col = 32 * dt + 16 * (grp & 1) + 4 * (s & 3);
  const int c = col >> 3, half = (col >> 2) & 1;
  const int dr = 4 * g + (s >> 2);
  const auto* pa = lds + L::off(ra + dr, c) + 4 * half;
  const auto* pb = lds + L::off(rb + dr, c) + 4 * half;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)pa);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)pb);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(typename M::frag, v);
}

}  // namespace sdpa

namespace sdpa {

// Per-lane element offsets into swizzled 16-bit tiles, computed once per
// kernel so that every operand read in the hot loops is one LDS instruction
// whose tile, stage and row block are folded into its immediate offset.
//   row[st]: chunk 2*st + g of row r (row_frag of any 32-row block);
//   tra[dt] / trb[dt]: the transposing-read addresses of tr_frag for rows
//   4g + (s>>2) and 8 + 4g + (s>>2) of any 16-row block, column block dt.
template <typename M, int D>
struct LdsOffsets {
  using L = Swz<D>;
  static constexpr int NS = D / 16, DVT = (D + 31) / 32;
  int row[NS], tra[DVT], trb[DVT];
  __device__ __forceinline__ void init(int lane) {
    const int r = lane & 31, g = lane >> 5, s = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int st = 0; st < NS; ++st) row[st] = L::off(r, 2 * st + g);
    const int dr = 4 * g + (s >> 2);
#pragma unroll
    for (int dt = 0; dt < DVT; ++dt) {
      const int col = 32 * dt + 16 * (grp & 1) + 4 * (s & 3);
      const int c = col >> 3, half = (col >> 2) & 1;
      tra[dt] = L::off(dr, c) + 4 * half;
      trb[dt] = L::off(8 + dr, c) + 4 * half;
    }
  }
};

// A operand straight from rows: row block starting at element offset `base`
// (a multiple of 16 rows), K step st.
template <typename M>
__device__ __forceinline__ typename M::frag ld_row(const typename M::elem* lds, int off) {
  return *reinterpret_cast<const typename M::frag*>(lds + off);
}

// A operand by transposing reads (see tr_frag): `lds` points at the first
// row of a 16-row block.
template <typename M>
__device__ __forceinline__ typename M::frag ld_tr(const typename M::elem* lds, int offa, int offb) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(lds + offa));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(lds + offb));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(typename M::frag, v);
}

// Buffer resource for direct global->LDS loads at byte offsets from `base`:
// raw (stride 0), range 2^31 - 1 bytes (callers keep every offset below
// it), word 3 = 32-bit data format as the gfx9 family expects.  Loads
// through a buffer resource are tracked by the compiler as vector-memory
// loads only, so waits on LDS reads issued after them stay partial.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

// One lane's share of copying a ROWS-row tile into a swizzled LDS tile with
// direct loads, NW waves splitting the 1 KiB instructions (64 lanes x 16
// bytes, RPI rows each).  Byte offsets of the lane's chunks in a full tile
// are computed once; they are taken from the tile's lowest-addressed row, so
// a negative row stride works too.  Rows at or beyond `nvalid` (>= 1)
// repeat row nvalid-1, so every loaded value is a finite input value.  The
// loads are asynchronous: a barrier after `s_waitcnt vmcnt(0)` publishes
// them.
template <typename T, int D, int ROWS, int NW>
struct DmaLane {
  using L = Swz<D>;
  static constexpr int RPI = 64 / L::SLOTS, NI = ROWS / RPI, PER = (NI + NW - 1) / NW;
  static_assert(ROWS % RPI == 0, "tile rows");
  int boff[PER];  // byte offset of the lane's chunk in a full tile
  static __device__ __forceinline__ int row_of(int u, int wave, int lane) {
    return (wave + u * NW) * RPI + lane / L::SLOTS;
  }
  static __device__ __forceinline__ int chunk_of(int row, int lane) { return (lane % L::SLOTS) ^ L::sigma(row); }
  static __device__ __forceinline__ long long lowest(long long row_stride) {
    return row_stride < 0 ? (long long)(ROWS - 1) * row_stride : 0;
  }
  __device__ __forceinline__ void init(long long row_stride, int wave, int lane) {
    const long long lo = lowest(row_stride);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int row = row_of(u, wave, lane);
      boff[u] = (int)(((long long)row * row_stride - lo) * (long long)sizeof(T)) + chunk_of(row, lane) * 16;
    }
  }
  // Copies the tile whose first row is g (rows >= nvalid repeat row nvalid-1).
  __device__ __forceinline__ void issue(T* lds, const T* __restrict__ g, long long row_stride, int nvalid,
                                        int wave, int lane) const {
    const long long lo = lowest(row_stride);
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(g + lo);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = wave + u * NW;
      if (NI % NW == 0 || i < NI) {
        const int row = row_of(u, wave, lane);
        if (L::CH == L::SLOTS || chunk_of(row, lane) < L::CH) {
          const int off = nvalid >= ROWS ? boff[u]
                                         : (int)(((long long)min(row, nvalid - 1) * row_stride - lo) *
                                                 (long long)sizeof(T)) + chunk_of(row, lane) * 16;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + i * RPI * L::PITCH), 16, off, 0, 0, 0);
        }
      }
    }
  }
};

}  // namespace sdpa

namespace sdpa {

// Tiles t (of T rows or keys) whose start t*T lies in [lo, hi]: [t0, t1],
// empty when t1 < t0.  Used for the range of tiles a window leaves whole,
// computed once per wave so the hot loop tests two integers per tile.
struct TileRange {
  int t0, t1;
};
__host__ __device__ __forceinline__ TileRange tiles_starting_in(long long lo, long long hi, int T) {
  const long long a = lo <= 0 ? 0 : (lo + T - 1) / T;
  const long long b = hi < 0 ? -1 : hi / T;
  return TileRange{(int)(a > 0x7fffffffLL ? 0x7fffffffLL : a), (int)(b > 0x7fffffffLL ? 0x7fffffffLL : b)};
}

}  // namespace sdpa

namespace sdpa {

// Masking of one 32 x 32 accumulator block without compares.  Element e of
// half-wave g sits at row offset acc_row(e, g) = 8*(e/4) + 4*g + e%4 of the
// block; with base = block row 0 + 4*g, the elements whose row offset
// r(e) = 8*(e/4) + e%4 satisfies lo <= r(e) <= hi are visible.  vis_bits
// turns [lo, hi] into a 32-bit mask (bit r visible); mask_block keeps the
// visible scores and sets the others to -inf with a bit-select per element.
__host__ __device__ __forceinline__ uint32_t vis_bits(long long lo, long long hi) {
  const int a = (int)(lo < 0 ? 0 : (lo > 32 ? 32 : lo));
  const int b = (int)(hi < -1 ? -1 : (hi > 31 ? 31 : hi));
  const uint32_t below_a = a >= 32 ? 0xffffffffu : ((1u << a) - 1u);      // bits < a
  const uint32_t upto_b = b >= 31 ? 0xffffffffu : ((1u << (b + 1)) - 1u);  // bits <= b
  return upto_b & ~below_a;
}

__device__ __forceinline__ void mask_block(f32x16& s, uint32_t vis) {
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int bit = 8 * (e >> 2) + (e & 3);
    const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)vis, bit, 1);  // all ones if visible
    s[e] = __uint_as_float((__float_as_uint(s[e]) & keep) | (0xff800000u & ~keep));
  }
}

}  // namespace sdpa
