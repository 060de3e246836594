// attn_feat.hpp - the optional features of a call, on the device: an additive
// bias on the logits, ALiBi, and dropout with a Philox4x32-10 keep mask.
// Only the kernels built with their FEAT template flag read these; the other
// kernels never see a call that has any of them.
//
// Logits in the kernels' log2 domain: x_ij = c s_ij + log2(e) (bias_ij +
// alibi_ij), with c = scale log2(e) and s_ij = q_i.k_j.  The bias is
// stored in the input type and converted to fp32 before any arithmetic (the
// fp32 cast of the AOTriton 0.14b notes, "Kernel Bug Fixes").  ALiBi adds
// -slope_h |i + sk - sq - j| (query i at key position i + sk - sq).
// Dropout keeps (i, j) iff word j % 4 of Philox4x32-10 (Salmon et al., SC
// 2011; the generator of the AOTriton 0.10b notes, "Major Changes") at
// counter (lo, hi of offset + ((b H + h) Sq + i) ceil(Sk / 4) + j / 4, 0, 0)
// and key (lo, hi of seed) is >= the threshold floor(p 2^32); the four words
// of a counter serve four consecutive keys in generation order (the AOTriton
// 0.14b notes, "Minor Changes").  Kept probabilities are multiplied by
// 1 / (1 - p).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

struct FeatArgs {
  const void* bias;                // null: none; [b, h, i, j], key stride 1
  long long bsb, bsh, bss;         // element strides of the bias
  const float* alibi;              // null: none; one slope per head
  unsigned long long offset;       // Philox counter offset
  unsigned int seed_lo, seed_hi;   // Philox key
  unsigned int drop_thresh;        // keep iff word >= drop_thresh; 0: no dropout
  float drop_scale;                // 1 / (1 - p)
  float* dbias;                    // backward output d loss / d logit (null: none)
  long long dsb, dsh, dss;         // element strides of dbias
};

// Philox4x32 with ten rounds: (hi0, lo0) = M0 c0, (hi1, lo1) = M1 c2,
// c = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0), the key bumped by the Weyl
// constants before every round but the first.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += W0;
      k1 += W1;
    }
    const uint32_t hi0 = __umulhi(M0, c.x), lo0 = M0 * c.x;
    const uint32_t hi1 = __umulhi(M1, c.z), lo1 = M1 * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// Keep decisions of keys j0 .. j0+3 (j0 a multiple of 4) of local query row
// i of (sequence b, head h), as bits 0..3.  sq_max, sk_max: the problem's
// seqlen_q / seqlen_k (the counters' row length).
template <class FA>
__device__ __forceinline__ uint32_t keep4(const FA& f, int b, int h, int H, int i, int j0, int sq_max, int sk_max) {
  const unsigned long long groups = (unsigned long long)((sk_max + 3) >> 2);
  const unsigned long long row = ((unsigned long long)b * H + h) * (unsigned long long)sq_max + (unsigned)i;
  const unsigned long long n = f.offset + row * groups + (unsigned)(j0 >> 2);
  const uint4 w = philox4x32_10(make_uint4((uint32_t)n, (uint32_t)(n >> 32), 0u, 0u), f.seed_lo, f.seed_hi);
  return (uint32_t)(w.x >= f.drop_thresh) | ((uint32_t)(w.y >= f.drop_thresh) << 1) |
         ((uint32_t)(w.z >= f.drop_thresh) << 2) | ((uint32_t)(w.w >= f.drop_thresh) << 3);
}

// Keep decision of the single pair (i, j).
template <class FA>
__device__ __forceinline__ bool keep1(const FA& f, int b, int h, int H, int i, int j, int sq_max, int sk_max) {
  return (keep4(f, b, h, H, i, j & ~3, sq_max, sk_max) >> (j & 3)) & 1u;
}

// log2(e) (bias_ij + alibi_ij) for the pair (i, j) of a sequence of sq
// queries and sk keys; 0 for a pair outside it (never read there).  T: the
// stored type of the bias.
template <typename T, class FA>
__device__ __forceinline__ float extra_log2(const FA& f, int b, int h, int i, int j, int sq, int sk) {
  if (i >= sq || j >= sk || i < 0 || j < 0) return 0.f;
  float add = 0.f;
  if (f.bias)
    add = (float)((const T*)f.bias)[b * f.bsb + h * f.bsh + (long long)i * f.bss + j];
  if (f.alibi) {
    const long long dist = (long long)i + sk - sq - j;
    add -= f.alibi[h] * (float)(dist < 0 ? -dist : dist);
  }
  return add * 1.4426950408889634f;
}

}  // namespace sdpa
