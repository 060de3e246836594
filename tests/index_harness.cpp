// Host-side harness over the index helpers the kernels use (window bounds,
// tile classification, the per-wave range of unmasked tiles, the visibility
// bit masks, XCD block remap, operand permutations).  Built with hipcc for
// the host only; no kernel is launched.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <vector>

#include "attn_device.hpp"

int main(int argc, char** argv) {
  using namespace sdpa;
  if (argc > 1 && strcmp(argv[1], "vis") == 0) {
    // Lines "sq sk wl wr diag qi jb": the 32-bit mask of keys jb .. jb+31
    // visible to query qi, as the forward and dQ kernels build it.
    int sq, sk, wl, wr, diag, qi;
    long long jb;
    while (scanf("%d %d %d %d %d %d %lld", &sq, &sk, &wl, &wr, &diag, &qi, &jb) == 7) {
      const Window w = seq_window(wl, wr, diag, sq, sk);
      printf("%u\n", vis_bits((long long)qi + w.lo - jb, std::min((long long)qi + w.hi, (long long)sk - 1) - jb));
    }
    return 0;
  }
  // 1. xcd_remap is a bijection of [0, n).
  for (int n = 1; n <= 3000; ++n) {
    std::vector<int> seen(n, 0);
    for (int hw = 0; hw < n; ++hw) {
      const int l = xcd_remap(hw, n);
      if (l < 0 || l >= n || seen[l]++) {
        printf("remap_fail %d %d\n", n, hw);
        return 1;
      }
    }
  }
  printf("remap_ok\n");
  // 1b. grid_pos maps [0, nseq * nbh) one to one onto (bh, i) pairs, dense
  //     and packed; and for packed sequences with nbh a multiple of 8 every
  //     XCD (hw mod 8) gets the same positions i of the same bh mod 8.
  for (int varlen = 0; varlen < 2; ++varlen)
    for (int nbh = 1; nbh <= 40; ++nbh)
      for (int nseq = 1; nseq <= 40; ++nseq) {
        const int n = nseq * nbh;
        std::vector<int> seen(n, 0);
        for (int hw = 0; hw < n; ++hw) {
          const GridPos p = grid_pos(hw, n, nseq, nbh, varlen != 0);
          if (p.bh < 0 || p.bh >= nbh || p.i < 0 || p.i >= nseq || seen[p.bh * nseq + p.i]++) {
            printf("grid_fail %d %d %d %d\n", varlen, nbh, nseq, hw);
            return 1;
          }
          if (varlen && nbh % 8 == 0 && p.bh % 8 != hw % 8) {
            printf("grid_xcd_fail %d %d %d\n", nbh, nseq, hw);
            return 1;
          }
        }
      }
  printf("grid_ok\n");
  // 2. perm_pos(e, g) == perm16(acc_row(e, g)) on every 32-row block.
  for (int g = 0; g < 2; ++g)
    for (int e = 0; e < 16; ++e)
      if (perm_pos(e, g) != perm16(acc_row(e, g))) {
        printf("perm_fail %d %d\n", e, g);
        return 1;
      }
  printf("perm_ok\n");
  // 3. The per-wave range of unmasked tiles equals the tiles classify()
  //    calls FULL, for waves of WR rows and tiles of BN keys.
  {
    const int INF = kWindowInf;
    const int wls[] = {INF, 0, 1, 5, 37, -3, 64, 100}, wrs[] = {INF, 0, 2, 9, -2, 70};
    for (int sq : {1, 17, 64, 65, 130, 300})
      for (int sk : {1, 31, 64, 65, 129, 300})
        for (int wl : wls)
          for (int wr : wrs)
            for (int diag = 0; diag < 2; ++diag) {
              const Window w = seq_window(wl, wr, diag, sq, sk);
              for (int BN : {32, 64, 128})
                for (int WR : {32, 64})
                  for (int iw0 = 0; iw0 < sq; iw0 += WR) {
                    const TileRange full = tiles_starting_in(
                        (long long)iw0 + WR - 1 + w.lo, std::min((long long)iw0 + w.hi, (long long)sk - 1) - BN + 1, BN);
                    for (int t = 0; t * BN < sk; ++t)
                      if ((classify(w, iw0, WR, (long long)t * BN, BN, sk) == kFull) != (t >= full.t0 && t <= full.t1)) {
                        printf("full_fail %d %d %d %d %d %d %d %d %d\n", sq, sk, wl, wr, diag, BN, WR, iw0, t);
                        return 1;
                      }
                  }
            }
  }
  printf("full_ok\n");
  // 4. classify rectangles read from stdin: sq sk wl wr diag i0 nr j0 nc
  int sq, sk, wl, wr, diag, nr, nc;
  long long i0, j0;
  while (scanf("%d %d %d %d %d %lld %d %lld %d", &sq, &sk, &wl, &wr, &diag, &i0, &nr, &j0, &nc) ==
         9) {
    const Window w = seq_window(wl, wr, diag, sq, sk);
    printf("%d\n", classify(w, i0, nr, j0, nc, sk));
  }
  return 0;
}
