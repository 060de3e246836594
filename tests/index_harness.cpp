// Host-side harness over the index helpers the kernels use (window bounds,
// tile classification, XCD block remap, operand permutations).  Built with
// hipcc for the host only; no kernel is launched.
#include <cstdio>
#include <vector>

#include "attn_device.hpp"

int main(int argc, char** argv) {
  using namespace sdpa;
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
  // 2. perm_pos(e, g) == perm16(acc_row(e, g)) on every 32-row block.
  for (int g = 0; g < 2; ++g)
    for (int e = 0; e < 16; ++e)
      if (perm_pos(e, g) != perm16(acc_row(e, g))) {
        printf("perm_fail %d %d\n", e, g);
        return 1;
      }
  printf("perm_ok\n");
  // 3. classify rectangles read from stdin: sq sk wl wr diag i0 nr j0 nc
  int sq, sk, wl, wr, diag, nr, nc;
  long long i0, j0;
  while (scanf("%d %d %d %d %d %lld %d %lld %d", &sq, &sk, &wl, &wr, &diag, &i0, &nr, &j0, &nc) ==
         9) {
    const Window w = seq_window(wl, wr, diag, sq, sk);
    printf("%d\n", classify(w, i0, nr, j0, nc, sk));
  }
  return 0;
}
