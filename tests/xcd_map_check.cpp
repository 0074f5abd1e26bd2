// Host-only check of the workgroup-id maps of the attention kernels (built from
// the library's own internal header): for every grid of nbh heads x nqb query
// blocks given on stdin, xcd_remap and xcd_head_remap must each be a bijection
// on [0, nbh*nqb), give XCD x (ids with id % 8 == x) the same number of ids, and
// xcd_head_remap must walk the heads in order on every XCD with a contiguous
// ascending slice of each. Prints "ok" or the first failure.
#include <cstdio>
#include <vector>

#include "ab_internal.h"

int main() {
  int nbh, nqb;
  long long grids = 0;
  while (std::scanf("%d %d", &nbh, &nqb) == 2) {
    const int n = nbh * nqb;
    std::vector<int> seen_a(n, 0), seen_b(n, 0);
    for (int pid = 0; pid < n; ++pid) {
      const int a = ab::xcd_remap(pid, n), b = ab::xcd_head_remap(pid, nbh, nqb);
      if (a < 0 || a >= n || b < 0 || b >= n) {
        std::printf("out of range: nbh %d nqb %d pid %d -> %d %d\n", nbh, nqb, pid, a, b);
        return 1;
      }
      ++seen_a[a];
      ++seen_b[b];
    }
    for (int v = 0; v < n; ++v)
      if (seen_a[v] != 1 || seen_b[v] != 1) {
        std::printf("not a bijection: nbh %d nqb %d id %d (%d, %d)\n", nbh, nqb, v, seen_a[v], seen_b[v]);
        return 1;
      }
    // per XCD: heads in order, each head's blocks one ascending contiguous run
    for (int x = 0; x < ab::kXcds; ++x) {
      int prev = -1;
      for (int pid = x; pid < n; pid += ab::kXcds) {
        const int b = ab::xcd_head_remap(pid, nbh, nqb);
        if (prev >= 0) {
          const bool same_head = b / nqb == prev / nqb;
          if ((same_head && b != prev + 1) || (!same_head && b / nqb < prev / nqb)) {
            std::printf("order: nbh %d nqb %d xcd %d: %d after %d\n", nbh, nqb, x, b, prev);
            return 1;
          }
        }
        prev = b;
      }
    }
    ++grids;
  }
  std::printf("ok %lld grids\n", grids);
  return 0;
}
