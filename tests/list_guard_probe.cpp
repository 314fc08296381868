// Host build of the kept-list guard that the attention and decode kernels
// apply to every list entry (pisa_row_geometry + pisa_list_entry_kept from
// the library's internal header, the same inline code the kernels compile).
// Reads lines "L block window causal start k j_0 .. j_{k-1}" and prints
// "own lo nc kept..." with the entries the guard keeps, in list order.
#include <cstdio>

#include "pisa_internal.h"

int main() {
  int L, bs, window, causal, start, k;
  while (std::scanf("%d %d %d %d %d %d", &L, &bs, &window, &causal, &start, &k) == 6) {
    PisaDims dm{};
    dm.L = L;
    dm.bs = bs;
    dm.n_blk = (L + bs - 1) / bs;
    dm.window = window;
    dm.causal = causal;
    int own = -1, lo = -1;
    const int nc = pisa_row_geometry(dm, start, &own, &lo);
    std::printf("%d %d %d", own, lo, nc);
    for (int i = 0; i < k; ++i) {
      int j;
      if (std::scanf("%d", &j) != 1) return 2;
      if (pisa_list_entry_kept(j, nc)) std::printf(" %d", j);
    }
    std::printf("\n");
  }
  return 0;
}
