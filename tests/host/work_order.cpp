// Host check of the work-order maps that the kernels use to place work on
// XCDs: both are bijections over every size tried.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <vector>
#include "moe_internal.h"
int main() {
  int bad = 0;
  for (int total = 1; total <= 3000; ++total) {
    std::vector<int> seen(total, 0);
    for (int l = 0; l < total; ++l) { int i = moe::xcd_contiguous(l, total); if (i < 0 || i >= total || seen[i]++) bad++; }
  }
  for (int nt = 1; nt <= 40; ++nt) for (int nbx = 1; nbx <= 50; ++nbx) for (int gc = 1; gc <= nbx; ++gc) {
    std::vector<int> seen(nt * nbx, 0);
    for (int it = 0; it < nt * nbx; ++it) { int t, b; moe::item_tile_block(it, nt, nbx, gc, t, b);
      if (t < 0 || t >= nt || b < 0 || b >= nbx || seen[t * nbx + b]++) bad++; }
  }
  printf("bad=%d\n", bad); return bad != 0;
}
