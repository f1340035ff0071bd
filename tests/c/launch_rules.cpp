// Prints the kernel the fused launcher picks for each (hidden, element bytes,
// partials, rows, CUs) line on stdin: "all", "seq", "strided" or "both", together
// with the geometry (threads per workgroup, vectors per thread) and the round
// size on that many CUs.  Built with the host compiler against the
// launcher's own geometry header; no GPU and no HIP runtime involved.

#include <cstdint>
#include <cstdio>

#include "geometry.h"

int main() {
  long long h = 0, es = 0, n = 0, rows = 0, cus = 0;
  while (std::scanf("%lld %lld %lld %lld %lld", &h, &es, &n, &rows, &cus) == 5) {
    const int g = tw::geometry_index(h * es / 16);
    if (g < 0) {
      std::printf("none\n");
      continue;
    }
    const tw::Geometry geo = tw::fused_geometry(g, (int)n);
    const tw::RowKernel rk = tw::fused_row_kernel(g, (int)n, rows, (int)cus);
    const char* name = rk == tw::RowKernel::kStrided     ? "strided"
                       : rk == tw::RowKernel::kSequenced ? "seq"
                       : rk == tw::RowKernel::kBothSlots ? "both"
                                                         : "all";
    std::printf("%s %d %d %lld\n", name, geo.block, geo.vpt,
                (long long)tw::round_rows(geo.block, (int)cus));
  }
  return 0;
}
