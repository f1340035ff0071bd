// Row geometry of the row-per-workgroup kernels: threads per workgroup and
// 16-byte vectors per thread, chosen from the row width alone.  Every kernel
// that normalizes rows uses this table, so the per-row arithmetic (and its
// reduction order) never depends on the launch.
#pragma once

#include <cstdint>

namespace tw {

struct Geometry {
  int block;          // threads per workgroup
  int vpt;            // 16-byte vectors per thread
  int waves_per_eu;   // occupancy the compiler must allow (1: no constraint)
  int chunk;          // vector slots whose loads are issued together (divides vpt)
};

// (threads per workgroup, vectors per thread) by 16-byte vectors per row: the
// first entry whose capacity covers the row.  Measured on MI355X at 184-738 MB
// per launch, N = 8 bf16:
//  * h = 8192 (1024 vectors): 512 x 2 at 6 waves per SIMD (at most 80 VGPRs,
//    three workgroups per CU) 31.5 us; uncapped 32.7 us; 1024 x 1 33.4 us;
//    256 x 4 36.0-36.5 us.
//  * h = 4096 (512 vectors): 512 x 1 at 8 waves per SIMD 122.9-123.2 us
//    (T = 8192); 256 x 2 128.9 us.
//  * h = 16384 (2048 vectors): 512 x 4 at 4 waves per SIMD, loads two slots
//    at a time, 123.9 us (T = 2048); 1024 x 2 133.4 us; 256 x 8 132.1 us.
// The occupancy cap applies up to N = 8 partials, where it costs no scratch;
// with more partials the compiler's own allocation is kept.
constexpr Geometry kGeometry[] = {
    {64, 1, 1, 1},  {128, 1, 1, 1}, {256, 1, 1, 1},  {512, 1, 8, 1},
    {512, 2, 6, 2}, {512, 4, 4, 2}, {1024, 4, 1, 1}, {1024, 8, 1, 1}};
constexpr int kMaxCappedPartials = 8;

// The geometry the fused kernels use for row class g and N partials.  Up to
// kMaxCappedPartials the table entry applies with its occupancy cap.  Above
// it the cap is dropped (it would force spills), and the 512 x 2 class runs
// 1024 x 1 instead: at N = 16, T = 1024, h = 8192 it took 54.8 us (62 VGPRs)
// against 57.6 us for uncapped 512 x 2.
constexpr Geometry fused_geometry(int g, int n) {
  if (n <= kMaxCappedPartials) return kGeometry[g];
  if (kGeometry[g].block == 512 && kGeometry[g].vpt == 2) return Geometry{1024, 1, 1, 1};
  return Geometry{kGeometry[g].block, kGeometry[g].vpt, 1, kGeometry[g].chunk};
}
constexpr int kNumGeometries = sizeof(kGeometry) / sizeof(kGeometry[0]);
constexpr int kMaxVectors = 8192;

inline int geometry_index(int64_t nvec) {
  for (int g = 0; g < kNumGeometries; ++g)
    if (nvec <= (int64_t)kGeometry[g].block * kGeometry[g].vpt) return g;
  return -1;
}

}  // namespace tw
