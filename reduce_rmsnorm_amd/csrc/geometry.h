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
};

// (threads per workgroup, vectors per thread) by 16-byte vectors per row: the
// first entry whose capacity covers the row.  Measured on MI355X at 184-738 MB
// per launch (h = 8192 bf16 has 1024 vectors): 512 x 2 beat 256 x 4 and
// 1024 x 1; at h = 4096 512 x 1, at h = 16384 1024 x 2.  The occupancy entry
// lets more rows be resident per CU: 512 x 2 at 6 waves per SIMD (at most 80
// VGPRs, three workgroups per CU instead of two) took 31.6-31.9 us against
// 32.6-32.8 us at T = 1024; 1024 x 2 at 5 waves per SIMD 132 us against
// 137 us at h = 16384; 512 x 1 at 8 waves per SIMD 122.9 us against 123.7 us
// at h = 4096.  The cap applies up to N = 8 partials, where it costs no
// scratch; with more partials the compiler's own allocation is kept.
constexpr Geometry kGeometry[] = {
    {64, 1, 1},  {128, 1, 1},  {256, 1, 1},  {512, 1, 8},
    {512, 2, 6}, {1024, 2, 5}, {1024, 4, 1}, {1024, 8, 1}};
constexpr int kMaxCappedPartials = 8;
constexpr int kNumGeometries = sizeof(kGeometry) / sizeof(kGeometry[0]);
constexpr int kMaxVectors = 8192;

inline int geometry_index(int64_t nvec) {
  for (int g = 0; g < kNumGeometries; ++g)
    if (nvec <= (int64_t)kGeometry[g].block * kGeometry[g].vpt) return g;
  return -1;
}

}  // namespace tw
