// Internal interface between the C ABI (api.cpp, host-only C++) and the HIP
// kernels (fused_reduce_rmsnorm.hip).  Not installed, not part of the ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include "geometry.h"

namespace tw {

constexpr int kMaxPartials = 16;

// The most work-items one dispatch carries.  The dispatch packet holds the
// grid size in work-items as a 32-bit field; staying below 2^31 also keeps
// every count a non-negative int.  Launches over more rows than
// kMaxLaunchWorkItems / block are split into several dispatches over
// consecutive row ranges (one-workgroup-per-row kernels), or have their
// workgroup count capped (consecutive-rows kernel).  The per-row code is the
// same either way, so the results do not change.
constexpr int64_t kMaxLaunchWorkItems = 0x7FFFFFFF;
inline int64_t max_rows_per_dispatch(int block) { return kMaxLaunchWorkItems / block; }

// The most bytes one dispatch of the one-row-per-workgroup fused kernel
// streams: single launches lose speed beyond about 768 MiB, in proportion to
// the bytes rather than the rows (profiles/launch_rules_mi355x.md, "Dispatch
// size").  Longer launches are therefore cut into dispatches over consecutive
// row ranges of about equal size, none above this many bytes unless one round
// of resident workgroups alone streams more.
constexpr int64_t kMaxDispatchBytes = int64_t(768) << 20;

// The most rows one dispatch takes, for rows of row_bytes (all tensors of a
// row, read and written) when round_rows workgroups are resident at once: a
// whole number of rounds within kMaxDispatchBytes (at least one round), and
// never above the work-item limit.
inline int64_t fused_rows_per_dispatch(int block, int64_t row_bytes, int64_t round_rows) {
  int64_t cap = kMaxDispatchBytes / row_bytes;
  cap -= cap % round_rows;
  if (cap < round_rows) cap = round_rows;
  const int64_t hard = max_rows_per_dispatch(block);
  return cap < hard ? cap : hard;
}

// How a fused call of `rows` rows is laid out: its row class and geometry,
// the round of resident workgroups on num_cus CUs, and the consecutive row
// ranges of about equal size it is cut into.  geometry < 0: no compiled
// kernel covers rows of nvec vectors.
struct FusedPlan {
  int geometry;
  Geometry geo;
  int64_t round;
  int64_t rows_per_dispatch;
  int64_t dispatches;
};

inline FusedPlan plan_fused(int64_t nvec, int num_partials, int64_t rows, int num_cus) {
  FusedPlan p{};
  p.geometry = geometry_index(nvec);
  if (p.geometry < 0 || nvec > kMaxVectors || rows <= 0 || num_cus < 1) {
    p.geometry = p.geometry < 0 || nvec > kMaxVectors ? -1 : p.geometry;
    return p;
  }
  p.geo = fused_geometry(p.geometry, num_partials);
  p.round = round_rows(p.geo.block, num_cus);
  const int64_t row_bytes = (int64_t)(num_partials + 3) * nvec * 16;
  const int64_t cap = fused_rows_per_dispatch(p.geo.block, row_bytes, p.round);
  const int64_t pieces = (rows + cap - 1) / cap;
  p.rows_per_dispatch = (rows + pieces - 1) / pieces;
  p.dispatches = (rows + p.rows_per_dispatch - 1) / p.rows_per_dispatch;
  return p;
}

struct FusedLaunch {
  const void* partials[kMaxPartials];
  int32_t num_partials;
  const void* residual;
  const void* weight;
  void* out;
  void* residual_out;
  int64_t row_begin;   // first row this launch processes
  int64_t num_rows;    // rows processed: [row_begin, row_begin + num_rows)
  int64_t hidden;
  float eps;
  int32_t dtype;       // tw_dtype value
  void* stream;        // hipStream_t
  int64_t max_workgroups;   // <= 0: one workgroup per row; else at most this many
  int32_t num_cus;     // CUs the stream's launches may use (sizes a round of workgroups)
};

// Enqueues the kernel.  Returns 0 on success; otherwise writes a message to
// err (NUL-terminated, at most errlen bytes) and returns a nonzero HIP error.
int launch_fused(const FusedLaunch& a, char* err, size_t errlen);

// Unfused comparator: reduced = round(sum of partials), one row per workgroup.
struct ReduceLaunch {
  const void* partials[kMaxPartials];
  int32_t num_partials;
  void* reduced;
  int64_t num_rows;
  int64_t hidden;
  int32_t dtype;
  void* stream;
  int32_t num_cus;     // CUs the stream's launches may use
};
int launch_reduce(const ReduceLaunch& a, char* err, size_t errlen);

// Unfused comparator: two-pass residual-add + RMSNorm (reads the tensor twice).
struct AddNormLaunch {
  const void* input;
  const void* residual;
  const void* weight;
  void* out;
  void* residual_out;
  int64_t num_rows;
  int64_t hidden;
  float eps;
  int32_t dtype;
  void* stream;
};
int launch_add_rmsnorm(const AddNormLaunch& a, char* err, size_t errlen);

// Threads per workgroup and 16-byte vectors per thread that the fused kernel
// uses for a given hidden size, element size and partial count.  Depends on
// nothing else, so every launch over rows of the same shape runs the same
// per-row code.
void kernel_geometry(int64_t hidden, int32_t elem_bytes, int32_t num_partials, int* block,
                     int* vecs_per_thread);

}  // namespace tw
