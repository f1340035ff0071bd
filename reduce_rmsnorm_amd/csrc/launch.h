// Internal interface between the C ABI (api.cpp, host-only C++) and the HIP
// kernels (fused_reduce_rmsnorm.hip).  Not installed, not part of the ABI.
#pragma once

#include <cstddef>
#include <cstdint>

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
