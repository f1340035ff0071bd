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

// The most bytes one dispatch of the one-row-per-workgroup fused kernel
// streams.  Measured on MI355X (N = 8 bf16, inputs and outputs rotated past
// the MALL): one launch streams 79% of peak at 738 MB (T = 4096, h = 8192),
// 78.7% at 1.1 GB and 77% at 1.5 GB and beyond, and a 1.5 GB launch takes as
// long at h = 4096 as at h = 8192.  Longer launches are therefore cut into
// dispatches over consecutive row ranges of about equal size, none above this
// many bytes and each at least one round of resident workgroups.
constexpr int64_t kMaxDispatchBytes = int64_t(768) << 20;

// Rows per dispatch for rows of row_bytes (all tensors of a row, read and
// written) when round_rows workgroups are resident at once: a whole number of
// rounds within kMaxDispatchBytes (at least one round), and never above the
// work-item limit.
inline int64_t fused_rows_per_dispatch(int block, int64_t row_bytes, int64_t round_rows) {
  int64_t cap = kMaxDispatchBytes / row_bytes;
  cap -= cap % round_rows;
  if (cap < round_rows) cap = round_rows;
  const int64_t hard = max_rows_per_dispatch(block);
  return cap < hard ? cap : hard;
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
