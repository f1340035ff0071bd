// C ABI entry points: argument validation (before any HIP call), shard row
// ranges, and the hand-off to the kernel launcher.  Host-only C++.

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include <hip/hip_runtime_api.h>

#include "launch.h"
#include "tokenweave.h"

namespace tw {

namespace {
thread_local char g_last_error[512] = "";
}

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

namespace {

std::atomic<int> g_pointer_checks{0};

// CUs of each device, queried once (0: not yet known).
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_cus[kMaxDevices];
// Used when the runtime cannot say (an MI355X has 256).
constexpr int kFallbackCUs = 256;
// 32-bit words of a stream's CU mask that are read: up to 1024 CUs.
constexpr uint32_t kMaskWords = 32;

int device_cus(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return 0;
  int n = g_device_cus[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    return 0;
  }
  g_device_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

// The CUs the launches of `stream` may use, which size a round of resident
// workgroups in the launch rules: the device's CU count, or the number of
// CUs in the stream's CU mask when that is smaller (a stream made with
// hipExtStreamCreateWithCUMask).  Runtime queries only, no launch.
int stream_cus(void* stream) {
  int dev = -1;
  const hipError_t e = stream != nullptr
                           ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                           : hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return kFallbackCUs;
  }
  int n = device_cus(dev);
  if (n < 1) return kFallbackCUs;
  if (stream != nullptr) {
    uint32_t mask[kMaskWords] = {};
    if (hipExtStreamGetCUMask(static_cast<hipStream_t>(stream), kMaskWords, mask) == hipSuccess) {
      int bits = 0;
      for (uint32_t w = 0; w < kMaskWords; ++w) bits += __builtin_popcount(mask[w]);
      if (bits > 0 && bits < n) n = bits;
    } else {
      (void)hipGetLastError();
    }
  }
  return n;
}

// With pointer checks on: is [p, p + bytes) device memory inside one
// allocation?  Uses runtime queries only (no launch); clears the runtime's
// last error when a query fails.
bool device_range_ok(const void* p, uint64_t bytes, const char* what, const char* who) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    set_error("%s: %s is not memory the HIP runtime knows", who, what);
    return false;
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) {
    set_error("%s: %s is not device memory", who, what);
    return false;
  }
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
    (void)hipGetLastError();
    set_error("%s: no allocation found for %s", who, what);
    return false;
  }
  const uintptr_t lo = reinterpret_cast<uintptr_t>(base);
  const uintptr_t ptr = reinterpret_cast<uintptr_t>(p);
  if (ptr < lo || ptr + bytes > lo + size) {
    set_error("%s: %s spans %llu bytes past its allocation", who, what,
              (unsigned long long)(ptr + bytes > lo + size ? ptr + bytes - (lo + size) : 0));
    return false;
  }
  return true;
}

// One tensor argument of an entry point: where it is, how many bytes the call
// touches, its name in messages, and whether the call writes it.
struct Tensor {
  const void* p;
  uint64_t bytes;
  char name[24];
  bool output;
};

Tensor tensor(const void* p, uint64_t bytes, const char* name, bool output) {
  Tensor t{p, bytes, {}, output};
  std::snprintf(t.name, sizeof(t.name), "%s", name);
  return t;
}

bool overlap(const Tensor& a, const Tensor& b) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Scalar arguments shared by every row entry point.  Sets *elem_bytes.
tw_status check_scalars(int32_t n, int64_t T, int64_t h, float eps, tw_dtype dtype,
                        const char* who, int64_t* elem_bytes) {
  if (n < 1 || n > TW_MAX_PARTIALS) {
    set_error("%s: num_partials=%d outside [1, %d]", who, n, TW_MAX_PARTIALS);
    return TW_ERR_INVALID_ARG;
  }
  if (T < 0 || h < 1) {
    set_error("%s: num_tokens=%lld must be >= 0 and hidden=%lld >= 1", who, (long long)T,
              (long long)h);
    return TW_ERR_INVALID_ARG;
  }
  if (!std::isfinite(eps) || eps < 0.0f) {
    set_error("%s: eps=%g must be finite and >= 0", who, (double)eps);
    return TW_ERR_INVALID_ARG;
  }
  if (dtype != TW_F32 && dtype != TW_BF16) {
    set_error("%s: unknown dtype %d", who, (int)dtype);
    return TW_ERR_INVALID_ARG;
  }
  const int64_t es = dtype == TW_BF16 ? 2 : 4;
  if (h > TW_MAX_ROW_BYTES / es) {             // before any product with h
    set_error("%s: hidden=%lld exceeds %lld elements", who, (long long)h,
              (long long)(TW_MAX_ROW_BYTES / es));
    return TW_ERR_UNSUPPORTED;
  }
  if ((h * es) % 16 != 0) {
    set_error("%s: hidden=%lld is not a multiple of %lld elements (16 bytes)", who,
              (long long)h, (long long)(16 / es));
    return TW_ERR_UNSUPPORTED;
  }
  if (T > TW_MAX_TOKENS) {
    set_error("%s: num_tokens=%lld exceeds %lld", who, (long long)T, (long long)TW_MAX_TOKENS);
    return TW_ERR_UNSUPPORTED;
  }
  *elem_bytes = es;
  return TW_OK;
}

// Tensor arguments: none NULL, all 16-byte aligned, no output overlapping any
// other argument except the one allowed in-place pair (output t[in_place_out]
// at exactly the address of input t[in_place_in]; -1: none), and, with pointer
// checks on, all device memory inside one allocation each.
tw_status check_tensors(const Tensor* t, int count, const char* who, int in_place_out = -1,
                        int in_place_in = -1) {
  for (int i = 0; i < count; ++i) {
    if (t[i].p == nullptr) {
      set_error("%s: %s is NULL", who, t[i].name);
      return TW_ERR_INVALID_ARG;
    }
  }
  for (int i = 0; i < count; ++i) {
    if ((reinterpret_cast<uintptr_t>(t[i].p) & 15u) != 0) {
      set_error("%s: %s is not 16-byte aligned", who, t[i].name);
      return TW_ERR_UNSUPPORTED;
    }
  }
  for (int i = 0; i < count; ++i) {
    if (!t[i].output) continue;
    for (int j = 0; j < count; ++j) {
      if (j == i || (t[j].output && j < i)) continue;     // each output pair once
      // The exemption is for that one pair, at exactly the same address.
      const bool allowed = i == in_place_out && j == in_place_in && t[i].p == t[j].p &&
                           t[i].bytes == t[j].bytes;
      if (!allowed && overlap(t[i], t[j])) {
        set_error("%s: %s overlaps %s%s", who, t[i].name, t[j].name,
                  in_place_out >= 0 ? " (only residual_out == residual is allowed)" : "");
        return TW_ERR_INVALID_ARG;
      }
    }
  }
  if (g_pointer_checks.load(std::memory_order_relaxed)) {
    for (int i = 0; i < count; ++i)
      if (!device_range_ok(t[i].p, t[i].bytes, t[i].name, who)) return TW_ERR_INVALID_ARG;
  }
  return TW_OK;
}

// Validation of the fused, shard and grid entries (and of tw_add_rmsnorm with
// its input as the one partial).  With num_tokens == 0 the pointers are not
// inspected.
tw_status validate(const void* const* partials, int32_t n, const void* residual,
                   const void* weight, void* out, void* residual_out, int64_t T, int64_t h,
                   float eps, tw_dtype dtype, const char* who,
                   const char* partial_name = "partials") {
  int64_t es = 0;
  const tw_status s = check_scalars(n, T, h, eps, dtype, who, &es);
  if (s != TW_OK || T == 0) return s;
  if (partials == nullptr) {
    set_error("%s: %s array is NULL", who, partial_name);
    return TW_ERR_INVALID_ARG;
  }
  const uint64_t tb = (uint64_t)T * (uint64_t)h * (uint64_t)es;
  Tensor t[TW_MAX_PARTIALS + 4];
  char name[24];
  for (int32_t i = 0; i < n; ++i) {
    if (n == 1 && partial_name[0] != 'p') std::snprintf(name, sizeof(name), "%s", partial_name);
    else std::snprintf(name, sizeof(name), "%s[%d]", partial_name, i);
    t[i] = tensor(partials[i], tb, name, false);
  }
  t[n] = tensor(residual, tb, "residual", false);
  t[n + 1] = tensor(weight, (uint64_t)h * es, "weight", false);
  t[n + 2] = tensor(out, tb, "out", true);
  t[n + 3] = tensor(residual_out, tb, "residual_out", true);
  return check_tensors(t, n + 4, who, /*in_place_out=*/n + 3, /*in_place_in=*/n);
}

tw_status launch_rows(const void* const* partials, int32_t n, const void* residual,
                      const void* weight, void* out, void* residual_out, int64_t row_begin,
                      int64_t row_end, int64_t h, float eps, tw_dtype dtype, void* stream,
                      int64_t max_workgroups = 0) {
  if (row_end <= row_begin) return TW_OK;
  FusedLaunch L{};
  for (int32_t i = 0; i < n; ++i) L.partials[i] = partials[i];
  L.num_partials = n;
  L.residual = residual;
  L.weight = weight;
  L.out = out;
  L.residual_out = residual_out;
  L.row_begin = row_begin;
  L.num_rows = row_end - row_begin;
  L.hidden = h;
  L.eps = eps;
  L.dtype = (int32_t)dtype;
  L.stream = stream;
  L.max_workgroups = max_workgroups;
  L.num_cus = stream_cus(stream);
  char msg[256];
  if (launch_fused(L, msg, sizeof(msg)) != 0) {
    set_error("%s", msg);
    return TW_ERR_DEVICE;
  }
  return TW_OK;
}

}  // namespace
}  // namespace tw

extern "C" {

int32_t tw_abi_version(void) { return TW_ABI_VERSION; }

void tw_set_pointer_checks(int32_t enabled) {
  tw::g_pointer_checks.store(enabled != 0 ? 1 : 0, std::memory_order_relaxed);
}

tw_status tw_fused_reduce_rmsnorm(const void* const* partials, int32_t num_partials,
                                  const void* residual, const void* weight, void* out,
                                  void* residual_out, int64_t num_tokens, int64_t hidden,
                                  float eps, tw_dtype dtype, void* stream) {
  const tw_status s = tw::validate(partials, num_partials, residual, weight, out, residual_out,
                                   num_tokens, hidden, eps, dtype, "tw_fused_reduce_rmsnorm");
  if (s != TW_OK || num_tokens == 0) return s;
  return tw::launch_rows(partials, num_partials, residual, weight, out, residual_out, 0,
                         num_tokens, hidden, eps, dtype, stream);
}

tw_status tw_fused_reduce_rmsnorm_grid(const void* const* partials, int32_t num_partials,
                                       const void* residual, const void* weight, void* out,
                                       void* residual_out, int64_t num_tokens, int64_t hidden,
                                       float eps, tw_dtype dtype, int32_t num_workgroups,
                                       void* stream) {
  const tw_status s = tw::validate(partials, num_partials, residual, weight, out, residual_out,
                                   num_tokens, hidden, eps, dtype, "tw_fused_reduce_rmsnorm_grid");
  if (s != TW_OK) return s;
  if (num_workgroups < 1) {
    tw::set_error("tw_fused_reduce_rmsnorm_grid: num_workgroups=%d must be >= 1", num_workgroups);
    return TW_ERR_INVALID_ARG;
  }
  if (num_tokens == 0) return TW_OK;
  return tw::launch_rows(partials, num_partials, residual, weight, out, residual_out, 0,
                         num_tokens, hidden, eps, dtype, stream, num_workgroups);
}

tw_status tw_shard_rmsnorm(const void* const* partials, int32_t num_partials,
                           const void* residual, const void* weight, void* out,
                           void* residual_out, int64_t num_tokens, int64_t hidden, float eps,
                           tw_dtype dtype, int32_t shard_index, void* stream) {
  const tw_status s = tw::validate(partials, num_partials, residual, weight, out, residual_out,
                                   num_tokens, hidden, eps, dtype, "tw_shard_rmsnorm");
  if (s != TW_OK) return s;
  if (shard_index < 0 || shard_index >= num_partials) {
    tw::set_error("tw_shard_rmsnorm: shard_index=%d outside [0, %d)", shard_index, num_partials);
    return TW_ERR_INVALID_ARG;
  }
  if (num_tokens == 0) return TW_OK;
  // Rows [floor(k*T/N), floor((k+1)*T/N)); T < 2^31 and N <= 16, so no overflow.
  const int64_t lo = (int64_t)shard_index * num_tokens / num_partials;
  const int64_t hi = ((int64_t)shard_index + 1) * num_tokens / num_partials;
  return tw::launch_rows(partials, num_partials, residual, weight, out, residual_out, lo, hi,
                         hidden, eps, dtype, stream);
}

tw_status tw_reduce_partials(const void* const* partials, int32_t num_partials, void* reduced,
                             int64_t num_tokens, int64_t hidden, tw_dtype dtype, void* stream) {
  const char* who = "tw_reduce_partials";
  int64_t es = 0;
  tw_status s = tw::check_scalars(num_partials, num_tokens, hidden, 0.0f, dtype, who, &es);
  if (s != TW_OK || num_tokens == 0) return s;
  if (partials == nullptr) {
    tw::set_error("%s: partials array is NULL", who);
    return TW_ERR_INVALID_ARG;
  }
  const uint64_t tb = (uint64_t)num_tokens * (uint64_t)hidden * (uint64_t)es;
  tw::Tensor t[TW_MAX_PARTIALS + 1];
  char name[24];
  for (int32_t i = 0; i < num_partials; ++i) {
    std::snprintf(name, sizeof(name), "partials[%d]", i);
    t[i] = tw::tensor(partials[i], tb, name, false);
  }
  t[num_partials] = tw::tensor(reduced, tb, "reduced", true);
  s = tw::check_tensors(t, num_partials + 1, who);
  if (s != TW_OK) return s;
  tw::ReduceLaunch L{};
  for (int32_t i = 0; i < num_partials; ++i) L.partials[i] = partials[i];
  L.num_partials = num_partials;
  L.reduced = reduced;
  L.num_rows = num_tokens;
  L.hidden = hidden;
  L.dtype = (int32_t)dtype;
  L.stream = stream;
  L.num_cus = tw::stream_cus(stream);
  char msg[256];
  if (tw::launch_reduce(L, msg, sizeof(msg)) != 0) {
    tw::set_error("%s", msg);
    return TW_ERR_DEVICE;
  }
  return TW_OK;
}

tw_status tw_add_rmsnorm(const void* input, const void* residual, const void* weight, void* out,
                         void* residual_out, int64_t num_tokens, int64_t hidden, float eps,
                         tw_dtype dtype, void* stream) {
  const void* parts[1] = {input};
  const tw_status s = tw::validate(parts, 1, residual, weight, out, residual_out, num_tokens,
                                   hidden, eps, dtype, "tw_add_rmsnorm", "input");
  if (s != TW_OK || num_tokens == 0) return s;
  tw::AddNormLaunch L{};
  L.input = input;
  L.residual = residual;
  L.weight = weight;
  L.out = out;
  L.residual_out = residual_out;
  L.num_rows = num_tokens;
  L.hidden = hidden;
  L.eps = eps;
  L.dtype = (int32_t)dtype;
  L.stream = stream;
  char msg[256];
  if (tw::launch_add_rmsnorm(L, msg, sizeof(msg)) != 0) {
    tw::set_error("%s", msg);
    return TW_ERR_DEVICE;
  }
  return TW_OK;
}

tw_status tw_fused_launch_info(int32_t num_partials, int64_t num_tokens, int64_t hidden,
                               tw_dtype dtype, void* stream, tw_launch_info* out) {
  const char* who = "tw_fused_launch_info";
  if (out == nullptr) {
    tw::set_error("%s: NULL result pointer", who);
    return TW_ERR_INVALID_ARG;
  }
  int64_t es = 0;
  const tw_status s = tw::check_scalars(num_partials, num_tokens, hidden, 0.0f, dtype, who, &es);
  if (s != TW_OK) return s;
  tw_launch_info r{};
  r.num_cus = tw::stream_cus(stream);
  const tw::FusedPlan p = tw::plan_fused(hidden * es / 16, num_partials, num_tokens, r.num_cus);
  r.threads_per_workgroup = tw::fused_geometry(p.geometry, num_partials).block;
  r.vectors_per_thread = tw::fused_geometry(p.geometry, num_partials).vpt;
  r.round_rows = tw::round_rows(r.threads_per_workgroup, r.num_cus);
  r.rows_per_dispatch = p.rows_per_dispatch;
  r.dispatches = p.dispatches;
  r.kernel = -1;
  if (num_tokens > 0) {
    const tw::RowKernel rk = tw::fused_row_kernel(p.geometry, num_partials, p.rows_per_dispatch,
                                                  r.num_cus);
    r.kernel = rk == tw::RowKernel::kStrided     ? TW_KERNEL_STRIDED
               : rk == tw::RowKernel::kSequenced ? TW_KERNEL_SEQUENCED
               : rk == tw::RowKernel::kBothSlots ? TW_KERNEL_BOTH_SLOTS
                                                 : TW_KERNEL_ALL_AT_ONCE;
  }
  *out = r;
  return TW_OK;
}

const char* tw_status_string(tw_status s) {
  switch (s) {
    case TW_OK: return "TW_OK";
    case TW_ERR_INVALID_ARG: return "TW_ERR_INVALID_ARG: argument out of range";
    case TW_ERR_UNSUPPORTED: return "TW_ERR_UNSUPPORTED: outside what the kernels handle";
    case TW_ERR_DEVICE: return "TW_ERR_DEVICE: the HIP runtime reported an error";
  }
  return "unknown tw_status";
}

const char* tw_last_error(void) { return tw::g_last_error; }

}  // extern "C"
