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

struct Range {
  uintptr_t lo, hi;   // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range range_of(const void* p, uint64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + (uintptr_t)bytes};
}

// Shared checks of the fused and shard entries; TW_OK when the arguments are
// valid.  With num_tokens == 0 the pointers are not inspected.
tw_status validate(const void* const* partials, int32_t n, const void* residual,
                   const void* weight, void* out, void* residual_out, int64_t T, int64_t h,
                   float eps, tw_dtype dtype, const char* who, bool outputs_alias = false) {
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
  if ((h * es) % 16 != 0) {
    set_error("%s: hidden=%lld is not a multiple of %lld elements (16 bytes)", who,
              (long long)h, (long long)(16 / es));
    return TW_ERR_UNSUPPORTED;
  }
  if (h * es > TW_MAX_ROW_BYTES) {
    set_error("%s: hidden=%lld exceeds %lld elements", who, (long long)h,
              (long long)(TW_MAX_ROW_BYTES / es));
    return TW_ERR_UNSUPPORTED;
  }
  if (T > TW_MAX_TOKENS) {
    set_error("%s: num_tokens=%lld exceeds %lld", who, (long long)T, (long long)TW_MAX_TOKENS);
    return TW_ERR_UNSUPPORTED;
  }
  if (T == 0) return TW_OK;
  if (partials == nullptr || residual == nullptr || weight == nullptr || out == nullptr ||
      residual_out == nullptr) {
    set_error("%s: NULL tensor pointer", who);
    return TW_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (partials[i] == nullptr) {
      set_error("%s: partials[%d] is NULL", who, i);
      return TW_ERR_INVALID_ARG;
    }
  }
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
  for (int32_t i = 0; i < n; ++i) {
    if (misaligned(partials[i])) {
      set_error("%s: partials[%d] is not 16-byte aligned", who, i);
      return TW_ERR_UNSUPPORTED;
    }
  }
  if (misaligned(residual) || misaligned(weight) || misaligned(out) || misaligned(residual_out)) {
    set_error("%s: residual, weight, out and residual_out must be 16-byte aligned", who);
    return TW_ERR_UNSUPPORTED;
  }
  const uint64_t tensor_bytes = (uint64_t)T * (uint64_t)h * (uint64_t)es;
  const Range r_out = range_of(out, tensor_bytes);
  const Range r_res_out = range_of(residual_out, tensor_bytes);
  const Range r_res = range_of(residual, tensor_bytes);
  const Range r_w = range_of(weight, (uint64_t)h * es);
  if (!outputs_alias && overlaps(r_out, r_res_out)) {
    set_error("%s: out and residual_out overlap", who);
    return TW_ERR_INVALID_ARG;
  }
  // With outputs_alias the caller has one output (passed as both) and the
  // residual/weight slots hold a partial; only the partials are checked.
  const bool in_place = residual_out == residual;
  const int32_t last_input = outputs_alias ? n - 1 : n + 1;
  for (int32_t i = 0; i <= last_input; ++i) {
    const Range in = i < n ? range_of(partials[i], tensor_bytes) : (i == n ? r_res : r_w);
    if (overlaps(r_out, in)) {
      set_error("%s: out overlaps an input (%s)", who,
                i < n ? "a partial" : (i == n ? "residual" : "weight"));
      return TW_ERR_INVALID_ARG;
    }
    if (i == n && in_place) continue;
    if (overlaps(r_res_out, in)) {
      set_error("%s: residual_out overlaps an input (%s); only residual_out == residual is "
                "allowed", who, i < n ? "a partial" : (i == n ? "residual" : "weight"));
      return TW_ERR_INVALID_ARG;
    }
  }
  if (g_pointer_checks.load(std::memory_order_relaxed)) {
    char what[32];
    for (int32_t i = 0; i < n; ++i) {
      std::snprintf(what, sizeof(what), "partials[%d]", i);
      if (!device_range_ok(partials[i], tensor_bytes, what, who)) return TW_ERR_INVALID_ARG;
    }
    if (!device_range_ok(residual, tensor_bytes, "residual", who) ||
        !device_range_ok(weight, (uint64_t)h * es, "weight", who) ||
        !device_range_ok(out, tensor_bytes, "out", who) ||
        !device_range_ok(residual_out, tensor_bytes, "residual_out", who))
      return TW_ERR_INVALID_ARG;
  }
  return TW_OK;
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
  // Same checks as the fused entry with the reduced tensor standing in for
  // both outputs' ranges; a zero eps and the partials as residual/weight
  // placeholders keep the shared validation meaningful.
  const char* who = "tw_reduce_partials";
  if (num_tokens > 0 && reduced == nullptr) {
    tw::set_error("%s: NULL tensor pointer", who);
    return TW_ERR_INVALID_ARG;
  }
  const void* any = (partials != nullptr && num_partials >= 1) ? partials[0] : nullptr;
  tw_status s = tw::validate(partials, num_partials, any, any, reduced, reduced, num_tokens,
                             hidden, 0.0f, dtype, who, /*outputs_alias=*/true);
  if (s != TW_OK || num_tokens == 0) return s;
  tw::ReduceLaunch L{};
  for (int32_t i = 0; i < num_partials; ++i) L.partials[i] = partials[i];
  L.num_partials = num_partials;
  L.reduced = reduced;
  L.num_rows = num_tokens;
  L.hidden = hidden;
  L.dtype = (int32_t)dtype;
  L.stream = stream;
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
                                   hidden, eps, dtype, "tw_add_rmsnorm");
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
