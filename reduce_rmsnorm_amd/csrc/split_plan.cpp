// Wave-aware prefix/suffix split planner (host only, integer arithmetic).
//
// Rule from the blog post "TokenWeave: Why Hiding Tensor-Parallel
// Communication Needs Wave Arithmetic, Not Finer Tiles":
//  * "The overlap trap": a GEMM of C CTAs on S SMs runs ceil(C / S) waves.
//  * "Fix one: split at wave boundaries, unequally": split the batch exactly
//    in two, prefix = half + offset and suffix = half - offset with the offset
//    from {0, 64, 128, 192, 256, 512} kept below half, such that the two
//    pieces together take no more waves than the whole; do not split a batch
//    that is already one wave, nor one below the per-model token threshold.
// The page picks the offset by timing the GEMMs offline; with no GEMM to time
// this planner takes the first offset (in the given order) that meets the wave
// condition.  For odd T the suffix is T - prefix, so no token is dropped.

#include <cstdint>
#include <cstdio>

#include "tokenweave.h"

namespace tw {

void set_error(const char* fmt, ...);

namespace {

constexpr int32_t kDefaultOffsets[] = {0, 64, 128, 192, 256, 512};
constexpr int64_t kMaxTokens = int64_t(1) << 40;
constexpr int64_t kMaxTiles = int64_t(1) << 20;

// a >= 0, b >= 1; no intermediate can overflow, whatever b is.
int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0 ? 1 : 0); }

struct WaveModel {
  int64_t tokens_per_cta, tiles, slots;
  int64_t waves(int64_t m) const { return ceil_div(ceil_div(m, tokens_per_cta) * tiles, slots); }
};

}  // namespace
}  // namespace tw

extern "C" tw_status tw_split_plan(const tw_split_problem* in, tw_split_plan_result* out) {
  using namespace tw;
  if (in == nullptr || out == nullptr) {
    set_error("tw_split_plan: NULL problem or result pointer");
    return TW_ERR_INVALID_ARG;
  }
  const tw_split_problem p = *in;
  if (p.num_tokens < 0 || p.tokens_per_cta < 1 || p.ctas_per_token_tile < 1 || p.num_cus < 1 ||
      p.ctas_per_cu < 1 || p.min_split_tokens < 0 || p.num_offsets < 0 ||
      (p.offsets == nullptr && p.num_offsets != 0)) {
    set_error("tw_split_plan: field out of range (num_tokens=%lld tokens_per_cta=%lld "
              "ctas_per_token_tile=%lld num_cus=%d ctas_per_cu=%d min_split_tokens=%lld "
              "num_offsets=%d)",
              (long long)p.num_tokens, (long long)p.tokens_per_cta,
              (long long)p.ctas_per_token_tile, p.num_cus, p.ctas_per_cu,
              (long long)p.min_split_tokens, p.num_offsets);
    return TW_ERR_INVALID_ARG;
  }
  const int32_t* offs = p.offsets ? p.offsets : kDefaultOffsets;
  const int32_t n_offs = p.offsets ? p.num_offsets : (int32_t)(sizeof(kDefaultOffsets) / sizeof(int32_t));
  for (int32_t i = 0; i < n_offs; ++i) {
    if (offs[i] < 0 || (i > 0 && offs[i] <= offs[i - 1])) {
      set_error("tw_split_plan: offsets must be >= 0 and strictly ascending (index %d)", i);
      return TW_ERR_INVALID_ARG;
    }
  }
  if (p.num_tokens > kMaxTokens || p.ctas_per_token_tile > kMaxTiles) {
    set_error("tw_split_plan: num_tokens above 2^40 or ctas_per_token_tile above 2^20");
    return TW_ERR_UNSUPPORTED;
  }
  const WaveModel wm{p.tokens_per_cta, p.ctas_per_token_tile,
                     (int64_t)p.num_cus * (int64_t)p.ctas_per_cu};
  const int64_t T = p.num_tokens;
  const int64_t W = wm.waves(T);
  if (W > INT32_MAX) {
    set_error("tw_split_plan: wave count does not fit in int32");
    return TW_ERR_UNSUPPORTED;
  }

  tw_split_plan_result r{};
  r.prefix_tokens = T;
  r.suffix_tokens = 0;
  r.offset = -1;
  r.waves_unsplit = (int32_t)W;
  r.waves_prefix = (int32_t)W;
  r.waves_suffix = 0;
  if (T == 0) {
    r.reason = TW_PLAN_EMPTY;
  } else if (T < p.min_split_tokens) {
    r.reason = TW_PLAN_BELOW_THRESHOLD;
  } else if (W <= 1) {
    r.reason = TW_PLAN_SINGLE_WAVE;
  } else {
    r.reason = TW_PLAN_NO_FEASIBLE_OFFSET;
    const int64_t half = T / 2;
    for (int32_t i = 0; i < n_offs; ++i) {
      const int64_t off = offs[i];
      if (off >= half) continue;
      const int64_t prefix = half + off;
      const int64_t suffix = T - prefix;
      const int64_t wp = wm.waves(prefix), ws = wm.waves(suffix);
      if (wp + ws <= W) {
        r.prefix_tokens = prefix;
        r.suffix_tokens = suffix;
        r.offset = (int32_t)off;
        r.waves_prefix = (int32_t)wp;
        r.waves_suffix = (int32_t)ws;
        r.reason = TW_PLAN_SPLIT;
        break;
      }
    }
  }
  *out = r;
  return TW_OK;
}
