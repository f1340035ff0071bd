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
// The page picks the offset by timing the GEMMs offline and keeps the winner
// per shape in a table.  tw_split_plan, with no GEMM to time, takes the first
// offset (in the given order) that meets the wave condition;
// tw_split_plan_measured looks the shape up in a caller's measured table
// first and holds the table's offset to the same wave condition.  For odd T
// the suffix is T - prefix, so no token is dropped.

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

// Checks the problem's fields and its offset list; fills the wave model, the
// offsets to search and the unsplit wave count.
tw_status check_problem(const tw_split_problem* in, const char* who, WaveModel* wm,
                        const int32_t** offs, int32_t* n_offs, int64_t* W) {
  const tw_split_problem p = *in;
  if (p.num_tokens < 0 || p.tokens_per_cta < 1 || p.ctas_per_token_tile < 1 || p.num_cus < 1 ||
      p.ctas_per_cu < 1 || p.min_split_tokens < 0 || p.num_offsets < 0 ||
      (p.offsets == nullptr && p.num_offsets != 0)) {
    set_error("%s: field out of range (num_tokens=%lld tokens_per_cta=%lld "
              "ctas_per_token_tile=%lld num_cus=%d ctas_per_cu=%d min_split_tokens=%lld "
              "num_offsets=%d)",
              who, (long long)p.num_tokens, (long long)p.tokens_per_cta,
              (long long)p.ctas_per_token_tile, p.num_cus, p.ctas_per_cu,
              (long long)p.min_split_tokens, p.num_offsets);
    return TW_ERR_INVALID_ARG;
  }
  *offs = p.offsets ? p.offsets : kDefaultOffsets;
  *n_offs = p.offsets ? p.num_offsets : (int32_t)(sizeof(kDefaultOffsets) / sizeof(int32_t));
  for (int32_t i = 0; i < *n_offs; ++i) {
    if ((*offs)[i] < 0 || (i > 0 && (*offs)[i] <= (*offs)[i - 1])) {
      set_error("%s: offsets must be >= 0 and strictly ascending (index %d)", who, i);
      return TW_ERR_INVALID_ARG;
    }
  }
  if (p.num_tokens > kMaxTokens || p.ctas_per_token_tile > kMaxTiles) {
    set_error("%s: num_tokens above 2^40 or ctas_per_token_tile above 2^20", who);
    return TW_ERR_UNSUPPORTED;
  }
  *wm = WaveModel{p.tokens_per_cta, p.ctas_per_token_tile, (int64_t)p.num_cus * (int64_t)p.ctas_per_cu};
  *W = wm->waves(p.num_tokens);
  if (*W > INT32_MAX) {
    set_error("%s: wave count does not fit in int32", who);
    return TW_ERR_UNSUPPORTED;
  }
  return TW_OK;
}

// The plan that keeps all T tokens in the prefix.
tw_split_plan_result whole(int64_t T, int64_t W, int32_t reason) {
  tw_split_plan_result r{};
  r.prefix_tokens = T;
  r.suffix_tokens = 0;
  r.offset = -1;
  r.waves_unsplit = (int32_t)W;
  r.waves_prefix = (int32_t)W;
  r.waves_suffix = 0;
  r.reason = reason;
  return r;
}

// The rules that come before any offset is tried: an empty batch, a batch
// below the threshold and a batch of one wave stay whole.  Returns false when
// none applies.
bool early_rule(int64_t T, int64_t min_split_tokens, int64_t W, tw_split_plan_result* r) {
  if (T == 0) *r = whole(T, W, TW_PLAN_EMPTY);
  else if (T < min_split_tokens) *r = whole(T, W, TW_PLAN_BELOW_THRESHOLD);
  else if (W <= 1) *r = whole(T, W, TW_PLAN_SINGLE_WAVE);
  else return false;
  return true;
}

// The two pieces of offset `off`, or false when they break the wave condition.
bool pieces(const WaveModel& wm, int64_t T, int64_t W, int64_t off, int32_t reason,
            tw_split_plan_result* r) {
  const int64_t prefix = T / 2 + off;
  const int64_t suffix = T - prefix;
  const int64_t wp = wm.waves(prefix), ws = wm.waves(suffix);
  if (wp + ws > W) return false;
  *r = whole(T, W, reason);
  r->prefix_tokens = prefix;
  r->suffix_tokens = suffix;
  r->offset = (int32_t)off;
  r->waves_prefix = (int32_t)wp;
  r->waves_suffix = (int32_t)ws;
  return true;
}

// The analytic search: the first offset below floor(T/2), in the given order,
// whose pieces meet the wave condition.
tw_split_plan_result search(const WaveModel& wm, int64_t T, int64_t W, const int32_t* offs,
                            int32_t n_offs) {
  tw_split_plan_result r = whole(T, W, TW_PLAN_NO_FEASIBLE_OFFSET);
  for (int32_t i = 0; i < n_offs; ++i) {
    if (offs[i] >= T / 2) continue;
    if (pieces(wm, T, W, offs[i], TW_PLAN_SPLIT, &r)) break;
  }
  return r;
}

}  // namespace
}  // namespace tw

extern "C" tw_status tw_split_plan(const tw_split_problem* in, tw_split_plan_result* out) {
  using namespace tw;
  if (in == nullptr || out == nullptr) {
    set_error("tw_split_plan: NULL problem or result pointer");
    return TW_ERR_INVALID_ARG;
  }
  WaveModel wm{};
  const int32_t* offs = nullptr;
  int32_t n_offs = 0;
  int64_t W = 0;
  const tw_status s = check_problem(in, "tw_split_plan", &wm, &offs, &n_offs, &W);
  if (s != TW_OK) return s;
  tw_split_plan_result r{};
  if (!early_rule(in->num_tokens, in->min_split_tokens, W, &r))
    r = search(wm, in->num_tokens, W, offs, n_offs);
  *out = r;
  return TW_OK;
}

extern "C" tw_status tw_split_plan_measured(const tw_split_problem* in,
                                            const tw_split_entry* table, int32_t table_len,
                                            tw_split_plan_result* out) {
  using namespace tw;
  const char* who = "tw_split_plan_measured";
  if (in == nullptr || out == nullptr) {
    set_error("%s: NULL problem or result pointer", who);
    return TW_ERR_INVALID_ARG;
  }
  if (table_len < 0 || (table == nullptr && table_len != 0)) {
    set_error("%s: table_len=%d with a %s table", who, table_len, table ? "non-NULL" : "NULL");
    return TW_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < table_len; ++i) {
    const tw_split_entry e = table[i];
    if (e.num_tokens < 1 || (i > 0 && e.num_tokens <= table[i - 1].num_tokens)) {
      set_error("%s: table token counts must be >= 1 and strictly ascending (index %d)", who, i);
      return TW_ERR_INVALID_ARG;
    }
    if (e.offset < -1 || (e.offset >= 0 && e.offset >= e.num_tokens / 2)) {
      set_error("%s: table entry %d (num_tokens=%lld) has offset %d outside [0, T/2) or -1",
                who, i, (long long)e.num_tokens, e.offset);
      return TW_ERR_INVALID_ARG;
    }
  }
  WaveModel wm{};
  const int32_t* offs = nullptr;
  int32_t n_offs = 0;
  int64_t W = 0;
  const tw_status s = check_problem(in, who, &wm, &offs, &n_offs, &W);
  if (s != TW_OK) return s;
  const int64_t T = in->num_tokens;
  tw_split_plan_result r{};
  if (!early_rule(T, in->min_split_tokens, W, &r)) {
    // Binary search of the ascending table.
    int32_t lo = 0, hi = table_len;
    while (lo < hi) {
      const int32_t mid = lo + (hi - lo) / 2;
      if (table[mid].num_tokens < T) lo = mid + 1;
      else hi = mid;
    }
    if (lo == table_len || table[lo].num_tokens != T) r = search(wm, T, W, offs, n_offs);
    else if (table[lo].offset < 0) r = whole(T, W, TW_PLAN_MEASURED_UNSPLIT);
    else if (!pieces(wm, T, W, table[lo].offset, TW_PLAN_MEASURED_SPLIT, &r))
      r = whole(T, W, TW_PLAN_MEASURED_OVER_WAVES);
  }
  *out = r;
  return TW_OK;
}
