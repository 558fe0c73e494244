// plan.cpp -- the broadcast schedule of Pyramid Attention Broadcast.
//
// PAB article, "Implementation": attention changes a lot in the first and
// last 15% of the denoising steps and little in the middle 70%; in that
// middle one step's attention output is broadcast to several following
// steps, over a range chosen per attention type (wider for types that change
// less; PAB abstract calls the set of ranges a pyramid).  Figure 2 caption:
// at run time the broadcast output replaces the next few steps' attention.
//
// Integer arithmetic only, so the result is exact and platform-independent.
// The window test is evaluated on i/N as 100*i against pct*N.
#include <stdint.h>

#include <algorithm>
#include <limits>

#include "abi.hpp"

using namespace pab;

extern "C" int pab_plan_schedule(int32_t num_steps, int32_t num_types, const int32_t* ranges,
                                 int32_t window_lo_pct, int32_t window_hi_pct,
                                 uint8_t* recompute, int32_t* source_step,
                                 int32_t* recompute_count) {
  if (num_steps < 1) return fail(PAB_ERR_INVALID_ARG, "pab_plan_schedule: num_steps must be >= 1");
  if (num_types < 1 || num_types > 32)
    return fail(PAB_ERR_INVALID_ARG, "pab_plan_schedule: num_types must be in [1, 32]");
  if (!ranges || !recompute) return fail(PAB_ERR_INVALID_ARG, "pab_plan_schedule: NULL array");
  if (!(0 <= window_lo_pct && window_lo_pct <= window_hi_pct && window_hi_pct <= 100))
    return fail(PAB_ERR_INVALID_ARG, "pab_plan_schedule: need 0 <= lo <= hi <= 100");
  for (int a = 0; a < num_types; ++a)
    if (ranges[a] < 0) return fail(PAB_ERR_INVALID_ARG, "pab_plan_schedule: negative range");

  const int64_t n = num_steps;
  // First step of the stable window, and its length.
  int64_t w0 = -1, w = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (100 * i >= (int64_t)window_lo_pct * n && 100 * i < (int64_t)window_hi_pct * n) {
      if (w0 < 0) w0 = i;
      ++w;
    }
  }
  for (int a = 0; a < num_types; ++a) {
    const int64_t period = (int64_t)ranges[a] + 1;
    int32_t count = 0, src = 0;
    for (int64_t i = 0; i < n; ++i) {
      const bool inside = w > 0 && i >= w0 && i < w0 + w;
      const bool fresh = !inside || ((i - w0) % period) == 0;
      if (fresh) {
        src = (int32_t)i;
        ++count;
      }
      recompute[i * num_types + a] = fresh ? 1 : 0;
      if (source_step) source_step[i * num_types + a] = src;
    }
    if (recompute_count) recompute_count[a] = count;
  }
  return ok();
}

// Broadcast ranges from a measured attention difference.  PAB article,
// "Implementation": each type's range follows how much its output changes
// between consecutive steps inside the stable window (the less, the wider),
// that change being the MSE of Figure 1.  A type's score is the mean of its
// differences over every block and the steps whose output and
// predecessor's output both lie in the window (summed block by block, each
// block's steps in step order, fp64); candidates are handed out by rank,
// the largest score receiving the smallest candidate (ties: the lower type
// index counts as larger).
extern "C" int pab_plan_calibrate(int32_t num_blocks, int32_t num_steps, int32_t num_types,
                                  const double* diff, int32_t window_lo_pct, int32_t window_hi_pct,
                                  const int32_t* candidate_ranges, int32_t* ranges_out,
                                  double* score_out) {
  const char* fn = "pab_plan_calibrate";
  if (num_blocks < 1) return fail(PAB_ERR_INVALID_ARG, fmt("%s: num_blocks must be >= 1", fn));
  if (num_steps < 1) return fail(PAB_ERR_INVALID_ARG, fmt("%s: num_steps must be >= 1", fn));
  if (num_types < 1 || num_types > 32)
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: num_types must be in [1, 32]", fn));
  if (!diff || !candidate_ranges || !ranges_out)
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: NULL array", fn));
  if (!(0 <= window_lo_pct && window_lo_pct <= window_hi_pct && window_hi_pct <= 100))
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: need 0 <= lo <= hi <= 100", fn));
  for (int a = 0; a < num_types; ++a)
    if (candidate_ranges[a] < 0) return fail(PAB_ERR_INVALID_ARG, fmt("%s: negative candidate range", fn));

  const int64_t n = num_steps;
  auto inside = [&](int64_t i) {
    return 100 * i >= (int64_t)window_lo_pct * n && 100 * i < (int64_t)window_hi_pct * n;
  };
  int64_t counted = 0;
  for (int64_t i = 1; i < n; ++i)
    if (inside(i) && inside(i - 1)) ++counted;
  if (counted == 0)
    return fail(PAB_ERR_INVALID_ARG,
                fmt("%s: the window holds no two consecutive steps", fn));
  double score[32];
  for (int a = 0; a < num_types; ++a) score[a] = 0.0;
  for (int64_t b = 0; b < num_blocks; ++b) {
    const double* db = diff + b * n * num_types;
    for (int64_t i = 1; i < n; ++i) {
      if (!(inside(i) && inside(i - 1))) continue;
      for (int a = 0; a < num_types; ++a) {
        const double d = db[i * num_types + a];
        if (!(d >= 0.0) || d == std::numeric_limits<double>::infinity())
          return fail(PAB_ERR_INVALID_ARG,
                      fmt("%s: difference at block %lld, step %lld, type %d is not finite and >= 0",
                          fn, (long long)b, (long long)i, a));
        score[a] += d;
      }
    }
  }
  for (int a = 0; a < num_types; ++a) score[a] /= (double)(counted * num_blocks);

  // Rank: largest score first, lower index first among equals.
  int order[32];
  for (int a = 0; a < num_types; ++a) order[a] = a;
  std::stable_sort(order, order + num_types, [&](int x, int y) { return score[x] > score[y]; });
  int32_t ascending[32];
  for (int a = 0; a < num_types; ++a) ascending[a] = candidate_ranges[a];
  std::sort(ascending, ascending + num_types);
  for (int k = 0; k < num_types; ++k) ranges_out[order[k]] = ascending[k];
  if (score_out)
    for (int a = 0; a < num_types; ++a) score_out[a] = score[a];
  return ok();
}
