// Host side of the boundary: error text, the static keep-mask schedule and
// the cache layout.  Plain C++17, no device code.
//
// The schedule follows the HeatKV project page, Method steps 3-5 (rank
// head-scale pairs by their contribution to future predictions, remove
// low-ranked pairs to meet the budget, always keep the early sink scales, one
// static prompt-independent schedule) and the Figure 4 caption on the Pith
// page of arXiv 2605.14877 (per-source-scale orderings of the heads, pruning
// set = union of a prefix of each ordering).
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "../../include/heatkv.h"
#include "status.h"

namespace hk {

static thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

}  // namespace hk

extern "C" const char* hk_last_error(void) { return hk::g_last_error.c_str(); }

extern "C" int hk_build_schedule(int L, int H, int K, const int32_t* scale_tokens,
                                 const float* scas, double budget_frac, int n_sink,
                                 uint8_t* keep_out, int64_t* retained_out,
                                 int32_t* n_pruned_out) {
  using hk::fail;
  if (L < 1 || H < 1 || K < 1) return fail(HK_EINVAL, "L, H, K must be >= 1");
  if (!scale_tokens || !scas || !keep_out) return fail(HK_EINVAL, "null argument");
  for (int s = 0; s < K; ++s)
    if (scale_tokens[s] < 1) return fail(HK_EINVAL, "scale %d has no tokens", s);
  if (n_sink < 0 || n_sink > K - 1) return fail(HK_EINVAL, "n_sink must be in [0, K-1]");
  if (!(budget_frac > 0.0 && budget_frac <= 1.0))
    return fail(HK_EINVAL, "budget_frac must be in (0, 1]");

  const int64_t heads = int64_t(L) * H;
  const auto at = [&](int64_t f, int t, int s) -> double {
    return double(scas[(f * K + t) * K + s]);
  };

  // Token-slot costs per sequence.
  int64_t cached_tokens = 0, sink_tokens = 0, prunable_tokens = 0;
  for (int s = 0; s <= K - 2; ++s) {
    cached_tokens += scale_tokens[s];
    if (s < n_sink) sink_tokens += scale_tokens[s];
    else prunable_tokens += scale_tokens[s];
  }
  const int64_t full = heads * cached_tokens;
  const int64_t budget = int64_t(std::floor(budget_frac * double(full)));
  const int64_t sink_cost = heads * sink_tokens;
  if (budget < sink_cost)
    return fail(HK_EBUDGET, "budget of %lld token slots is below the sink cost %lld",
                (long long)budget, (long long)sink_cost);
  const int64_t kept =
      prunable_tokens == 0 ? heads : std::min(heads, (budget - sink_cost) / prunable_tokens);
  const int64_t n_prune = heads - kept;

  // Every cacheable scale starts kept; the final scale is never cached.
  for (int64_t f = 0; f < heads; ++f)
    for (int s = 0; s < K; ++s) keep_out[f * K + s] = s <= K - 2 ? 1 : 0;

  if (n_prune > 0) {
    std::vector<double> imp(heads);
    std::vector<int64_t> order(heads);
    for (int s = n_sink; s <= K - 2; ++s) {
      // Future dependence of each head on source scale s.
      for (int64_t f = 0; f < heads; ++f) {
        double acc = 0.0;
        for (int t = s + 1; t < K; ++t) acc += at(f, t, s);
        imp[f] = acc;
      }
      std::iota(order.begin(), order.end(), int64_t(0));
      // Least dependent first; equal importance drops the lower flat index first.
      std::sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
        return imp[a] < imp[b] || (imp[a] == imp[b] && a < b);
      });
      for (int64_t i = 0; i < n_prune; ++i) keep_out[order[i] * K + s] = 0;
    }
  }

  if (retained_out) {
    int64_t running = 0;
    for (int k = 0; k < K; ++k) {
      if (k <= K - 2) {
        int64_t kept_heads = 0;
        for (int64_t f = 0; f < heads; ++f) kept_heads += keep_out[f * K + k];
        running += kept_heads * scale_tokens[k];
      }
      retained_out[k] = running;
    }
  }
  if (n_pruned_out) *n_pruned_out = int32_t(n_prune);
  return HK_OK;
}

extern "C" int hk_layout(int L, int H, int K, const int32_t* scale_tokens, const uint8_t* keep,
                         int B, int D, int64_t* cache_elems_out, int64_t* cap_out,
                         int64_t* base_out) {
  using hk::fail;
  if (L < 1 || H < 1 || K < 1 || B < 1 || D < 1) return fail(HK_EINVAL, "sizes must be >= 1");
  if (!scale_tokens || !keep || !cache_elems_out) return fail(HK_EINVAL, "null argument");
  int64_t offset = 0;
  for (int64_t f = 0; f < int64_t(L) * H; ++f) {
    int64_t cap = 0;
    for (int s = 0; s <= K - 2; ++s) {
      if (scale_tokens[s] < 1) return fail(HK_EINVAL, "scale %d has no tokens", s);
      if (keep[f * K + s]) cap += scale_tokens[s];
    }
    if (cap_out) cap_out[f] = cap;
    if (base_out) base_out[f] = offset;
    offset += cap * B * D;
  }
  *cache_elems_out = offset;
  return HK_OK;
}
