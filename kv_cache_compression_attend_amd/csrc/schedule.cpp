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
#include "layout.h"
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

namespace {

using hk::fail;

int check_schedule_args(int L, int H, int K, const int32_t* scale_tokens, const void* scas,
                        double budget_frac, int n_sink) {
  if (L < 1 || H < 1 || K < 1) return fail(HK_EINVAL, "L, H, K must be >= 1");
  if (!scale_tokens || !scas) return fail(HK_EINVAL, "null argument");
  for (int s = 0; s < K; ++s)
    if (scale_tokens[s] < 1) return fail(HK_EINVAL, "scale %d has no tokens", s);
  if (n_sink < 0 || n_sink > K - 1) return fail(HK_EINVAL, "n_sink must be in [0, K-1]");
  if (!(budget_frac > 0.0 && budget_frac <= 1.0))
    return fail(HK_EINVAL, "budget_frac must be in (0, 1]");
  return HK_OK;
}

// O_s: the flat head indices ascending by (importance, index), where the
// importance of head f for source scale s is its S-CAS mass summed over the
// later target scales t > s, in double, ascending t.
void ordering(const float* scas, int64_t heads, int K, int s, std::vector<double>& imp,
              std::vector<int64_t>& order) {
  imp.assign(heads, 0.0);
  for (int64_t f = 0; f < heads; ++f) {
    double acc = 0.0;
    for (int t = s + 1; t < K; ++t) acc += double(scas[(f * K + t) * K + s]);
    imp[f] = acc;
  }
  order.resize(heads);
  std::iota(order.begin(), order.end(), int64_t(0));
  // Least dependent first; equal importance drops the lower flat index first.
  std::sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
    return imp[a] < imp[b] || (imp[a] == imp[b] && a < b);
  });
}

}  // namespace

extern "C" int hk_build_schedule(int L, int H, int K, const int32_t* scale_tokens,
                                 const float* scas, double budget_frac, int n_sink,
                                 uint8_t* keep_out, int64_t* retained_out,
                                 int32_t* n_pruned_out) {
  int rc = check_schedule_args(L, H, K, scale_tokens, scas, budget_frac, n_sink);
  if (rc != HK_OK) return rc;
  if (!keep_out) return fail(HK_EINVAL, "null argument");
  const int64_t heads = int64_t(L) * H;

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
    std::vector<double> imp;
    std::vector<int64_t> order;
    for (int s = n_sink; s <= K - 2; ++s) {
      ordering(scas, heads, K, s, imp, order);
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

extern "C" int hk_scas_mean(int L, int H, int K, const double* scas_sum, double images,
                            float* scas_out) {
  if (L < 1 || H < 1 || K < 1) return fail(HK_EINVAL, "L, H, K must be >= 1");
  if (!scas_sum || !scas_out) return fail(HK_EINVAL, "null argument");
  if (!(images > 0.0)) return fail(HK_EINVAL, "images must be positive");
  const int64_t n = int64_t(L) * H * K * K;
  for (int64_t i = 0; i < n; ++i) scas_out[i] = float(scas_sum[i] / images);
  return HK_OK;
}

extern "C" int hk_ranking_stability(int L, int H, int K, const int32_t* scale_tokens,
                                    const float* scas_a, const float* scas_b, double budget_frac,
                                    int n_sink, double* rho_out, double* jaccard_out) {
  int rc = check_schedule_args(L, H, K, scale_tokens, scas_a, budget_frac, n_sink);
  if (rc != HK_OK) return rc;
  if (!scas_b || !rho_out || !jaccard_out) return fail(HK_EINVAL, "null argument");
  const int64_t heads = int64_t(L) * H;
  std::vector<double> imp;
  std::vector<int64_t> oa, ob, pos_a(heads), pos_b(heads);
  for (int s = 0; s < K; ++s) {
    rho_out[s] = std::nan("");
    if (s < n_sink || s > K - 2 || heads < 2) continue;
    ordering(scas_a, heads, K, s, imp, oa);
    ordering(scas_b, heads, K, s, imp, ob);
    for (int64_t i = 0; i < heads; ++i) {
      pos_a[oa[i]] = i;
      pos_b[ob[i]] = i;
    }
    // Spearman's rho of two permutations: 1 - 6 sum d^2 / (n (n^2 - 1)).
    double d2 = 0.0;
    for (int64_t f = 0; f < heads; ++f) {
      const double d = double(pos_a[f] - pos_b[f]);
      d2 += d * d;
    }
    const double n = double(heads);
    rho_out[s] = 1.0 - 6.0 * d2 / (n * (n * n - 1.0));
  }
  std::vector<uint8_t> ka(heads * K), kb(heads * K);
  rc = hk_build_schedule(L, H, K, scale_tokens, scas_a, budget_frac, n_sink, ka.data(), nullptr,
                         nullptr);
  if (rc != HK_OK) return rc;
  rc = hk_build_schedule(L, H, K, scale_tokens, scas_b, budget_frac, n_sink, kb.data(), nullptr,
                         nullptr);
  if (rc != HK_OK) return rc;
  int64_t inter = 0, uni = 0;
  for (int64_t f = 0; f < heads; ++f)
    for (int s = 0; s <= K - 2; ++s) {
      const bool pa = !ka[f * K + s], pb = !kb[f * K + s];
      inter += pa && pb;
      uni += pa || pb;
    }
  *jaccard_out = uni == 0 ? 1.0 : double(inter) / double(uni);
  return HK_OK;
}

extern "C" int hk_layout_expiry(int L, int H, int K, const int32_t* scale_tokens,
                                const uint8_t* expire, int B, int D, int64_t* cache_elems_out,
                                int64_t* cap_out, int64_t* base_out) {
  if (L < 1 || H < 1 || K < 1 || B < 1 || D < 1) return fail(HK_EINVAL, "sizes must be >= 1");
  if (!scale_tokens || !expire || !cache_elems_out) return fail(HK_EINVAL, "null argument");
  for (int s = 0; s < K; ++s)
    if (scale_tokens[s] < 1) return fail(HK_EINVAL, "scale %d has no tokens", s);
  const int64_t heads = int64_t(L) * H;
  const int64_t bad = hk::first_bad_expire(expire, heads, K);
  if (bad >= 0)
    return fail(HK_EINVAL, "expire[%lld] = %d outside [scale, K-1]", (long long)bad, int(expire[bad]));
  std::vector<int32_t> lenb;
  std::vector<int64_t> cap;
  hk::step_tables(expire, scale_tokens, heads, K, lenb, cap);
  int64_t offset = 0;
  for (int64_t f = 0; f < heads; ++f) {
    if (cap_out) cap_out[f] = cap[f];
    if (base_out) base_out[f] = offset;
    offset += cap[f] * B * D;
  }
  *cache_elems_out = offset;
  return HK_OK;
}

extern "C" int hk_layout_pooled(int L, int H, int K, const int32_t* scale_tokens,
                                const uint8_t* expire, int B, int D, int64_t* pool_elems_out,
                                int64_t* pool_rows_out, int32_t* seg_rows_out) {
  if (L < 1 || H < 1 || K < 1 || B < 1 || D < 1) return fail(HK_EINVAL, "sizes must be >= 1");
  if (!scale_tokens || !expire || !pool_elems_out) return fail(HK_EINVAL, "null argument");
  for (int s = 0; s < K; ++s)
    if (scale_tokens[s] < 1) return fail(HK_EINVAL, "scale %d has no tokens", s);
  const int64_t heads = int64_t(L) * H;
  const int64_t bad = hk::first_bad_expire(expire, heads, K);
  if (bad >= 0)
    return fail(HK_EINVAL, "expire[%lld] = %d outside [scale, K-1]", (long long)bad, int(expire[bad]));
  hk::PoolPlan p;
  hk::pool_plan(expire, scale_tokens, L, H, K, p);
  if (p.rows > INT32_MAX) return fail(HK_EINVAL, "pool exceeds 2^31 rows");
  *pool_elems_out = p.rows * B * D;
  if (pool_rows_out) *pool_rows_out = p.rows;
  if (seg_rows_out) {
    int64_t per_head = 0;
    for (int s = 0; s <= K - 2; ++s) per_head += scale_tokens[s];
    for (int64_t f = 0; f < heads; ++f) {
      int64_t off = f * per_head;
      for (int s = 0; s <= K - 2; ++s) {
        const int64_t first = p.seg_first[f * K + s];
        for (int i = 0; i < scale_tokens[s]; ++i) seg_rows_out[off + i] = first >= 0 ? p.rows_of[first + i] : -1;
        off += scale_tokens[s];
      }
    }
  }
  return HK_OK;
}

extern "C" int hk_layout_int4(int L, int H, int K, const int32_t* scale_tokens,
                              const uint8_t* keep, int B, int D, int sub_blocks,
                              int64_t* store_bytes_out, int64_t* param_offset_out) {
  if (L < 1 || H < 1 || K < 1 || B < 1) return fail(HK_EINVAL, "sizes must be >= 1");
  if (!scale_tokens || !keep || !store_bytes_out) return fail(HK_EINVAL, "null argument");
  if (D != 128) return fail(HK_EUNSUPPORTED, "4-bit storage needs head_dim 128 (got %d)", D);
  if (sub_blocks < 1 || sub_blocks > 64) return fail(HK_EINVAL, "sub_blocks must be in [1, 64]");
  for (int s = 0; s < K; ++s)
    if (scale_tokens[s] < 1) return fail(HK_EINVAL, "scale %d has no tokens", s);
  const int64_t heads = int64_t(L) * H;
  std::vector<uint8_t> expire, kept(heads * K);
  hk::expire_from_keep(keep, heads, K, expire);
  for (int64_t i = 0; i < heads * K; ++i) kept[i] = expire[i] == K - 1 && i % K <= K - 2;
  std::vector<int32_t> lenb, gcap;
  std::vector<int64_t> cap, code_base, param_base;
  hk::step_tables(expire.data(), scale_tokens, heads, K, lenb, cap);
  *store_bytes_out =
      hk::int4_layout(kept.data(), cap, heads, K, B, D, sub_blocks, code_base, param_base, gcap);
  if (param_offset_out) *param_offset_out = heads > 0 ? param_base[0] : 0;
  return HK_OK;
}

extern "C" int hk_layout(int L, int H, int K, const int32_t* scale_tokens, const uint8_t* keep,
                         int B, int D, int64_t* cache_elems_out, int64_t* cap_out,
                         int64_t* base_out) {
  if (L < 1 || H < 1 || K < 1 || B < 1 || D < 1) return fail(HK_EINVAL, "sizes must be >= 1");
  if (!scale_tokens || !keep || !cache_elems_out) return fail(HK_EINVAL, "null argument");
  std::vector<uint8_t> expire;
  hk::expire_from_keep(keep, int64_t(L) * H, K, expire);
  return hk_layout_expiry(L, H, K, scale_tokens, expire.data(), B, D, cache_elems_out, cap_out,
                          base_out);
}

extern "C" int hk_cache_size_after_layer(int L, int H, int K, const int32_t* scale_tokens,
                                         const uint8_t* expire, int step, int layer,
                                         int64_t* out) {
  if (L < 1 || H < 1 || K < 1) return fail(HK_EINVAL, "L, H, K must be >= 1");
  if (!scale_tokens || !expire || !out) return fail(HK_EINVAL, "null argument");
  if (step < 0 || step >= K) return fail(HK_EINVAL, "step %d out of [0, %d)", step, K);
  if (layer < 0 || layer >= L) return fail(HK_EINVAL, "layer %d out of [0, %d)", layer, L);
  const int64_t heads = int64_t(L) * H;
  const int64_t bad = hk::first_bad_expire(expire, heads, K);
  if (bad >= 0)
    return fail(HK_EINVAL, "expire[%lld] = %d outside [scale, K-1]", (long long)bad, int(expire[bad]));
  // Layers up to `layer` have finished the step; the later ones still hold
  // what they held at the end of the previous step.
  int64_t total = 0;
  for (int64_t f = 0; f < heads; ++f) {
    const bool done = f / H <= layer;
    if (done) total += hk::rows_at_end(expire + f * K, scale_tokens, K, step);
    else if (step > 0) total += hk::rows_at_end(expire + f * K, scale_tokens, K, step - 1);
  }
  *out = total;
  return HK_OK;
}

extern "C" int hk_build_progressive_schedule(int L, int H, int K, const int32_t* scale_tokens,
                                             const float* scas, double budget_frac, int n_sink,
                                             int per_layer, uint8_t* expire_out,
                                             int32_t* prefix_out, int64_t* live_out) {
  int rc = check_schedule_args(L, H, K, scale_tokens, scas, budget_frac, n_sink);
  if (rc != HK_OK) return rc;
  if (!expire_out) return fail(HK_EINVAL, "null argument");
  const int64_t heads = int64_t(L) * H;
  int64_t cached_tokens = 0;
  for (int s = 0; s <= K - 2; ++s) cached_tokens += scale_tokens[s];
  const int64_t budget = int64_t(std::floor(budget_frac * double(heads * cached_tokens)));

  // Orderings of the prunable scales n_sink..K-2.
  std::vector<std::vector<int64_t>> orders(K);
  {
    std::vector<double> imp;
    for (int s = n_sink; s <= K - 2; ++s) ordering(scas, heads, K, s, imp, orders[s]);
  }
  for (int64_t i = 0; i < heads * K; ++i) expire_out[i] = uint8_t(K - 1);
  std::vector<uint8_t> pruned(heads * K, 0);
  std::vector<int64_t> pending(L, 0), done(L, 0), sizes(L, 0);
  int64_t n = 0;
  for (int k = 0; k <= K - 2; ++k) {
    // Start of step k: every layer holds its end-of-(k-1) rows; the prefix of
    // O_k at the current length is pruned before segment k is ever stored.
    if (k >= n_sink)
      for (int64_t i = 0; i < n; ++i) pruned[orders[k][i] * K + k] = 1;
    for (int l = 0; l < L; ++l) {
      done[l] = pending[l];
      for (int h = 0; h < H; ++h)
        if (!pruned[(int64_t(l) * H + h) * K + k]) done[l] += scale_tokens[k];
    }
    for (;;) {
      // Size after layer l: layers 0..l finished, the rest still pending.
      int64_t total_pending = 0;
      for (int l = 0; l < L; ++l) total_pending += pending[l];
      int64_t run_done = 0, run_pending = total_pending, worst = 0;
      for (int l = 0; l < L; ++l) {
        run_done += done[l];
        run_pending -= pending[l];
        sizes[l] = run_done + run_pending;
        worst = std::max(worst, sizes[l]);
      }
      if ((per_layer ? worst : sizes[L - 1]) <= budget) break;
      if (n == heads)
        return fail(HK_EBUDGET, "budget of %lld token slots cannot hold scale %d",
                    (long long)budget, k);
      // Grow the prefix by one: the next head of every ordering i <= k.
      for (int i = n_sink; i <= k; ++i) {
        const int64_t f = orders[i][n];
        if (pruned[f * K + i]) continue;
        pruned[f * K + i] = 1;
        done[f / H] -= scale_tokens[i];
      }
      ++n;
    }
    for (int64_t f = 0; f < heads; ++f)
      for (int i = 0; i <= k; ++i)
        if (pruned[f * K + i] && expire_out[f * K + i] == K - 1) expire_out[f * K + i] = uint8_t(k);
    if (prefix_out) prefix_out[k] = int32_t(n);
    if (live_out)
      for (int l = 0; l < L; ++l) live_out[int64_t(k) * L + l] = sizes[l];
    pending = done;
  }
  if (K >= 2) {
    if (prefix_out) prefix_out[K - 1] = int32_t(n);
    if (live_out)
      for (int l = 0; l < L; ++l) live_out[int64_t(K - 1) * L + l] = sizes[L - 1];
  } else {
    if (prefix_out) prefix_out[0] = 0;
    if (live_out)
      for (int l = 0; l < L; ++l) live_out[l] = 0;
  }
  return HK_OK;
}

extern "C" int hk_build_scale_window_schedule(int L, int H, int K, const int32_t* scale_tokens,
                                              int n_condensed, int window, int window_demanding,
                                              const float* similarity, int n_demanding,
                                              uint8_t* expire_out) {
  if (L < 1 || H < 1 || K < 1) return fail(HK_EINVAL, "L, H, K must be >= 1");
  if (!scale_tokens || !expire_out) return fail(HK_EINVAL, "null argument");
  for (int s = 0; s < K; ++s)
    if (scale_tokens[s] < 1) return fail(HK_EINVAL, "scale %d has no tokens", s);
  if (n_condensed < 0 || n_condensed > K) return fail(HK_EINVAL, "n_condensed must be in [0, K]");
  if (window < 0 || window_demanding < 0) return fail(HK_EINVAL, "windows must be >= 0");
  if (n_demanding < 0 || n_demanding > L) return fail(HK_EINVAL, "n_demanding must be in [0, L]");
  if (n_demanding > 0 && !similarity)
    return fail(HK_EINVAL, "n_demanding > 0 needs a similarity score per layer");
  // Cache-demanding layers: the n_demanding lowest similarity scores, ties
  // by the lower layer index.
  std::vector<int> order(L);
  std::iota(order.begin(), order.end(), 0);
  std::vector<uint8_t> wide(L, 0);
  if (n_demanding > 0) {
    std::sort(order.begin(), order.end(), [&](int a, int b) {
      return similarity[a] < similarity[b] || (similarity[a] == similarity[b] && a < b);
    });
    for (int i = 0; i < n_demanding; ++i) wide[order[i]] = 1;
  }
  for (int l = 0; l < L; ++l) {
    const int64_t w = wide[l] ? window_demanding : window;
    for (int h = 0; h < H; ++h)
      for (int s = 0; s < K; ++s)
        expire_out[(int64_t(l) * H + h) * K + s] =
            uint8_t(s < n_condensed ? K - 1 : std::min<int64_t>(s + w, K - 1));
  }
  return HK_OK;
}
