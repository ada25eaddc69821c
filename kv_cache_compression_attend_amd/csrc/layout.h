// Host-side cache layout of a schedule given as expiry steps.
//
// expire[f][s] (f = l*H + h) is the step at whose end segment s of head f
// leaves the cache: the queries of scales t with s < t <= expire read it from
// the cache, expire == s means it is never stored, expire == K-1 means it
// stays to the end.  A static keep-mask is the case expire = K-1 (kept) or s
// (pruned).  Pruning sets that grow from scale to scale (Pith page of arXiv
// 2605.14877, Figure 4 caption: G_k is the union of prefixes of length N_k,
// absent by the end of scale k) give expiry steps between s and K-1: the
// segment is dropped from the middle of the head's cache at that step.
#pragma once

#include <algorithm>
#include <cstdint>
#include <vector>

namespace hk {

inline void expire_from_keep(const uint8_t* keep, int64_t heads, int K, std::vector<uint8_t>& out) {
  out.resize(heads * K);
  for (int64_t f = 0; f < heads; ++f)
    for (int s = 0; s < K; ++s)
      out[f * K + s] = uint8_t(keep[f * K + s] && s <= K - 2 ? K - 1 : s);
}

// Index of the first entry outside [s, K-1], or -1 when all are valid.
inline int64_t first_bad_expire(const uint8_t* expire, int64_t heads, int K) {
  for (int64_t f = 0; f < heads; ++f)
    for (int s = 0; s < K; ++s)
      if (expire[f * K + s] < s || expire[f * K + s] > K - 1) return f * K + s;
  return -1;
}

// Rows of head f (per batch entry) at the end of step k; nothing changes
// after step K-2 because the final scale is never cached.
inline int64_t rows_at_end(const uint8_t* exp_f, const int32_t* tokens, int K, int k) {
  const int kk = std::min(k, K - 2);
  int64_t rows = 0;
  for (int s = 0; s <= kk; ++s)
    if (exp_f[s] > kk) rows += tokens[s];
  return rows;
}

// lenb[(t*heads + f)*K + s]: first cache row of segment s while step t is
// attended (segments s < t that are still held, in scale order); entry t is
// the number of held rows, entry t+1 that plus n_t when segment t is stored
// (equal to the rows at the end of step t when nothing leaves at t), later
// entries repeat entry t+1.  cap[f] is the most rows head f holds at the end
// of any step: segments leaving at step t are gone before segment t is
// stored, so the two never occupy the cache together.
inline void step_tables(const uint8_t* expire, const int32_t* tokens, int64_t heads, int K,
                        std::vector<int32_t>& lenb, std::vector<int64_t>& cap) {
  lenb.assign(int64_t(K) * heads * K, 0);
  cap.assign(heads, 0);
  for (int t = 0; t < K; ++t)
    for (int64_t f = 0; f < heads; ++f) {
      const uint8_t* e = expire + f * K;
      int32_t* row = lenb.data() + (int64_t(t) * heads + f) * K;
      int64_t run = 0;
      for (int s = 0; s < K; ++s) {
        row[s] = int32_t(run);
        if (s < t && s <= K - 2 && e[s] >= t) run += tokens[s];
        if (s == t && t <= K - 2 && e[t] > t) run += tokens[t];
      }
      cap[f] = std::max<int64_t>(cap[f], rows_at_end(e, tokens, K, t));
    }
}

// Moves of step t for head f: the held segments that outlive step t, shifted
// down over the segments that expire at t.  Consecutive surviving segments
// with the same shift form one run (dst, src, rows), in ascending order.
struct MoveRun {
  int32_t dst, src, rows;
};

inline void step_moves(const uint8_t* exp_f, const int32_t* tokens, int K, int t,
                       std::vector<MoveRun>& runs) {
  runs.clear();
  if (t > K - 2) return;
  int32_t src = 0, dst = 0;
  for (int s = 0; s < t; ++s) {
    if (s > K - 2 || exp_f[s] < t) continue;  // not held at step t
    const int32_t n = tokens[s];
    if (exp_f[s] > t) {
      if (dst != src) {
        if (!runs.empty() && runs.back().src + runs.back().rows == src &&
            runs.back().dst + runs.back().rows == dst)
          runs.back().rows += n;
        else
          runs.push_back(MoveRun{dst, src, n});
      }
      dst += n;
    }
    src += n;
  }
}

// 4-bit storage of a static keep-mask (one buffer each for K and V, bytes):
// codes of head f at code_base[f], [B][cap[f]][D/2]; then, from
// param_offset (256-byte aligned), the group parameters of head f at
// param_base[f], [B][gcap[f]][D] float2 (step, lo), gcap[f] = m * (number of
// stored segments), segment s's m groups following those of the stored
// segments before it.
inline int64_t int4_layout(const uint8_t* keep, const std::vector<int64_t>& cap, int64_t heads,
                           int K, int B, int D, int m, std::vector<int64_t>& code_base,
                           std::vector<int64_t>& param_base, std::vector<int32_t>& gcap) {
  code_base.assign(heads, 0);
  param_base.assign(heads, 0);
  gcap.assign(heads, 0);
  int64_t off = 0;
  for (int64_t f = 0; f < heads; ++f) {
    code_base[f] = off;
    off += int64_t(B) * cap[f] * (D / 2);
    int stored = 0;
    for (int s = 0; s <= K - 2; ++s) stored += keep[f * K + s] ? 1 : 0;
    gcap[f] = m * stored;
  }
  const int64_t param_offset = (off + 255) / 256 * 256;
  off = param_offset;
  for (int64_t f = 0; f < heads; ++f) {
    param_base[f] = off;
    off += int64_t(B) * gcap[f] * D * 8;
  }
  return off;
}

// One pool of rows shared by every head (per batch entry and per K or V
// buffer), for schedules whose segments leave the cache after they were
// stored: rows freed by a dropped segment are reused by later segments, so
// nothing ever moves and the pool holds exactly the most token slots the
// cache holds at once.  Events are taken in generation order -- for each
// scale k, for each layer l: the queries of (l, k) read the cache, then the
// segments of layer l that expire at k give back their rows and the stored
// segments (l, h, k) take rows -- the order of the per-layer accounting of
// Algorithm 2 (Pith page of arXiv 2605.14877, Appendix A).  Rows are taken
// lowest first, so a segment is one run of consecutive rows unless it fills
// holes.
struct PoolPlan {
  int64_t rows = 0;                // pool rows per batch entry
  std::vector<int64_t> seg_first;  // [heads][K]: first entry in rows_of, -1 if not stored
  std::vector<int32_t> rows_of;    // pool rows of the stored segments, in event order
};

inline void pool_plan(const uint8_t* expire, const int32_t* tokens, int L, int H, int K,
                      PoolPlan& p) {
  const int64_t heads = int64_t(L) * H;
  p.rows = 0;
  p.seg_first.assign(heads * K, -1);
  p.rows_of.clear();
  std::vector<std::pair<int64_t, int64_t>> free_runs;  // (start, length), sorted by start
  auto give_back = [&](int64_t first, int n) {
    // the segment's rows as runs of consecutive rows
    int i = 0;
    while (i < n) {
      int j = i + 1;
      while (j < n && p.rows_of[first + j] == p.rows_of[first + j - 1] + 1) ++j;
      const int64_t a = p.rows_of[first + i], len = j - i;
      auto it = std::lower_bound(free_runs.begin(), free_runs.end(), std::make_pair(a, int64_t(0)));
      it = free_runs.insert(it, {a, len});
      // merge with the next and the previous run
      if (it + 1 != free_runs.end() && it->first + it->second == (it + 1)->first) {
        it->second += (it + 1)->second;
        free_runs.erase(it + 1);
      }
      if (it != free_runs.begin() && (it - 1)->first + (it - 1)->second == it->first) {
        (it - 1)->second += it->second;
        free_runs.erase(it);
      }
      i = j;
    }
  };
  auto take = [&](int n) {
    const int64_t first = int64_t(p.rows_of.size());
    while (n > 0 && !free_runs.empty()) {
      auto& r = free_runs.front();
      const int64_t m = std::min<int64_t>(n, r.second);
      for (int64_t q = 0; q < m; ++q) p.rows_of.push_back(int32_t(r.first + q));
      r.first += m;
      r.second -= m;
      n -= int(m);
      if (r.second == 0) free_runs.erase(free_runs.begin());
    }
    for (; n > 0; --n) p.rows_of.push_back(int32_t(p.rows++));
    return first;
  };
  for (int k = 0; k < K; ++k)
    for (int l = 0; l < L; ++l) {
      for (int h = 0; h < H; ++h) {
        const int64_t f = int64_t(l) * H + h;
        for (int s = 0; s < k && s <= K - 2; ++s)
          if (expire[f * K + s] == k && p.seg_first[f * K + s] >= 0)
            give_back(p.seg_first[f * K + s], tokens[s]);
      }
      if (k > K - 2) continue;
      for (int h = 0; h < H; ++h) {
        const int64_t f = int64_t(l) * H + h;
        if (expire[f * K + k] > k) p.seg_first[f * K + k] = take(tokens[k]);
      }
    }
}

}  // namespace hk
