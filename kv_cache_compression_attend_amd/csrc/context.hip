// Context and per-scale entry points of the C ABI: argument checks, the
// per-layer scale-order state, the small device tables and the kernel
// launches.  Every entry point returns a status code and records text for
// hk_last_error(); nothing here aborts.
#include <math.h>

#include <algorithm>
#include <cstdint>
#include <vector>

#include "../../include/heatkv.h"
#include "device.h"
#include "layout.h"
#include "status.h"

struct hk_ctx {
  int L, H, D, B, K, dtype, device;
  int elem_bytes;
  std::vector<int32_t> tokens;
  std::vector<uint8_t> expire;    // [L][H][K] step at whose end a segment leaves
  std::vector<int64_t> cap;       // [L][H]
  std::vector<int64_t> base;      // [L][H] element offsets
  std::vector<int32_t> lenb;      // [K][L][H][K] segment start rows while step t is attended
  std::vector<int64_t> retained;  // [K]
  // Compaction descriptors: for scale t, the (l, h) that store segment t,
  // sorted by l; the ones of layer l are desc_first[t*(L+1)+l] ..
  // desc_first[t*(L+1)+l+1].
  std::vector<int64_t> desc_first;
  // Gather descriptors (heads whose held segments move at step t), indexed
  // the same way, and whether any head of layer l drops a held segment at
  // step t ([K][L]); a dropped tail segment moves nothing but still changes
  // where segment t is stored.
  std::vector<int64_t> gdesc_first;
  std::vector<uint8_t> drops;
  void* kcache;
  void* vcache;
  int64_t* d_base = nullptr;
  int32_t* d_cap = nullptr;
  int32_t* d_lenb = nullptr;
  // Heads of each (step, layer) heaviest first ([K][L][H]) and whether the
  // bf16 attend launch of (step, layer) uses that order ([K][L]): only when
  // its heads hold different numbers of keys and B is a multiple of the die
  // count.
  std::vector<int32_t> order;
  std::vector<uint8_t> ordered;
  int32_t* d_order = nullptr;
  hk::CopyDesc* d_desc = nullptr;
  hk::GatherDesc* d_gdesc = nullptr;
  hk::GatherRun* d_gruns = nullptr;
  int64_t* d_rowdst = nullptr;    // [K][L][H] byte offset where (l, h) stores scale t, or -1
  float* d_partials = nullptr;
  std::vector<int> rows;          // [K] query rows per workgroup of each scale's attend launch
  std::vector<int> splits;        // [K] key-range splits of each scale's attend launch
  std::vector<int> rows_scas;     // [K] query rows per workgroup with S-CAS (never split)
  float* d_ws_o = nullptr;        // split workspace: unnormalised outputs
  float2* d_ws_ml = nullptr;      // split workspace: (max, denominator)
  std::vector<int> appended;      // last scale appended per layer (-1: none)
  std::vector<int> attended;      // last scale attended per layer (-1: none)
  // 4-bit storage (quant_m > 0 sub-blocks per segment): kstore/vstore are the
  // caller's code + parameter buffers; kcache/vcache then point at the
  // context's bf16 scratch for one layer, which base[] indexes per layer.
  int quant_m = 0;
  void* kstore = nullptr;
  void* vstore = nullptr;
  std::vector<int64_t> qdesc_first;   // [K][L+1] quantize descriptors of (t, l)
  std::vector<int64_t> uitem_first;   // [L] unpack items of layer l (sorted by scale)
  std::vector<int64_t> uitem_count;   // [K][L] items attend(l, t) unpacks (a prefix)
  hk::QuantDesc* d_qdesc = nullptr;
  hk::UnpackItem* d_uitems = nullptr;
  float2* d_qminmax = nullptr;        // split-quantizer workspace
  int64_t qminmax_slots = 0;          // its capacity in (desc, sub-block, chunk, b) slots
  // Pooled cache: every head's rows in one pool of pool_rows rows per batch
  // entry; d_map holds, per (step, layer, head), the pool row of each row the
  // head holds while the step is attended (offsets d_mapoff [K][L][H]);
  // pdesc_first[t*(L+1)+l] indexes the stored segments of (t, l) in d_pdesc.
  bool pooled = false;
  int64_t pool_rows = 0;
  int32_t* d_map = nullptr;
  int64_t* d_mapoff = nullptr;
  int32_t* d_poolrows = nullptr;
  hk::PoolDesc* d_pdesc = nullptr;
  std::vector<int64_t> pdesc_first;
};

namespace {

using hk::fail;

// Makes the context's device current for the duration of a call.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_fail(hipError_t e, const char* what) {
  return fail(HK_EHIP, "%s: %s", what, hipGetErrorString(e));
}

void free_tables(hk_ctx* c) {
  (void)hipFree(c->d_base);
  (void)hipFree(c->d_cap);
  (void)hipFree(c->d_lenb);
  (void)hipFree(c->d_order);
  c->d_order = nullptr;
  (void)hipFree(c->d_desc);
  (void)hipFree(c->d_gdesc);
  (void)hipFree(c->d_gruns);
  (void)hipFree(c->d_rowdst);
  c->d_rowdst = nullptr;
  (void)hipFree(c->d_qdesc);
  (void)hipFree(c->d_uitems);
  (void)hipFree(c->d_qminmax);
  c->d_qminmax = nullptr;
  if (c->quant_m > 0) {
    (void)hipFree(c->kcache);
    (void)hipFree(c->vcache);
    c->kcache = nullptr;
    c->vcache = nullptr;
  }
  (void)hipFree(c->d_map);
  (void)hipFree(c->d_mapoff);
  (void)hipFree(c->d_poolrows);
  (void)hipFree(c->d_pdesc);
  c->d_map = nullptr;
  c->d_mapoff = nullptr;
  c->d_poolrows = nullptr;
  c->d_pdesc = nullptr;
  (void)hipFree(c->d_partials);
  (void)hipFree(c->d_ws_o);
  (void)hipFree(c->d_ws_ml);
  c->d_ws_o = nullptr;
  c->d_ws_ml = nullptr;
  c->d_base = nullptr;
  c->d_cap = nullptr;
  c->d_lenb = nullptr;
  c->d_desc = nullptr;
  c->d_gdesc = nullptr;
  c->d_gruns = nullptr;
  c->d_qdesc = nullptr;
  c->d_uitems = nullptr;
  c->d_partials = nullptr;
}

template <typename T>
hipError_t upload(T** dst, const std::vector<T>& src) {
  const size_t bytes = std::max<size_t>(src.size(), 1) * sizeof(T);
  hipError_t e = hipMalloc(reinterpret_cast<void**>(dst), bytes);
  if (e != hipSuccess) return e;
  if (src.empty()) return hipSuccess;
  return hipMemcpy(*dst, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice);
}

// Chunks of kQuantChunkRows rows covering the largest of m sub-blocks of n rows.
int quant_chunks(int n, int m) {
  const int rows = (n + m - 1) / m;
  return std::max(1, (rows + hk::kQuantChunkRows - 1) / hk::kQuantChunkRows);
}

int check_step_args(const hk_ctx* c, int layer, int step) {
  if (!c) return fail(HK_EINVAL, "null context");
  if (layer < 0 || layer >= c->L) return fail(HK_EINVAL, "layer %d out of [0, %d)", layer, c->L);
  if (step < 0 || step >= c->K) return fail(HK_EINVAL, "step %d out of [0, %d)", step, c->K);
  return HK_OK;
}

int append_launch(hk_ctx* c, int layer_begin, int layer_end, int step, const void* k_cur,
                  const void* v_cur, int64_t layer_stride_elems, void* hip_stream);

// A pooled cache gives the rows of segments dropped at step-1 and earlier
// (by any layer), and at this step by the layers before this one, to the
// segment appended here; their readers must be done: every layer has
// appended step-1 (so it has attended it) and the layers before this one
// have appended this step.
int pool_append_order(const hk_ctx* c, int layer, int step) {
  if (!c->pooled) return HK_OK;
  for (int l = 0; l < c->L; ++l)
    if (c->appended[l] < (l < layer ? step : step - 1))
      return fail(HK_EORDER, "append(layer %d, step %d) on a pooled cache before layer %d has "
                  "appended step %d", layer, step, l, l < layer ? step : step - 1);
  return HK_OK;
}

int attend_common(hk_ctx* c, int layer, int step, const void* q, const void* k_cur,
                  const void* v_cur, void* out, float softmax_scale, float* scas_table,
                  bool scas, bool append, void* hip_stream, double* scas_sum = nullptr) {
  int rc = check_step_args(c, layer, step);
  if (rc != HK_OK) return rc;
  if (!q || !k_cur || !v_cur || !out) return fail(HK_EINVAL, "null tensor pointer");
  if (scas && !scas_table && !scas_sum) return fail(HK_EINVAL, "null S-CAS table");
  if (!aligned16(q) || !aligned16(k_cur) || !aligned16(v_cur) || !aligned16(out))
    return fail(HK_EINVAL, "tensor pointers must be 16-byte aligned");
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale))
    return fail(HK_EINVAL, "softmax_scale must be positive and finite");
  if (step > 0 && c->appended[layer] < step - 1)
    return fail(HK_EORDER, "attend(layer %d, step %d) needs scale %d appended first (last: %d)",
                layer, step, step - 1, c->appended[layer]);
  // A pooled cache reuses the rows of dropped segments, so a step is attended
  // only before its own append (its rows may be reused afterwards).
  if (c->pooled && c->appended[layer] != step - 1)
    return fail(HK_EORDER, "attend(layer %d, step %d) on a pooled cache after its append (last "
                "appended: %d)", layer, step, c->appended[layer]);
  // Segments that leave the cache at a step are overwritten by that step's
  // append (the gather moves the survivors down): once the append of any
  // step u >= step that drops segments has run, this step's layout is gone.
  const bool drops = c->drops[int64_t(step) * c->L + layer] != 0;
  for (int u = step; u <= c->appended[layer]; ++u)
    if (c->drops[int64_t(u) * c->L + layer])
      return fail(HK_EORDER, "attend(layer %d, step %d) after the append of step %d, which moved "
                  "the segments this step reads", layer, step, u);
  // Appending this scale as well needs the layer's cache to end at scale step-1.
  append = append && step <= c->K - 2;
  if (append && c->appended[layer] != step - 1)
    return fail(HK_EORDER, "append(layer %d, step %d) out of order (last appended: %d)", layer,
                step, c->appended[layer]);
  if (append) {
    rc = pool_append_order(c, layer, step);
    if (rc != HK_OK) return rc;
  }

  DeviceGuard g(c->device);
  if (!g.ok) return fail(HK_EHIP, "cannot select device %d", c->device);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);

  hk::AttendArgs a{};
  a.q = q;
  a.kcur = k_cur;
  a.vcur = v_cur;
  a.out = out;
  a.kcache = c->kcache;
  a.vcache = c->vcache;
  a.base = c->d_base + int64_t(layer) * c->H;
  a.cap = c->d_cap + int64_t(layer) * c->H;
  a.lenb = c->d_lenb + (int64_t(step) * c->L + layer) * c->H * c->K;
  a.order = c->ordered[int64_t(step) * c->L + layer] ? c->d_order + (int64_t(step) * c->L + layer) * c->H
                                                      : nullptr;
  a.partials = c->d_partials;
  if (c->pooled) {
    a.map = c->d_map;
    a.mapoff = c->d_mapoff + (int64_t(step) * c->L + layer) * c->H;
  }
  a.ws_o = c->d_ws_o;
  a.ws_ml = c->d_ws_ml;
  a.rows = scas ? c->rows_scas[step] : c->rows[step];
  a.n_split = scas ? 1 : c->splits[step];
  a.B = c->B;
  a.H = c->H;
  a.n = c->tokens[step];
  a.K = c->K;
  a.step = step;
  a.n_qtiles = (a.n + a.rows - 1) / a.rows;
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  // bf16 kernels append in the same launch, unless segments leave at this
  // step (segment t is then stored where the attention still reads, after
  // the survivors); otherwise the gather and compaction kernels run after the
  // attention kernel.
  const bool fused = append && c->dtype == HK_DTYPE_BF16 && !drops && c->quant_m == 0 && !c->pooled;
  a.append = fused;

  hipError_t e = hipSuccess;
  if (c->quant_m > 0) {
    // 4-bit storage: unpack the layer's held rows into the bf16 scratch the
    // attend kernel reads; the scale itself is quantized by the append.
    a.append = 0;
    hk::UnpackArgs u{};
    u.items = c->d_uitems + c->uitem_first[layer];
    u.n_items = int(c->uitem_count[int64_t(step) * c->L + layer]);
    u.kstore = static_cast<const uint8_t*>(c->kstore);
    u.vstore = static_cast<const uint8_t*>(c->vstore);
    u.kscratch = static_cast<uint16_t*>(c->kcache);
    u.vscratch = static_cast<uint16_t*>(c->vcache);
    u.B = c->B;
    e = hk::launch_unpack(u, s);
    if (e != hipSuccess) return hip_fail(e, "unpack launch");
  }
  e = c->dtype == HK_DTYPE_BF16 ? hk::launch_attend_bf16_d128(a, scas, s)
                                : hk::launch_attend_f32(a, c->D, scas, s);
  if (e != hipSuccess) return hip_fail(e, "attend launch");
  c->attended[layer] = step;
  if (scas) {
    e = scas_sum ? hk::launch_scas_accumulate(c->d_partials, scas_sum, layer, c->H, c->K, c->B,
                                              a.n, step, a.n_qtiles, s)
                 : hk::launch_scas_finalize(c->d_partials, scas_table, layer, c->H, c->K, c->B,
                                            a.n, step, a.n_qtiles, s);
    if (e != hipSuccess) return hip_fail(e, "S-CAS finalize launch");
  }
  if (append) {
    if (fused) {
      c->appended[layer] = step;
    } else {
      rc = append_launch(c, layer, layer + 1, step, k_cur, v_cur, 0, hip_stream);
      if (rc != HK_OK) return rc;
    }
  }
  return HK_OK;
}

}  // namespace

namespace {

// Builds a context for an expiry-step schedule.  quant_m > 0: 4-bit storage
// in k_cache / v_cache (a static schedule, bf16 head_dim 128).
int create_impl(hk_ctx** out, int L, int H, int D, int B, int K, const int32_t* scale_tokens,
                const uint8_t* expire, int dtype, void* k_cache, void* v_cache, int quant_m,
                bool pooled = false) {
  if (!out) return fail(HK_EINVAL, "null output pointer");
  *out = nullptr;
  if (L < 1 || H < 1 || B < 1 || K < 1) return fail(HK_EINVAL, "L, H, B, K must be >= 1");
  if (K > HK_MAX_SCALES) return fail(HK_EUNSUPPORTED, "K = %d exceeds %d scales", K, HK_MAX_SCALES);
  if (!scale_tokens || !expire) return fail(HK_EINVAL, "null scale_tokens or schedule");
  if (dtype == HK_DTYPE_BF16) {
    if (D != 128) return fail(HK_EUNSUPPORTED, "bf16 needs head_dim 128 (got %d)", D);
  } else if (dtype == HK_DTYPE_F32) {
    if (D != 16 && D != 32 && D != 64 && D != 128)
      return fail(HK_EUNSUPPORTED, "f32 needs head_dim 16, 32, 64 or 128 (got %d)", D);
  } else {
    return fail(HK_EUNSUPPORTED, "unknown dtype %d", dtype);
  }
  for (int s = 0; s < K; ++s)
    if (scale_tokens[s] < 1) return fail(HK_EINVAL, "scale %d has no tokens", s);
  const int64_t heads = int64_t(L) * H;
  const int64_t bad = hk::first_bad_expire(expire, heads, K);
  if (bad >= 0)
    return fail(HK_EINVAL, "expire[%lld] = %d outside [scale, K-1]", (long long)bad, int(expire[bad]));

  if (pooled && (dtype != HK_DTYPE_BF16 || D != 128 || quant_m > 0))
    return fail(HK_EUNSUPPORTED, "pooled caches take bf16 tensors with head_dim 128");

  auto* c = new hk_ctx();
  c->L = L; c->H = H; c->D = D; c->B = B; c->K = K; c->dtype = dtype;
  c->pooled = pooled;
  c->elem_bytes = dtype == HK_DTYPE_BF16 ? 2 : 4;
  c->tokens.assign(scale_tokens, scale_tokens + K);
  c->expire.assign(expire, expire + heads * K);
  c->kcache = k_cache;
  c->vcache = v_cache;
  c->appended.assign(L, -1);
  c->attended.assign(L, -1);

  hk::step_tables(expire, scale_tokens, heads, K, c->lenb, c->cap);
  c->base.assign(heads, 0);
  int64_t offset = 0, scratch_elems = 0;
  for (int64_t f = 0; f < heads; ++f) {
    if (c->cap[f] > INT32_MAX) { delete c; return fail(HK_EINVAL, "head cache exceeds 2^31 rows"); }
    // 4-bit storage: base[] indexes the one-layer bf16 scratch, so it
    // restarts with every layer.
    if (quant_m > 0 && f % H == 0) offset = 0;
    c->base[f] = offset;
    offset += c->cap[f] * B * D;
    scratch_elems = std::max(scratch_elems, offset);
  }
  hk::PoolPlan plan;
  if (pooled) {
    // One pool per batch entry shared by every head (base 0, cap = pool rows).
    hk::pool_plan(expire, scale_tokens, L, H, K, plan);
    if (plan.rows * D * c->elem_bytes > INT32_MAX) {
      delete c;
      return fail(HK_EINVAL, "pool of %lld rows exceeds 2^31 bytes per batch entry",
                  (long long)plan.rows);
    }
    c->pool_rows = plan.rows;
    for (int64_t f = 0; f < heads; ++f) {
      c->base[f] = 0;
      c->cap[f] = plan.rows;
    }
    offset = plan.rows * B * D;
  }
  const int64_t cache_bytes = quant_m > 0 ? 0 : offset * c->elem_bytes;
  std::vector<int64_t> code_base, param_base;
  std::vector<int32_t> gcap;
  std::vector<uint8_t> keep(heads * K);
  for (int64_t i = 0; i < heads * K; ++i) keep[i] = expire[i] == K - 1 && i % K <= K - 2;
  const int64_t store_bytes =
      quant_m > 0 ? hk::int4_layout(keep.data(), c->cap, heads, K, B, D, quant_m, code_base,
                                    param_base, gcap)
                  : cache_bytes;
  if (store_bytes > 0 && (!k_cache || !v_cache)) {
    delete c;
    return fail(HK_EINVAL, "null cache buffer");
  }
  if (!aligned16(k_cache) || !aligned16(v_cache)) {
    delete c;
    return fail(HK_EINVAL, "cache buffers must be 16-byte aligned");
  }
  if (quant_m > 0) {
    c->quant_m = quant_m;
    c->kstore = k_cache;
    c->vstore = v_cache;
    c->kcache = nullptr;
    c->vcache = nullptr;
  }
  auto lenb_at = [&](int t, int64_t f, int s) { return c->lenb[(int64_t(t) * heads + f) * K + s]; };

  c->retained.assign(K, 0);
  for (int k = 0; k < K; ++k)
    for (int64_t f = 0; f < heads; ++f)
      c->retained[k] += hk::rows_at_end(expire + f * K, scale_tokens, K, k);

  // Per step: the heads that store segment t (at its row once the segments
  // expiring at t are gone) and the heads whose held segments move.
  std::vector<hk::CopyDesc> desc;
  std::vector<int64_t> rowdst(int64_t(K) * heads, -1);
  std::vector<hk::GatherDesc> gdesc;
  std::vector<hk::GatherRun> gruns;
  std::vector<hk::MoveRun> runs;
  c->desc_first.assign(int64_t(K) * (L + 1), 0);
  c->gdesc_first.assign(int64_t(K) * (L + 1), 0);
  c->drops.assign(int64_t(K) * L, 0);
  for (int t = 0; t < K; ++t) {
    for (int l = 0; l < L; ++l) {
      c->desc_first[int64_t(t) * (L + 1) + l] = int64_t(desc.size());
      c->gdesc_first[int64_t(t) * (L + 1) + l] = int64_t(gdesc.size());
      if (t > K - 2 || quant_m > 0) continue;
      if (pooled) {
        for (int h = 0; h < H; ++h) {
          const int64_t f = int64_t(l) * H + h;
          for (int sd = 0; sd < t; ++sd)
            if (expire[f * K + sd] == t) c->drops[int64_t(t) * L + l] = 1;
        }
        continue;
      }
      for (int h = 0; h < H; ++h) {
        const int64_t f = int64_t(l) * H + h;
        for (int sd = 0; sd < t; ++sd)
          if (expire[f * K + sd] == t) c->drops[int64_t(t) * L + l] = 1;
        hk::step_moves(expire + f * K, scale_tokens, K, t, runs);
        if (!runs.empty()) {
          hk::GatherDesc g{};
          g.base = c->base[f] * c->elem_bytes;
          g.cap = int32_t(c->cap[f]);
          g.run_first = int32_t(gruns.size());
          g.n_runs = int32_t(runs.size());
          g.dst_begin = runs.front().dst;
          g.dst_end = runs.back().dst + runs.back().rows;
          for (const auto& r : runs) gruns.push_back(hk::GatherRun{r.dst, r.src, r.rows});
          gdesc.push_back(g);
        }
        if (expire[f * K + t] <= t) continue;
        hk::CopyDesc d{};
        d.dst = (c->base[f] + int64_t(lenb_at(t + 1, f, t)) * D) * c->elem_bytes;
        rowdst[int64_t(t) * heads + f] = d.dst;
        d.cap = int32_t(c->cap[f]);
        d.head = h;
        d.layer = l;
        desc.push_back(d);
      }
    }
    c->desc_first[int64_t(t) * (L + 1) + L] = int64_t(desc.size());
    c->gdesc_first[int64_t(t) * (L + 1) + L] = int64_t(gdesc.size());
  }

  // Pooled cache: the map of every (step, layer, head) -- the pool rows of
  // the segments the head holds while the step is attended, in scale order
  // -- and one descriptor per stored segment.
  std::vector<int32_t> map;
  std::vector<int64_t> mapoff;
  std::vector<hk::PoolDesc> pdesc;
  c->pdesc_first.assign(int64_t(K) * (L + 1), 0);
  if (pooled) {
    mapoff.assign(int64_t(K) * heads, 0);
    for (int t = 0; t < K; ++t) {
      for (int64_t f = 0; f < heads; ++f) {
        mapoff[int64_t(t) * heads + f] = int64_t(map.size());
        for (int sd = 0; sd < t && sd <= K - 2; ++sd) {
          const int64_t first = plan.seg_first[f * K + sd];
          if (first < 0 || expire[f * K + sd] < t) continue;
          map.insert(map.end(), plan.rows_of.begin() + first,
                     plan.rows_of.begin() + first + scale_tokens[sd]);
        }
      }
      for (int l = 0; l < L; ++l) {
        c->pdesc_first[int64_t(t) * (L + 1) + l] = int64_t(pdesc.size());
        if (t > K - 2) continue;
        for (int h = 0; h < H; ++h) {
          const int64_t f = int64_t(l) * H + h;
          if (plan.seg_first[f * K + t] >= 0)
            pdesc.push_back(hk::PoolDesc{plan.seg_first[f * K + t], h, l});
        }
      }
      c->pdesc_first[int64_t(t) * (L + 1) + L] = int64_t(pdesc.size());
    }
  }

  // 4-bit storage: one quantize descriptor per stored (t, l, h); unpack
  // items per layer in scale order (chunks of at most kUnpackRows rows of
  // one sub-block group), so attend(l, t) unpacks a prefix of layer l's list.
  std::vector<hk::QuantDesc> qdesc;
  std::vector<hk::UnpackItem> uitems;
  c->qdesc_first.assign(int64_t(K) * (L + 1), 0);
  c->uitem_first.assign(L + 1, 0);
  c->uitem_count.assign(int64_t(K) * L, 0);
  if (quant_m > 0) {
    for (int t = 0; t < K; ++t) {
      for (int l = 0; l < L; ++l) {
        c->qdesc_first[int64_t(t) * (L + 1) + l] = int64_t(qdesc.size());
        if (t > K - 2) continue;
        for (int h = 0; h < H; ++h) {
          const int64_t f = int64_t(l) * H + h;
          if (!keep[f * K + t]) continue;
          int before = 0;
          for (int s2 = 0; s2 < t; ++s2) before += keep[f * K + s2];
          hk::QuantDesc q{};
          q.code_off = code_base[f] + int64_t(lenb_at(t + 1, f, t)) * hk::kQuantRowBytes;
          q.param_off = param_base[f] + int64_t(quant_m) * before * D * int64_t(sizeof(float2));
          q.cap = int32_t(c->cap[f]);
          q.gcap = gcap[f];
          q.head = h;
          q.layer = l;
          qdesc.push_back(q);
        }
      }
      c->qdesc_first[int64_t(t) * (L + 1) + L] = int64_t(qdesc.size());
    }
    for (int l = 0; l < L; ++l) {
      c->uitem_first[l] = int64_t(uitems.size());
      for (int s2 = 0; s2 <= K - 2; ++s2) {
        // Steps t > s2 read segment s2: every later step's prefix includes it.
        for (int h = 0; h < H; ++h) {
          const int64_t f = int64_t(l) * H + h;
          if (!keep[f * K + s2]) continue;
          int before = 0;
          for (int s3 = 0; s3 < s2; ++s3) before += keep[f * K + s3];
          const int n = scale_tokens[s2];
          const int row0 = lenb_at(K - 1, f, s2);
          for (int j = 0; j < quant_m; ++j) {
            const int a = int(int64_t(j) * n / quant_m), b = int(int64_t(j + 1) * n / quant_m);
            for (int r = a; r < b; r += hk::kUnpackRows) {
              hk::UnpackItem u{};
              u.code_off = code_base[f] + int64_t(row0 + r) * hk::kQuantRowBytes;
              u.param_off = param_base[f] +
                            (int64_t(quant_m) * before + j) * D * int64_t(sizeof(float2));
              u.scratch_off = c->base[f] + int64_t(row0 + r) * D;
              u.rows = std::min(hk::kUnpackRows, b - r);
              u.cap = int32_t(c->cap[f]);
              u.gcap = gcap[f];
              uitems.push_back(u);
            }
          }
        }
        for (int t = s2 + 1; t < K; ++t)
          c->uitem_count[int64_t(t) * L + l] = int64_t(uitems.size()) - c->uitem_first[l];
      }
    }
    c->uitem_first[L] = int64_t(uitems.size());
    for (int t = 0; t <= K - 2; ++t) {
      const int64_t nd = c->qdesc_first[int64_t(t) * (L + 1) + L] - c->qdesc_first[int64_t(t) * (L + 1)];
      c->qminmax_slots = std::max<int64_t>(
          c->qminmax_slots, nd * quant_m * quant_chunks(scale_tokens[t], quant_m) * B);
    }
  }

  // Attend plans per scale: query rows per workgroup and key-range splits
  // (bf16 launches without S-CAS may split the keys of a launch that would
  // not fill the chip), the S-CAS partial rows and the split workspace the
  // largest launch needs.  fp32 launches take 64 query rows, unsplit.
  c->rows.assign(K, 64);
  c->rows_scas.assign(K, 64);
  c->splits.assign(K, 1);
  int64_t max_partials = 1;
  int64_t ws_rows = 0;
  for (int t = 0; t < K; ++t) {
    if (dtype == HK_DTYPE_BF16) {
      int max_keys = 0;
      for (int64_t f = 0; f < heads; ++f)
        max_keys = std::max<int>(max_keys, lenb_at(t, f, t) + scale_tokens[t]);
      const hk::AttendPlan p = hk::attend_bf16_plan(B, H, scale_tokens[t], max_keys, true);
      c->rows[t] = p.rows;
      c->splits[t] = p.splits;
      c->rows_scas[t] = hk::attend_bf16_plan(B, H, scale_tokens[t], max_keys, false).rows;
      if (p.splits > 1)
        ws_rows = std::max<int64_t>(ws_rows, int64_t(p.splits) * B * scale_tokens[t] * H);
    }
    const int64_t qt = (scale_tokens[t] + c->rows_scas[t] - 1) / c->rows_scas[t];
    max_partials = std::max<int64_t>(max_partials, int64_t(B) * H * qt);
  }

  // Dispatch order of each (step, layer): heads by keys held, most first
  // (ties by index).
  c->order.assign(int64_t(K) * heads, 0);
  c->ordered.assign(int64_t(K) * L, 0);
  for (int t = 0; t < K; ++t)
    for (int l = 0; l < L; ++l) {
      int32_t* ord = c->order.data() + (int64_t(t) * L + l) * H;
      auto keys = [&](int h) { return lenb_at(t, int64_t(l) * H + h, t); };
      for (int h = 0; h < H; ++h) ord[h] = h;
      std::stable_sort(ord, ord + H, [&](int x, int y) { return keys(x) > keys(y); });
      c->ordered[int64_t(t) * L + l] =
          dtype == HK_DTYPE_BF16 && B % hk::kXcds == 0 && keys(ord[0]) != keys(ord[H - 1]);
    }

  hipError_t e = hipGetDevice(&c->device);
  if (e == hipSuccess) e = upload(&c->d_base, c->base);
  if (e == hipSuccess) e = upload(&c->d_order, c->order);
  std::vector<int32_t> cap32(c->cap.begin(), c->cap.end());
  if (e == hipSuccess) e = upload(&c->d_cap, cap32);
  if (e == hipSuccess) e = upload(&c->d_lenb, c->lenb);
  if (e == hipSuccess) e = upload(&c->d_desc, desc);
  if (e == hipSuccess) e = upload(&c->d_gdesc, gdesc);
  if (e == hipSuccess && quant_m == 0) e = upload(&c->d_rowdst, rowdst);
  if (e == hipSuccess) e = upload(&c->d_gruns, gruns);
  if (e == hipSuccess) e = upload(&c->d_qdesc, qdesc);
  if (e == hipSuccess) e = upload(&c->d_uitems, uitems);
  if (e == hipSuccess && pooled) e = upload(&c->d_map, map);
  if (e == hipSuccess && pooled) e = upload(&c->d_mapoff, mapoff);
  if (e == hipSuccess && pooled) e = upload(&c->d_poolrows, plan.rows_of);
  if (e == hipSuccess && pooled) e = upload(&c->d_pdesc, pdesc);
  if (e == hipSuccess && c->qminmax_slots > 0)
    e = hipMalloc(reinterpret_cast<void**>(&c->d_qminmax),
                  size_t(c->qminmax_slots) * 2 * hk::kQuantD * sizeof(float2));
  if (e == hipSuccess && quant_m > 0) {
    const size_t bytes = size_t(std::max<int64_t>(scratch_elems, 1)) * sizeof(uint16_t);
    e = hipMalloc(&c->kcache, bytes);
    if (e == hipSuccess) e = hipMalloc(&c->vcache, bytes);
  }
  if (e == hipSuccess)
    e = hipMalloc(reinterpret_cast<void**>(&c->d_partials),
                  size_t(max_partials) * hk::kMaxScales * sizeof(float));
  if (e == hipSuccess && ws_rows > 0)
    e = hipMalloc(reinterpret_cast<void**>(&c->d_ws_o), size_t(ws_rows) * D * sizeof(float));
  if (e == hipSuccess && ws_rows > 0)
    e = hipMalloc(reinterpret_cast<void**>(&c->d_ws_ml), size_t(ws_rows) * sizeof(float2));
  if (e != hipSuccess) {
    free_tables(c);
    delete c;
    return hip_fail(e, "context tables");
  }
  *out = c;
  return HK_OK;
}

}  // namespace

extern "C" int hk_create_expiry(hk_ctx** out, int L, int H, int D, int B, int K,
                                const int32_t* scale_tokens, const uint8_t* expire, int dtype,
                                void* k_cache, void* v_cache) {
  return create_impl(out, L, H, D, B, K, scale_tokens, expire, dtype, k_cache, v_cache, 0);
}

extern "C" int hk_create_pooled(hk_ctx** out, int L, int H, int D, int B, int K,
                                const int32_t* scale_tokens, const uint8_t* expire, void* k_pool,
                                void* v_pool) {
  return create_impl(out, L, H, D, B, K, scale_tokens, expire, HK_DTYPE_BF16, k_pool, v_pool, 0,
                     true);
}

extern "C" int hk_create_int4(hk_ctx** out, int L, int H, int D, int B, int K,
                              const int32_t* scale_tokens, const uint8_t* keep, int sub_blocks,
                              void* k_store, void* v_store) {
  if (!out) return fail(HK_EINVAL, "null output pointer");
  *out = nullptr;
  if (L < 1 || H < 1 || B < 1 || K < 1) return fail(HK_EINVAL, "L, H, B, K must be >= 1");
  if (!scale_tokens || !keep) return fail(HK_EINVAL, "null scale_tokens or keep");
  if (D != hk::kQuantD) return fail(HK_EUNSUPPORTED, "4-bit storage needs head_dim 128 (got %d)", D);
  if (sub_blocks < 1 || sub_blocks > 64) return fail(HK_EINVAL, "sub_blocks must be in [1, 64]");
  std::vector<uint8_t> expire;
  hk::expire_from_keep(keep, int64_t(L) * H, K, expire);
  return create_impl(out, L, H, D, B, K, scale_tokens, expire.data(), HK_DTYPE_BF16, k_store,
                     v_store, sub_blocks);
}

extern "C" int hk_create(hk_ctx** out, int L, int H, int D, int B, int K,
                         const int32_t* scale_tokens, const uint8_t* keep, int dtype,
                         void* k_cache, void* v_cache) {
  if (!out) return fail(HK_EINVAL, "null output pointer");
  *out = nullptr;
  if (L < 1 || H < 1 || B < 1 || K < 1) return fail(HK_EINVAL, "L, H, B, K must be >= 1");
  if (!scale_tokens || !keep) return fail(HK_EINVAL, "null scale_tokens or keep");
  std::vector<uint8_t> expire;
  hk::expire_from_keep(keep, int64_t(L) * H, K, expire);
  return hk_create_expiry(out, L, H, D, B, K, scale_tokens, expire.data(), dtype, k_cache, v_cache);
}

extern "C" int hk_destroy(hk_ctx* c) {
  if (!c) return HK_OK;
  int rc = HK_OK;
  {
    DeviceGuard g(c->device);
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) rc = hip_fail(e, "synchronise before destroy");
    free_tables(c);
  }
  delete c;
  return rc;
}

extern "C" int hk_reset(hk_ctx* c) {
  if (!c) return fail(HK_EINVAL, "null context");
  c->appended.assign(c->L, -1);
  c->attended.assign(c->L, -1);
  return HK_OK;
}

extern "C" int hk_attend(hk_ctx* c, int layer, int step, const void* q, const void* k_cur,
                         const void* v_cur, void* out, float softmax_scale, void* hip_stream) {
  return attend_common(c, layer, step, q, k_cur, v_cur, out, softmax_scale, nullptr, false, false,
                       hip_stream);
}

extern "C" int hk_attend_with_scas(hk_ctx* c, int layer, int step, const void* q,
                                   const void* k_cur, const void* v_cur, void* out,
                                   float softmax_scale, float* scas_table, void* hip_stream) {
  return attend_common(c, layer, step, q, k_cur, v_cur, out, softmax_scale, scas_table, true, false,
                       hip_stream);
}

extern "C" int hk_attend_with_scas_sum(hk_ctx* c, int layer, int step, const void* q,
                                       const void* k_cur, const void* v_cur, void* out,
                                       float softmax_scale, double* scas_sum, void* hip_stream) {
  if (!scas_sum) return fail(HK_EINVAL, "null S-CAS sum table");
  return attend_common(c, layer, step, q, k_cur, v_cur, out, softmax_scale, nullptr, true, false,
                       hip_stream, scas_sum);
}

extern "C" int hk_attend_append(hk_ctx* c, int layer, int step, const void* q, const void* k_cur,
                                const void* v_cur, void* out, float softmax_scale,
                                float* scas_table, void* hip_stream) {
  return attend_common(c, layer, step, q, k_cur, v_cur, out, softmax_scale, scas_table,
                       scas_table != nullptr, true, hip_stream);
}

extern "C" int hk_append_scale(hk_ctx* c, int layer_begin, int layer_end, int step,
                               const void* k_cur, const void* v_cur, int64_t layer_stride_elems,
                               void* hip_stream) {
  if (!c) return fail(HK_EINVAL, "null context");
  if (layer_begin < 0 || layer_end > c->L || layer_begin >= layer_end)
    return fail(HK_EINVAL, "layer range [%d, %d) invalid for %d layers", layer_begin, layer_end, c->L);
  if (step < 0 || step > c->K - 2)
    return fail(HK_EINVAL, "step %d cannot be appended (cached scales are 0..%d)", step, c->K - 2);
  if (!k_cur || !v_cur) return fail(HK_EINVAL, "null tensor pointer");
  if (!aligned16(k_cur) || !aligned16(v_cur))
    return fail(HK_EINVAL, "tensor pointers must be 16-byte aligned");
  const int nl = layer_end - layer_begin;
  if (nl > 1 && (layer_stride_elems < 0 ||
                 (layer_stride_elems * c->elem_bytes) % 16 != 0))
    return fail(HK_EINVAL, "layer stride must be non-negative and a multiple of 16 bytes");
  for (int l = layer_begin; l < layer_end; ++l) {
    if (c->appended[l] != step - 1)
      return fail(HK_EORDER, "append(layer %d, step %d) out of order (last appended: %d)", l,
                  step, c->appended[l]);
    if (c->drops[int64_t(step) * c->L + l] && c->attended[l] != step)
      return fail(HK_EORDER, "append(layer %d, step %d) overwrites segments that attend(layer %d, "
                  "step %d) reads: attend first", l, step, l, step);
  }
  const int rc = pool_append_order(c, layer_begin, step);
  if (rc != HK_OK) return rc;
  return append_launch(c, layer_begin, layer_end, step, k_cur, v_cur, layer_stride_elems,
                       hip_stream);
}

namespace {

// Launches the compaction of scale `step` for layers [layer_begin, layer_end)
// (arguments already checked) and records the layers as appended.
int append_launch(hk_ctx* c, int layer_begin, int layer_end, int step, const void* k_cur,
                  const void* v_cur, int64_t layer_stride_elems, void* hip_stream) {
  const int nl = layer_end - layer_begin;
  if (c->quant_m > 0) {
    const int64_t qfirst = c->qdesc_first[int64_t(step) * (c->L + 1) + layer_begin];
    const int64_t qlast = c->qdesc_first[int64_t(step) * (c->L + 1) + layer_end];
    if (qlast > qfirst) {
      DeviceGuard g(c->device);
      if (!g.ok) return fail(HK_EHIP, "cannot select device %d", c->device);
      hk::QuantArgs q{};
      q.desc = c->d_qdesc + qfirst;
      q.kcur = static_cast<const uint16_t*>(k_cur);
      q.vcur = static_cast<const uint16_t*>(v_cur);
      q.kstore = static_cast<uint8_t*>(c->kstore);
      q.vstore = static_cast<uint8_t*>(c->vstore);
      q.layer_stride = nl > 1 ? layer_stride_elems : 0;
      q.n_desc = int(qlast - qfirst);
      q.m = c->quant_m;
      q.B = c->B;
      q.n = c->tokens[step];
      q.H = c->H;
      q.layer_begin = layer_begin;
      // Cut long sub-blocks into chunks when one workgroup per sub-block
      // would leave most of the chip idle.
      const int64_t single = int64_t(q.n_desc) * q.m * q.B * 2;
      q.nch = single >= 2048 ? 1 : quant_chunks(q.n, q.m);
      q.minmax = c->d_qminmax;
      hipError_t e = hk::launch_quantize(q, static_cast<hipStream_t>(hip_stream));
      if (e != hipSuccess) return hip_fail(e, "quantize launch");
    }
    for (int l = layer_begin; l < layer_end; ++l) c->appended[l] = step;
    return HK_OK;
  }
  if (c->pooled) {
    const int64_t pf = c->pdesc_first[int64_t(step) * (c->L + 1) + layer_begin];
    const int64_t pl = c->pdesc_first[int64_t(step) * (c->L + 1) + layer_end];
    if (pl > pf) {
      DeviceGuard g(c->device);
      if (!g.ok) return fail(HK_EHIP, "cannot select device %d", c->device);
      hk::PoolArgs a{};
      a.desc = c->d_pdesc + pf;
      a.rows = c->d_poolrows;
      a.kcur = static_cast<const uint8_t*>(k_cur);
      a.vcur = static_cast<const uint8_t*>(v_cur);
      a.kpool = static_cast<uint8_t*>(c->kcache);
      a.vpool = static_cast<uint8_t*>(c->vcache);
      a.layer_stride_bytes = nl > 1 ? layer_stride_elems * c->elem_bytes : 0;
      a.pool_rows = c->pool_rows;
      a.n_desc = int(pl - pf);
      a.B = c->B;
      a.n = c->tokens[step];
      a.H = c->H;
      a.layer_begin = layer_begin;
      a.row_bytes = c->D * c->elem_bytes;
      a.cpr_shift = 0;
      while ((16 << a.cpr_shift) < a.row_bytes) ++a.cpr_shift;
      a.rows_per_block = std::min(hk::kCopyBlockBytes / a.row_bytes, a.n);
      a.chunks = (a.n + a.rows_per_block - 1) / a.rows_per_block;
      hipError_t e = hk::launch_compact_pooled(a, static_cast<hipStream_t>(hip_stream));
      if (e != hipSuccess) return hip_fail(e, "compact launch");
    }
    for (int l = layer_begin; l < layer_end; ++l) c->appended[l] = step;
    return HK_OK;
  }
  const int64_t gfirst = c->gdesc_first[int64_t(step) * (c->L + 1) + layer_begin];
  const int64_t glast = c->gdesc_first[int64_t(step) * (c->L + 1) + layer_end];
  const int64_t first = c->desc_first[int64_t(step) * (c->L + 1) + layer_begin];
  const int64_t last = c->desc_first[int64_t(step) * (c->L + 1) + layer_end];
  if (glast > gfirst) {
    // Drop the segments that expire at this step before storing it.
    DeviceGuard g(c->device);
    if (!g.ok) return fail(HK_EHIP, "cannot select device %d", c->device);
    hk::GatherArgs a{};
    a.desc = c->d_gdesc + gfirst;
    a.runs = c->d_gruns;
    a.kcache = static_cast<uint8_t*>(c->kcache);
    a.vcache = static_cast<uint8_t*>(c->vcache);
    a.n_desc = int(glast - gfirst);
    a.B = c->B;
    a.row_bytes = c->D * c->elem_bytes;
    // Column parts of whole 128-byte lines (rows of 128 bytes or less: one
    // part); both sizes are powers of two here.
    a.parts = std::max(1, a.row_bytes / hk::kGatherPartBytes);
    a.cpp_shift = 0;
    while ((a.parts * 16 << a.cpp_shift) < a.row_bytes) ++a.cpp_shift;
    a.rows_per_chunk = (hk::kGatherChunkBytes / 16) >> a.cpp_shift;
    hipError_t e = hk::launch_gather(a, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "gather launch");
  }
  const int row_bytes = c->D * c->elem_bytes;
  const int rows_per_block = hk::kCopyBlockBytes / row_bytes;
  if (last > first && 2 * (last - first) >= int64_t(nl) * c->H && c->H <= hk::kRowsMaxHeads) {
    // A scale that most heads store: copy whole token blocks (contiguous
    // reads across the heads, every head's rows written from one workgroup),
    // faster than per-head workgroups whose reads stride over the tokens.
    DeviceGuard g(c->device);
    if (!g.ok) return fail(HK_EHIP, "cannot select device %d", c->device);
    hk::RowsArgs a{};
    a.dst = c->d_rowdst + (int64_t(step) * c->L + layer_begin) * c->H;
    a.cap = c->d_cap + int64_t(layer_begin) * c->H;
    a.kcur = static_cast<const uint8_t*>(k_cur);
    a.vcur = static_cast<const uint8_t*>(v_cur);
    a.kcache = static_cast<uint8_t*>(c->kcache);
    a.vcache = static_cast<uint8_t*>(c->vcache);
    a.layer_stride_bytes = nl > 1 ? layer_stride_elems * c->elem_bytes : 0;
    a.n_layers = nl;
    a.B = c->B;
    a.n = c->tokens[step];
    a.H = c->H;
    a.row_bytes = row_bytes;
    // Tokens per workgroup: at least two and at least 8 KB per tensor, at
    // most 16 KB (and at least one token).  Measured on the 32-layer,
    // 16-head, batch-4 full-cache appends: two tokens (8 KB per tensor)
    // 5.43-5.47 TB/s against 5.29-5.33 with four (16 KB), 5.31 with three and
    // 4.95-4.97 with one; at 28 heads, batch 16, two tokens (14 KB) 5.20
    // against 5.06-5.08 with one and 5.04 with three.
    const int tok_bytes = c->H * row_bytes;
    a.rows = std::max(1, std::min(hk::kCopyBlockBytes / tok_bytes,
                                  std::max(hk::kRowsTokens, hk::kCopyBlockBytes / 2 / tok_bytes)));
    hipError_t e = hk::launch_compact_rows(a, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "compact launch");
  } else if (last > first) {
    DeviceGuard g(c->device);
    if (!g.ok) return fail(HK_EHIP, "cannot select device %d", c->device);
    hk::CompactArgs a{};
    a.desc = c->d_desc + first;
    a.kcur = static_cast<const uint8_t*>(k_cur);
    a.vcur = static_cast<const uint8_t*>(v_cur);
    a.kcache = static_cast<uint8_t*>(c->kcache);
    a.vcache = static_cast<uint8_t*>(c->vcache);
    a.layer_stride_bytes = nl > 1 ? layer_stride_elems * c->elem_bytes : 0;
    a.n_desc = int(last - first);
    a.B = c->B;
    a.n = c->tokens[step];
    a.H = c->H;
    a.row_bytes = c->D * c->elem_bytes;
    // One block per tensor per workgroup; the large block when the launch
    // has enough of them.
    const int large_rows = hk::kCopyBlockBytesLarge / row_bytes;
    const int64_t large_blocks = (last - first) * c->B * ((a.n + large_rows - 1) / large_rows);
    const int block_rows = large_blocks >= hk::kCopyLargeMinBlocks ? large_rows : rows_per_block;
    a.rows_per_block = std::min(std::max(1, block_rows), a.n);
    a.chunks = (a.n + a.rows_per_block - 1) / a.rows_per_block;
    a.layer_begin = layer_begin;
    hipError_t e = hk::launch_compact(a, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "compact launch");
  }
  for (int l = layer_begin; l < layer_end; ++l) c->appended[l] = step;
  return HK_OK;
}

}  // namespace

extern "C" int hk_retained_tokens(const hk_ctx* c, int step, int64_t* out) {
  if (!c || !out) return fail(HK_EINVAL, "null argument");
  if (step < 0 || step >= c->K) return fail(HK_EINVAL, "step %d out of [0, %d)", step, c->K);
  *out = c->retained[step];
  return HK_OK;
}

extern "C" int hk_plan_attend_bf16(int B, int H, int n, int max_keys, int allow_split,
                                   int32_t* rows_per_wg, int32_t* splits) {
  if (!rows_per_wg || !splits) return fail(HK_EINVAL, "null argument");
  if (B < 1 || H < 1 || n < 1 || max_keys < 1)
    return fail(HK_EINVAL, "B, H, n and max_keys must be >= 1");
  const hk::AttendPlan p = hk::attend_bf16_plan(B, H, n, max_keys, allow_split != 0);
  *rows_per_wg = p.rows;
  *splits = p.splits;
  return HK_OK;
}

extern "C" int hk_attend_plan(const hk_ctx* c, int step, int with_scas, int32_t* rows_per_wg,
                              int32_t* splits) {
  if (!c || !rows_per_wg || !splits) return fail(HK_EINVAL, "null argument");
  if (step < 0 || step >= c->K) return fail(HK_EINVAL, "step %d out of [0, %d)", step, c->K);
  *rows_per_wg = with_scas ? c->rows_scas[step] : c->rows[step];
  *splits = with_scas ? 1 : c->splits[step];
  return HK_OK;
}
