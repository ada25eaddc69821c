// Attention of one layer and scale that allocates nothing: a variant of
// hk_attend_with_scas / hk_attend for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that
// forbid allocation).  It needs no context: the caller passes one layer's
// static keep-mask and that layer's cache (laid out as hk_layout lays out a
// layer), and the per-head tables the attend kernels read, together with the
// S-CAS partial sums, live in a file-scope device array (one copy per GPU,
// held until the process ends) instead of in a context's allocations.
//
// The scratch array holds, at offset 0, the per-head tables of the call
// (written by a small kernel from its by-value arguments, so no host memory
// is read after the call returns) and, from kTablesBytes on, the S-CAS
// partial sums.  Every call overwrites what it reads, so nothing needs
// clearing; calls that overlap on one GPU (other streams, other threads)
// share the array and race.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "../../include/heatkv.h"
#include "device.h"
#include "status.h"

namespace hk {
namespace {

constexpr int kNaMaxHeads = HK_NOALLOC_MAX_HEADS;
constexpr size_t kScratchBytes = size_t(HK_NOALLOC_SCRATCH_BYTES);
constexpr size_t kTablesBytes = 4096;
constexpr int kNaMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

// The tables of one call, passed by value to the kernel that stores them.
struct NaTables {
  int64_t base[kNaMaxHeads];                // element offset of head h in the layer's cache
  int32_t cap[kNaMaxHeads];                 // rows per batch entry of head h
  int32_t lenb[kNaMaxHeads * kMaxScales];   // [H][K] segment starts while `step` is attended
};
static_assert(sizeof(NaTables) <= kTablesBytes, "tables exceed their scratch region");
static_assert(kTablesBytes % 256 == 0, "partials must stay 256-byte aligned");

__global__ void noalloc_tables_kernel(NaTables t, int H, int K, unsigned char* dst) {
  NaTables* d = reinterpret_cast<NaTables*>(dst);
  for (int i = threadIdx.x; i < H; i += blockDim.x) {
    d->base[i] = t.base[i];
    d->cap[i] = t.cap[i];
  }
  for (int i = threadIdx.x; i < H * K; i += blockDim.x) d->lenb[i] = t.lenb[i];
}

std::mutex g_mu;
unsigned char* g_scratch[kNaMaxDevices] = {};

// The device address of this GPU's scratch array, taken once per device with
// that device current.  The array's name is a host-side stand-in and is never
// passed to a kernel or copy.
int scratch_of(int dev, unsigned char** out) {
  if (dev < 0 || dev >= kNaMaxDevices) return fail(HK_EUNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(HK_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch[dev] = static_cast<unsigned char*>(p);
  }
  *out = g_scratch[dev];
  return HK_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace hk

extern "C" int hk_attend_noalloc(int H, int B, int K, const int32_t* scale_tokens,
                                 const uint8_t* keep, int step, const void* k_cache,
                                 const void* v_cache, const void* q, const void* k_cur,
                                 const void* v_cur, void* out, float softmax_scale,
                                 float* scas_table, void* hip_stream) {
  using hk::fail;
  if (H < 1 || B < 1 || K < 1) return fail(HK_EINVAL, "H, B, K must be >= 1");
  if (H > hk::kNaMaxHeads)
    return fail(HK_EINVAL, "hk_attend_noalloc takes at most %d heads (got %d)", hk::kNaMaxHeads, H);
  if (K > HK_MAX_SCALES) return fail(HK_EUNSUPPORTED, "K = %d exceeds %d scales", K, HK_MAX_SCALES);
  if (step < 0 || step >= K) return fail(HK_EINVAL, "step %d out of [0, %d)", step, K);
  if (!scale_tokens || !keep) return fail(HK_EINVAL, "null scale_tokens or keep");
  if (!q || !k_cur || !v_cur || !out) return fail(HK_EINVAL, "null tensor pointer");
  if (!hk::aligned16(q) || !hk::aligned16(k_cur) || !hk::aligned16(v_cur) ||
      !hk::aligned16(out) || !hk::aligned16(k_cache) || !hk::aligned16(v_cache))
    return fail(HK_EINVAL, "tensor and cache pointers must be 16-byte aligned");
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale))
    return fail(HK_EINVAL, "softmax_scale must be positive and finite");
  for (int s = 0; s < K; ++s)
    if (scale_tokens[s] < 1) return fail(HK_EINVAL, "scale %d has no tokens", s);

  // Tables of a static keep-mask (no heap: fixed-size arrays on the stack).
  hk::NaTables t{};
  int64_t off = 0, held_max = 0;
  for (int h = 0; h < H; ++h) {
    const uint8_t* kp = keep + int64_t(h) * K;
    int64_t cap = 0, run = 0;
    for (int s = 0; s <= K - 2; ++s) cap += kp[s] ? scale_tokens[s] : 0;
    for (int s = 0; s < K; ++s) {
      t.lenb[h * K + s] = int32_t(run);
      if (s < step && s <= K - 2 && kp[s]) run += scale_tokens[s];
      if (s == step && step <= K - 2 && kp[step]) run += scale_tokens[step];
    }
    if (cap > INT32_MAX) return fail(HK_EINVAL, "head %d holds more than 2^31 rows", h);
    t.base[h] = off;
    t.cap[h] = int32_t(cap);
    off += int64_t(B) * cap * 128;
    held_max = std::max<int64_t>(held_max, t.lenb[h * K + step]);
  }
  if (off > 0 && (!k_cache || !v_cache)) return fail(HK_EINVAL, "null cache buffer");

  const int n = scale_tokens[step];
  const hk::AttendPlan plan = hk::attend_bf16_plan(B, H, n, int(held_max + n), false);
  const int n_qtiles = (n + plan.rows - 1) / plan.rows;
  const int64_t partial_bytes = int64_t(B) * H * n_qtiles * hk::kMaxScales * int64_t(sizeof(float));
  if (partial_bytes > int64_t(hk::kScratchBytes - hk::kTablesBytes))
    return fail(HK_EINVAL,
                "S-CAS partial sums need %lld bytes, beyond the %lld this entry point holds "
                "(B * H * query tiles too large)",
                (long long)partial_bytes, (long long)(hk::kScratchBytes - hk::kTablesBytes));

  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(HK_EHIP, "no current device");
  unsigned char* scr = nullptr;
  int rc = hk::scratch_of(dev, &scr);
  if (rc != HK_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  hipLaunchKernelGGL(hk::noalloc_tables_kernel, dim3(1), dim3(256), 0, s, t, H, K, scr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HK_EHIP, "table launch: %s", hipGetErrorString(e));

  const hk::NaTables* dt = reinterpret_cast<const hk::NaTables*>(scr);
  hk::AttendArgs a{};
  a.q = q;
  a.kcur = k_cur;
  a.vcur = v_cur;
  a.out = out;
  a.kcache = k_cache;
  a.vcache = v_cache;
  a.base = dt->base;
  a.cap = dt->cap;
  a.lenb = dt->lenb;
  a.partials = reinterpret_cast<float*>(scr + hk::kTablesBytes);
  a.ws_o = nullptr;
  a.ws_ml = nullptr;
  a.rows = plan.rows;
  a.n_split = 1;
  a.B = B;
  a.H = H;
  a.n = n;
  a.K = K;
  a.step = step;
  a.n_qtiles = n_qtiles;
  a.append = 0;
  a.order = nullptr;
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  const bool scas = scas_table != nullptr;
  e = hk::launch_attend_bf16_d128(a, scas, s);
  if (e != hipSuccess) return fail(HK_EHIP, "attend launch: %s", hipGetErrorString(e));
  if (scas) {
    e = hk::launch_scas_finalize(a.partials, scas_table, 0, H, K, B, n, step, n_qtiles, s);
    if (e != hipSuccess) return fail(HK_EHIP, "S-CAS finalize launch: %s", hipGetErrorString(e));
  }
  return HK_OK;
}
