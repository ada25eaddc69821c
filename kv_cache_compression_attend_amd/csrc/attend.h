// Attention launch arguments and plan, shared by the attend kernels and the
// host code that launches them.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hk {

constexpr int kMaxScales = 16;   // S-CAS accumulators per query row
constexpr int kXcds = 8;         // MI355X: 8 accelerator dies, 32 CUs each

// A dispatch packet holds 32-bit grid sizes in work-items; launchers refuse
// a grid that would not fit (hipErrorInvalidConfiguration) instead of
// truncating it.  y and z stay within the runtime's 16-bit limits.
inline bool grid_fits(int64_t blocks_x, int threads, int64_t y = 1, int64_t z = 1) {
  return blocks_x >= 0 && blocks_x * threads <= 0xFFFFFFFFll && y >= 1 && y <= 65535 && z >= 1 &&
         z <= 65535;
}

// Arguments of one attend launch: one layer, one scale step.
struct AttendArgs {
  const void* q;          // [B][n][H][D]
  const void* kcur;       // [B][n][H][D]
  const void* vcur;       // [B][n][H][D]
  void* out;              // [B][n][H][D]
  const void* kcache;     // whole K cache buffer
  const void* vcache;     // whole V cache buffer
  const int64_t* base;    // [H] element offset of head (layer, h)
  const int32_t* cap;     // [H] cache rows per batch entry of head (layer, h)
  const int32_t* lenb;    // [H][K] rows cached before each scale
  float* partials;        // S-CAS partial sums [B*H*n_qtiles][kMaxScales]
  float* ws_o;            // split launches: unnormalised outputs [n_split][B][n][H][D] fp32
  float2* ws_ml;          // split launches: (running max, denominator) [n_split][B][n][H]
  int B, H, n, K, step, n_qtiles;
  int rows;               // bf16: query rows per workgroup (128 or 256)
  int n_split;            // key-range splits per query tile (1: no split)
  int append;             // 1: the workgroups also write this scale's kept K/V
                          // rows into the cache, key tile t by q-tile t mod
                          // n_qtiles (fused append)
  const int32_t* order;   // [H] heads heaviest first, or null; set only when B
                          // is a multiple of kXcds (see attend_coords)
  float scale;            // softmax scale alpha
  float scale_log2;       // alpha * log2(e)
  // Pooled cache (null otherwise): every head's rows sit in one pool per
  // batch entry (base 0, cap = pool rows); cache row r of head h at this
  // step is pool row map[mapoff[h] + r].  No fused append with a pool.
  const int32_t* map;
  const int64_t* mapoff;  // [H]
};

// Workgroups are handed to the 8 dies round-robin (workgroup i runs on die
// i % 8).  This maps the hardware index to a logical index so that each die
// receives one contiguous range of logical work, keeping a head's query tiles
// (which read the same keys and values) on one die and its L2.
__device__ __forceinline__ int xcd_logical(int i, int n) {
  const int q = n / kXcds, r = n % kXcds;
  const int x = i % kXcds, k = i / kXcds;
  return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

// Work item of attend workgroup i: (batch entry, head, key-range split,
// query tile).  Without a head order, logical index xcd_logical(i) in
// (b, h, split, q-tile) order, q-tile fastest.  With one (the heads of a
// pruned schedule hold different numbers of keys), die x takes batch entries
// [x B/8, (x+1) B/8) and runs their work heaviest head first: (head rank,
// batch entry, split, q-tile), so every die gets the same work and the
// longest workgroups start first instead of forming the launch's tail.
struct AttendItem {
  int b, h, split, qt;
};
__device__ __forceinline__ AttendItem attend_coords(int i, int n, int B, int H, int n_split,
                                                    int n_qtiles, const int32_t* order) {
  AttendItem it;
  if (order) {
    const int x = i % kXcds, k = i / kXcds;
    const int per_die = B / kXcds;
    it.qt = k % n_qtiles;
    int r = k / n_qtiles;
    it.split = r % n_split;
    r /= n_split;
    it.b = x * per_die + r % per_die;
    it.h = order[r / per_die];
  } else {
    const int wg = xcd_logical(i, n);
    it.qt = wg % n_qtiles;
    const int rest = wg / n_qtiles;
    it.split = rest % n_split;
    const int bh = rest / n_split;
    it.h = bh % H;
    it.b = bh / H;
  }
  return it;
}

// Query rows per workgroup (128 or 256) and key-range splits of one bf16
// attend launch.
struct AttendPlan {
  int rows;
  int splits;
};

// The plan for a scale of n tokens whose longest head holds max_keys keys
// (its cached rows plus the scale's own): the (rows, splits) pair of least
// modelled time.  The model counts launch rounds (one 256-query workgroup or
// two 128-query workgroups per CU), key tiles per split plus a per-workgroup
// set-up cost, and the merge of split partials.  allow_split false (S-CAS
// launches) keeps one split.
AttendPlan attend_bf16_plan(int B, int H, int n, int max_keys, bool allow_split);

// Launchers (defined next to their kernels).  For the bf16 launch a.rows,
// a.n_split and a.n_qtiles = ceil(n / rows) follow an attend_bf16_plan (S-CAS
// launches: one split); a split launch also merges the splits into a.out.
hipError_t launch_attend_bf16_d128(const AttendArgs& a, bool scas, hipStream_t s);
hipError_t launch_attend_f32(const AttendArgs& a, int D, bool scas, hipStream_t s);

}  // namespace hk
