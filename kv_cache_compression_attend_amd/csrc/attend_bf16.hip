// Block-causal multi-scale attention over kept head-scale segments, bf16
// inputs, head_dim 128, on the gfx950 matrix cores.
//
// What it computes: every query of scale t in head (layer, h) attends to the
// kept segments s < t of that head, read from the ragged cache in scale
// order, followed by the keys of scale t itself (HeatKV project page,
// Abstract and Method step 5; Pith page of arXiv 2605.14877, Figure 2
// caption).  With S-CAS on, it also accumulates the probability mass each
// query puts on each source scale (HeatKV project page, Method step 2).
//
// Shared design:
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: each lane owns one query column and 16 key
//     rows per 32x32 block, so a query's max and sum stay in the lane and
//     the lane 32 apart that holds the query's other 16 keys (the two
//     combine only when a block's exact max is needed, and once at the end
//     for the denominator).
//   * The key rows fed to the score product are permuted (bits 2 and 3 of the
//     row index swapped) so that each lane's score registers already hold,
//     for every 16-key step of the value product, the 8 consecutive keys the
//     B operand of O^T = V^T P^T needs: probabilities go from the score
//     registers straight into the value product.
//   * K tiles are staged row-major in LDS; V tiles are transposed on the way
//     in (4 keys x 8 dims per lane, repacked in registers with byte
//     permutes) so the A operand of the value product is one 16-byte LDS
//     read.  Row strides are padded
//     so the operand reads are free of bank conflicts.
//   * Global loads are buffer loads from per-tile scalar descriptors whose
//     size ends at the last valid row, so rows past the end read as zero and
//     the per-lane offsets stay constant.  A 64-key tile lies in the cache,
//     in the current scale, or (at most once) across the junction, where each
//     row picks its source; the junction needs no padding.
//   * fp32 online softmax in base 2 (alpha * log2 e folded into one fma).
//     The running max is raised only when a block's max exceeds it by more
//     than 2^8, so the output accumulators are rescaled on a few blocks
//     rather than on every one; probabilities stay below 256, which bf16 and
//     fp32 hold as precisely as values below 1.  The exponentials are taken
//     first, against the running max; only when a lane's probabilities sum
//     to more than 2^7 (which any probability above 2^8 forces) does the
//     wave take the block's exact max and, if it must, rescale and take the
//     exponentials again.  The common block thus spends nothing on its max
//     or on the cross-lane exchange the max needs.
//   * Without S-CAS and for alpha * log2 e <= 2, Q is multiplied by
//     alpha * log2 e once per workgroup (and rounded to bf16), so the score
//     products come out in base-2 units,
//     and the 256-query tiling runs the middle key tiles of a wave without
//     any running max while its scores stay within +-64 of zero (2^64 and
//     2^-64 are far inside fp32 and bf16 range): the exponentials then take
//     the accumulators as they are, with no scaling or subtraction.  A block
//     whose probabilities sum above 2^64 raises the running max at once and
//     the wave continues in the general form.  (With S-CAS the scores keep
//     the exact bf16 Q: the per-source mass of a single query is compared
//     to 1e-4.)
//   * Without S-CAS the softmax denominator is summed from the same bf16
//     probabilities the value product uses (v_dot2 against ones: half the
//     adds).  With S-CAS it is summed in fp32 together with per-source
//     accumulators, rescaled with the running max, reduced across the
//     workgroup into one partial row per workgroup; a second kernel adds the
//     partials in a fixed order (no float atomics, deterministic).
//
// Two tilings, chosen per launch by a cost model (attend_bf16_plan):
//   * 128 queries per workgroup of 4 waves, two workgroups per CU; the 64-key
//     tile is scored, normalised and accumulated in sequence.  Used for the
//     smallest launches and for S-CAS launches that would not fill the chip
//     with 256-query workgroups.
//   * 256 queries per workgroup of 8 waves (two per SIMD), optionally with
//     each head's key range split over several workgroups whose (output,
//     max, denominator) partials a merge kernel combines.  Per 32-key unit u
//     a wave runs the score product QK(u) (8 MFMAs), the softmax SM(u) and
//     the value product PV(u) (8 MFMAs), pipelined as step
//     i = { QK(u_{i+1}), PV(u_{i-1}) } on the matrix cores beside SM(u_i) on
//     the vector ALUs.  Each step is written as 16 fixed slots (LDS read of
//     the fragment two slots ahead, one MFMA, one exponential and its share of
//     the packing and sum) fenced by scheduling barriers, so LDS latency hides
//     behind the MFMA before it and the exponentials fill the MFMA shadow.
//     Tiles go from memory straight into LDS (buffer loads with the LDS
//     flag; waves 4-7 load K, waves 0-3 load V) in four LDS buffers per
//     operand, in pairs: one barrier per two 64-key tiles publishes the next
//     two tiles of K and V, the K waves load two tiles at that barrier and
//     the V waves two at the start of the following tile.  V stays
//     row-major and the value product reads its transposed fragments with
//     the CDNA4 transposing LDS read.  Pooled
//     caches, whose rows are found through a map, read each burst's pool
//     rows one burst ahead.  The first and last tiles are separate
//     instantiations, so the steady-state step is straight-line code.  (The
//     128-query tiling stages through registers, V transposed on the way.)
#include <math.h>

#include <algorithm>

#include <type_traits>

#include "attend.h"

namespace hk {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;        // head_dim
constexpr int BN = 64;        // keys per staged tile
constexpr int KSTR = D + 8;   // K tile row stride (bf16 elements): 272 bytes
constexpr int VSTR = BN + 8;  // V^T tile row stride (bf16 elements): 144 bytes
constexpr int kRowBytes = D * 2;
constexpr int kMaxSplits = 16;  // key-range splits per head in one launch
constexpr float kRescaleSlack = 8.f;  // log2 units
constexpr float kSumTrigger = 128.f;   // 2^(kRescaleSlack - 1)
constexpr float kFastRange = 64.f;     // log2 units: |first block max| allowed in fast mode
constexpr float kFastTrigger = 1.8446744e19f;  // 2^kFastRange
// Largest alpha * log2 e for which Q is pre-scaled.  Rounding alpha * log2 e
// * q to bf16 moves each term of a score's dot product by up to 2^-8 of
// itself, so the score error grows with the scale: up to 2 (alpha ~1.4, the
// workloads' alpha = 1) it perturbs a probability about as much as its own
// bf16 rounding before the value product; a softmax scale of 6 measured
// twice the bf16 parity bar, so larger scales keep the exact Q.
constexpr float kPreMaxScale = 2.f;
constexpr unsigned kOutOfRange = 0x80000000u;
// s_waitcnt operand: vector memory count 0 and LDS count 0 (export count
// not waited on).
constexpr unsigned kWaitVmLds = 0x0070u;
constexpr int kRsrcFlags = 0x00020000;
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;

union Vec16 {
  u32x4 u;
  bf16x8 b;
  uint32_t w[4];
};

// Key row (within a 32-key block) that feeds row i of the score product.
__device__ __forceinline__ int permuted_row(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Key (within a 32-key block) held in score register v of a lane in half hf.
__device__ __forceinline__ int key_of(int v, int hf) {
  const int kp = v >> 2, r = v & 3;
  return 16 * (kp >> 1) + 8 * hf + 4 * (kp & 1) + r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}


// acc + lo(w) + hi(w), the two bf16 halves of w summed in fp32.
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                         __builtin_bit_cast(bf16x2, kOnesBf16x2), acc, false);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int nrec = bytes <= 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : int(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nrec, kRsrcFlags);
}

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0);
}

// Where the keys (or values) of one (batch, head) live: cache rows [0, Lc),
// then the current scale's rows; Ltot keys in all.
struct KeySource {
  const char* cache;  // row r at cache + r * kRowBytes (pooled: at cache + map[r] * kRowBytes)
  const char* cur;    // row r at cur + r * tokb
  int Lc, Ltot, n, tokb;
  const int32_t* map;  // pooled caches: pool row of each held row, else null
  int pool_bytes;      // pooled caches: bytes of the batch entry's pool
};

// Four 16-byte vectors of the 64-row tile starting at key k0: rows
// r0 + rstep * i (i = 0..3), 16-byte chunk c.  Rows past the end read 0.
// PAGED: cache rows are found through the map (one 4-byte load per row,
// then the row itself).
template <bool PAGED>
__device__ __forceinline__ void load_rows(const KeySource& s, int k0, int r0, int rstep, int c,
                                          u32x4 (&reg)[4]) {
  if (k0 + BN <= s.Lc) {  // all rows in the cache
    if constexpr (PAGED) {
      const auto rm = rsrc(s.map + k0, BN * 4);
      const auto rp = rsrc(s.cache, s.pool_bytes);
      unsigned pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pr[i] = __builtin_amdgcn_raw_buffer_load_b32(rm, (r0 + rstep * i) * 4, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) reg[i] = bload(rp, pr[i] * unsigned(kRowBytes) + 16u * c);
    } else {
      const auto r = rsrc(s.cache + int64_t(k0) * kRowBytes, BN * kRowBytes);
#pragma unroll
      for (int i = 0; i < 4; ++i) reg[i] = bload(r, unsigned(r0 + rstep * i) * kRowBytes + 16u * c);
    }
  } else if (k0 >= s.Lc) {  // all rows in the current scale
    const int64_t q0 = k0 - s.Lc;
    const auto r = rsrc(s.cur + q0 * s.tokb, int64_t(s.n - q0 - 1) * s.tokb + kRowBytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) reg[i] = bload(r, unsigned(r0 + rstep * i) * s.tokb + 16u * c);
  } else {  // junction: rows below split from the cache, the rest from the current scale
    const int split = s.Lc - k0;
    const auto ru = rsrc(s.cur - int64_t(split) * s.tokb, int64_t(split + s.n - 1) * s.tokb + kRowBytes);
    if constexpr (PAGED) {
      const auto rm = rsrc(s.map + k0, split * 4);
      const auto rp = rsrc(s.cache, s.pool_bytes);
      unsigned pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pr[i] = __builtin_amdgcn_raw_buffer_load_b32(rm, (r0 + rstep * i) * 4, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = r0 + rstep * i;
        const unsigned oc = row < split ? pr[i] * unsigned(kRowBytes) + 16u * c : kOutOfRange;
        const unsigned ou = row >= split ? unsigned(row) * s.tokb + 16u * c : kOutOfRange;
        reg[i] = bload(rp, oc) | bload(ru, ou);
      }
    } else {
      const auto rc = rsrc(s.cache + int64_t(k0) * kRowBytes, int64_t(split) * kRowBytes);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = r0 + rstep * i;
        const unsigned oc = row < split ? unsigned(row) * kRowBytes + 16u * c : kOutOfRange;
        const unsigned ou = row >= split ? unsigned(row) * s.tokb + 16u * c : kOutOfRange;
        reg[i] = bload(rc, oc) | bload(ru, ou);
      }
    }
  }
}

// K staging over 256 lanes: lane l holds chunk l & 15 of rows (l >> 4) + 16 i.
template <bool PAGED>
__device__ __forceinline__ void load_k(const KeySource& s, int k0, int l, u32x4 (&reg)[4]) {
  load_rows<PAGED>(s, k0, l >> 4, 16, l & 15, reg);
}
__device__ __forceinline__ void store_k(uint16_t* sK, int l, const u32x4 (&reg)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<u32x4*>(&sK[((l >> 4) + 16 * i) * KSTR + 8 * (l & 15)]) = reg[i];
}

// V staging over 256 lanes: lane l holds chunk l >> 4 of rows 4 (l & 15) + r,
// written transposed (dims x keys).
template <bool PAGED>
__device__ __forceinline__ void load_v(const KeySource& s, int k0, int l, u32x4 (&reg)[4]) {
  load_rows<PAGED>(s, k0, 4 * (l & 15), 1, l >> 4, reg);
}
__device__ __forceinline__ void store_v(uint16_t* sV, int l, const u32x4 (&reg)[4]) {
  const int g = l & 15, c = l >> 4;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t a0 = reg[0][w], a1 = reg[1][w], a2 = reg[2][w], a3 = reg[3][w];
    uint2 even, odd;
    even.x = __builtin_amdgcn_perm(a1, a0, 0x05040100u);
    even.y = __builtin_amdgcn_perm(a3, a2, 0x05040100u);
    odd.x = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
    odd.y = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
    const int d = 8 * c + 2 * w;
    *reinterpret_cast<uint2*>(&sV[d * VSTR + 4 * g]) = even;
    *reinterpret_cast<uint2*>(&sV[(d + 1) * VSTR + 4 * g]) = odd;
  }
}

// ---------------------------------------------------------------------------
// Direct staging (256-query tiling):
// tiles go from memory straight into LDS (buffer loads with the LDS flag:
// lane l of a wave's load writes its 16 bytes at the load's LDS base + 16 l;
// a lane whose offset is out of range writes zeros), with no pass through
// registers.  A wave's load fills 1 KB of a tile's LDS buffer, i.e. 64
// consecutive 16-byte chunk slots; a tile row occupies CH slots, of which
// the first 16 hold the row's 256 bytes and the rest are padding (read out
// of range).  K rows keep the 272-byte stride of the score product's
// fragment reads (CH = 17); V stays row-major (keys x dims) with a 320-byte
// stride (CH = 20), which the transposing LDS reads of the value product
// take without bank conflicts.
// ---------------------------------------------------------------------------
constexpr int VROW = D + 32;               // row-major V tile row stride (bf16 elements)
constexpr int kKChunks = KSTR / 8;         // 17
constexpr int kVChunks = VROW / 8;         // 20
constexpr int kKLoads = BN * kKChunks / 64;  // 17 wave loads per K tile
constexpr int kVLoads = BN * kVChunks / 64;  // 20 per V tile
static_assert(BN * kKChunks % 64 == 0 && BN * kVChunks % 64 == 0, "whole wave loads per tile");

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

// Waits for all of this wave's vector memory operations (its direct loads
// included) and LDS operations.
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(kWaitVmLds); }

// Workgroup barrier that does not itself wait for this wave's outstanding
// direct loads (the fenced barrier would; the callers wait with wait_loads
// where the next steps read what the loads bring); the empty asm statements
// keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_keep_loads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const void* lds, unsigned voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds), 16, int(voff), 0, 0, 0);
}

// One wave's share of a tile's direct loads (the four waves of a stager
// group take loads i = w, w + 4, ...): for its m-th load, this lane's byte
// offsets in a 64-row block of the cache (rows kRowBytes apart) and of the
// current scale (rows tokb apart), or kOutOfRange for a padding slot.
struct DmaLane {
  unsigned vc[5], vu[5];
  int w, n;  // first load index, loads of this wave (wave-uniform)
};

template <int CH, int NLOADS>
__device__ __forceinline__ DmaLane dma_lane(int w, int lane, int tokb) {
  DmaLane d;
  d.w = w;
  d.n = (NLOADS - w + 3) / 4;
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    const int i = w + 4 * m;
    const int q = 64 * i + lane, row = q / CH, c = q % CH;
    const bool ok = i < NLOADS && c < 16;
    d.vc[m] = ok ? unsigned(row * kRowBytes + 16 * c) : kOutOfRange;
    d.vu[m] = ok ? unsigned(row) * unsigned(tokb) + 16u * c : kOutOfRange;
  }
  return d;
}

// Pooled caches: the pool row of the row each of this wave's loads of the
// tile at key x0 takes from the cache (0 for rows past the held ones, which
// come from the current scale, and for padding slots), read from the map one
// burst of loads ahead of its use.
__device__ __forceinline__ void map_prefetch(const KeySource& s, int x0, const DmaLane& d,
                                             unsigned (&mv)[5]) {
  const int held = min(s.Lc - x0, BN);
  if (held <= 0) return;
  const auto r = rsrc(s.map + x0, int64_t(held) * 4);
#pragma unroll
  for (int m = 0; m < 5; ++m)
    if (m < d.n) mv[m] = __builtin_amdgcn_raw_buffer_load_b32(r, int((d.vc[m] >> 8) * 4u), 0, 0);
}

// Issues this wave's loads of the tile at key k0 into the LDS buffer buf.
// Rows past the end of the keys are read as zeros.  PAGED: cache rows come
// from the pool rows in mv (map_prefetch of the same tile).
template <bool PAGED>
__device__ __forceinline__ void dma_tile(const KeySource& s, int k0, const uint16_t* buf,
                                         const DmaLane& d, const unsigned (&mv)[5]) {
  const char* const lds = reinterpret_cast<const char*>(buf);
  // Byte offset of the cache part of load m: the pool row's, or the row's
  // within the tile's contiguous block.
  auto coff = [&](int m) {
    if constexpr (PAGED)
      return d.vc[m] == kOutOfRange ? kOutOfRange : mv[m] * unsigned(kRowBytes) + (d.vc[m] & 255u);
    else
      return d.vc[m];
  };
  if (k0 + BN <= s.Lc) {  // all rows in the cache
    const auto r = PAGED ? rsrc(s.cache, s.pool_bytes)
                         : rsrc(s.cache + int64_t(k0) * kRowBytes, BN * kRowBytes);
#pragma unroll
    for (int m = 0; m < 5; ++m)
      if (m < d.n) dma16(r, lds + 1024 * (d.w + 4 * m), coff(m));
  } else if (k0 >= s.Lc) {  // all rows in the current scale
    const int64_t q0 = k0 - s.Lc;
    const auto r = rsrc(s.cur + q0 * s.tokb, int64_t(s.n - q0 - 1) * s.tokb + kRowBytes);
#pragma unroll
    for (int m = 0; m < 5; ++m)
      if (m < d.n) dma16(r, lds + 1024 * (d.w + 4 * m), d.vu[m]);
  } else {  // junction: rows below split from the cache, the rest from the current scale
    const int split = s.Lc - k0;
    const auto rc = PAGED ? rsrc(s.cache, s.pool_bytes)
                          : rsrc(s.cache + int64_t(k0) * kRowBytes, int64_t(split) * kRowBytes);
    const auto ru = rsrc(s.cur - int64_t(split) * s.tokb, int64_t(split + s.n - 1) * s.tokb + kRowBytes);
#pragma unroll
    for (int m = 0; m < 5; ++m) {
      if (m < d.n) {
        // Padding slots (kOutOfRange) take the second branch and read zeros.
        if (int(d.vc[m] >> 8) < split) dma16(rc, lds + 1024 * (d.w + 4 * m), coff(m));
        else dma16(ru, lds + 1024 * (d.w + 4 * m), d.vu[m]);
      }
    }
  }
}

// Fused append with direct staging: the 256 lanes of a stager group copy the
// rows of the staged tile at key k0 (LDS row stride RS bytes) that belong to
// the current scale into the cache rows of the same keys.
template <int RS>
__device__ __forceinline__ void append_from_lds(const KeySource& s, char* cache, int k0,
                                                const uint16_t* buf, int l) {
  if (k0 + BN <= s.Lc) return;
  const int c = l & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (l >> 4) + 16 * i, key = k0 + row;
    if (key >= s.Lc && key < s.Ltot)
      *reinterpret_cast<u32x4*>(cache + int64_t(key) * kRowBytes + 16 * c) =
          *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(buf) + row * RS + 16 * c);
  }
}

// A-operand fragment of the value product from a row-major V tile: dims
// 32 db + (lane mod 32), keys 16 st + 8 (lane / 32) + 0..7, as two
// transposing reads of four keys.  Within each 16-lane group the read hands
// lane i element (i mod 4) of the row addressed by lane 4 r + i / 4, for
// r = 0..3; lane a of group g therefore addresses key row
// 8 (g / 2) + a / 4 (+ 4 for the second read) at dims
// 32 db + 16 (g mod 2) + 4 (a mod 4) .. + 3.  voff: that byte offset for
// st = db = 0.
__device__ __forceinline__ int vtr_lane_offset(int lane) {
  const int g = lane >> 4, a = lane & 15;
  return (8 * (g >> 1) + (a >> 2)) * VROW * 2 + 32 * (g & 1) + 8 * (a & 3);
}
__device__ __forceinline__ u32x4 vfrag_tr(const uint16_t* Vt, int voff, int st, int db) {
  const char* p = reinterpret_cast<const char*>(Vt) + voff + st * 16 * VROW * 2 + db * 64;
  const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p));
  const v4i16 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p + 4 * VROW * 2));
  const uint2 xa = __builtin_bit_cast(uint2, x), ya = __builtin_bit_cast(uint2, y);
  return u32x4{xa.x, xa.y, ya.x, ya.y};
}

// Fused append: the 16-byte chunks held in reg (rows r0 + rstep * i, chunk c
// of the tile at key k0) whose key falls in the current scale are written to
// the same key's row of the cache, where the scale's segment starts at row Lc.
template <bool PAGED>
__device__ __forceinline__ void append_rows(const KeySource& s, char* cache, int k0, int r0, int rstep,
                                            int c, const u32x4 (&reg)[4]) {
  if constexpr (PAGED) return;  // pooled caches are appended by their own kernel
  if (k0 + BN <= s.Lc) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = k0 + r0 + rstep * i;
    if (key >= s.Lc && key < s.Ltot)
      *reinterpret_cast<u32x4*>(cache + int64_t(key) * kRowBytes + 16 * c) = reg[i];
  }
}

// Per-workgroup setup shared by both tilings.
struct Head {
  KeySource ks, vs;
  const char* q;      // (b, row 0, h) of the query tensor
  int n, tokb, Lc, Ltot, h, b, qt, split;
  const int32_t* lenb;
  bool append;        // this workgroup writes the current scale's rows to the cache
};

__device__ __forceinline__ Head setup(const AttendArgs& a) {
  Head hd;
  // The workgroups that read the same key range of a head are adjacent on
  // one die (q-tile fastest).
  const AttendItem it = attend_coords(blockIdx.x, gridDim.x, a.B, a.H, a.n_split, a.n_qtiles, a.order);
  hd.qt = it.qt;
  hd.split = it.split;
  hd.h = it.h;
  hd.b = it.b;
  hd.n = a.n;
  const int64_t tok = int64_t(a.H) * D;
  hd.tokb = int(tok * 2);
  const int cap = a.cap[hd.h];
  const int64_t hb = (a.base[hd.h] + int64_t(hd.b) * cap * D) * 2;
  hd.lenb = a.lenb + hd.h * a.K;
  hd.Lc = hd.lenb[a.step];
  hd.Ltot = hd.Lc + hd.n;
  const int64_t curoff = (int64_t(hd.b) * hd.n * tok + hd.h * D) * 2;
  // A pooled cache: every head's rows sit in the batch entry's pool of cap
  // rows (base 0), found through this step's map of the head.
  const int32_t* map = a.map ? a.map + a.mapoff[hd.h] : nullptr;
  const int pool_bytes = a.map ? cap * kRowBytes : 0;
  hd.ks = KeySource{static_cast<const char*>(a.kcache) + hb, static_cast<const char*>(a.kcur) + curoff,
                    hd.Lc, hd.Ltot, hd.n, hd.tokb, map, pool_bytes};
  hd.vs = KeySource{static_cast<const char*>(a.vcache) + hb, static_cast<const char*>(a.vcur) + curoff,
                    hd.Lc, hd.Ltot, hd.n, hd.tokb, map, pool_bytes};
  hd.q = static_cast<const char*>(a.q) + curoff;
  // Every workgroup of a (b, h, split) stages all of its key tiles; the
  // append of tile t falls to the one with q-tile t mod n_qtiles, so the
  // writes are spread over the workgroups.  A pruned segment (no cache rows
  // reserved for this scale) is never written, and nothing is written past
  // the head's capacity.
  hd.append = a.append && a.step + 1 < a.K && hd.lenb[a.step + 1] > hd.Lc &&
              hd.lenb[a.step + 1] <= cap;
  return hd;
}

// The first key tile at or after t whose append falls to this workgroup
// (tiles t' with t' mod n_qtiles == q-tile); later ones follow every
// n_qtiles tiles.
__device__ __forceinline__ int first_append_tile(const AttendArgs& a, const Head& hd, int t) {
  return t + (hd.qt - t % a.n_qtiles + a.n_qtiles) % a.n_qtiles;
}

// Q^T fragments of query qrow: dims 16*kk + 8*hf + [0, 8); zero past the end.
__device__ __forceinline__ void load_q(const Head& hd, int qrow, int hf, Vec16 (&qf)[8]) {
  const auto rq = rsrc(hd.q, int64_t(hd.n - 1) * hd.tokb + kRowBytes);
  const unsigned off = qrow < hd.n ? unsigned(qrow) * unsigned(hd.tokb) + 16u * hf : kOutOfRange;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) qf[kk].u = bload(rq, off + 32u * kk);
}

// out[b][qrow][h][:] = O / l, bf16.
__device__ __forceinline__ void store_out(const AttendArgs& a, const Head& hd, int qrow, int hf,
                                          const f32x16 (&o)[4], float inv) {
  if (qrow >= hd.n) return;
  uint16_t* op = static_cast<uint16_t*>(a.out) +
                 (int64_t(hd.b) * hd.n + qrow) * (int64_t(a.H) * D) + hd.h * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
      const int d = 32 * db + 8 * kp + 4 * hf;
      uint2 w;
      w.x = pack_bf16x2(o[db][4 * kp + 0] * inv, o[db][4 * kp + 1] * inv);
      w.y = pack_bf16x2(o[db][4 * kp + 2] * inv, o[db][4 * kp + 3] * inv);
      *reinterpret_cast<uint2*>(op + d) = w;
    }
}

// This lane's 16 probabilities of one 32-key block, 2^(s * c2 - m), packed
// to bf16 pairs as the B operand of the value product (p[0]: keys of the
// first 16-key step, p[1]: the second).  Returns their sum: of the fp32
// values with F32SUM, else of the bf16 values the value product uses.
template <bool F32SUM>
__device__ __forceinline__ float exp_pack(const f32x16& s, float c2, float m, Vec16 (&p)[2]) {
  float sum = 0.f;
#pragma unroll
  for (int v = 0; v < 16; v += 2) {
    const float e0 = __builtin_amdgcn_exp2f(fmaf(s[v], c2, -m));
    const float e1 = __builtin_amdgcn_exp2f(fmaf(s[v + 1], c2, -m));
    uint32_t& w = p[v >> 3].w[(v & 7) >> 1];
    w = pack_bf16x2(e0, e1);
    if constexpr (F32SUM) sum += e0 + e1;
    else sum = add_bf16x2(w, sum);
  }
  return sum;
}

// The probability of score register v, recomputed exactly as exp_pack and
// the pipelined step compute it.
struct ProbOf {
  const f32x16& s;
  float c2, m;
  __device__ __forceinline__ float operator()(int v) const {
    return __builtin_amdgcn_exp2f(fmaf(s[v], c2, -m));
  }
};

// A split's unnormalised output row (fp32) and its (running max, denominator)
// into the split workspace, for attend_combine_kernel.
__device__ __forceinline__ void write_split(const AttendArgs& a, const Head& hd, int qrow, int hf,
                                            const f32x16 (&o)[4], float m, float l) {
  if (qrow >= hd.n) return;
  const int64_t row = (int64_t(hd.split) * a.B + hd.b) * hd.n * a.H + int64_t(qrow) * a.H + hd.h;
  float* op = a.ws_o + row * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int kp = 0; kp < 4; ++kp)
      *reinterpret_cast<float4*>(op + 32 * db + 8 * kp + 4 * hf) =
          make_float4(o[db][4 * kp], o[db][4 * kp + 1], o[db][4 * kp + 2], o[db][4 * kp + 3]);
  if (hf == 0) a.ws_ml[row] = make_float2(m, l);
}

// The head's segment bounds for S-CAS: cache rows held before scale src.
// The table is not written while a launch runs, so it is read through the
// constant address space: the loads are scalar (their waits do not wait for
// the tiles in flight, as vector loads' would) and land in scalar registers.
typedef __attribute__((address_space(4))) const int32_t const_i32;
__device__ __forceinline__ int seg_lo(const Head& hd, int src) {
  return ((const const_i32*)hd.lenb)[src];
}

// Adds this lane's probabilities of keys [kblk, kblk + 32) to the
// accumulator of every source segment they fall in.  Source src < step
// covers cache rows [lenb[src], lenb[src+1]); the current scale covers
// [Lc, Ltot).
template <typename Prob>
__device__ __forceinline__ void scas_add(const AttendArgs& a, const Head& hd, int hf,
                                         const Prob& prob, float psum, int kblk,
                                         float (&sc)[kMaxScales]) {
#pragma unroll
  for (int src = 0; src < kMaxScales; ++src) {
    if (src > a.step) continue;  // (not break: the loop must unroll fully, sc stays in registers)
    const int lo = seg_lo(hd, src);
    const int hi = src < a.step ? seg_lo(hd, src + 1) : hd.Ltot;
    if (lo < hi && lo < kblk + 32 && hi > kblk) {
      float acc = 0.f;
      if (lo <= kblk && hi >= kblk + 32) {
        acc = psum;
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kblk + key_of(v, hf);
          acc += (key >= lo && key < hi) ? prob(v) : 0.f;
        }
      }
      sc[src] += acc;
    }
  }
}

// Per-lane S-CAS accumulators: sc[src] is this query's unnormalised mass on
// source src, relative to the running max.  Most 32-key blocks lie inside
// one source segment, so their mass goes to one open accumulator (acc, for
// source cur, whose keys end at hi); only a block that crosses a segment
// boundary walks the segment list (scas_add) and moves the open segment on,
// at most once per source per workgroup.  The per-source sums are indexed
// only by unrolled loops (cur is wave-uniform), so they stay in registers.
struct ScasAcc {
  float sc[kMaxScales];
  float acc;
  int cur, hi;
};

__device__ __forceinline__ int seg_hi(const AttendArgs& a, const Head& hd, int src) {
  return src < a.step ? seg_lo(hd, src + 1) : hd.Ltot;
}

// The open segment: the first source whose keys end after key k.
__device__ __forceinline__ void scas_open(const AttendArgs& a, const Head& hd, ScasAcc& x, int k) {
  int src = 0;
  while (src < a.step && seg_hi(a, hd, src) <= k) ++src;
  x.cur = src;
  x.hi = seg_hi(a, hd, src);
}

__device__ __forceinline__ void scas_init(const AttendArgs& a, const Head& hd, ScasAcc& x) {
#pragma unroll
  for (int s = 0; s < kMaxScales; ++s) x.sc[s] = 0.f;
  x.acc = 0.f;
  scas_open(a, hd, x, 0);
}

__device__ __forceinline__ void scas_flush(ScasAcc& x) {
#pragma unroll
  for (int s = 0; s < kMaxScales; ++s)
    if (s == x.cur) x.sc[s] += x.acc;
  x.acc = 0.f;
}

__device__ __forceinline__ void scas_rescale(ScasAcc& x, float corr) {
#pragma unroll
  for (int s = 0; s < kMaxScales; ++s) x.sc[s] *= corr;
  x.acc *= corr;
}

// Adds one 32-key block (keys kblk.., this lane's probabilities prob(v),
// v = 0..15, summing to psum); blocks are added in key order.
template <typename Prob>
__device__ __forceinline__ void scas_block(const AttendArgs& a, const Head& hd, int hf,
                                           const Prob& prob, float psum, int kblk, ScasAcc& x) {
  if (kblk + 32 <= x.hi) {
    x.acc += psum;
    return;
  }
  scas_flush(x);
  scas_add(a, hd, hf, prob, psum, kblk, x.sc);
  scas_open(a, hd, x, kblk + 32);
}

// Sums each source's normalised mass over the workgroup's valid queries and
// writes the workgroup's partial row.
template <int WAVES>
__device__ __forceinline__ void scas_reduce(const AttendArgs& a, const Head& hd, int qrow,
                                            float inv, const ScasAcc& x, float* sRed) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int src = 0; src < kMaxScales; ++src) {
    const float own = x.sc[src];
    float m = (own + __shfl_xor(own, 32)) * inv;
    m = qrow < hd.n ? m : 0.f;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) m += __shfl_xor(m, off);
    if (lane == 0) sRed[wave * kMaxScales + src] = m;
  }
  __syncthreads();
  if (threadIdx.x < kMaxScales) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) tot += sRed[w * kMaxScales + threadIdx.x];
    const int64_t row = (int64_t(hd.b) * a.H + hd.h) * a.n_qtiles + hd.qt;
    a.partials[row * kMaxScales + threadIdx.x] = tot;
  }
}

// ---------------------------------------------------------------------------
// 128 queries per workgroup, 32 per wave, two workgroups per CU.
// ---------------------------------------------------------------------------
// With S-CAS the per-lane source accumulators do not fit beside the rest in
// 256 registers, so that variant runs one wave per SIMD instead of spilling.
template <bool SCAS, bool PAGED>
__global__ __launch_bounds__(256, SCAS ? 1 : 2) void attend_q128_kernel(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * VSTR];
  __shared__ float sRed[SCAS ? 4 * kMaxScales : 1];

  const Head hd = setup(a);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, hf = lane >> 5;
  const int qrow = hd.qt * 128 + wave * 32 + j;
  Vec16 qf[8];
  load_q(hd, qrow, hf, qf);

  u32x4 kreg[4], vreg[4];
  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  ScasAcc sa;
  if constexpr (SCAS) scas_init(a, hd, sa);

  const int kb_row = permuted_row(j);
  const int Ltot = hd.Ltot;
  const float c2 = a.scale_log2;
  // Key tiles [t_lo, t_hi): this tiling is never split.
  const int t_lo = 0;
  const int t_hi = (Ltot + BN - 1) / BN;

  char* const kc_w = const_cast<char*>(hd.ks.cache);
  char* const vc_w = const_cast<char*>(hd.vs.cache);
  int next_append = first_append_tile(a, hd, t_lo);
  auto append_tile = [&](int t) {
    if (hd.append && t == next_append) {
      append_rows<PAGED>(hd.ks, kc_w, t * BN, tid >> 4, 16, tid & 15, kreg);
      append_rows<PAGED>(hd.vs, vc_w, t * BN, 4 * (tid & 15), 1, tid >> 4, vreg);
      next_append += a.n_qtiles;
    }
  };

  if (t_lo < t_hi) {
    load_k<PAGED>(hd.ks, t_lo * BN, tid, kreg);
    load_v<PAGED>(hd.vs, t_lo * BN, tid, vreg);
    store_k(sK[0], tid, kreg);
    store_v(sV[0], tid, vreg);
    append_tile(t_lo);
    if (t_lo + 1 < t_hi) {
      load_k<PAGED>(hd.ks, (t_lo + 1) * BN, tid, kreg);
      load_v<PAGED>(hd.vs, (t_lo + 1) * BN, tid, vreg);
    }
  }
  __syncthreads();

  for (int it = t_lo; it < t_hi; ++it) {
    const int k0 = it * BN;
    const int buf = (it - t_lo) & 1;
    if (it + 1 < t_hi) {
      store_k(sK[buf ^ 1], tid, kreg);
      store_v(sV[buf ^ 1], tid, vreg);
      append_tile(it + 1);
    }
    if (it + 2 < t_hi) {
      load_k<PAGED>(hd.ks, k0 + 2 * BN, tid, kreg);
      load_v<PAGED>(hd.vs, k0 + 2 * BN, tid, vreg);
    }

    // Scores S^T for two 32-key blocks.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const uint16_t* kp = &sK[buf][(32 * kb + kb_row) * KSTR + 8 * hf];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        Vec16 kf;
        kf.u = *reinterpret_cast<const u32x4*>(kp + 16 * kk);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.b, qf[kk].b, s[kb], 0, 0, 0);
      }
    }

    if (k0 + BN > Ltot) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (k0 + 32 * kb + key_of(v, hf) >= Ltot) s[kb][v] = -INFINITY;
    }

    // Exponentials against the running max, then the lazy-max check (the
    // same rule as the 256-query kernel; no value product of this tile has
    // been issued yet, so a rescale covers all of the accumulators).
    Vec16 pb[2][2];
    float ps[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) ps[kb] = exp_pack<SCAS>(s[kb], c2, m_run, pb[kb]);
    if (__builtin_expect(__any(!(ps[0] + ps[1] <= kSumTrigger)), 0)) {
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, s[kb][v]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mt = tmax * c2;
      if (__any(mt > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mt);
        const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= corr;
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[db] *= corr;
        if constexpr (SCAS) scas_rescale(sa, corr);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) ps[kb] = exp_pack<SCAS>(s[kb], c2, m_run, pb[kb]);
      }
    }
    l_run += ps[0] + ps[1];
    if constexpr (SCAS) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) scas_block(a, hd, hf, ProbOf{s[kb], c2, m_run}, ps[kb], k0 + 32 * kb, sa);
    }

#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        Vec16 vf;
        vf.u = *reinterpret_cast<const u32x4*>(&sV[buf][(32 * db + j) * VSTR + 16 * st + 8 * hf]);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf.b, pb[st >> 1][st & 1].b, oacc[db], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  const float inv = 1.f / (l_run + __shfl_xor(l_run, 32));
  store_out(a, hd, qrow, hf, oacc, inv);
  if constexpr (SCAS) {
    scas_flush(sa);
    scas_reduce<4>(a, hd, qrow, inv, sa, sRed);
  }
}

// Merges the splits of one output row: with M the largest split max and
// w_s = 2^(m_s - M), out = sum_s w_s O_s / sum_s w_s l_s, added in split
// order.  32 lanes per row, 4 dims per lane.  Every split's (max, sum) and
// output slice are loaded before any is used, so a row costs one memory
// latency rather than one per split; MAXS (>= n_split) bounds the registers
// this takes.
template <int MAXS>
__global__ __launch_bounds__(256) void attend_combine_kernel(const float* ws_o, const float2* ws_ml,
                                                             uint16_t* out, int64_t rows, int n_split) {
  const int64_t row = int64_t(blockIdx.x) * 8 + (threadIdx.x >> 5);
  if (row >= rows) return;
  const int d0 = 4 * (threadIdx.x & 31);
  float2 ml[MAXS];
  float4 o[MAXS];
#pragma unroll
  for (int sp = 0; sp < MAXS; ++sp) {
    if (sp < n_split) {
      ml[sp] = ws_ml[sp * rows + row];
      o[sp] = *reinterpret_cast<const float4*>(ws_o + (sp * rows + row) * D + d0);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < MAXS; ++sp)
    if (sp < n_split) M = fmaxf(M, ml[sp].x);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int sp = 0; sp < MAXS; ++sp) {
    if (sp < n_split) {
      const float w = __builtin_amdgcn_exp2f(ml[sp].x - M);
      L = fmaf(w, ml[sp].y, L);
      acc.x = fmaf(w, o[sp].x, acc.x);
      acc.y = fmaf(w, o[sp].y, acc.y);
      acc.z = fmaf(w, o[sp].z, acc.z);
      acc.w = fmaf(w, o[sp].w, acc.w);
    }
  }
  const float inv = 1.f / L;
  uint2 wv;
  wv.x = pack_bf16x2(acc.x * inv, acc.y * inv);
  wv.y = pack_bf16x2(acc.z * inv, acc.w * inv);
  *reinterpret_cast<uint2*>(out + row * D + d0) = wv;
}

// ---------------------------------------------------------------------------
// 256 queries per workgroup of 8 waves, 32 per wave, software-pipelined.
// ---------------------------------------------------------------------------
// SPLIT: the launch splits each head's key range (a.n_split > 1); a separate
// instantiation, so the unsplit kernel carries no split code.
// PRE (never with S-CAS): Q scaled by alpha * log2 e and rounded to bf16,
// with the fast mode; only for alpha * log2 e <= kPreMaxScale.
// PAGED: the cache is a pool whose rows the per-(step, layer, head) map
// gives (tile loads take per-lane pool offsets).
template <bool SCAS, bool SPLIT, bool PAGED, bool PRE>
__global__ __launch_bounds__(512) void attend_q256_kernel(AttendArgs a) {
  // LDS buffers per operand: tiles in pairs (PD = 2, one barrier per two
  // tiles) in four.
  constexpr int NBUF = 4;
  constexpr int PD = NBUF - 2;
  __shared__ __attribute__((aligned(16))) uint16_t sK[NBUF][BN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sV[NBUF][BN * VROW];
  __shared__ float sRed[SCAS ? 8 * kMaxScales : 1];

  const Head hd = setup(a);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, hf = lane >> 5;
  // Waves 4-7 stage K, waves 0-3 V (wave-uniform, read as a scalar so that
  // the loads' count is one).
  const bool kstager = __builtin_amdgcn_readfirstlane(tid) >= 256;
  const int stid = tid & 255;
  const int qrow = hd.qt * 256 + wave * 32 + j;
  Vec16 qf[8];
  load_q(hd, qrow, hf, qf);
  // Without S-CAS, Q is scaled by alpha * log2 e once (rounded to bf16), so
  // the score products come out in base-2 units.  While a wave's scores stay
  // within +-kFastRange of zero no running max is subtracted at all (fast
  // mode): the exponentials take the accumulators as they are.  A block whose
  // probabilities sum above 2^kFastRange (or a first block outside the range)
  // moves the wave to the running-max form at the end of its key tile.
  static_assert(!(PRE && SCAS), "S-CAS keeps the exact bf16 Q");
  if constexpr (PRE) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = qf[kk].w[w];
        const float lo = __builtin_bit_cast(float, x << 16) * a.scale_log2;
        const float hi = __builtin_bit_cast(float, x & 0xFFFF0000u) * a.scale_log2;
        qf[kk].w[w] = pack_bf16x2(lo, hi);
      }
  }
  bool fast = false;

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  ScasAcc sa;
  if constexpr (SCAS) scas_init(a, hd, sa);

  const int kb_row = permuted_row(j);
  const int Ltot = hd.Ltot;
  const float c2 = PRE ? 1.f : a.scale_log2;
  // Key tiles [t_lo, t_hi) of this workgroup's split.
  const int ntiles_all = (Ltot + BN - 1) / BN;
  const int per_split = SPLIT ? (ntiles_all + a.n_split - 1) / a.n_split : ntiles_all;
  const int t_lo = SPLIT ? hd.split * per_split : 0;
  const int t_hi = SPLIT ? min(ntiles_all, t_lo + per_split) : ntiles_all;
  if (SPLIT && t_lo >= t_hi) {
    // A head with fewer key tiles than splits: an empty partial (weight 0 in
    // the merge).  The whole workgroup leaves before any barrier.
    write_split(a, hd, qrow, hf, o, -INFINITY, 0.f);
    return;
  }

  auto qk = [&](const uint16_t* Kt, int kb, f32x16& s) {
    s = f32x16{};
    const uint16_t* kp = Kt + (32 * kb + kb_row) * KSTR + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      Vec16 kf;
      kf.u = *reinterpret_cast<const u32x4*>(kp + 16 * kk);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.b, qf[kk].b, s, 0, 0, 0);
    }
  };
  // This lane's share of the direct loads: K by waves 4-7, V by waves 0-3.
  const int stw = __builtin_amdgcn_readfirstlane(wave) & 3;
  DmaLane dma;
  // Pooled caches: pool rows of the rows this wave loads in its next burst
  // (one tile, or two with paired tiles).
  unsigned mv[2][5];
  if (kstager) dma = dma_lane<kKChunks, kKLoads>(stw, lane, hd.tokb);
  else dma = dma_lane<kVChunks, kVLoads>(stw, lane, hd.tokb);
  const int voff = vtr_lane_offset(lane);
  // V^T fragment (dims 32 db + j, keys 16 st + 8 hf + 0..7) of a staged V tile.
  auto vfrag = [&](const uint16_t* Vt, int st, int db) {
    Vec16 vf;
    vf.u = vfrag_tr(Vt, voff, st, db);
    return vf;
  };
  auto pv = [&](const uint16_t* Vt, int kb, const Vec16 (&p)[2]) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int st = 2 * kb + half;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const Vec16 vf = vfrag(Vt, st, db);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf.b, p[half].b, o[db], 0, 0, 0);
      }
    }
  };
  // Keys past the end of the last tile score -inf.
  auto mask_tail = [&](f32x16& s, int kblk) {
    if (kblk + 32 > Ltot) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (kblk + key_of(v, hf) >= Ltot) s[v] = -INFINITY;
    }
  };
  // Lazy max, checked after the exponentials: they are taken against the
  // running max, and only when some probability may exceed 2^8 (a lane's sum
  // above 2^7 covers it, bf16 rounding included; a NaN sum, from the first
  // unit's infinite max, too) does the wave take the block's exact max.  Where
  // that lies more than 2^8 above the running max, the max is raised, the
  // output accumulators (which already hold the previous unit's value
  // product), the denominator and the S-CAS sums are rescaled, and the unit's
  // exponentials are taken again.
  // Fast mode (scores relative to m_run, which is 0 until the wave leaves
  // the mode): a block sum above 2^kFastRange raises m_run by the block's
  // max (where positive), rescales, and ends fast mode after this tile; the
  // next unit's scores, when this tile still takes their exponentials
  // (shift_next), are moved to the new reference.
  auto settle_fast = [&](const f32x16& s, Vec16 (&p)[2], float& psum, f32x16& snext,
                         bool shift_next) {
    if (__builtin_expect(__any(!(psum <= kFastTrigger)), 0)) {
      float t = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) t = fmaxf(t, s[v]);
      t = fmaxf(t, __shfl_xor(t, 32));
      const float d = fmaxf(t, 0.f);
      m_run += d;
      const float corr = __builtin_amdgcn_exp2f(-d);
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= corr;
      psum = exp_pack<SCAS>(s, 1.f, d, p);
      if (shift_next) {
#pragma unroll
        for (int v = 0; v < 16; ++v) snext[v] -= d;
      }
      fast = false;
    }
    l_run += psum;
  };
  auto settle = [&](const f32x16& s, Vec16 (&p)[2], float& psum) {
    if (__builtin_expect(__any(!(psum <= kSumTrigger)), 0)) {
      float t = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) t = fmaxf(t, s[v]);
      t = fmaxf(t, __shfl_xor(t, 32));
      const float mt = t * c2;
      if (__any(mt > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mt);
        const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= corr;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= corr;
        if constexpr (SCAS) scas_rescale(sa, corr);
        psum = exp_pack<SCAS>(s, c2, m_run, p);
      }
    }
    l_run += psum;
  };
  // One pipelined step in 16 fixed slots: slot i issues the LDS read of the
  // fragment two slots ahead, one MFMA (score product of the next unit in
  // slots 0-7, value product of the previous unit in slots 8-15: the next
  // step's exponentials read the score product, which so completes earlier;
  // measured 1% fewer cycles than the other order) and 1/16 of the
  // current unit's exponentials, packing and denominator.
  auto step = [&](const uint16_t* Vt, int kbv, const Vec16 (&pprev)[2], auto do_pv_c,
                  const uint16_t* Kt, int kbk, f32x16& snext, auto do_qk_c, f32x16& s,
                  Vec16 (&p)[2], auto fast_c) {
    constexpr bool DO_PV = decltype(do_pv_c)::value;
    constexpr bool DO_QK = decltype(do_qk_c)::value;
    constexpr bool FAST = decltype(fast_c)::value;
    const uint16_t* kp = Kt + (32 * kbk + kb_row) * KSTR + 8 * hf;
    auto frag = [&](int i) {
      Vec16 f;
      if (i < 8) {
        const int half = i >> 2, db = i & 3;
        f = vfrag(Vt, 2 * kbv + half, db);
      } else {
        f.u = *reinterpret_cast<const u32x4*>(kp + 16 * (i - 8));
      }
      return f;
    };
    // Operation op_of(i) of slot i: 0-7 value product fragments, 8-15 score
    // product fragments; seq lists the enabled ones in slot order (all
    // compile-time: the loops unroll).
    auto op_of = [](int i) { return (i + 8) & 15; };
    auto enabled = [](int op) { return op < 8 ? DO_PV : DO_QK; };
    int seq[16];
    int nen = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (enabled(op_of(i))) seq[nen++] = op_of(i);
    Vec16 fr[3];
    if (nen > 0) fr[0] = frag(seq[0]);
    if (nen > 1) fr[1] = frag(seq[1]);
    if constexpr (DO_QK) snext = f32x16{};
    float psum = 0.f, l1 = 0.f, e[2];
    int k = 0;  // enabled slots so far
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int op = op_of(i);
      if (enabled(op)) {
        if (k + 2 < nen) fr[(k + 2) % 3] = frag(seq[k + 2]);
        __builtin_amdgcn_sched_barrier(0);
        if (op < 8) {
          const int half = op >> 2, db = op & 3;
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[k % 3].b, pprev[half].b, o[db], 0, 0, 0);
        } else {
          snext = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[k % 3].b, qf[op - 8].b, snext, 0, 0, 0);
        }
        ++k;
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (FAST) e[i & 1] = __builtin_amdgcn_exp2f(s[i]);
      else e[i & 1] = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -m_run));
      if (i & 1) {
        const int half = i >> 3, w = (i & 7) >> 1;
        p[half].w[w] = pack_bf16x2(e[0], e[1]);
        if constexpr (SCAS) {
          psum += e[0];
          l1 += e[1];
        } else {
          if (w & 1) l1 = add_bf16x2(p[half].w[w], l1);
          else psum = add_bf16x2(p[half].w[w], psum);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return psum + l1;
  };

  f32x16 s0, s1;
  Vec16 p0[2], p1[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) p1[half].u = u32x4{0, 0, 0, 0};

  // Prologue: K(t_lo), K(t_lo + 1), K(t_lo + 2) (waves 4-7) and V(t_lo),
  // V(t_lo + 1) (waves 0-3) in LDS buffers 0, 1, 2.  Every split holds at
  // least one tile.
  char* const kc_w = const_cast<char*>(hd.ks.cache);
  char* const vc_w = const_cast<char*>(hd.vs.cache);
  const int k_lo = t_lo * BN;
  // Whether this workgroup writes key tile x of the current scale into the
  // cache (fused append: tile x falls to the q-tile x mod n_qtiles).
  auto owns = [&](int x) { return hd.append && x % a.n_qtiles == hd.qt; };
  // Pooled caches read each tile's pool rows first (map_prefetch), the
  // prologue's tiles one after another and the first burst's ahead.
  if (kstager) {
#pragma unroll
    for (int x = 0; x <= PD; ++x) {
      if (t_lo + x < t_hi) {
        if constexpr (PAGED) map_prefetch(hd.ks, k_lo + x * BN, dma, mv[0]);
        dma_tile<PAGED>(hd.ks, k_lo + x * BN, sK[x], dma, mv[0]);
      }
    }
    if constexpr (PAGED)
#pragma unroll
      for (int x = PD + 1; x <= 2 * PD; ++x)
        if (t_lo + x < t_hi) map_prefetch(hd.ks, k_lo + x * BN, dma, mv[x - PD - 1]);
  } else {
#pragma unroll
    for (int x = 0; x < PD; ++x) {
      if (t_lo + x < t_hi) {
        if constexpr (PAGED) map_prefetch(hd.vs, k_lo + x * BN, dma, mv[0]);
        dma_tile<PAGED>(hd.vs, k_lo + x * BN, sV[x], dma, mv[0]);
      }
    }
    if constexpr (PAGED)
#pragma unroll
      for (int x = PD; x < 2 * PD; ++x)
        if (t_lo + x < t_hi) map_prefetch(hd.vs, k_lo + x * BN, dma, mv[x - PD]);
  }
  wait_loads();
  barrier_keep_loads();
  if (kstager && owns(t_lo)) append_from_lds<KSTR * 2>(hd.ks, kc_w, k_lo, sK[0], stid);
  // A wave whose 32 queries all lie past the scale's end (the last query tile
  // of a scale that does not fill it) computes nothing: it only stages its
  // share of the tiles and meets the barriers, so its SIMD's other wave has
  // the matrix pipe to itself.
  const bool idle = __builtin_amdgcn_readfirstlane(hd.qt * 256 + wave * 32) >= hd.n;
  if (!idle) qk(sK[0], 0, s0);
  if (PRE && !idle) {
    // The first unit (it always holds a valid key) sets the reference: 0
    // when its exact max lies within +-kFastRange for every query of the
    // wave (the first tile's probabilities are then already those of fast
    // mode, none pending needs converting), else that max.
    mask_tail(s0, k_lo);
    float t = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) t = fmaxf(t, s0[v]);
    t = fmaxf(t, __shfl_xor(t, 32));
    m_run = __all(t >= -kFastRange && t <= kFastRange) ? 0.f : t;
  }

  // One 64-key tile; FIRST (the split's first tile) drops the value product
  // of the absent previous unit, LAST (its last) the score product of the
  // absent next tile and enables the tail mask, which only the head's final
  // tile needs.
  int bk = 0;  // LDS buffer of K(t) and of V(t)
  auto tile = [&](int t, auto first_c, auto last_c, auto fast_c, auto idle_c) {
    constexpr bool FIRST = decltype(first_c)::value;
    constexpr bool LAST = decltype(last_c)::value;
    constexpr bool FAST = decltype(fast_c)::value;
    constexpr bool IDLE = decltype(idle_c)::value;
    const int k0 = t * BN;
    const int bn = bk == NBUF - 1 ? 0 : bk + 1;
    const int bp = bk == 0 ? NBUF - 1 : bk - 1;
    if constexpr (PD == 2) {
      // Paired tiles, odd tile t (no barrier): the V-staging waves load
      // V(t + 1) and V(t + 2) into the buffers of V(t - 3) and V(t - 2), both
      // last read in step a of tile t - 1, before the previous barrier.  The
      // K-staging waves load at the even tiles' barriers, so the two waves of
      // a SIMD never issue their loads at the same time (measured: 6% fewer
      // cycles than both at the barrier).
      if (((t - t_lo) & 1) == 1 && !kstager) {
#pragma unroll
        for (int x = 1; x <= 2; ++x)
          if (t + x < t_hi) dma_tile<PAGED>(hd.vs, k0 + x * BN, sV[(bk + x) % NBUF], dma, mv[x - 1]);
        if constexpr (PAGED)
#pragma unroll
          for (int x = 3; x <= 4; ++x)
            if (t + x < t_hi) map_prefetch(hd.vs, k0 + x * BN, dma, mv[x - 3]);
      }
    }
    // step a: unit (t, keys 0..31)
    if constexpr (!IDLE) {
      if constexpr (LAST) mask_tail(s0, k0);
      float e0 = step(sV[bp], 1, p1, std::integral_constant<bool, !FIRST>{}, sK[bk], 1, s1,
                      std::true_type{}, s0, p0, fast_c);
      if constexpr (FAST) settle_fast(s0, p0, e0, s1, true);
      else settle(s0, p0, e0);
      if constexpr (SCAS) scas_block(a, hd, hf, ProbOf{s0, c2, m_run}, e0, k0, sa);
    }
    if constexpr (PD == 2) {
      // Paired tiles, one barrier every second tile (t - t_lo even).  By the
      // barrier of tile t, K(t + 1), K(t + 2), V(t) and V(t + 1) have landed
      // (loaded two tiles back, or in the prologue; each wave waits for its
      // own loads, the barrier publishes them): steps b(t), a(t + 1), b(t + 1)
      // and a(t + 2) read nothing else.  Then the appends of those tiles that
      // fall to this workgroup, and the K-staging waves' loads of K(t + 3) and
      // K(t + 4) into the buffers of K(t - 1) and K(t), both last read in step
      // a of tile t at the latest (V: at the start of tile t + 1).
      if (((t - t_lo) & 1) == 0) {
        wait_loads();
        barrier_keep_loads();
        if (kstager) {
#pragma unroll
          for (int x = 1; x <= 2; ++x)
            if (t + x < t_hi && owns(t + x))
              append_from_lds<KSTR * 2>(hd.ks, kc_w, k0 + x * BN, sK[(bk + x) % NBUF], stid);
#pragma unroll
          for (int x = 3; x <= 4; ++x)
            if (t + x < t_hi) dma_tile<PAGED>(hd.ks, k0 + x * BN, sK[(bk + x) % NBUF], dma, mv[x - 3]);
          if constexpr (PAGED)
#pragma unroll
            for (int x = 5; x <= 6; ++x)
              if (t + x < t_hi) map_prefetch(hd.ks, k0 + x * BN, dma, mv[x - 5]);
        } else {
#pragma unroll
          for (int x = 0; x <= 1; ++x)
            if (t + x < t_hi && owns(t + x))
              append_from_lds<VROW * 2>(hd.vs, vc_w, k0 + x * BN, sV[(bk + x) % NBUF], stid);
        }
      }
    }

    // step b: unit (t, keys 32..63)
    if constexpr (!IDLE) {
      if constexpr (LAST) mask_tail(s1, k0 + 32);
      float e1 = step(sV[bk], 0, p0, std::true_type{}, sK[bn], 0, s0,
                      std::integral_constant<bool, !LAST>{}, s1, p1, fast_c);
      if constexpr (FAST) settle_fast(s1, p1, e1, s0, false);
      else settle(s1, p1, e1);
      if constexpr (SCAS) scas_block(a, hd, hf, ProbOf{s1, c2, m_run}, e1, k0 + 32, sa);
    }
    bk = bn;
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (idle) {
    // The same tiles, so the same loads, appends and barriers.
    for (int t = t_lo; t < t_hi; ++t) tile(t, F_{}, F_{}, F_{}, T_{});
  } else if (t_hi - t_lo == 1) {
    tile(t_lo, T_{}, T_{}, F_{}, F_{});
  } else {
    tile(t_lo, T_{}, F_{}, F_{}, F_{});
    int t = t_lo + 1;
    if constexpr (PRE) {
      // Where the reference is still 0 after the first tile for every query
      // of the wave, the middle tiles run in fast mode until a block leaves
      // the range.
      fast = __all(m_run == 0.f);
      for (; fast && t + 1 < t_hi; ++t) tile(t, F_{}, F_{}, T_{}, F_{});
    }
    for (; t + 1 < t_hi; ++t) tile(t, F_{}, F_{}, F_{}, F_{});
    tile(t_hi - 1, F_{}, T_{}, F_{}, F_{});
  }
  if (!idle) pv(sV[bk == 0 ? NBUF - 1 : bk - 1], 1, p1);

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if constexpr (SPLIT) {
    // Unnormalised output and (max, denominator) of this split, merged later.
    write_split(a, hd, qrow, hf, o, m_run, l_tot);
    return;
  }
  const float inv = 1.f / l_tot;
  store_out(a, hd, qrow, hf, o, inv);
  if constexpr (SCAS) {
    scas_flush(sa);
    scas_reduce<8>(a, hd, qrow, inv, sa, sRed);
  }
}

}  // namespace

// Plan model, in microseconds, fitted to every (rows, splits) choice for
// scales 2-11 of the 16-head full-cache layer at batch 1 and 8 on the MI355X
// (random bf16 data): a 64-key tile of a 256-query workgroup (one resident
// per CU) takes kTile256, of a 128-query workgroup (two resident per CU)
// kTile128; a workgroup's set-up (query load, first staging) adds kSetup*
// tiles; a split launch adds the merge, kMerge plus kMergeRow per partial
// output row.  Costs common to every choice (the launch) are left out.  A
// split may be a single tile: timed inside whole generation passes, scale 5
// of that layer at batch 1 (5 tiles, 16 workgroups) took 15.0-16.5 us in 5
// one-tile splits against 20.6 us unsplit.
namespace {
constexpr double kTile256 = 1.80;
constexpr double kTile128 = 2.00;
constexpr double kSetup256 = 0.17;
constexpr double kSetup128 = 0.0;
constexpr double kMerge = 3.15;
constexpr double kMergeRow = 0.00024;
constexpr int kMinTilesPerSplit = 1;
}  // namespace

AttendPlan attend_bf16_plan(int B, int H, int n, int max_keys, bool allow_split) {
  const int tiles = std::max(1, (max_keys + BN - 1) / BN);
  AttendPlan best{256, 1};
  double best_cost = 1e300;
  for (const int rows : {256, 128}) {
    const int64_t wg = int64_t(B) * H * ((n + rows - 1) / rows);
    const int64_t slots = rows == 256 ? 256 : 512;
    const double tile_us = rows == 256 ? kTile256 : kTile128;
    const double setup = rows == 256 ? kSetup256 : kSetup128;
    for (int sp = 1; sp <= (rows == 256 ? kMaxSplits : 1); ++sp) {
      if (sp > 1 && (!allow_split || tiles < kMinTilesPerSplit * sp)) break;
      const double rounds = double((wg * sp + slots - 1) / slots);
      const double per_split = double((tiles + sp - 1) / sp);
      double cost = rounds * (per_split + setup) * tile_us;
      if (sp > 1) cost += kMerge + kMergeRow * double(sp) * B * n * H;
      if (cost < best_cost * (1 - 1e-9)) {
        best_cost = cost;
        best = AttendPlan{rows, sp};
      }
    }
  }
  return best;
}

namespace {

template <bool PAGED>
hipError_t launch_attend(const AttendArgs& a, bool scas, hipStream_t s) {
  const int64_t blocks = int64_t(a.B) * a.H * a.n_qtiles * a.n_split;
  const bool pre = a.scale_log2 <= kPreMaxScale;
  if (a.n_split > 1) {
    if (pre)
      hipLaunchKernelGGL((attend_q256_kernel<false, true, PAGED, true>), dim3(unsigned(blocks)), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((attend_q256_kernel<false, true, PAGED, false>), dim3(unsigned(blocks)), dim3(512), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t out_rows = int64_t(a.B) * a.n * a.H;
    const dim3 grid(unsigned((out_rows + 7) / 8));
    uint16_t* out = static_cast<uint16_t*>(a.out);
    if (a.n_split <= 4)
      hipLaunchKernelGGL(attend_combine_kernel<4>, grid, dim3(256), 0, s, a.ws_o, a.ws_ml, out, out_rows, a.n_split);
    else if (a.n_split <= 8)
      hipLaunchKernelGGL(attend_combine_kernel<8>, grid, dim3(256), 0, s, a.ws_o, a.ws_ml, out, out_rows, a.n_split);
    else
      hipLaunchKernelGGL(attend_combine_kernel<kMaxSplits>, grid, dim3(256), 0, s, a.ws_o, a.ws_ml, out,
                         out_rows, a.n_split);
    return hipGetLastError();
  }
  if (a.rows == 256) {
    if (scas)
      hipLaunchKernelGGL((attend_q256_kernel<true, false, PAGED, false>), dim3(unsigned(blocks)), dim3(512), 0, s, a);
    else if (pre)
      hipLaunchKernelGGL((attend_q256_kernel<false, false, PAGED, true>), dim3(unsigned(blocks)), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((attend_q256_kernel<false, false, PAGED, false>), dim3(unsigned(blocks)), dim3(512), 0, s, a);
  } else {
    if (scas)
      hipLaunchKernelGGL((attend_q128_kernel<true, PAGED>), dim3(unsigned(blocks)), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((attend_q128_kernel<false, PAGED>), dim3(unsigned(blocks)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_bf16_d128(const AttendArgs& a, bool scas, hipStream_t s) {
  const int rows = a.rows;
  const int64_t blocks = int64_t(a.B) * a.H * a.n_qtiles * a.n_split;
  if ((rows != 128 && rows != 256) || a.n_qtiles != (a.n + rows - 1) / rows ||
      (a.order && a.B % kXcds != 0))
    return hipErrorInvalidValue;
  if (a.n_split < 1 || a.n_split > kMaxSplits ||
      (a.n_split > 1 && (scas || rows != 256 || !a.ws_o || !a.ws_ml)))
    return hipErrorInvalidValue;
  if ((a.map != nullptr) != (a.mapoff != nullptr) || (a.map && a.append))
    return hipErrorInvalidValue;
  if (!grid_fits(blocks, 512) || !grid_fits((int64_t(a.B) * a.n * a.H + 7) / 8, 256))
    return hipErrorInvalidConfiguration;
  return a.map ? launch_attend<true>(a, scas, s) : launch_attend<false>(a, scas, s);
}

}  // namespace hk
