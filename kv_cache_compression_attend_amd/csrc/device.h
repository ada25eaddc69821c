// Device-side types and launch descriptors shared by the kernels and the
// host launch code.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attend.h"

namespace hk {

// Copy geometry shared by the compaction kernels and the host code that
// sizes their grids: a workgroup of kCopyThreads lanes moves one block per
// tensor in a single pass, kCopyBlockBytes (4 16-byte vectors per lane in
// flight) or kCopyBlockBytesLarge (8).  Measured on the MI355X: 4 per lane is
// the fastest plain contiguous copy and the faster compaction of launches
// with few head runs; 8 per lane the faster one when a launch has at least
// kCopyLargeMinBlocks blocks of the large size.  The in-place gather walks its
// region in chunks of kGatherChunkBytes per column part, one pass each; a
// part is at most kGatherPartBytes of every row.  Scales that most heads
// store are copied in token blocks (contiguous reads across all heads) when a
// layer has at most kRowsMaxHeads heads (their destinations sit in LDS), at
// least kRowsTokens tokens and half a block per workgroup where a block holds
// that many.
constexpr int kCopyThreads = 256;
constexpr int kCopyBlockBytes = 16384;
constexpr int kCopyBlockBytesLarge = 32768;
constexpr int64_t kCopyLargeMinBlocks = 16384;
constexpr int kGatherChunkBytes = 32768;
constexpr int kGatherPartBytes = 128;
constexpr int kRowsMaxHeads = 1024;
constexpr int kRowsTokens = 2;

// One kept (layer, head) segment of a completed scale, to be copied into the cache.
struct CopyDesc {
  int64_t dst;            // byte offset of row len_before(l,h,t) of (l,h,b=0)
  int32_t cap;            // rows per batch entry of (l,h)
  int32_t head;
  int32_t layer;
  int32_t pad;
};

struct CompactArgs {
  const CopyDesc* desc;   // descriptors of this launch
  const uint8_t* kcur;    // byte views
  const uint8_t* vcur;
  uint8_t* kcache;
  uint8_t* vcache;
  int64_t layer_stride_bytes;
  int n_desc, B, n, H;
  int layer_begin;        // layer whose tensor starts at kcur / vcur
  int row_bytes;          // D * element size, a multiple of 16
  int rows_per_block;
  int chunks;             // row blocks per (desc, b)
};

// Token-block compaction: a workgroup copies `rows` consecutive tokens of one
// (layer, batch entry) for every head at once, reading them contiguously
// ([n][H][D] source) and writing each stored head's run to its cache rows.
struct RowsArgs {
  const int64_t* dst;     // [layers][H] byte offset of row len_before of (l, h, b=0); -1: not stored
  const int32_t* cap;     // [layers][H] rows per batch entry
  const uint8_t* kcur;
  const uint8_t* vcur;
  uint8_t* kcache;
  uint8_t* vcache;
  int64_t layer_stride_bytes;
  int n_layers, B, n, H;
  int row_bytes;          // a multiple of 16
  int rows;               // tokens per workgroup
};

// One stored (layer, head) segment of a completed scale in a pooled cache:
// its n rows go to pool rows rows[rows_first + i], i < n (the same rows in
// every batch entry's pool).
struct PoolDesc {
  int64_t rows_first;
  int32_t head;
  int32_t layer;
};

struct PoolArgs {
  const PoolDesc* desc;   // descriptors of this launch
  const int32_t* rows;    // pool rows of every stored segment
  const uint8_t* kcur;    // byte views, [B][n][H][D] per layer
  const uint8_t* vcur;
  uint8_t* kpool;         // [B][pool_rows][D]
  uint8_t* vpool;
  int64_t layer_stride_bytes;
  int64_t pool_rows;
  int n_desc, B, n, H;
  int layer_begin;        // layer whose tensor starts at kcur / vcur
  int row_bytes;          // 16 << cpr_shift
  int cpr_shift;
  int rows_per_block;     // kCopyBlockBytes / row_bytes
  int chunks;             // row blocks per (desc, b)
};

// One (layer, head) whose cache loses segments at a step: the held segments
// that outlive the step move down over the dropped ones.  The moves are runs
// (dst row, src row, rows) in ascending order with dst < src, covering
// destination rows [dst_begin, dst_end) without gaps.
struct GatherRun {
  int32_t dst, src, rows;
};

struct GatherDesc {
  int64_t base;           // byte offset of (l, h, b=0)'s region
  int32_t cap;            // rows per batch entry of (l, h)
  int32_t run_first;      // first run in the launch's run table
  int32_t n_runs;         // <= kMaxScales
  int32_t dst_begin;
  int32_t dst_end;
  int32_t pad;
};

struct GatherArgs {
  const GatherDesc* desc;
  const GatherRun* runs;
  uint8_t* kcache;
  uint8_t* vcache;
  int n_desc, B;
  int row_bytes;          // D * element size, a multiple of 16
  int parts;              // column parts per region: row_bytes = parts * 16 << cpp_shift
  int cpp_shift;          // log2 of the 16-byte vectors per row in one part
  int rows_per_chunk;     // rows moved per barrier interval: kCopyThreads * kGatherItems >> cpp_shift
};

// 4-bit storage (head_dim 128): a row of 128 channels is 64 bytes of codes
// (two per byte, even channel in the low nibble); every (sub-block, channel)
// group has a float2 (step, lo).
constexpr int kQuantD = 128;
constexpr int kQuantRowBytes = kQuantD / 2;

// Quantize one stored segment of a completed scale (one per (l, h) that
// keeps scale t); the workgroup handles sub-block blockIdx.x % m.
struct QuantDesc {
  int64_t code_off;       // bytes: codes of (l, h, b=0), first row of the segment
  int64_t param_off;      // bytes: params of (l, h, b=0), first group of the segment
  int32_t cap;            // rows per batch entry of (l, h)
  int32_t gcap;           // groups per batch entry of (l, h)
  int32_t head;
  int32_t layer;
};

struct QuantArgs {
  const QuantDesc* desc;
  const uint16_t* kcur;   // bf16 [layers][B][n][H][D]
  const uint16_t* vcur;
  uint8_t* kstore;
  uint8_t* vstore;
  int64_t layer_stride;   // elements between consecutive layers' tensors
  int n_desc, m, B, n, H, layer_begin;
  // Split form (nch > 1): each sub-block's rows are cut into nch chunks of
  // kQuantChunkRows; a first launch writes per-chunk (min, max) pairs to
  // minmax [n_desc][m][nch][B][2][D] (float2), a second one combines them
  // and writes the codes.
  int nch;
  float2* minmax;
};
constexpr int kQuantChunkRows = 256;

// Unpack a run of stored rows (one sub-block group, at most kUnpackRows
// rows) of one head into the bf16 scratch that attend reads.
struct UnpackItem {
  int64_t code_off;       // bytes: codes of (l, h, b=0), first row of the run
  int64_t param_off;      // bytes: params of (l, h, b=0), the run's group
  int64_t scratch_off;    // elements: scratch of (h, b=0), first row of the run
  int32_t rows;
  int32_t cap;            // rows per batch entry (codes and scratch)
  int32_t gcap;           // groups per batch entry
  int32_t pad;
};
constexpr int kUnpackRows = 256;

struct UnpackArgs {
  const UnpackItem* items;
  const uint8_t* kstore;
  const uint8_t* vstore;
  uint16_t* kscratch;     // bf16
  uint16_t* vscratch;
  int n_items, B;
};

// Launchers, defined next to their kernels; each returns the launch status.
hipError_t launch_scas_finalize(const float* partials, float* table, int layer, int H, int K,
                                int B, int n, int step, int n_qtiles, hipStream_t s);
hipError_t launch_scas_accumulate(const float* partials, double* table, int layer, int H, int K,
                                  int B, int n, int step, int n_qtiles, hipStream_t s);
hipError_t launch_compact(const CompactArgs& a, hipStream_t s);
hipError_t launch_compact_rows(const RowsArgs& a, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);
hipError_t launch_compact_pooled(const PoolArgs& a, hipStream_t s);
hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);
hipError_t launch_unpack(const UnpackArgs& a, hipStream_t s);

}  // namespace hk
