// Compaction: copy the kept (layer, head) segments of a completed scale into
// the ragged per-head cache (HeatKV project page, Method step 5: pruning
// during inference as new scales are generated; a pruned segment is simply
// never written).
//
// A pure copy, bound by HBM bandwidth.  Two grids: token blocks (a scale
// that most heads store: a workgroup reads a few consecutive whole tokens
// (8-16 KB per tensor), every head's row of each, and writes each head's
// rows to that head's run) and per head (one block of rows of one (segment, batch entry);
// reads stride over the tokens).  Every lane moves 16-byte vectors; per-head
// workgroups keep four (16 KB blocks) or, for launches with many head runs,
// eight (32 KB blocks) loads per tensor in flight before storing, one pass
// per workgroup.  Loads and stores are nontemporal: the source is read once
// and the next reader of the cache is a later attend launch.  Measured on
// the MI355X with 1 GiB of K and of V: a contiguous copy with this structure
// moves 6.1 TB/s (5.75 with ordinary loads), the token-block pattern 5.96,
// the per-head pattern (256 bytes per 4 KB token row) 5.30.
#include "device.h"

namespace hk {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyItems = kCopyBlockBytes / (16 * kCopyThreads);      // per lane per tensor
constexpr int kGatherItems = kGatherChunkBytes / (16 * kCopyThreads);  // per lane per tensor
static_assert(kCopyBlockBytesLarge == 2 * kCopyBlockBytes, "block sizes");

// ITEMS: 16-byte vectors per lane per tensor; a.rows_per_block rows hold
// exactly kCopyThreads * ITEMS of them (one pass).
template <int ITEMS>
__global__ __launch_bounds__(kCopyThreads) void compact_kernel(CompactArgs a) {
  const int chunk = blockIdx.x % a.chunks;
  const int rest = blockIdx.x / a.chunks;
  const int b = rest % a.B;
  const int di = rest / a.B;
  const CopyDesc d = a.desc[di];

  const int cpr = a.row_bytes >> 4;                 // vectors per row
  const int row0 = chunk * a.rows_per_block;
  const int rows = min(a.rows_per_block, a.n - row0);
  const int items = rows * cpr;

  const int64_t tok_stride = int64_t(a.H) * a.row_bytes;
  const int64_t src0 = int64_t(d.layer - a.layer_begin) * a.layer_stride_bytes +
                       (int64_t(b) * a.n + row0) * tok_stride + int64_t(d.head) * a.row_bytes;
  const int64_t dst_row0 = d.dst + (int64_t(b) * d.cap + row0) * a.row_bytes;

  for (int base = threadIdx.x; base < items; base += kCopyThreads * ITEMS) {
    u32x4 kv[ITEMS], vv[ITEMS];
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      const int it = base + u * kCopyThreads;
      if (it < items) {
        const int r = it / cpr, c = it % cpr;
        const int64_t off = src0 + r * tok_stride + c * 16;
        kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.kcur + off));
        vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.vcur + off));
      }
    }
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      const int it = base + u * kCopyThreads;
      if (it < items) {
        const int64_t off = dst_row0 + int64_t(it) * 16;
        __builtin_nontemporal_store(kv[u], reinterpret_cast<u32x4*>(a.kcache + off));
        __builtin_nontemporal_store(vv[u], reinterpret_cast<u32x4*>(a.vcache + off));
      }
    }
  }
}

// In-place gather of one (layer, head, batch entry) cache region: the
// segments that outlive the step move down over the dropped ones (Pith page
// of arXiv 2605.14877, Figure 4 caption: a pruning set that grows is to be gone
// from the cache once its scale is done, so segments leave from the middle of the cache).
//
// Destination rows are rewritten in ascending chunks by one workgroup per
// (region, column part).  Every destination row's source row lies at or above
// it, so within a chunk all loads finish (barrier) before any store, and the
// loads of later chunks start above every row stored so far: no byte is read
// after this launch has written it, and no source byte is overwritten before
// it is read.  A region's rows are split by columns into a.parts parts of
// whole 128-byte lines (blockIdx.z): the parts touch disjoint bytes, so each
// is an independent move of its own, and a region's chain of chunks is
// a.parts times shorter than with one workgroup per region.
__global__ __launch_bounds__(kCopyThreads) void gather_kernel(GatherArgs a) {
  __shared__ GatherRun runs[kMaxScales];
  const GatherDesc d = a.desc[blockIdx.x];
  if (threadIdx.x < unsigned(d.n_runs)) runs[threadIdx.x] = a.runs[d.run_first + threadIdx.x];
  __syncthreads();

  const int64_t region = d.base + int64_t(blockIdx.y) * d.cap * a.row_bytes;
  uint8_t* kc = a.kcache + region;
  uint8_t* vc = a.vcache + region;
  const int cmask = (1 << a.cpp_shift) - 1;              // vectors per part - 1
  const int col0 = int(blockIdx.z) << a.cpp_shift;       // first vector of this part
  for (int row0 = d.dst_begin; row0 < d.dst_end; row0 += a.rows_per_chunk) {
    const int items = min(a.rows_per_chunk, d.dst_end - row0) << a.cpp_shift;
    u32x4 kv[kGatherItems], vv[kGatherItems];
#pragma unroll
    for (int u = 0; u < kGatherItems; ++u) {
      const int it = threadIdx.x + u * kCopyThreads;
      if (it < items) {
        const int row = row0 + (it >> a.cpp_shift);
        int src = row;
        for (int r = 0; r < d.n_runs; ++r)
          if (row < runs[r].dst + runs[r].rows) {
            src = runs[r].src + (row - runs[r].dst);
            break;
          }
        const int64_t off = int64_t(src) * a.row_bytes + (col0 + (it & cmask)) * 16;
        kv[u] = *reinterpret_cast<const u32x4*>(kc + off);
        vv[u] = *reinterpret_cast<const u32x4*>(vc + off);
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kGatherItems; ++u) {
      const int it = threadIdx.x + u * kCopyThreads;
      if (it < items) {
        const int64_t off = int64_t(row0 + (it >> a.cpp_shift)) * a.row_bytes + (col0 + (it & cmask)) * 16;
        __builtin_nontemporal_store(kv[u], reinterpret_cast<u32x4*>(kc + off));
        __builtin_nontemporal_store(vv[u], reinterpret_cast<u32x4*>(vc + off));
      }
    }
  }
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  if (a.n_desc == 0) return hipSuccess;
  if (a.parts < 1 || (a.parts << a.cpp_shift) * 16 != a.row_bytes ||
      (a.rows_per_chunk << a.cpp_shift) != kCopyThreads * kGatherItems)
    return hipErrorInvalidValue;
  if (!grid_fits(a.n_desc, kCopyThreads, a.B, a.parts)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(gather_kernel, dim3(unsigned(a.n_desc), unsigned(a.B), unsigned(a.parts)),
                     dim3(kCopyThreads), 0, s, a);
  return hipGetLastError();
}

// grid: (n_layers * B * ceil(n / rows)).  Item i of a workgroup is the i-th
// 16-byte vector of its token block, so the loads walk the source
// contiguously; a vector of a head that does not store this scale is skipped.
// The layer's per-head destinations (a.H <= kRowsMaxHeads) are read once
// into LDS.
__global__ __launch_bounds__(kCopyThreads) void compact_rows_kernel(RowsArgs a) {
  __shared__ int64_t s_dst[kRowsMaxHeads];
  __shared__ int32_t s_cap[kRowsMaxHeads];
  const int nblk = (a.n + a.rows - 1) / a.rows;
  const int blk = blockIdx.x % nblk;
  const int b = (blockIdx.x / nblk) % a.B;
  const int l = blockIdx.x / (nblk * a.B);
  const int cpr = a.row_bytes >> 4;
  const int per_tok = a.H * cpr;
  const int r0 = blk * a.rows;
  const int items = min(a.rows, a.n - r0) * per_tok;
  const int64_t src0 = int64_t(l) * a.layer_stride_bytes + (int64_t(b) * a.n + r0) * per_tok * 16;
  for (int i = threadIdx.x; i < a.H; i += kCopyThreads) {
    s_dst[i] = a.dst[int64_t(l) * a.H + i];
    s_cap[i] = a.cap[int64_t(l) * a.H + i];
  }
  __syncthreads();
  const int64_t* dst = s_dst;
  const int32_t* cap = s_cap;
  for (int base = threadIdx.x; base < items; base += kCopyThreads * kCopyItems) {
    u32x4 kv[kCopyItems], vv[kCopyItems];
    int64_t off[kCopyItems];
#pragma unroll
    for (int u = 0; u < kCopyItems; ++u) {
      const int it = base + u * kCopyThreads;
      off[u] = -1;
      if (it < items) {
        const int r = it / per_tok, h = (it / cpr) % a.H, c = it % cpr;
        const int64_t d = dst[h];
        if (d >= 0) {
          off[u] = d + (int64_t(b) * cap[h] + r0 + r) * a.row_bytes + c * 16;
          kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.kcur + src0 + int64_t(it) * 16));
          vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.vcur + src0 + int64_t(it) * 16));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyItems; ++u) {
      if (off[u] >= 0) {
        __builtin_nontemporal_store(kv[u], reinterpret_cast<u32x4*>(a.kcache + off[u]));
        __builtin_nontemporal_store(vv[u], reinterpret_cast<u32x4*>(a.vcache + off[u]));
      }
    }
  }
}

hipError_t launch_compact_rows(const RowsArgs& a, hipStream_t s) {
  const int64_t blocks = int64_t(a.n_layers) * a.B * ((a.n + a.rows - 1) / a.rows);
  if (blocks == 0) return hipSuccess;
  if (a.H > kRowsMaxHeads) return hipErrorInvalidValue;
  if (!grid_fits(blocks, kCopyThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(compact_rows_kernel, dim3(unsigned(blocks)), dim3(kCopyThreads), 0, s, a);
  return hipGetLastError();
}

// Pooled caches: the stored segments of a completed scale go to their pool
// rows (one workgroup per (segment, batch entry, block of rows)); nothing
// already in the pool moves.  Reads stride over the [B][n][H][D] source,
// writes are whole 256-byte rows wherever the pool placed them.
__global__ __launch_bounds__(kCopyThreads) void compact_pooled_kernel(PoolArgs a) {
  const int chunk = blockIdx.x % a.chunks;
  const int rest = blockIdx.x / a.chunks;
  const int b = rest % a.B;
  const PoolDesc d = a.desc[rest / a.B];
  const int row0 = chunk * a.rows_per_block;
  const int rows = min(a.rows_per_block, a.n - row0);
  const int items = rows << a.cpr_shift;
  const int cmask = (1 << a.cpr_shift) - 1;
  const int64_t tok_stride = int64_t(a.H) * a.row_bytes;
  const int64_t src0 = int64_t(d.layer - a.layer_begin) * a.layer_stride_bytes +
                       (int64_t(b) * a.n + row0) * tok_stride + int64_t(d.head) * a.row_bytes;
  const int64_t pool0 = int64_t(b) * a.pool_rows * a.row_bytes;
  const int32_t* prow = a.rows + d.rows_first + row0;
  u32x4 kv[kCopyItems], vv[kCopyItems];
  int64_t dst[kCopyItems];
#pragma unroll
  for (int u = 0; u < kCopyItems; ++u) {
    const int it = threadIdx.x + u * kCopyThreads;
    if (it < items) {
      const int r = it >> a.cpr_shift, c = it & cmask;
      const int64_t off = src0 + r * tok_stride + c * 16;
      kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.kcur + off));
      vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.vcur + off));
      dst[u] = pool0 + int64_t(prow[r]) * a.row_bytes + c * 16;
    }
  }
#pragma unroll
  for (int u = 0; u < kCopyItems; ++u) {
    const int it = threadIdx.x + u * kCopyThreads;
    if (it < items) {
      __builtin_nontemporal_store(kv[u], reinterpret_cast<u32x4*>(a.kpool + dst[u]));
      __builtin_nontemporal_store(vv[u], reinterpret_cast<u32x4*>(a.vpool + dst[u]));
    }
  }
}

hipError_t launch_compact_pooled(const PoolArgs& a, hipStream_t s) {
  const int64_t blocks = int64_t(a.n_desc) * a.B * a.chunks;
  if (blocks == 0) return hipSuccess;
  if ((16 << a.cpr_shift) != a.row_bytes || int64_t(a.rows_per_block) * a.row_bytes > kCopyBlockBytes)
    return hipErrorInvalidValue;
  if (!grid_fits(blocks, kCopyThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(compact_pooled_kernel, dim3(unsigned(blocks)), dim3(kCopyThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  const int64_t blocks = int64_t(a.n_desc) * a.B * a.chunks;
  if (blocks == 0) return hipSuccess;
  if (!grid_fits(blocks, kCopyThreads)) return hipErrorInvalidConfiguration;
  if (int64_t(a.rows_per_block) * a.row_bytes > kCopyBlockBytes)
    hipLaunchKernelGGL(compact_kernel<2 * kCopyItems>, dim3(unsigned(blocks)), dim3(kCopyThreads), 0, s, a);
  else
    hipLaunchKernelGGL(compact_kernel<kCopyItems>, dim3(unsigned(blocks)), dim3(kCopyThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hk
