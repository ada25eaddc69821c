// 4-bit storage of the ragged cache: quantize a completed scale's stored
// segments, and unpack a layer's stored rows into the bf16 scratch that the
// attend kernels read.
//
// Groups follow the VAR-Q summary page (Key contributions, Method): one group
// per (block, channel), where a block is one scale's segment, optionally cut
// into m sub-blocks along the token axis (sub-block j of an n-token segment
// is rows [j*n/m, (j+1)*n/m), rounded down).  Values are packed two per byte
// when written and unpacked for attention.  Each group stores (step, lo) in
// float32: lo = min, step = (max - min) / 15, code = round-half-even((x -
// lo) / step) clamped to [0, 15] (0 when step = 0); an empty sub-block
// stores (0, 0).  The value read back is lo + code * step, rounded to bf16
// for the matrix cores.
//
// Both kernels are bound by HBM bandwidth: the quantizer reads each bf16 row
// twice (min/max pass, then codes; the second read hits L2) and writes 64
// bytes per row; the unpacker reads 64 bytes and writes 256.
#include "device.h"

namespace hk {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ unsigned code_of(float x, float step, float lo) {
  if (step == 0.f) return 0u;
  const float q = rintf((x - lo) / step);
  return unsigned(fminf(fmaxf(q, 0.f), 15.f));
}

}  // namespace

// grid: (n_desc * m, B, 2): segment, sub-block, batch entry, K (z=0) or V (z=1).
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantArgs a) {
  __shared__ float sLo[16][kQuantD];
  __shared__ float sHi[16][kQuantD];
  __shared__ float sStep[kQuantD];
  __shared__ float sBase[kQuantD];

  const int j = blockIdx.x % a.m;
  const QuantDesc d = a.desc[blockIdx.x / a.m];
  const int b = blockIdx.y;
  const bool is_v = blockIdx.z == 1;
  const int64_t tok = int64_t(a.H) * kQuantD;
  const uint16_t* src = (is_v ? a.vcur : a.kcur) + int64_t(d.layer - a.layer_begin) * a.layer_stride +
                        int64_t(b) * a.n * tok + int64_t(d.head) * kQuantD;
  uint8_t* store = is_v ? a.vstore : a.kstore;
  uint8_t* codes = store + d.code_off + int64_t(b) * d.cap * kQuantRowBytes;
  float2* params = reinterpret_cast<float2*>(store + d.param_off +
                                             int64_t(b) * d.gcap * kQuantD * int64_t(sizeof(float2))) +
                   j * kQuantD;
  const int r0 = (j * a.n) / a.m, r1 = ((j + 1) * a.n) / a.m;

  // Pass 1: per-channel min and max; lane (row r0 + i + 16k, channels 8c..8c+7).
  {
    const int i = threadIdx.x >> 4, c8 = (threadIdx.x & 15) * 8;
    float lo[8], hi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = INFINITY;
      hi[e] = -INFINITY;
    }
    for (int r = r0 + i; r < r1; r += 16) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(src + r * tok + c8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = bf16_lo(w[e]), x1 = bf16_hi(w[e]);
        lo[2 * e] = fminf(lo[2 * e], x0);
        hi[2 * e] = fmaxf(hi[2 * e], x0);
        lo[2 * e + 1] = fminf(lo[2 * e + 1], x1);
        hi[2 * e + 1] = fmaxf(hi[2 * e + 1], x1);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sLo[i][c8 + e] = lo[e];
      sHi[i][c8 + e] = hi[e];
    }
  }
  __syncthreads();
  if (threadIdx.x < kQuantD) {
    const int c = threadIdx.x;
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      lo = fminf(lo, sLo[i][c]);
      hi = fmaxf(hi, sHi[i][c]);
    }
    float step = 0.f, base = 0.f;
    if (r1 > r0) {
      base = lo;
      step = (hi - lo) / 15.f;
    }
    sStep[c] = step;
    sBase[c] = base;
    params[c] = make_float2(step, base);
  }
  __syncthreads();

  // Pass 2: codes; lane (row r0 + i + 64k, channels 32c..32c+31) -> 16 bytes.
  const int i = threadIdx.x >> 2, c32 = (threadIdx.x & 3) * 32;
  float step[32], base[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    step[e] = sStep[c32 + e];
    base[e] = sBase[c32 + e];
  }
  for (int r = r0 + i; r < r1; r += 64) {
    const u32x4* p = reinterpret_cast<const u32x4*>(src + r * tok + c32);
    u32x4 w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = p[k];
    u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const unsigned word = w[e / 8][(e % 8) / 2];
      const float x = (e % 2) ? bf16_hi(word) : bf16_lo(word);
      out[e / 8] |= code_of(x, step[e], base[e]) << (4 * (e % 8));
    }
    __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(codes + int64_t(r) * kQuantRowBytes +
                                                               (threadIdx.x & 3) * 16));
  }
}

// grid: (n_items, B, 2).  Lane (row i + 64k of the run, channels 32c..32c+31).
__global__ __launch_bounds__(kThreads) void unpack_kernel(UnpackArgs a) {
  const UnpackItem it = a.items[blockIdx.x];
  const int b = blockIdx.y;
  const bool is_v = blockIdx.z == 1;
  const uint8_t* store = is_v ? a.vstore : a.kstore;
  uint16_t* scratch = is_v ? a.vscratch : a.kscratch;
  const int c = threadIdx.x & 3, i = threadIdx.x >> 2;

  const f32x4* pp = reinterpret_cast<const f32x4*>(
      store + it.param_off + int64_t(b) * it.gcap * kQuantD * int64_t(sizeof(float2))) + c * 16;
  float step[32], lo[32];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const f32x4 v = pp[k];   // (step, lo) of channels 2k, 2k+1 of this lane's 32
    step[2 * k] = v[0];
    lo[2 * k] = v[1];
    step[2 * k + 1] = v[2];
    lo[2 * k + 1] = v[3];
  }
  const uint8_t* codes = store + it.code_off + int64_t(b) * it.cap * kQuantRowBytes + c * 16;
  uint16_t* out = scratch + it.scratch_off + int64_t(b) * it.cap * kQuantD + c * 32;
  for (int r = i; r < it.rows; r += 64) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(codes + int64_t(r) * kQuantRowBytes);
    u32x4 o[4];
#pragma unroll
    for (int e = 0; e < 32; e += 2) {
      const float x0 = fmaf(float((w[e / 8] >> (4 * (e % 8))) & 15u), step[e], lo[e]);
      const float x1 = fmaf(float((w[e / 8] >> (4 * (e % 8) + 4)) & 15u), step[e + 1], lo[e + 1]);
      o[e / 8][(e % 8) / 2] = pack_bf16x2(x0, x1);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(out + int64_t(r) * kQuantD);
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[k] = o[k];
  }
}

// Split form, first launch.  grid: (n_desc * m * nch, B, 2): per-channel
// (min, max) of one chunk of a sub-block's rows ((+inf, -inf) when empty).
__global__ __launch_bounds__(kThreads) void quantize_minmax_kernel(QuantArgs a) {
  __shared__ float sLo[16][kQuantD];
  __shared__ float sHi[16][kQuantD];
  const int ch = blockIdx.x % a.nch;
  const int j = (blockIdx.x / a.nch) % a.m;
  const int di = blockIdx.x / (a.nch * a.m);
  const QuantDesc d = a.desc[di];
  const int b = blockIdx.y;
  const bool is_v = blockIdx.z == 1;
  const int64_t tok = int64_t(a.H) * kQuantD;
  const uint16_t* src = (is_v ? a.vcur : a.kcur) + int64_t(d.layer - a.layer_begin) * a.layer_stride +
                        int64_t(b) * a.n * tok + int64_t(d.head) * kQuantD;
  const int g0 = (j * a.n) / a.m, g1 = ((j + 1) * a.n) / a.m;
  const int r0 = g0 + ch * kQuantChunkRows, r1 = min(g1, r0 + kQuantChunkRows);
  const int i = threadIdx.x >> 4, c8 = (threadIdx.x & 15) * 8;
  float lo[8], hi[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lo[e] = INFINITY;
    hi[e] = -INFINITY;
  }
  for (int r = r0 + i; r < r1; r += 16) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(src + r * tok + c8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = bf16_lo(w[e]), x1 = bf16_hi(w[e]);
      lo[2 * e] = fminf(lo[2 * e], x0);
      hi[2 * e] = fmaxf(hi[2 * e], x0);
      lo[2 * e + 1] = fminf(lo[2 * e + 1], x1);
      hi[2 * e + 1] = fmaxf(hi[2 * e + 1], x1);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    sLo[i][c8 + e] = lo[e];
    sHi[i][c8 + e] = hi[e];
  }
  __syncthreads();
  if (threadIdx.x < kQuantD) {
    const int c = threadIdx.x;
    float l = INFINITY, h = -INFINITY;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      l = fminf(l, sLo[k][c]);
      h = fmaxf(h, sHi[k][c]);
    }
    const int64_t slot = ((int64_t(di) * a.m + j) * a.nch + ch) * a.B + b;
    a.minmax[(slot * 2 + (is_v ? 1 : 0)) * kQuantD + c] = make_float2(l, h);
  }
}

// Split form, second launch.  Same grid: the group's (min, max) from its
// chunks (min and max are exact, so the order does not matter), the group
// parameters (chunk 0 writes them), then this chunk's codes.
__global__ __launch_bounds__(kThreads) void quantize_codes_kernel(QuantArgs a) {
  __shared__ float sStep[kQuantD];
  __shared__ float sBase[kQuantD];
  const int ch = blockIdx.x % a.nch;
  const int j = (blockIdx.x / a.nch) % a.m;
  const int di = blockIdx.x / (a.nch * a.m);
  const QuantDesc d = a.desc[di];
  const int b = blockIdx.y;
  const bool is_v = blockIdx.z == 1;
  const int64_t tok = int64_t(a.H) * kQuantD;
  const uint16_t* src = (is_v ? a.vcur : a.kcur) + int64_t(d.layer - a.layer_begin) * a.layer_stride +
                        int64_t(b) * a.n * tok + int64_t(d.head) * kQuantD;
  uint8_t* store = is_v ? a.vstore : a.kstore;
  uint8_t* codes = store + d.code_off + int64_t(b) * d.cap * kQuantRowBytes;
  const int g0 = (j * a.n) / a.m, g1 = ((j + 1) * a.n) / a.m;
  if (threadIdx.x < kQuantD) {
    const int c = threadIdx.x;
    float lo = INFINITY, hi = -INFINITY;
    for (int k = 0; k < a.nch; ++k) {
      const int64_t slot = ((int64_t(di) * a.m + j) * a.nch + k) * a.B + b;
      const float2 v = a.minmax[(slot * 2 + (is_v ? 1 : 0)) * kQuantD + c];
      lo = fminf(lo, v.x);
      hi = fmaxf(hi, v.y);
    }
    float step = 0.f, base = 0.f;
    if (g1 > g0) {
      base = lo;
      step = (hi - lo) / 15.f;
    }
    sStep[c] = step;
    sBase[c] = base;
    if (ch == 0) {
      float2* params = reinterpret_cast<float2*>(store + d.param_off +
                                                 int64_t(b) * d.gcap * kQuantD * int64_t(sizeof(float2))) +
                       j * kQuantD;
      params[c] = make_float2(step, base);
    }
  }
  __syncthreads();
  const int r0 = g0 + ch * kQuantChunkRows, r1 = min(g1, r0 + kQuantChunkRows);
  const int i = threadIdx.x >> 2, c32 = (threadIdx.x & 3) * 32;
  float step[32], base[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    step[e] = sStep[c32 + e];
    base[e] = sBase[c32 + e];
  }
  for (int r = r0 + i; r < r1; r += 64) {
    const u32x4* p = reinterpret_cast<const u32x4*>(src + r * tok + c32);
    u32x4 w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = p[k];
    u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const unsigned word = w[e / 8][(e % 8) / 2];
      const float x = (e % 2) ? bf16_hi(word) : bf16_lo(word);
      out[e / 8] |= code_of(x, step[e], base[e]) << (4 * (e % 8));
    }
    __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(codes + int64_t(r) * kQuantRowBytes +
                                                               (threadIdx.x & 3) * 16));
  }
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  if (a.n_desc == 0) return hipSuccess;
  if (!grid_fits(int64_t(a.n_desc) * a.m * (a.nch > 1 ? a.nch : 1), kThreads, a.B, 2))
    return hipErrorInvalidConfiguration;
  if (a.nch <= 1) {
    hipLaunchKernelGGL(quantize_kernel, dim3(unsigned(a.n_desc * a.m), unsigned(a.B), 2u),
                       dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
  const dim3 grid(unsigned(a.n_desc * a.m * a.nch), unsigned(a.B), 2u);
  hipLaunchKernelGGL(quantize_minmax_kernel, grid, dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quantize_codes_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_unpack(const UnpackArgs& a, hipStream_t s) {
  if (a.n_items == 0) return hipSuccess;
  if (!grid_fits(a.n_items, kThreads, a.B, 2)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(unpack_kernel, dim3(unsigned(a.n_items), unsigned(a.B), 2u), dim3(kThreads), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace hk
