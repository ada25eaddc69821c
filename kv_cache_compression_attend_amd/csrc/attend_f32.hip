// Block-causal multi-scale attention over kept head-scale segments, fp32
// inputs, small head_dim (16..128), on the vector ALUs.
//
// Same operation as the bf16 matrix-core kernel (HeatKV project page,
// Abstract and Method step 5; Pith page of arXiv 2605.14877, Figure 2
// caption), for fp32 workloads such as the tiny parity case.  One lane per
// query; all lanes of a workgroup belong to one (batch, head) and read the
// same key row at the same time.  Two passes over the keys: the first finds
// the query's maximum score, the second sums exp(score - max) into the
// output, the normaliser and the per-source S-CAS mass, so no rescaling is
// needed.  Scores, softmax and outputs are fp32.
#include <math.h>

#include "device.h"

namespace hk {

namespace {

constexpr int kThreads = 64;

template <int D, bool SCAS>
__global__ __launch_bounds__(kThreads) void attend_f32_kernel(AttendArgs a) {
  __shared__ float sRed[SCAS ? kMaxScales : 1];
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n = a.n;
  const int qrow = qt * kThreads + threadIdx.x;
  const bool qvalid = qrow < n;
  const int64_t tok = int64_t(a.H) * D;
  const float* kcur = static_cast<const float*>(a.kcur) + int64_t(b) * n * tok + h * D;
  const float* vcur = static_cast<const float*>(a.vcur) + int64_t(b) * n * tok + h * D;
  const int cap = a.cap[h];
  const int64_t hb = a.base[h] + int64_t(b) * cap * D;
  const float* kc = static_cast<const float*>(a.kcache) + hb;
  const float* vc = static_cast<const float*>(a.vcache) + hb;
  const int32_t* lenb = a.lenb + h * a.K;
  const int Lc = lenb[a.step];
  const int Ltot = Lc + n;

  float q[D];
  {
    const float* qp = static_cast<const float*>(a.q) + (int64_t(b) * n + (qvalid ? qrow : 0)) * tok + h * D;
#pragma unroll
    for (int d = 0; d < D; ++d) q[d] = qvalid ? qp[d] : 0.f;
  }

  auto krow = [&](int key) { return key < Lc ? kc + int64_t(key) * D : kcur + int64_t(key - Lc) * tok; };
  auto vrow = [&](int key) { return key < Lc ? vc + int64_t(key) * D : vcur + int64_t(key - Lc) * tok; };
  auto score = [&](int key) {
    const float* k = krow(key);
    float acc = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) acc = fmaf(q[d], k[d], acc);
    return acc * a.scale;
  };

  float m = -INFINITY;
  for (int key = 0; key < Ltot; ++key) m = fmaxf(m, score(key));

  float o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = 0.f;
  float l = 0.f;
  float mass[SCAS ? kMaxScales : 1];
#pragma unroll
  for (int s = 0; s < (SCAS ? kMaxScales : 1); ++s) mass[s] = 0.f;

  // Walk the keys segment by segment: kept sources s < step, then the current scale.
  for (int src = 0; src <= a.step; ++src) {
    const int lo = lenb[src];
    const int hi = src < a.step ? lenb[src + 1] : Ltot;
    float part = 0.f;
    for (int key = lo; key < hi; ++key) {
      const float p = expf(score(key) - m);
      const float* v = vrow(key);
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, v[d], o[d]);
      part += p;
    }
    l += part;
    if constexpr (SCAS) {
#pragma unroll
      for (int s = 0; s < kMaxScales; ++s)
        if (s == src) mass[s] = part;
    }
  }

  const float inv = 1.f / l;
  if (qvalid) {
    float* op = static_cast<float*>(a.out) + (int64_t(b) * n + qrow) * tok + h * D;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
  }

  if constexpr (SCAS) {
#pragma unroll
    for (int s = 0; s < kMaxScales; ++s) {
      float v = qvalid ? mass[s] * inv : 0.f;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
      if (threadIdx.x == 0) sRed[s] = v;
    }
    __syncthreads();
    if (threadIdx.x < kMaxScales) {
      const int64_t row = (int64_t(b) * a.H + h) * a.n_qtiles + qt;
      a.partials[row * kMaxScales + threadIdx.x] = sRed[threadIdx.x];
    }
  }
}

template <int D>
hipError_t launch_d(const AttendArgs& a, bool scas, hipStream_t s) {
  if (!grid_fits(a.n_qtiles, kThreads, a.H, a.B)) return hipErrorInvalidConfiguration;
  const dim3 grid(a.n_qtiles, a.H, a.B);
  if (scas)
    hipLaunchKernelGGL((attend_f32_kernel<D, true>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((attend_f32_kernel<D, false>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_f32(const AttendArgs& a, int D, bool scas, hipStream_t s) {
  switch (D) {
    case 16: return launch_d<16>(a, scas, s);
    case 32: return launch_d<32>(a, scas, s);
    case 64: return launch_d<64>(a, scas, s);
    case 128: return launch_d<128>(a, scas, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hk
