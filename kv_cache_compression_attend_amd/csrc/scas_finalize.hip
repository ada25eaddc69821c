// S-CAS row of one (layer, step): the per-workgroup partial sums of the
// attention kernels, added in a fixed order (batch entry, then query tile) in
// double and divided by the number of queries B * n_t, so the row is the mean
// over the scale's queries and the batch of the mass each query puts on each
// source scale (HeatKV project page, Abstract and Method step 2).  No float
// atomics: the result is the same on every run.
#include "device.h"

namespace hk {

namespace {

__global__ void scas_finalize_kernel(const float* partials, float* table, int layer, int H, int K,
                                     int B, int n, int step, int n_qtiles) {
  const int h = blockIdx.x;
  const int s = threadIdx.x;
  if (s > step) return;
  double acc = 0.0;
  for (int b = 0; b < B; ++b)
    for (int qt = 0; qt < n_qtiles; ++qt)
      acc += double(partials[((int64_t(b) * H + h) * n_qtiles + qt) * kMaxScales + s]);
  table[((int64_t(layer) * H + h) * K + step) * K + s] = float(acc / (double(B) * double(n)));
}

// Streaming form: adds the sum over the batch of per-image S-CAS (partials
// added in the same fixed order, divided by the n queries) to a double table.
__global__ void scas_accumulate_kernel(const float* partials, double* table, int layer, int H,
                                       int K, int B, int n, int step, int n_qtiles) {
  const int h = blockIdx.x;
  const int s = threadIdx.x;
  if (s > step) return;
  double acc = 0.0;
  for (int b = 0; b < B; ++b)
    for (int qt = 0; qt < n_qtiles; ++qt)
      acc += double(partials[((int64_t(b) * H + h) * n_qtiles + qt) * kMaxScales + s]);
  table[((int64_t(layer) * H + h) * K + step) * K + s] += acc / double(n);
}

}  // namespace

hipError_t launch_scas_accumulate(const float* partials, double* table, int layer, int H, int K,
                                  int B, int n, int step, int n_qtiles, hipStream_t s) {
  hipLaunchKernelGGL(scas_accumulate_kernel, dim3(H), dim3(kMaxScales), 0, s, partials, table,
                     layer, H, K, B, n, step, n_qtiles);
  return hipGetLastError();
}

hipError_t launch_scas_finalize(const float* partials, float* table, int layer, int H, int K,
                                int B, int n, int step, int n_qtiles, hipStream_t s) {
  hipLaunchKernelGGL(scas_finalize_kernel, dim3(H), dim3(kMaxScales), 0, s, partials, table, layer,
                     H, K, B, n, step, n_qtiles);
  return hipGetLastError();
}

}  // namespace hk
