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
// Design (one workgroup = 4 waves = 128 queries of one (batch, head)):
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: each lane then owns one query column and 16
//     key rows per 32x32 block, so a query's running max and sum stay in the
//     lane (one exchange with the lane 32 apart per key tile).
//   * The key rows fed to the score product are permuted (bits 2 and 3 of the
//     row index swapped) so that the score accumulator of each lane already
//     holds, for every 16-key step of the value product, the 8 consecutive
//     keys the B operand of O^T = V^T P^T needs: probabilities go from the
//     score registers straight into the value product, without LDS.
//   * K tiles are staged row-major in LDS; V tiles are transposed on the way
//     in (4 keys x 8 dims per lane, repacked in registers) so the A operand
//     of the value product is one 16-byte LDS read.  Row strides are padded
//     so both the staging writes and the operand reads are free of bank
//     conflicts.
//   * The next tile's global loads are issued before the current tile is
//     computed; the key index selects the source row: the cache for the
//     first len_before keys, the current scale's K/V rows after that, so the
//     junction needs no padding.
//   * fp32 online softmax in base 2 (alpha * log2 e folded into one multiply).
//   * S-CAS: per-lane fp32 accumulators for up to 16 source scales, rescaled
//     with the running max, reduced across the workgroup and written as one
//     partial row per workgroup; a second kernel sums the partials in a fixed
//     order (no float atomics, deterministic).
#include <math.h>

#include "device.h"

namespace hk {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int D = 128;        // head_dim
constexpr int BM = 128;       // queries per workgroup
constexpr int BN = 64;        // keys per tile
constexpr int KSTR = D + 8;   // K tile row stride (bf16 elements): 272 bytes
constexpr int VSTR = BN + 8;  // V^T tile row stride (bf16 elements): 144 bytes
constexpr int kThreads = 256;

union Vec16 {
  uint4 u;
  bf16x8 b;
  uint32_t w[4];
};

// Key row (within a 32-key block) that feeds row i of the score product.
__device__ __forceinline__ int permuted_row(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = __bf16(lo), b = __bf16(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, a)) |
         (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

template <bool SCAS>
__global__ __launch_bounds__(kThreads, 2) void attend_bf16_d128_kernel(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * VSTR];
  __shared__ float sRed[SCAS ? 4 * kMaxScales : 1];

  const int wg = xcd_logical(blockIdx.x, gridDim.x);
  const int qt = wg % a.n_qtiles;
  const int bh = wg / a.n_qtiles;
  const int h = bh % a.H;
  const int b = bh / a.H;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, hf = lane >> 5;

  const int n = a.n;
  const int64_t tok = int64_t(a.H) * D;  // elements between consecutive tokens
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* kcur = static_cast<const uint16_t*>(a.kcur) + int64_t(b) * n * tok + h * D;
  const uint16_t* vcur = static_cast<const uint16_t*>(a.vcur) + int64_t(b) * n * tok + h * D;
  const int cap = a.cap[h];
  const int64_t hb = a.base[h] + int64_t(b) * cap * D;
  const uint16_t* kc = static_cast<const uint16_t*>(a.kcache) + hb;
  const uint16_t* vc = static_cast<const uint16_t*>(a.vcache) + hb;
  const int32_t* lenb = a.lenb + h * a.K;
  const int Lc = lenb[a.step];
  const int Ltot = Lc + n;

  // Q^T fragments: lane (j, hf) holds query q0+j, dims 16*kk + 8*hf + [0, 8).
  const int qrow = qt * BM + wave * 32 + j;
  const bool qvalid = qrow < n;
  Vec16 qf[8];
  {
    const uint16_t* qp = q + (int64_t(b) * n + (qvalid ? qrow : 0)) * tok + h * D + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qf[kk].u = qvalid ? *reinterpret_cast<const uint4*>(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
    }
  }

  // Staging assignment.  K: 16-byte chunk kc_c of rows kr + 16*i.
  // V: key group vg (keys 4vg..4vg+3), 16-byte dim chunk vc_c.
  const int k_c = tid & 15, k_r = tid >> 4;
  const int v_g = tid & 15, v_c = tid >> 4;
  uint4 kreg[4], vreg[4];

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = k0 + k_r + 16 * i;
      const uint16_t* p = key < Lc ? kc + int64_t(key) * D : kcur + int64_t(key - Lc) * tok;
      kreg[i] = key < Ltot ? *reinterpret_cast<const uint4*>(p + 8 * k_c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = k0 + 4 * v_g + r;
      const uint16_t* p = key < Lc ? vc + int64_t(key) * D : vcur + int64_t(key - Lc) * tok;
      vreg[r] = key < Ltot ? *reinterpret_cast<const uint4*>(p + 8 * v_c) : make_uint4(0, 0, 0, 0);
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(&sK[(k_r + 16 * i) * KSTR + 8 * k_c]) = kreg[i];
    // Transpose 4 keys x 8 dims into 8 rows (dims) of 4 keys.
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[3]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint2 even, odd;
      even.x = (w0[w] & 0xFFFFu) | (w1[w] << 16);
      even.y = (w2[w] & 0xFFFFu) | (w3[w] << 16);
      odd.x = (w0[w] >> 16) | (w1[w] & 0xFFFF0000u);
      odd.y = (w2[w] >> 16) | (w3[w] & 0xFFFF0000u);
      const int d = 8 * v_c + 2 * w;
      *reinterpret_cast<uint2*>(&sV[d * VSTR + 4 * v_g]) = even;
      *reinterpret_cast<uint2*>(&sV[(d + 1) * VSTR + 4 * v_g]) = odd;
    }
  };

  // Running state of query j (both lane halves hold the same max; sums are per half).
  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  float sc[SCAS ? kMaxScales : 1];
#pragma unroll
  for (int s = 0; s < (SCAS ? kMaxScales : 1); ++s) sc[s] = 0.f;

  // Segment bounds for S-CAS: source s < step covers [lenb[s], lenb[s+1]),
  // the current scale covers [Lc, Ltot).
  int seg_lo[SCAS ? kMaxScales : 1], seg_hi[SCAS ? kMaxScales : 1];
  if constexpr (SCAS) {
#pragma unroll
    for (int s = 0; s < kMaxScales; ++s) {
      seg_lo[s] = s <= a.step ? lenb[s] : 0;
      seg_hi[s] = s < a.step ? lenb[s + 1] : (s == a.step ? Ltot : 0);
    }
  }

  const int kb_row = permuted_row(j);
  const int ntiles = (Ltot + BN - 1) / BN;
  load_tile(0);

  for (int it = 0; it < ntiles; ++it) {
    const int k0 = it * BN;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (it + 1 < ntiles) load_tile(k0 + BN);

    // Scores S^T for two 32-key blocks.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const uint16_t* kp = &sK[(32 * kb + kb_row) * KSTR + 8 * hf];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        Vec16 kf;
        kf.u = *reinterpret_cast<const uint4*>(kp + 16 * kk);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.b, qf[kk].b, s[kb], 0, 0, 0);
      }
    }

    // Register v = 4k'+r of block kb holds key 32kb + 16(k'>>1) + 8hf + 4(k'&1) + r.
    if (k0 + BN > Ltot) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kp = v >> 2, r = v & 3;
          const int key = k0 + 32 * kb + 16 * (kp >> 1) + 8 * hf + 4 * (kp & 1) + r;
          if (key >= Ltot) s[kb][v] = -INFINITY;
        }
    }

    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, s[kb][v]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax * a.scale_log2);
    const float corr = exp2f(m_run - m_new);
    m_run = m_new;

    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = exp2f(fmaf(s[kb][v], a.scale_log2, -m_new));
        s[kb][v] = p;
        psum += p;
      }
    l_run = fmaf(l_run, corr, psum);
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] *= corr;

    if constexpr (SCAS) {
#pragma unroll
      for (int src = 0; src < kMaxScales; ++src) {
        sc[src] *= corr;
        const int lo = seg_lo[src], hi = seg_hi[src];
        if (src <= a.step && lo < hi && lo < k0 + BN && hi > k0) {
          float acc = 0.f;
          if (lo <= k0 && hi >= k0 + BN) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int v = 0; v < 16; ++v) acc += s[kb][v];
          } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                const int kp = v >> 2, r = v & 3;
                const int key = k0 + 32 * kb + 16 * (kp >> 1) + 8 * hf + 4 * (kp & 1) + r;
                acc += (key >= lo && key < hi) ? s[kb][v] : 0.f;
              }
          }
          sc[src] += acc;
        }
      }
    }

    // Probabilities as the B operand of O^T += V^T P^T, 16 keys per step.
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kb = st >> 1, base = 8 * (st & 1);
      Vec16 pb;
#pragma unroll
      for (int w = 0; w < 4; ++w) pb.w[w] = pack_bf16x2(s[kb][base + 2 * w], s[kb][base + 2 * w + 1]);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        Vec16 vf;
        vf.u = *reinterpret_cast<const uint4*>(&sV[(32 * db + j) * VSTR + 16 * st + 8 * hf]);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf.b, pb.b, oacc[db], 0, 0, 0);
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;

  if (qvalid) {
    uint16_t* op = static_cast<uint16_t*>(a.out) + (int64_t(b) * n + qrow) * tok + h * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int kp = 0; kp < 4; ++kp) {
        const int d = 32 * db + 8 * kp + 4 * hf;
        uint2 w;
        w.x = pack_bf16x2(oacc[db][4 * kp + 0] * inv, oacc[db][4 * kp + 1] * inv);
        w.y = pack_bf16x2(oacc[db][4 * kp + 2] * inv, oacc[db][4 * kp + 3] * inv);
        *reinterpret_cast<uint2*>(op + d) = w;
      }
  }

  if constexpr (SCAS) {
    // Mass of query j on each source, summed over this workgroup's valid queries.
#pragma unroll
    for (int src = 0; src < kMaxScales; ++src) {
      float m = (sc[src] + __shfl_xor(sc[src], 32)) * inv;
      m = qvalid ? m : 0.f;
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) m += __shfl_xor(m, off);
      if (lane == 0) sRed[wave * kMaxScales + src] = m;
    }
    __syncthreads();
    if (tid < kMaxScales) {
      const float tot = sRed[tid] + sRed[kMaxScales + tid] + sRed[2 * kMaxScales + tid] +
                        sRed[3 * kMaxScales + tid];
      const int64_t row = (int64_t(b) * a.H + h) * a.n_qtiles + qt;
      a.partials[row * kMaxScales + tid] = tot;
    }
  }
}

}  // namespace

hipError_t launch_attend_bf16_d128(const AttendArgs& a, bool scas, hipStream_t s) {
  const int64_t blocks = int64_t(a.B) * a.H * a.n_qtiles;
  if (scas)
    hipLaunchKernelGGL(attend_bf16_d128_kernel<true>, dim3(unsigned(blocks)), dim3(kThreads), 0,
                       s, a);
  else
    hipLaunchKernelGGL(attend_bf16_d128_kernel<false>, dim3(unsigned(blocks)), dim3(kThreads), 0,
                       s, a);
  return hipGetLastError();
}

}  // namespace hk
