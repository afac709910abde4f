// Weight rescaling after the update (Osawa et al., "Large-Scale Distributed
// Second-Order Optimization Using Kronecker-Factored Approximate Curvature
// for Deep Convolutional Neural Networks", section 4.4): every listed weight
// W (a layer's d_out x d_in matrix, bias excluded) becomes
//     W * sqrt(2 d_out) / (||W||_F + eps)
// in place.  Two HBM-streaming launches over all listed weights:
//   rescale_norm_kernel   each workgroup sums the squares of its chunk of one
//                         weight (16-byte loads), wavefront sums in a fixed
//                         order, one partial per workgroup;
//   rescale_apply_kernel  each workgroup adds its weight's partials in order
//                         (the same sum in every workgroup of the weight),
//                         forms the scale and multiplies its chunk.
// No atomics: the result is bit-reproducible.
#include "common.h"

#include <algorithm>
#include <cmath>

namespace kfac {

namespace {

constexpr int kRsThreads = 256;
constexpr int kRsWaves = kRsThreads / kWave;
constexpr int kRsVec = 4;                                   // floats per load
constexpr int kRsUnroll = 8;                                // loads in flight per thread
constexpr int64_t kRsPerBlock = int64_t(kRsThreads) * kRsVec * kRsUnroll;
constexpr int kMaxRsSegs = 96;

struct RsItem {
  float* w;
  float* part;        // one partial per workgroup of this weight
  int64_t n;
  float target;       // sqrt(2 d_out)
  int32_t blk_begin;
  int32_t nblk;
  int32_t pad_;
};
struct RsTab {
  RsItem s[kMaxRsSegs];
  int32_t n;
  float eps;
};
static_assert(sizeof(RsTab) <= 4096, "kernel arguments");

__device__ inline int find_seg(const RsTab& t, int blk) {
  int lo = 0, hi = t.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (t.s[mid].blk_begin <= blk) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ inline float rs_wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__global__ void __launch_bounds__(kRsThreads) rescale_norm_kernel(RsTab tab) {
  __shared__ float red[kRsWaves];
  const RsItem& S = tab.s[find_seg(tab, blockIdx.x)];
  const int b = blockIdx.x - S.blk_begin;
  const int64_t base = static_cast<int64_t>(b) * kRsPerBlock;
  const int64_t end = min(S.n, base + kRsPerBlock);
  float acc = 0.f;
  if ((S.n & 3) == 0) {
    f32x4 v[kRsUnroll];
#pragma unroll
    for (int u = 0; u < kRsUnroll; ++u) {
      const int64_t e = base + (static_cast<int64_t>(u) * kRsThreads + threadIdx.x) * kRsVec;
      v[u] = e < end ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S.w + e)) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kRsUnroll; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = fmaf(v[u][q], v[u][q], acc);
  } else {
    for (int64_t e = base + threadIdx.x; e < end; e += kRsThreads) acc = fmaf(S.w[e], S.w[e], acc);
  }
  acc = rs_wave_sum(acc);
  const int wid = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  if (lane == 0) red[wid] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < kRsWaves; ++w) t += red[w];
    S.part[b] = t;
  }
}

__global__ void __launch_bounds__(kRsThreads) rescale_apply_kernel(RsTab tab) {
  __shared__ float scale;
  const RsItem& S = tab.s[find_seg(tab, blockIdx.x)];
  const int b = blockIdx.x - S.blk_begin;
  if (threadIdx.x < kWave) {
    // the weight's squared norm: its partials in a fixed order (lane-strided,
    // then a fixed shuffle tree), the same in every workgroup of the weight
    float t = 0.f;
    for (int i = threadIdx.x; i < S.nblk; i += kWave) t += S.part[i];
    t = rs_wave_sum(t);
    if (threadIdx.x == 0) scale = S.target / (sqrtf(t) + tab.eps);
  }
  __syncthreads();
  const float sc = scale;
  const int64_t base = static_cast<int64_t>(b) * kRsPerBlock;
  const int64_t end = min(S.n, base + kRsPerBlock);
  if ((S.n & 3) == 0) {
#pragma unroll
    for (int u = 0; u < kRsUnroll; ++u) {
      const int64_t e = base + (static_cast<int64_t>(u) * kRsThreads + threadIdx.x) * kRsVec;
      if (e >= end) continue;
      f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S.w + e));
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] *= sc;
      *reinterpret_cast<f32x4*>(S.w + e) = v;
    }
  } else {
    for (int64_t e = base + threadIdx.x; e < end; e += kRsThreads) S.w[e] *= sc;
  }
}

}  // namespace

int64_t rescale_blocks(int64_t n) { return (n + kRsPerBlock - 1) / kRsPerBlock; }

kfac_status_t launch_rescale(const std::vector<RescaleSeg>& segs, float eps, hipStream_t st) {
  for (int pass = 0; pass < 2; ++pass) {
    for (size_t g0 = 0; g0 < segs.size(); g0 += kMaxRsSegs) {
      const size_t g1 = std::min(segs.size(), g0 + kMaxRsSegs);
      RsTab T{};
      int blocks = 0;
      for (size_t i = g0; i < g1; ++i) {
        RsItem& it = T.s[i - g0];
        it.w = segs[i].w;
        it.part = segs[i].part;
        it.n = segs[i].n;
        it.target = std::sqrt(2.0f * static_cast<float>(segs[i].d_out));
        it.nblk = static_cast<int32_t>(rescale_blocks(segs[i].n));
        it.blk_begin = blocks;
        blocks += it.nblk;
      }
      T.n = static_cast<int32_t>(g1 - g0);
      T.eps = eps;
      if (pass == 0) hipLaunchKernelGGL(rescale_norm_kernel, dim3(blocks), dim3(kRsThreads), 0, st, T);
      else hipLaunchKernelGGL(rescale_apply_kernel, dim3(blocks), dim3(kRsThreads), 0, st, T);
      KFAC_HIP_TRY(hipGetLastError());
    }
  }
  return KFAC_OK;
}

}  // namespace kfac
