// Diagonal (AdaFisher-style) K-FAC step: the per-parameter FIM diagonal
// dG[o] * dA[j] (the diagonal of G kron A), its EMA, division of the gradient
// by (F + lambda), momentum, weight decay and the in-place parameter write
// (CAFIN briefing, "Introduction" and "Kernel Fusion Strategy").
//
// Three launches per step, all HBM-streaming.  The FACTORS phase is the first
// two (the streaming reduction into the workspace, then dA / dG from it,
// written to the descriptor's buffers for every layer kind); the UPDATE phase
// is the parameter pass, which reads dA / dG from those buffers.
//   diag_colsq_kernel   sum of squares down the rows of row-major matrices.
//                       Every reduction of the step is one of these: linear
//                       a [N, d_in] and g [N, d_out] give dA / dG directly; a
//                       conv input x [B, C*H*W] gives S = sum_b x^2 per pixel,
//                       a conv output gradient g [B, C*Ho*Wo] the same.  Each
//                       thread owns 4 adjacent columns and walks the rows in
//                       order: no atomics, no cross-lane reduction, the result
//                       is bit-reproducible.
//   diag_finish_kernel  conv: dA[c, kh, kw] = (1/N) * sum of S over the output
//                       positions' strided window (zero padding handled by the
//                       index range), dG[c] = (1/N) * sum of S over the plane;
//                       linear inputs larger than one row chunk: sum of the
//                       chunk partials in chunk order; bias entries dA[d_in] = 1.
//   diag_update_kernel  one float4-vectorised pass over every parameter
//                       segment: 4 loads + 3 stores of float32 per parameter.
// Batch-norm layers (Osawa et al. sections 1 and 5.4: a diagonal Fisher for
// batch normalisation) take one more FACTORS launch, diag_bn_kernel, which
// forms their gamma / beta Fisher diagonals directly; their parameters join
// the same parameter pass with their own damping.
#include "common.h"

#include <algorithm>
#include <mutex>
#include <vector>

namespace kfac {

namespace {

// 8 wavefronts split a workgroup's rows: at batch 128 each then issues its 16
// rows' loads in one round (4 wavefronts took two rounds, the second after the
// first returned): reduction phase 0.3995 -> 0.3970 ms on ResNet-18's shapes
constexpr int kColThreads = 512;
constexpr int kColWaves = kColThreads / 64;
constexpr int kColTile = 64 * 4;            // columns per workgroup (4 per lane; the wavefronts split the rows)
constexpr int kRowChunk = 512;              // rows per workgroup before chunking
constexpr int kMaxColTasks = 64;

struct ColTask {
  const float* src;   // [R][K] row-major
  float* dst;         // chunks == 1: dst[k] = scale * sum; else dst[chunk * K + k] = sum
  int64_t R;
  int32_t K;
  int32_t rc;         // rows per chunk
  int32_t tiles;      // column tiles
  int32_t blk_begin;
  int32_t chunks;
  float scale;
};
struct ColTasks {
  int32_t begin[kMaxColTasks];   // t[i].blk_begin, contiguous (one batch of scalar loads)
  ColTask t[kMaxColTasks];
  int32_t n;
};
static_assert(sizeof(ColTasks) <= 4096, "kernel arguments");

constexpr int kFinThreads = 512;
constexpr int kFinWaves = kFinThreads / kWave;
constexpr int kMaxFinTasks = 44;
constexpr int kMaxTab = 2048;        // plane rows / columns covered by the LDS tap-mask tables
constexpr int kFinPxPerLane = 16;    // team size target: about this many pixels per lane

enum FinKind : int32_t { FIN_WINDOW = 0, FIN_CHUNKSUM = 1 };

// Kernel rows handled by one window item for a k x k kernel: all of them for
// k <= 3 (at most 9 taps per pixel), two for k = 4, one above (each item then
// visits only the rows its kernel row reaches, stepping by the stride).
__host__ __device__ constexpr int fin_nkh(int k) { return k <= 3 ? k : (k == 4 ? 2 : 1); }

struct FinTask {
  const float* src;
  float* dst;
  int32_t kind;
  int32_t C, H, W, k, stride, pad, Ho, Wo;  // FIN_WINDOW: S is [C][H][W]
  int32_t K, chunks;                        // FIN_CHUNKSUM: partials [chunks][K]
  int32_t blk_begin;
  float scale;
  int32_t bias_index;                       // >= 0: dst[bias_index] = 1
  int32_t team;                             // FIN_WINDOW: wavefronts per item (1, 2, 4 or 8)
};
struct FinTasks {
  FinTask t[kMaxFinTasks];
  int32_t n;
};

constexpr int kUpdThreads = 256;
constexpr int kUpdUnroll = 2;   // float4 groups per thread (50 VGPRs: 8 wavefronts per SIMD)
constexpr int kUpdPerBlock = kUpdThreads * 4 * kUpdUnroll;
constexpr int kMaxSegs = 48;

struct Seg {
  const float* grad;
  float* w;
  float* mom;
  float* F;
  const float* dA;    // nullptr: the target of element e is dG[e] (a bias segment, whose dA entry is
                      // exactly 1, or a batch-norm parameter with its own Fisher diagonal in dG)
  const float* dG;
  int32_t n;
  int32_t cols;       // d_in for a weight segment
  int32_t blk_begin;
  float damping;      // lambda of this segment's layer
};
struct Segs {
  Seg s[kMaxSegs];
  int32_t n;
  float beta, one_minus_beta, weight_decay, momentum, lr;
  uint32_t* flags;
};
static_assert(sizeof(Segs) <= 4096, "kernel arguments");

// Batch-norm Fisher diagonals: one workgroup per channel c of a layer; its 4
// wavefronts take the samples b = w, w + 4, ...; per sample the per-sample
// gradients s1 = sum_hw g x_hat (gamma) and s2 = sum_hw g (beta) by a
// wavefront reduction, squared and summed; the 4 wavefront sums in order.
constexpr int kBnThreads = 256;
constexpr int kBnWaves = kBnThreads / kWave;
constexpr int kMaxBnTasks = 64;
struct BnTask {
  const float* x;     // x_hat [B, C, HW]
  const float* g;     // output gradient [B, C, HW]
  float* fg;          // [C] gamma Fisher diagonal
  float* fb;          // [C] beta Fisher diagonal
  int32_t C, B, HW, blk_begin;
  float scale;        // 1 / B
  int32_t pad_;
};
struct BnTasks {
  BnTask t[kMaxBnTasks];
  int32_t n;
};
static_assert(sizeof(BnTasks) <= 4096, "kernel arguments");

template <typename T, int N>
__device__ inline int find_task(const T (&t)[N], int n, int blk) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {          // last task with blk_begin <= blk
    int mid = (lo + hi + 1) >> 1;
    if (t[mid].blk_begin <= blk) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The last task whose first block is at or before `blk`, as a count over the
// contiguous start offsets: their loads go out together (a binary search
// waits for one round trip per step before the workgroup issues any load).
// Used by the column reduction (phase 0.3974 -> 0.3942 ms on ResNet-18's
// shapes); the batch-norm kernel's short per-channel workgroups were slower
// with it (0.449 -> 0.466 ms: 63 compares over a 64-entry table), so the
// other kernels keep the binary search.
template <int N>
__device__ inline int count_task(const int32_t (&begin)[N], int n, int blk) {
  int ti = 0;
#pragma unroll
  for (int i = 1; i < N; ++i) ti += (i < n && begin[i] <= blk) ? 1 : 0;
  return ti;
}

__global__ void __launch_bounds__(kColThreads) diag_colsq_kernel(ColTasks tasks) {
  __shared__ f32x4 part[kColWaves - 1][64];
  const int ti = count_task(tasks.begin, tasks.n, blockIdx.x);
  const ColTask& T = tasks.t[ti];
  const int b = blockIdx.x - T.blk_begin;
  const int tile = b % T.tiles;
  const int chunk = b / T.tiles;
  const int64_t r0 = static_cast<int64_t>(chunk) * T.rc;
  const int64_t r1 = min(T.R, r0 + T.rc);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int c0 = tile * kColTile + lane * 4;
  const int K = T.K;
  float* out = T.chunks == 1 ? T.dst : T.dst + static_cast<int64_t>(chunk) * K;
  const float s = T.chunks == 1 ? T.scale : 1.0f;
  // wavefront w sums rows r0 + w, r0 + w + kColWaves, ...; the partial sums
  // are added in wavefront order (deterministic)
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (c0 < K) {
    if ((K & 3) == 0) {
      const int64_t stride = static_cast<int64_t>(kColWaves) * K;
      const float* p = T.src + (r0 + wid) * K + c0;
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
      int64_t r = r0 + wid;
      for (; r + 15 * kColWaves < r1; r += 16 * kColWaves) {
        f32x4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + u * stride));
#pragma unroll
        for (int u = 0; u < 16; u += 2) {
          acc0 += v[u] * v[u];
          acc1 += v[u + 1] * v[u + 1];
        }
        p += 16 * stride;
      }
      for (; r < r1; r += kColWaves) {
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        acc0 += v * v;
        p += stride;
      }
      acc = acc0 + acc1;
    } else {
      for (int64_t r = r0 + wid; r < r1; r += kColWaves) {
        const float* p = T.src + r * K;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (c0 + q < K) acc[q] = fmaf(p[c0 + q], p[c0 + q], acc[q]);
      }
    }
  }
  if (wid > 0) part[wid - 1][lane] = acc;
  __syncthreads();
  if (wid != 0 || c0 >= K) return;
#pragma unroll
  for (int w = 0; w < kColWaves - 1; ++w) acc += part[w][lane];
  acc *= s;
  if ((K & 3) == 0) {
    *reinterpret_cast<f32x4*>(out + c0) = acc;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (c0 + q < K) out[c0 + q] = acc[q];
  }
}

// Sum over the wavefront, returned to every lane: butterflies within rows of
// 16 lanes by DPP moves (pairs, quads, half-row and row mirrors), then the
// four row sums by lane reads; no LDS round trips.
template <int CTRL>
__device__ inline float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

__device__ inline float wave_sum(float v) {
  v += dpp_mov<0xb1>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4e>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0x141>(v);   // row_half_mirror
  v += dpp_mov<0x140>(v);   // row_mirror
  const auto lane_v = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
  return (lane_v(0) + lane_v(16)) + (lane_v(32) + lane_v(48));
}

__global__ void __launch_bounds__(kBnThreads) diag_bn_kernel(BnTasks tasks) {
  __shared__ float red[kBnWaves][2];
  const BnTask& T = tasks.t[find_task(tasks.t, tasks.n, blockIdx.x)];
  const int c = blockIdx.x - T.blk_begin;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  float q1 = 0.f, q2 = 0.f;
  for (int b = wid; b < T.B; b += kBnWaves) {
    const int64_t off = (static_cast<int64_t>(b) * T.C + c) * T.HW;
    const float* xp = T.x + off;
    const float* gp = T.g + off;
    float s1 = 0.f, s2 = 0.f;
    if ((T.HW & 3) == 0) {
      // 16-byte loads, four of each tensor in flight per lane
      constexpr int kStep = 4 * kWave;
      int e = 4 * lane;
      for (; e + 3 * kStep < T.HW; e += 4 * kStep) {
        f32x4 xv[4], gv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          xv[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(xp + e + u * kStep));
          gv[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(gp + e + u * kStep));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            s1 = fmaf(gv[u][q], xv[u][q], s1);
            s2 += gv[u][q];
          }
      }
      for (; e < T.HW; e += kStep) {
        const f32x4 xv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(xp + e));
        const f32x4 gv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(gp + e));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          s1 = fmaf(gv[q], xv[q], s1);
          s2 += gv[q];
        }
      }
    } else {
      for (int e = lane; e < T.HW; e += kWave) {
        s1 = fmaf(gp[e], xp[e], s1);
        s2 += gp[e];
      }
    }
    s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    q1 = fmaf(s1, s1, q1);
    q2 = fmaf(s2, s2, q2);
  }
  if (lane == 0) {
    red[wid][0] = q1;
    red[wid][1] = q2;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float a1 = 0.f, a2 = 0.f;
    for (int w = 0; w < kBnWaves; ++w) {
      a1 += red[w][0];
      a2 += red[w][1];
    }
    T.fg[c] = a1 * T.scale;
    T.fb[c] = a2 * T.scale;
  }
}

// Bit t of the result is set when input row (or column) x is reached by
// kernel row (column) t from some output position: x = o * stride + t - pad
// with 0 <= o < n_out.
// (y = o * stride exactly when t = (x + pad) mod stride, mod stride; one
// division per call)
__device__ inline uint32_t tap_mask(int x, int k, int pad, int stride, int n_out) {
  const int base = x + pad;
  const int64_t lim = static_cast<int64_t>(n_out) * stride;   // o < n_out
  uint32_t m = 0;
  for (int t = base % stride; t < k; t += stride) {
    const int y = base - t;
    if (y >= 0 && y < lim) m |= 1u << t;
  }
  return m;
}

// One window item: channel c, kernel rows [kh0, kh0 + nk).  The team's lanes
// walk the rows these kernel rows reach (every row, or every stride-th one
// for a single kernel row) along the columns, VEC consecutive pixels per
// load; a pixel adds its value to every tap (kh, kw) of the item whose masks
// say it lies in that tap's window.  Each pixel of S is read once per item.
template <int K, int VEC, bool TABS>
__device__ __forceinline__ void fin_window(const FinTask& T, int c, int kh0, int nk, int tix, int nthr,
                                           const uint8_t* rowtab, const uint8_t* coltab,
                                           float (&acc)[fin_nkh(K) * K]) {
  constexpr int NKH = fin_nkh(K);
#pragma unroll
  for (int t = 0; t < NKH * K; ++t) acc[t] = 0.f;
  // rows reached by the item's kernel rows
  int hfirst = 1 << 30, hlast = -1;
  for (int r = 0; r < nk; ++r) {
    const int kh = kh0 + r;
    const int o0 = max(0, (T.pad - kh + T.stride - 1) / T.stride);          // first o with o*s + kh - pad >= 0
    const int o1 = min(T.Ho - 1, (T.H - 1 + T.pad - kh) / T.stride);        // last o with o*s + kh - pad < H
    if (T.H - 1 + T.pad - kh < 0 || o0 > o1) continue;
    hfirst = min(hfirst, o0 * T.stride + kh - T.pad);
    hlast = max(hlast, o1 * T.stride + kh - T.pad);
  }
  if (hlast < hfirst) return;
  const int hstep = nk == 1 ? T.stride : 1;
  const int nrows = (hlast - hfirst) / hstep + 1;
  const int wv = T.W / VEC;                       // loads per row
  const int nld = nrows * wv;
  const float* S = T.src + static_cast<int64_t>(c) * T.H * T.W;
  const uint32_t rsel = (1u << nk) - 1;
  // lane position (row i, load column x), stepped by nthr loads without division
  const int di = nthr / wv, dx = nthr - (nthr / wv) * wv;
  int i = tix / wv, x = tix - (tix / wv) * wv;
  // (2 loads in flight with the tables: 47 VGPRs, so 8 wavefronts per SIMD
  // and twice the resident workgroups of 8 loads in flight (86 VGPRs), which
  // the launch's ~2.7 rounds of short workgroups need more (19.3 -> 17.2 us);
  // the rare path without tables, which computes every tap mask, takes one
  // load at a time to stay small)
  constexpr int NL = TABS ? 2 : 1;
  for (int q0 = tix; q0 < nld; q0 += NL * nthr) {
    float v[NL][VEC];
    int hh[NL], ww[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const bool ok = q0 + u * nthr < nld;
      hh[u] = ok ? hfirst + i * hstep : -1;
      ww[u] = x * VEC;
      if (ok) {
        const float* ptr = S + static_cast<int64_t>(hh[u]) * T.W + ww[u];
        if constexpr (VEC == 4) {
          const f32x4 t4 = *reinterpret_cast<const f32x4*>(ptr);
          v[u][0] = t4[0]; v[u][1] = t4[1]; v[u][2] = t4[2]; v[u][3] = t4[3];
        } else {
          v[u][0] = *ptr;
        }
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[u][e] = 0.f;
      }
      i += di;
      x += dx;
      if (x >= wv) { x -= wv; ++i; }
    }
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      if (hh[u] < 0) continue;
      const uint32_t rm = (TABS ? rowtab[hh[u]] : tap_mask(hh[u], K, T.pad, T.stride, T.Ho)) >> kh0 & rsel;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const uint32_t cm = TABS ? coltab[ww[u] + e] : tap_mask(ww[u] + e, K, T.pad, T.stride, T.Wo);
#pragma unroll
        for (int r = 0; r < NKH; ++r)
#pragma unroll
          for (int kw = 0; kw < K; ++kw)
            acc[r * K + kw] += ((rm >> r) & (cm >> kw) & 1u) ? v[u][e] : 0.f;
      }
    }
  }
}

template <int K>
__device__ __forceinline__ void fin_window_block(const FinTask& T, int b, float (*red)[16], uint8_t* rowtab,
                                                 uint8_t* coltab) {
  constexpr int NKH = fin_nkh(K);
  const bool tabs = T.H <= kMaxTab && T.W <= kMaxTab;
  if (tabs) {
    for (int h = threadIdx.x; h < T.H; h += kFinThreads) rowtab[h] = tap_mask(h, K, T.pad, T.stride, T.Ho);
    for (int w = threadIdx.x; w < T.W; w += kFinThreads) coltab[w] = tap_mask(w, K, T.pad, T.stride, T.Wo);
  }
  __syncthreads();
  const int groups = (K + NKH - 1) / NKH;
  const int items = T.C * groups;
  const int teams = kFinWaves / T.team;
  const int wid = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int team = wid / T.team, tw = wid - team * T.team;
  const int item = b * teams + team;
  const int nthr = T.team * kWave, tix = tw * kWave + lane;
  const int c = item / groups, kh0 = (item - c * groups) * NKH, nk = min(NKH, K - kh0);
  float acc[NKH * K];
  if (item < items) {
    // (the tap masks come from the LDS tables unless the plane is too wide for
    // them; each body is compiled for one of the two, which keeps the code
    // of the common one within the instruction cache)
    const bool vec4 = (T.W & 3) == 0;   // plane starts and rows 16-byte aligned (S is 256-byte aligned)
    if (!tabs) fin_window<K, 1, false>(T, c, kh0, nk, tix, nthr, rowtab, coltab, acc);
    else if (vec4) fin_window<K, 4, true>(T, c, kh0, nk, tix, nthr, rowtab, coltab, acc);
    else fin_window<K, 1, true>(T, c, kh0, nk, tix, nthr, rowtab, coltab, acc);
  } else {
#pragma unroll
    for (int t = 0; t < NKH * K; ++t) acc[t] = 0.f;
  }
  float* out = T.dst + static_cast<int64_t>(c) * K * K + kh0 * K;
#pragma unroll
  for (int t = 0; t < NKH * K; ++t) {
    const float v = wave_sum(acc[t]);
    if (T.team == 1) {
      if (lane == 0 && item < items && t < nk * K) out[t] = v * T.scale;
    } else if (lane == 0) {
      red[wid][t] = v;
    }
  }
  if (T.team == 1) return;
  __syncthreads();
  if (tw == 0 && lane < nk * K && item < items) {
    float v = 0.f;
    for (int w = 0; w < T.team; ++w) v += red[team * T.team + w][lane];
    out[lane] = v * T.scale;
  }
}

__global__ void __launch_bounds__(kFinThreads) diag_finish_kernel(FinTasks tasks) {
  __shared__ float red[kFinWaves][16];
  __shared__ uint8_t rowtab[kMaxTab], coltab[kMaxTab];
  const int ti = find_task(tasks.t, tasks.n, blockIdx.x);  // uniform per block
  const FinTask T = tasks.t[ti];   // by value: the helpers take its address
  const int b = blockIdx.x - T.blk_begin;
  if (T.bias_index >= 0 && b == 0 && threadIdx.x == 0) T.dst[T.bias_index] = 1.0f;
  if (T.kind == FIN_CHUNKSUM) {
    const int c = b * kFinThreads + threadIdx.x;
    if (c < T.K) {
      float acc = 0.f;
      for (int ch = 0; ch < T.chunks; ++ch) acc += T.src[static_cast<int64_t>(ch) * T.K + c];
      T.dst[c] = acc * T.scale;
    }
    return;
  }
  // FIN_WINDOW: dA[c, kh, kw] = scale * sum over output positions of
  // S[c, ho * stride + kh - pad, wo * stride + kw - pad] (zero outside)
  switch (T.k) {
    case 1: fin_window_block<1>(T, b, red, rowtab, coltab); break;
    case 2: fin_window_block<2>(T, b, red, rowtab, coltab); break;
    case 3: fin_window_block<3>(T, b, red, rowtab, coltab); break;
    case 4: fin_window_block<4>(T, b, red, rowtab, coltab); break;
    case 5: fin_window_block<5>(T, b, red, rowtab, coltab); break;
    case 6: fin_window_block<6>(T, b, red, rowtab, coltab); break;
    default: fin_window_block<7>(T, b, red, rowtab, coltab); break;
  }
}

struct UpdOut {
  float w, v, f;
};

__device__ inline UpdOut upd_one(float g, float w, float v, float f, float target, float damping, const Segs& P) {
  UpdOut o;
  o.f = P.beta * f + P.one_minus_beta * target;
  const float p = g / (o.f + damping);
  const float d = fmaf(P.weight_decay, w, p);
  o.v = fmaf(P.momentum, v, d);
  o.w = fmaf(-P.lr, o.v, w);
  return o;
}

__global__ void __launch_bounds__(kUpdThreads) diag_update_kernel(Segs segs) {
  const int si = find_task(segs.s, segs.n, blockIdx.x);
  const Seg& S = segs.s[si];
  const int64_t base = static_cast<int64_t>(blockIdx.x - S.blk_begin) * kUpdPerBlock;
  bool bad = false;
  if ((S.n & 3) == 0) {
    f32x4 g[kUpdUnroll], w[kUpdUnroll], v[kUpdUnroll], f[kUpdUnroll];
    int e[kUpdUnroll];
#pragma unroll
    for (int u = 0; u < kUpdUnroll; ++u) {
      e[u] = static_cast<int>(base + u * (kUpdThreads * 4) + threadIdx.x * 4);
      if (e[u] < S.n) {
        // every parameter is read and written once per step: streaming loads
        // (measured 1.7% faster than cached ones for W, V and F)
        g[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S.grad + e[u]));
        w[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S.w + e[u]));
        v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S.mom + e[u]));
        f[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S.F + e[u]));
      }
    }
#pragma unroll
    for (int u = 0; u < kUpdUnroll; ++u) {
      if (e[u] >= S.n) continue;
      float tgt[4];
      if (S.dA && (S.cols & 3) == 0) {
        // the 4 elements share a row: one dG entry, 4 adjacent dA entries
        const int o = e[u] / S.cols;
        const int j = e[u] - o * S.cols;
        const float dg = S.dG[o];
        const f32x4 da = *reinterpret_cast<const f32x4*>(S.dA + j);
#pragma unroll
        for (int q = 0; q < 4; ++q) tgt[q] = dg * da[q];
      } else if (S.dA) {
        int o = e[u] / S.cols;
        int j = e[u] - o * S.cols;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          tgt[q] = S.dG[o] * S.dA[j];
          if (++j == S.cols) { j = 0; ++o; }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) tgt[q] = S.dG[e[u] + q];
      }
      f32x4 wn, vn, fn;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        UpdOut r = upd_one(g[u][q], w[u][q], v[u][q], f[u][q], tgt[q], S.damping, segs);
        wn[q] = r.w; vn[q] = r.v; fn[q] = r.f;
        bad |= !(isfinite(r.w) && isfinite(r.v));
      }
      *reinterpret_cast<f32x4*>(S.F + e[u]) = fn;
      *reinterpret_cast<f32x4*>(S.mom + e[u]) = vn;
      *reinterpret_cast<f32x4*>(S.w + e[u]) = wn;
    }
  } else {
    for (int u = 0; u < kUpdUnroll * 4; ++u) {
      const int64_t e = base + static_cast<int64_t>(u) * kUpdThreads + threadIdx.x;
      if (e >= S.n) continue;
      float tgt;
      if (S.dA) {
        const int o = static_cast<int>(e / S.cols);
        tgt = S.dG[o] * S.dA[e - static_cast<int64_t>(o) * S.cols];
      } else {
        tgt = S.dG[e];
      }
      UpdOut r = upd_one(S.grad[e], S.w[e], S.mom[e], S.F[e], tgt, S.damping, segs);
      S.F[e] = r.f; S.mom[e] = r.v; S.w[e] = r.w;
      bad |= !(isfinite(r.w) && isfinite(r.v));
    }
  }
  if (__any(bad) && (threadIdx.x & (kWave - 1)) == 0) raise_flag(segs.flags, KFAC_FLAG_NONFINITE);
}

// -------------------------------------------------------------------------
// planning

struct DiagPlan {
  std::vector<ColTask> col;
  std::vector<FinTask> fin;
  std::vector<BnTask> bn;
  std::vector<Seg> seg;
  std::vector<char> seg_bn;          // per segment: a batch-norm parameter (damping_bn)
  std::vector<RescaleSeg> rescale;   // conv / linear weights
  size_t ws_bytes = kFlagBytes;
};

// Wavefronts per window item: the smallest team (1, 2, 4 or 8 wavefronts)
// whose lanes see at most about kFinPxPerLane pixels each.
int window_team(int k, int stride, int H, int W, int Ho) {
  const int nkh = fin_nkh(k);
  const int64_t rows = nkh == 1 ? std::min<int64_t>(H, Ho) : H;
  const int64_t px = rows * W;
  int team = 1;
  while (team < kFinWaves && px > static_cast<int64_t>(kWave) * team * kFinPxPerLane) team *= 2;
  (void)stride;
  return team;
}

int fin_blocks(const FinTask& t) {
  if (t.kind == FIN_WINDOW) {
    const int items = t.C * ((t.k + fin_nkh(t.k) - 1) / fin_nkh(t.k));
    const int per_block = kFinWaves / t.team;
    return (items + per_block - 1) / per_block;
  }
  return t.chunks > 1 ? (t.K + kFinThreads - 1) / kFinThreads : 1;
}

// Builds the launch tables; with ws == nullptr only sizes are computed.
DiagPlan plan_diag(const kfac_layer_t* layers, int n, char* ws) {
  DiagPlan P;
  size_t off = kFlagBytes;
  auto carve = [&](size_t floats) -> float* {
    float* p = ws ? reinterpret_cast<float*>(ws + off) : nullptr;
    off = align_up(off + floats * sizeof(float), 256);
    return p;
  };
  int col_blk = 0, fin_blk = 0, upd_blk = 0;
  auto add_col = [&](const float* src, float* dst, int64_t R, int K, float scale, float* partials,
                     int chunks, int rc) {
    ColTask t{};
    t.src = src;
    t.R = R;
    t.K = K;
    t.rc = rc;
    t.tiles = (K + kColTile - 1) / kColTile;
    t.chunks = chunks;
    t.dst = chunks == 1 ? dst : partials;
    t.scale = scale;
    t.blk_begin = col_blk;
    col_blk += t.tiles * chunks;
    P.col.push_back(t);
  };
  auto add_fin = [&](FinTask t, int blocks) {
    t.blk_begin = fin_blk;
    fin_blk += blocks;
    P.fin.push_back(t);
  };
  int bn_blk = 0;
  for (int li = 0; li < n; ++li) {
    const kfac_layer_t& L = layers[li];
    const LayerGeom g = geom_of(L);
    const float invN = 1.0f / static_cast<float>(g.rows);
    if (g.bn) {
      // gamma / beta Fisher diagonals straight into dA / dG, then one
      // segment per parameter vector whose target is that diagonal
      BnTask t{};
      t.x = static_cast<const float*>(L.a);
      t.g = static_cast<const float*>(L.g);
      t.fg = L.dA;
      t.fb = L.dG;
      t.C = g.c_in;
      t.B = g.batch;
      t.HW = g.h * g.w;
      t.scale = 1.0f / static_cast<float>(g.batch);
      t.blk_begin = bn_blk;
      bn_blk += t.C;
      P.bn.push_back(t);
      for (int which = 0; which < (g.bias ? 2 : 1); ++which) {
        Seg sg{};
        sg.grad = which == 0 ? L.grad_w : L.grad_b;
        sg.w = which == 0 ? L.w : L.b;
        sg.mom = which == 0 ? L.mom_w : L.mom_b;
        sg.F = which == 0 ? L.F_w : L.F_b;
        sg.dA = nullptr;
        sg.dG = which == 0 ? L.dA : L.dG;
        sg.n = g.d_out;
        sg.cols = 1;
        sg.blk_begin = upd_blk;
        upd_blk += (sg.n + kUpdPerBlock - 1) / kUpdPerBlock;
        P.seg.push_back(sg);
        P.seg_bn.push_back(1);
      }
      continue;
    }
    {
      RescaleSeg r{};
      r.w = L.w;
      r.n = static_cast<int64_t>(g.d_out) * g.d_in;
      r.d_out = g.d_out;
      r.part = carve(static_cast<size_t>(rescale_blocks(r.n)));
      P.rescale.push_back(r);
    }
    if (g.conv) {
      // input: S_x[c*H*W + p] = sum_b x^2 ; then strided window sums
      const int Kx = g.c_in * g.h * g.w;
      float* Sx = carve(Kx);
      add_col(static_cast<const float*>(L.a), Sx, g.batch, Kx, 1.0f, nullptr, 1, g.batch);
      FinTask fx{};
      fx.src = Sx; fx.dst = L.dA; fx.kind = FIN_WINDOW;
      fx.C = g.c_in; fx.H = g.h; fx.W = g.w; fx.k = g.kh; fx.stride = g.stride; fx.pad = g.pad;
      fx.Ho = g.h_out; fx.Wo = g.w_out; fx.scale = invN; fx.bias_index = g.bias ? g.d_in : -1;
      fx.team = window_team(g.kh, g.stride, g.h, g.w, g.h_out);
      add_fin(fx, fin_blocks(fx));
      const int Kg = g.d_out * g.h_out * g.w_out;
      float* Sg = carve(Kg);
      add_col(static_cast<const float*>(L.g), Sg, g.batch, Kg, 1.0f, nullptr, 1, g.batch);
      FinTask fg{};
      fg.src = Sg; fg.dst = L.dG; fg.kind = FIN_WINDOW;
      fg.C = g.d_out; fg.H = g.h_out; fg.W = g.w_out; fg.k = 1; fg.stride = 1; fg.pad = 0;
      fg.Ho = g.h_out; fg.Wo = g.w_out; fg.scale = invN; fg.bias_index = -1;
      fg.team = window_team(1, 1, g.h_out, g.w_out, g.h_out);
      add_fin(fg, fin_blocks(fg));
    } else {
      const int64_t R = g.rows;
      const int chunks = static_cast<int>((R + kRowChunk - 1) / kRowChunk);
      const int rc = chunks == 1 ? static_cast<int>(R) : kRowChunk;
      for (int which = 0; which < 2; ++which) {
        const float* src = static_cast<const float*>(which == 0 ? L.a : L.g);
        float* dst = which == 0 ? L.dA : L.dG;
        const int K = which == 0 ? g.d_in : g.d_out;
        float* part = chunks > 1 ? carve(static_cast<size_t>(chunks) * K) : nullptr;
        add_col(src, dst, R, K, invN, part, chunks, rc);
        const int bias_idx = (which == 0 && g.bias) ? g.d_in : -1;
        if (chunks > 1 || bias_idx >= 0) {
          FinTask f{};
          f.src = part; f.dst = dst; f.kind = FIN_CHUNKSUM;
          f.K = chunks > 1 ? K : 0; f.chunks = chunks; f.scale = invN; f.bias_index = bias_idx;
          add_fin(f, fin_blocks(f));
        }
      }
    }
    // update segments
    {
      Seg s{};
      s.grad = L.grad_w; s.w = L.w; s.mom = L.mom_w; s.F = L.F_w; s.dA = L.dA; s.dG = L.dG;
      s.n = g.d_out * g.d_in; s.cols = g.d_in; s.blk_begin = upd_blk;
      upd_blk += (s.n + kUpdPerBlock - 1) / kUpdPerBlock;
      P.seg.push_back(s);
      P.seg_bn.push_back(0);
      if (g.bias) {
        Seg sb{};
        sb.grad = L.grad_b; sb.w = L.b; sb.mom = L.mom_b; sb.F = L.F_b; sb.dA = nullptr; sb.dG = L.dG;
        sb.n = g.d_out; sb.cols = 1; sb.blk_begin = upd_blk;
        upd_blk += (sb.n + kUpdPerBlock - 1) / kUpdPerBlock;
        P.seg.push_back(sb);
        P.seg_bn.push_back(0);
      }
    }
  }
  P.ws_bytes = off;
  return P;
}

}  // namespace

size_t diag_workspace_bytes(const kfac_layer_t* layers, int n) { return plan_diag(layers, n, nullptr).ws_bytes; }

namespace {

// The step's launches with the reduction's intermediate sums carved from `ws`
// (its first kFlagBytes are not used for them) and the flag word at `flags`.
kfac_status_t enqueue_steps(const kfac_layer_t* layers, int n, const kfac_hparams_t& hp, char* ws,
                            size_t ws_bytes, uint32_t* flags, hipStream_t stream, int phases) {
  DiagPlan P = plan_diag(layers, n, ws);
  if (P.ws_bytes > ws_bytes) return KFAC_ERR_WORKSPACE;
  if (phases & KFAC_PHASE_FACTORS) {
    for (size_t g0 = 0; g0 < P.col.size(); g0 += kMaxColTasks) {
      const size_t g1 = std::min(P.col.size(), g0 + kMaxColTasks);
      ColTasks T{};
      const int base = P.col[g0].blk_begin;
      int blocks = 0;
      for (size_t i = g0; i < g1; ++i) {
        T.t[i - g0] = P.col[i];
        T.t[i - g0].blk_begin -= base;
        T.begin[i - g0] = T.t[i - g0].blk_begin;
        blocks = T.t[i - g0].blk_begin + P.col[i].tiles * P.col[i].chunks;
      }
      T.n = static_cast<int>(g1 - g0);
      hipLaunchKernelGGL(diag_colsq_kernel, dim3(blocks), dim3(kColThreads), 0, stream, T);
      KFAC_HIP_TRY(hipGetLastError());
    }
    for (size_t g0 = 0; g0 < P.bn.size(); g0 += kMaxBnTasks) {
      const size_t g1 = std::min(P.bn.size(), g0 + kMaxBnTasks);
      BnTasks T{};
      const int base = P.bn[g0].blk_begin;
      for (size_t i = g0; i < g1; ++i) {
        T.t[i - g0] = P.bn[i];
        T.t[i - g0].blk_begin -= base;
      }
      const int blocks = P.bn[g1 - 1].blk_begin - base + P.bn[g1 - 1].C;
      T.n = static_cast<int>(g1 - g0);
      hipLaunchKernelGGL(diag_bn_kernel, dim3(blocks), dim3(kBnThreads), 0, stream, T);
      KFAC_HIP_TRY(hipGetLastError());
    }
    for (size_t g0 = 0; g0 < P.fin.size(); g0 += kMaxFinTasks) {
      const size_t g1 = std::min(P.fin.size(), g0 + kMaxFinTasks);
      FinTasks T{};
      const int base = P.fin[g0].blk_begin;
      int blocks = 0;
      for (size_t i = g0; i < g1; ++i) {
        T.t[i - g0] = P.fin[i];
        T.t[i - g0].blk_begin -= base;
      }
      blocks = P.fin[g1 - 1].blk_begin - base + fin_blocks(P.fin[g1 - 1]);
      T.n = static_cast<int>(g1 - g0);
      hipLaunchKernelGGL(diag_finish_kernel, dim3(blocks), dim3(kFinThreads), 0, stream, T);
      KFAC_HIP_TRY(hipGetLastError());
    }
  }
  if (phases & KFAC_PHASE_UPDATE) {
    for (size_t g0 = 0; g0 < P.seg.size(); g0 += kMaxSegs) {
      const size_t g1 = std::min(P.seg.size(), g0 + kMaxSegs);
      Segs S{};
      const int base = P.seg[g0].blk_begin;
      for (size_t i = g0; i < g1; ++i) {
        S.s[i - g0] = P.seg[i];
        S.s[i - g0].blk_begin -= base;
        S.s[i - g0].damping = P.seg_bn[i] ? hp.damping_bn : hp.damping;
      }
      const Seg& last = P.seg[g1 - 1];
      const int blocks = last.blk_begin - base + (last.n + kUpdPerBlock - 1) / kUpdPerBlock;
      S.n = static_cast<int>(g1 - g0);
      S.beta = hp.ema_decay;
      S.one_minus_beta = 1.0f - hp.ema_decay;
      S.weight_decay = hp.weight_decay;
      S.momentum = hp.momentum;
      S.lr = hp.lr;
      S.flags = flags;
      hipLaunchKernelGGL(diag_update_kernel, dim3(blocks), dim3(kUpdThreads), 0, stream, S);
      KFAC_HIP_TRY(hipGetLastError());
    }
  }
  if ((phases & KFAC_PHASE_RESCALE) && (hp.options & KFAC_OPT_RESCALE) && !P.rescale.empty()) {
    kfac_status_t r = launch_rescale(P.rescale, hp.rescale_eps, stream);
    if (r != KFAC_OK) return r;
  }
  return KFAC_OK;
}

}  // namespace

kfac_status_t diag_enqueue_into(const kfac_layer_t* layers, int n, const kfac_hparams_t& hp, char* ws,
                                size_t ws_bytes, uint32_t* flags, hipStream_t stream, int phases) {
  return enqueue_steps(layers, n, hp, ws, ws_bytes, flags, stream, phases);
}

kfac_status_t diag_enqueue(const kfac_layer_t* layers, int n, const kfac_hparams_t& hp, char* ws,
                           size_t ws_bytes, hipStream_t stream, int phases) {
  return enqueue_steps(layers, n, hp, ws, ws_bytes, reinterpret_cast<uint32_t*>(ws), stream, phases);
}

// ---------------------------------------------------------------------------
// The same step for callers that cannot allocate device memory: the
// reduction's intermediate sums (the only scratch the step's kernels use) live
// in `scratch`, a file-scope device array of kNoAllocScratchBytes that every
// GPU the library runs on holds until the process ends.  Its device address
// on each GPU is looked up once, with that GPU current, and kept; host code
// never passes the array's own name to a kernel.  Every call on one GPU uses
// the same array, so calls that can overlap on one GPU race; the sums are
// written by each FACTORS phase before they are read, so nothing in the
// array has to start at zero.

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

kfac_status_t scratch_address(char** out) {
  static std::mutex mu;
  static std::vector<char*> per_device;
  int dev = 0;
  KFAC_HIP_TRY(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(mu);
  if (per_device.size() <= static_cast<size_t>(dev)) per_device.resize(dev + 1, nullptr);
  if (!per_device[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return KFAC_ERR_HIP;
    per_device[dev] = static_cast<char*>(p);
  }
  *out = per_device[dev];
  return KFAC_OK;
}

}  // namespace

kfac_status_t diag_enqueue_noalloc(const kfac_layer_t* layers, int n, const kfac_hparams_t& hp, uint32_t* flags,
                                   hipStream_t stream, int phases) {
  if (diag_workspace_bytes(layers, n) > kNoAllocScratchBytes) return KFAC_ERR_WORKSPACE;
  char* base = nullptr;
  kfac_status_t r = scratch_address(&base);
  if (r != KFAC_OK) return r;
  return enqueue_steps(layers, n, hp, base, kNoAllocScratchBytes, flags, stream, phases);
}

}  // namespace kfac
