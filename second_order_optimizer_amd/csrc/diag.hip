// Diagonal (AdaFisher-style) K-FAC step: the per-parameter FIM diagonal
// dG[o] * dA[j] (the diagonal of G kron A), its EMA, division of the gradient
// by (F + lambda), momentum, weight decay and the in-place parameter write
// (CAFIN briefing, "Introduction" and "Kernel Fusion Strategy").
//
// Three launches per step, all HBM-streaming.  The FACTORS phase is the first
// (the streaming reduction, into the workspace); the UPDATE phase is the other
// two (dA / dG from the reduction, then the parameter pass).
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
#include "common.h"

#include <algorithm>
#include <vector>

namespace kfac {

namespace {

constexpr int kColThreads = 256;
constexpr int kColTile = kColThreads * 4;   // columns per workgroup
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
  ColTask t[kMaxColTasks];
  int32_t n;
};

constexpr int kFinThreads = 256;
constexpr int kMaxFinTasks = 44;
constexpr int kMaxTpb = 16;    // taps per finishing block

enum FinKind : int32_t { FIN_WINDOW = 0, FIN_CHUNKSUM = 1 };

struct FinTask {
  const float* src;
  float* dst;
  int32_t kind;
  int32_t C, H, W, k, stride, pad, Ho, Wo;  // FIN_WINDOW: S is [C][H][W]
  int32_t K, chunks;                        // FIN_CHUNKSUM: partials [chunks][K]
  int32_t blk_begin;
  float scale;
  int32_t bias_index;                       // >= 0: dst[bias_index] = 1
  int32_t tpb;                              // FIN_WINDOW: taps per unit (channel, tap group)
  int32_t upw;                              // FIN_WINDOW: 0 = one unit per block, else units per wavefront
};
struct FinTasks {
  FinTask t[kMaxFinTasks];
  int32_t n;
};

constexpr int kUpdThreads = 256;
constexpr int kUpdUnroll = 4;
constexpr int kUpdPerBlock = kUpdThreads * 4 * kUpdUnroll;
constexpr int kMaxSegs = 48;

struct Seg {
  const float* grad;
  float* w;
  float* mom;
  float* F;
  const float* dA;    // nullptr for a bias segment (its dA entry is exactly 1)
  const float* dG;
  int32_t n;
  int32_t cols;       // d_in for a weight segment
  int32_t blk_begin;
  int32_t pad_;
};
struct Segs {
  Seg s[kMaxSegs];
  int32_t n;
  float beta, one_minus_beta, damping, weight_decay, momentum, lr;
  uint32_t* flags;
};

template <typename T, int N>
__device__ inline int find_task(const T (&t)[N], int n, int blk) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {          // last task with blk_begin <= blk
    int mid = (lo + hi + 1) >> 1;
    if (t[mid].blk_begin <= blk) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ void __launch_bounds__(kColThreads) diag_colsq_kernel(ColTasks tasks) {
  const int ti = find_task(tasks.t, tasks.n, blockIdx.x);
  const ColTask& T = tasks.t[ti];
  const int b = blockIdx.x - T.blk_begin;
  const int tile = b % T.tiles;
  const int chunk = b / T.tiles;
  const int64_t r0 = static_cast<int64_t>(chunk) * T.rc;
  const int64_t r1 = min(T.R, r0 + T.rc);
  const int c0 = tile * kColTile + threadIdx.x * 4;
  const int K = T.K;
  if (c0 >= K) return;
  float* out = T.chunks == 1 ? T.dst : T.dst + static_cast<int64_t>(chunk) * K;
  const float s = T.chunks == 1 ? T.scale : 1.0f;
  if ((K & 3) == 0) {
    const float* p = T.src + r0 * K + c0;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    int64_t r = r0;
    for (; r + 16 <= r1; r += 16) {
      f32x4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + u * static_cast<int64_t>(K)));
#pragma unroll
      for (int u = 0; u < 16; u += 2) {
        acc0 += v[u] * v[u];
        acc1 += v[u + 1] * v[u + 1];
      }
      p += 16 * static_cast<int64_t>(K);
    }
    for (; r < r1; ++r) {
      f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
      acc0 += v * v;
      p += K;
    }
    f32x4 acc = acc0 + acc1;
    *reinterpret_cast<f32x4*>(out + c0) = acc * s;
  } else {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t r = r0; r < r1; ++r) {
      const float* p = T.src + r * K;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (c0 + q < K) acc[q] = fmaf(p[c0 + q], p[c0 + q], acc[q]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (c0 + q < K) out[c0 + q] = acc[q] * s;
  }
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__global__ void __launch_bounds__(kFinThreads) diag_finish_kernel(FinTasks tasks) {
  __shared__ float red[kFinThreads / kWave][kMaxTpb];
  const int ti = find_task(tasks.t, tasks.n, blockIdx.x);  // uniform per block
  const FinTask& T = tasks.t[ti];
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
  // FIN_WINDOW.  A unit is (channel c, tap group of `tpb` taps): the sum of S
  // at each tap's input pixel over all output positions.  Large units take a
  // block each (positions spread over 256 threads, block reduction); small
  // units (few output positions) go to single wavefronts, `upw` each, with a
  // shuffle reduction and no block barrier.
  const int k = T.k, taps = k * k, tpb = T.tpb;
  const int groups = (taps + tpb - 1) / tpb;
  const int units = T.C * groups;
  const int npos = T.Ho * T.Wo;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int nthr = T.upw ? kWave : kFinThreads;
  const int tix = T.upw ? lane : threadIdx.x;
  const int ubeg = T.upw ? (b * (kFinThreads / kWave) + wid) * T.upw : b;
  const int uend = T.upw ? min(units, ubeg + T.upw) : b + 1;
  for (int unit = ubeg; unit < uend; ++unit) {
    const int c = unit / groups, tg = unit - c * groups;
    const int t0 = tg * tpb, nt = min(tpb, taps - t0);
    const float* S = T.src + static_cast<int64_t>(c) * T.H * T.W;
    float acc[kMaxTpb];
    int dh[kMaxTpb], dw[kMaxTpb];
#pragma unroll
    for (int t = 0; t < kMaxTpb; ++t) {
      acc[t] = 0.f;
      const int tap = t0 + (t < nt ? t : 0);
      dh[t] = tap / k - T.pad;
      dw[t] = tap % k - T.pad;
    }
    // 8 independent loads in flight per thread per tap; the thread's output
    // position advances by nthr each time, (ho, wo) stepped without division
    const int sh = nthr / T.Wo, sw = nthr - sh * T.Wo;
    int ho = tix / T.Wo, wo = tix - (tix / T.Wo) * T.Wo;
    for (int q0 = tix; q0 < npos; q0 += nthr * 8) {
      int hb[8], wb[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        hb[u] = q0 + u * nthr < npos ? ho * T.stride : -(1 << 20);   // out of range -> every tap invalid
        wb[u] = wo * T.stride;
        ho += sh;
        wo += sw;
        if (wo >= T.Wo) { wo -= T.Wo; ++ho; }
      }
#pragma unroll
      for (int t = 0; t < kMaxTpb; ++t) {
        if (t >= nt) break;
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int hh = hb[u] + dh[t], ww = wb[u] + dw[t];
          v[u] = (hh >= 0 && hh < T.H && ww >= 0 && ww < T.W) ? S[hh * T.W + ww] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[t] += v[u];
      }
    }
    float* out = T.dst + static_cast<int64_t>(c) * taps + t0;
    if (T.upw) {
#pragma unroll
      for (int t = 0; t < kMaxTpb; ++t) {
        if (t >= nt) break;
        const float v = wave_sum(acc[t]);
        if (lane == 0) out[t] = v * T.scale;
      }
    } else {
#pragma unroll
      for (int t = 0; t < kMaxTpb; ++t) {
        if (t >= nt) break;
        const float v = wave_sum(acc[t]);
        if (lane == 0) red[wid][t] = v;
      }
      __syncthreads();
      if (threadIdx.x < nt) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kFinThreads / kWave; ++w) v += red[w][threadIdx.x];
        out[threadIdx.x] = v * T.scale;
      }
    }
  }
}

struct UpdOut {
  float w, v, f;
};

__device__ inline UpdOut upd_one(float g, float w, float v, float f, float target, const Segs& P) {
  UpdOut o;
  o.f = P.beta * f + P.one_minus_beta * target;
  const float p = g / (o.f + P.damping);
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
        g[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S.grad + e[u]));
        w[u] = *reinterpret_cast<const f32x4*>(S.w + e[u]);
        v[u] = *reinterpret_cast<const f32x4*>(S.mom + e[u]);
        f[u] = *reinterpret_cast<const f32x4*>(S.F + e[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kUpdUnroll; ++u) {
      if (e[u] >= S.n) continue;
      float tgt[4];
      if (S.dA) {
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
        UpdOut r = upd_one(g[u][q], w[u][q], v[u][q], f[u][q], tgt[q], segs);
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
      UpdOut r = upd_one(S.grad[e], S.w[e], S.mom[e], S.F[e], tgt, segs);
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
  std::vector<Seg> seg;
  size_t ws_bytes = kFlagBytes;
};

// Taps per unit: about 4096 position-taps of work per unit.
int window_tpb(int k, int positions) {
  const int taps = k * k;
  int tpb = std::max(1, 4096 / std::max(1, positions));
  return std::min(std::min(tpb, kMaxTpb), taps);
}

// Units per wavefront for small units (<= 1024 output positions): each unit
// costs a load round trip, so a wavefront takes at most 4; 0 = one unit per
// block.
int window_upw(int tpb, int positions) {
  if (positions > 1024) return 0;
  return std::min(4, std::max(1, 4096 / std::max(1, tpb * positions)));
}

int fin_blocks(const FinTask& t) {
  if (t.kind == FIN_WINDOW) {
    const int units = t.C * ((t.k * t.k + t.tpb - 1) / t.tpb);
    if (t.upw == 0) return units;
    const int per_block = t.upw * (kFinThreads / kWave);
    return (units + per_block - 1) / per_block;
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
  for (int li = 0; li < n; ++li) {
    const kfac_layer_t& L = layers[li];
    const LayerGeom g = geom_of(L);
    const float invN = 1.0f / static_cast<float>(g.rows);
    if (g.conv) {
      // input: S_x[c*H*W + p] = sum_b x^2 ; then strided window sums
      const int Kx = g.c_in * g.h * g.w;
      float* Sx = carve(Kx);
      add_col(static_cast<const float*>(L.a), Sx, g.batch, Kx, 1.0f, nullptr, 1, g.batch);
      FinTask fx{};
      fx.src = Sx; fx.dst = L.dA; fx.kind = FIN_WINDOW;
      fx.C = g.c_in; fx.H = g.h; fx.W = g.w; fx.k = g.kh; fx.stride = g.stride; fx.pad = g.pad;
      fx.Ho = g.h_out; fx.Wo = g.w_out; fx.scale = invN; fx.bias_index = g.bias ? g.d_in : -1;
      fx.tpb = window_tpb(g.kh, g.h_out * g.w_out);
      fx.upw = window_upw(fx.tpb, g.h_out * g.w_out);
      add_fin(fx, fin_blocks(fx));
      const int Kg = g.d_out * g.h_out * g.w_out;
      float* Sg = carve(Kg);
      add_col(static_cast<const float*>(L.g), Sg, g.batch, Kg, 1.0f, nullptr, 1, g.batch);
      FinTask fg{};
      fg.src = Sg; fg.dst = L.dG; fg.kind = FIN_WINDOW;
      fg.C = g.d_out; fg.H = g.h_out; fg.W = g.w_out; fg.k = 1; fg.stride = 1; fg.pad = 0;
      fg.Ho = g.h_out; fg.Wo = g.w_out; fg.scale = invN; fg.bias_index = -1;
      fg.tpb = 1;
      fg.upw = window_upw(1, g.h_out * g.w_out);
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
      if (g.bias) {
        Seg sb{};
        sb.grad = L.grad_b; sb.w = L.b; sb.mom = L.mom_b; sb.F = L.F_b; sb.dA = nullptr; sb.dG = L.dG;
        sb.n = g.d_out; sb.cols = 1; sb.blk_begin = upd_blk;
        upd_blk += (sb.n + kUpdPerBlock - 1) / kUpdPerBlock;
        P.seg.push_back(sb);
      }
    }
  }
  P.ws_bytes = off;
  return P;
}

}  // namespace

size_t diag_workspace_bytes(const kfac_layer_t* layers, int n) { return plan_diag(layers, n, nullptr).ws_bytes; }

kfac_status_t diag_enqueue(const kfac_layer_t* layers, int n, const kfac_hparams_t& hp, char* ws,
                           size_t ws_bytes, hipStream_t stream, int phases) {
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
        blocks = T.t[i - g0].blk_begin + P.col[i].tiles * P.col[i].chunks;
      }
      T.n = static_cast<int>(g1 - g0);
      hipLaunchKernelGGL(diag_colsq_kernel, dim3(blocks), dim3(kColThreads), 0, stream, T);
      KFAC_HIP_TRY(hipGetLastError());
    }
  }
  if (phases & KFAC_PHASE_UPDATE) {
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
    for (size_t g0 = 0; g0 < P.seg.size(); g0 += kMaxSegs) {
      const size_t g1 = std::min(P.seg.size(), g0 + kMaxSegs);
      Segs S{};
      const int base = P.seg[g0].blk_begin;
      for (size_t i = g0; i < g1; ++i) {
        S.s[i - g0] = P.seg[i];
        S.s[i - g0].blk_begin -= base;
      }
      const Seg& last = P.seg[g1 - 1];
      const int blocks = last.blk_begin - base + (last.n + kUpdPerBlock - 1) / kUpdPerBlock;
      S.n = static_cast<int>(g1 - g0);
      S.beta = hp.ema_decay;
      S.one_minus_beta = 1.0f - hp.ema_decay;
      S.damping = hp.damping;
      S.weight_decay = hp.weight_decay;
      S.momentum = hp.momentum;
      S.lr = hp.lr;
      S.flags = reinterpret_cast<uint32_t*>(ws);
      hipLaunchKernelGGL(diag_update_kernel, dim3(blocks), dim3(kUpdThreads), 0, stream, S);
      KFAC_HIP_TRY(hipGetLastError());
    }
  }
  return KFAC_OK;
}

}  // namespace kfac
