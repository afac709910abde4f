// Batched fp32 GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// A workgroup of 256 threads (4 wavefronts, 2 x 2) computes one 128 x 128
// output tile; each wavefront owns a 64 x 64 quarter as 2 x 2 MFMA 32 x 32
// blocks (64 accumulators per lane).  K advances 16 at a time: the next A/B
// slabs are fetched into registers while the current ones, staged in LDS as
// [k][m] rows (m contiguous, padded), feed the MFMAs.  fp32 in, fp32
// accumulate, fp32 out.
//
// One launch runs a table of independent problems (layers, matrices, K
// splits); each workgroup finds its problem by binary search over the
// table's block offsets.
#include "gemm.h"

#include <algorithm>

namespace kfac {

namespace {

constexpr int kThreads = 256;
constexpr int kLdsPad = 4;
constexpr int kLdsRow = kTile + kLdsPad;

struct GemmBatch {
  GemmProb p[kMaxGemmProbs];
  int32_t n;
  GemmScalars sc;
};

__device__ inline int find_prob(const GemmBatch& b, int blk) {
  int lo = 0, hi = b.n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (b.p[mid].blk_begin <= blk) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Loads this thread's share of a 16 x 128 operand slab (8 floats) into regs.
// MN layout: thread covers rows kk = t/32 and t/32 + 8, columns 4*(t%32)..+3.
// K layout : thread covers rows mm = t/4 and t/4 + 64, k = 4*(t%4)..+3.
template <int MODE, bool EXTRA>
__device__ inline void load_slab(float (&r)[8], const float* __restrict__ base, int ld, int m0, int mlim, int k0,
                                 int klim, int special, const float* __restrict__ extra) {
  const int t = threadIdx.x;
  if (MODE == OP_MN) {
    const int mm = (t & 31) * 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = k0 + (t >> 5) + 8 * h;
      const int m = m0 + mm;
      const bool kin = k < klim;
      const float* p = base + static_cast<int64_t>(k) * ld + m;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v = 0.f;
        if (kin) {
          if (m + q == special) v = 1.0f;          // virtual constant-1 (bias) column
          else if (m + q < mlim) v = p[q];
        }
        r[4 * h + q] = v;
      }
    }
  } else {
    const int kq = (t & 3) * 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = m0 + (t >> 2) + 64 * h;
      const int k = k0 + kq;
      const bool min_ = m < mlim;
      const float* p = base + static_cast<int64_t>(m) * ld + k;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v = 0.f;
        if (min_ && k + q < klim) {
          if (EXTRA && k + q == special) v = extra[m];   // extra column (bias gradient)
          else v = p[q];
        }
        r[4 * h + q] = v;
      }
    }
  }
}

template <int MODE>
__device__ inline void store_slab(float* __restrict__ s, const float (&r)[8]) {
  const int t = threadIdx.x;
  if (MODE == OP_MN) {
    const int mm = (t & 31) * 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kk = (t >> 5) + 8 * h;
      f32x4 v = {r[4 * h], r[4 * h + 1], r[4 * h + 2], r[4 * h + 3]};
      *reinterpret_cast<f32x4*>(s + kk * kLdsRow + mm) = v;
    }
  } else {
    const int kq = (t & 3) * 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int mm = (t >> 2) + 64 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q) s[(kq + q) * kLdsRow + mm] = r[4 * h + q];
    }
  }
}

__device__ inline void tile_coords(const GemmProb& P, int t, int& split, int& ti, int& tj) {
  int per;
  if (P.tri == TRI_FULL) per = P.tiles_m * P.tiles_n;
  else per = P.tiles_m * (P.tiles_m + 1) / 2;
  split = t / per;
  t -= split * per;
  if (P.tri == TRI_FULL) {
    ti = t / P.tiles_n;
    tj = t - ti * P.tiles_n;
  } else if (P.tri == TRI_UPPER) {
    const int T = P.tiles_m;
    ti = 0;
    while (t >= T - ti) { t -= T - ti; ++ti; }
    tj = ti + t;
  } else {
    ti = 0;
    while (t > ti) { t -= ti + 1; ++ti; }
    tj = t;
  }
}

template <int AMODE, int BMODE, int EPI>
__global__ void __launch_bounds__(kThreads) gemm_f32_kernel(GemmBatch batch) {
  __shared__ float sA[2][kTileK * kLdsRow];
  __shared__ float sB[2][kTileK * kLdsRow];
  const GemmProb& P = batch.p[find_prob(batch, blockIdx.x)];
  int split, ti, tj;
  tile_coords(P, blockIdx.x - P.blk_begin, split, ti, tj);
  const int i0 = ti * kTile, j0 = tj * kTile;
  int kb = P.kb, ke = P.ke;
  if (P.k_from_diag) kb = max(kb, max(i0, j0));
  if (P.nsplit > 1) {
    const int len = ((ke - kb + P.nsplit - 1) / P.nsplit + kTileK - 1) / kTileK * kTileK;
    const int s0 = kb + split * len;
    ke = min(ke, s0 + len);
    kb = s0;
  }
  float* C = P.C + static_cast<int64_t>(split) * P.split_stride;
  const float* Ab = static_cast<const float*>(P.A);
  const float* Bb = static_cast<const float*>(P.B);

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int wm = (wid >> 1) * 64, wn = (wid & 1) * 64;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  float ra[8], rb[8];
  int buf = 0;
  if (kb < ke) {
    load_slab<AMODE, true>(ra, Ab, P.lda, i0, P.M, kb, ke, P.a_special, P.A_extra);
    load_slab<BMODE, false>(rb, Bb, P.ldb, j0, P.N, kb, ke, P.b_special, Bb);
    store_slab<AMODE>(sA[0], ra);
    store_slab<BMODE>(sB[0], rb);
  }
  __syncthreads();
  for (int k0 = kb; k0 < ke; k0 += kTileK) {
    const bool more = k0 + kTileK < ke;
    if (more) {
      load_slab<AMODE, true>(ra, Ab, P.lda, i0, P.M, k0 + kTileK, ke, P.a_special, P.A_extra);
      load_slab<BMODE, false>(rb, Bb, P.ldb, j0, P.N, k0 + kTileK, ke, P.b_special, Bb);
    }
    const float* a = sA[buf];
    const float* b = sB[buf];
#pragma unroll
    for (int kk = 0; kk < kTileK; kk += 2) {
      const int row = (kk + (lane >> 5)) * kLdsRow;
      const float a0 = a[row + wm + (lane & 31)];
      const float a1 = a[row + wm + 32 + (lane & 31)];
      const float b0 = b[row + wn + (lane & 31)];
      const float b1 = b[row + wn + 32 + (lane & 31)];
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
    }
    if (more) {
      store_slab<AMODE>(sA[buf ^ 1], ra);
      store_slab<BMODE>(sB[buf ^ 1], rb);
    }
    __syncthreads();
    buf ^= 1;
  }

  // epilogue: accumulator r of block (si, sj) is C[row][col] with
  // row = i0 + wm + 32 si + 8 (r / 4) + 4 (lane / 32) + r % 4, col = j0 + wn + 32 sj + lane % 32
  bool bad = false;
  bool skip = false;
  if (EPI == EPI_SYM_IFOK) skip = *P.fail != 0;
#pragma unroll
  for (int si = 0; si < 2; ++si) {
#pragma unroll
    for (int sj = 0; sj < 2; ++sj) {
      const int col = j0 + wn + 32 * sj + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i0 + wm + 32 * si + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= P.M || col >= P.N) continue;
        const float v = acc[si][sj][r];
        const int64_t idx = static_cast<int64_t>(row) * P.ldc + col;
        if (EPI == EPI_STORE) {
          C[idx] = P.alpha * v;
        } else if (EPI == EPI_SUB) {
          C[idx] -= v;
        } else if (EPI == EPI_SYM_EMA) {
          if (row <= col) {
            const float o = P.beta * C[idx] + P.alpha * v;
            C[idx] = o;
            if (row != col) C[static_cast<int64_t>(col) * P.ldc + row] = o;
          }
        } else if (EPI == EPI_SYM_IFOK) {
          if (row <= col && !skip) {
            C[idx] = v;
            if (row != col) C[static_cast<int64_t>(col) * P.ldc + row] = v;
          }
        } else if (EPI == EPI_UPDATE) {
          float* wp;
          float* vp;
          if (col < P.d_in) {
            wp = P.W + static_cast<int64_t>(row) * P.d_in + col;
            vp = P.V + static_cast<int64_t>(row) * P.d_in + col;
          } else {
            wp = P.Wb + row;
            vp = P.Vb + row;
          }
          const float w = *wp;
          const float d = fmaf(batch.sc.weight_decay, w, v);
          const float vn = fmaf(batch.sc.momentum, *vp, d);
          const float wn2 = fmaf(-batch.sc.lr, vn, w);
          *vp = vn;
          *wp = wn2;
          bad |= !(isfinite(vn) && isfinite(wn2));
        }
      }
    }
  }
  if (EPI == EPI_UPDATE) {
    if (__any(bad) && lane == 0) raise_flag(batch.sc.flags, KFAC_FLAG_NONFINITE);
  }
}

template <int AM, int BM, int EPI>
kfac_status_t launch_group(const GemmBatch& b, int blocks, hipStream_t s) {
  hipLaunchKernelGGL((gemm_f32_kernel<AM, BM, EPI>), dim3(blocks), dim3(kThreads), 0, s, b);
  return hipGetLastError() == hipSuccess ? KFAC_OK : KFAC_ERR_HIP;
}

kfac_status_t dispatch(const GemmBatch& b, int blocks, int am, int bm, int epi, hipStream_t s) {
#define KFAC_GEMM_CASE(A_, B_, E_) \
  if (am == A_ && bm == B_ && epi == E_) return launch_group<A_, B_, E_>(b, blocks, s);
  KFAC_GEMM_CASE(OP_MN, OP_MN, EPI_SYM_EMA)
  KFAC_GEMM_CASE(OP_MN, OP_MN, EPI_STORE)
  KFAC_GEMM_CASE(OP_MN, OP_MN, EPI_UPDATE)
  KFAC_GEMM_CASE(OP_MN, OP_MN, EPI_SYM_IFOK)
  KFAC_GEMM_CASE(OP_K, OP_MN, EPI_STORE)
  KFAC_GEMM_CASE(OP_K, OP_MN, EPI_SUB)
  KFAC_GEMM_CASE(OP_K, OP_K, EPI_STORE)
  KFAC_GEMM_CASE(OP_K, OP_K, EPI_SUB)
#undef KFAC_GEMM_CASE
  return KFAC_ERR_UNSUPPORTED;
}

}  // namespace

void gemm_set_tiles(GemmProb& p) {
  p.tiles_m = (p.M + kTile - 1) / kTile;
  p.tiles_n = (p.N + kTile - 1) / kTile;
}

int gemm_blocks(const GemmProb& p) {
  const int per = p.tri == TRI_FULL ? p.tiles_m * p.tiles_n : p.tiles_m * (p.tiles_m + 1) / 2;
  return per * std::max(1, p.nsplit);
}

kfac_status_t launch_gemm(std::vector<GemmProb>& probs, int amode, int bmode, int epi, const GemmScalars& sc,
                          hipStream_t stream) {
  size_t i = 0;
  while (i < probs.size()) {
    GemmBatch b{};
    b.sc = sc;
    int blocks = 0;
    int n = 0;
    for (; i < probs.size() && n < kMaxGemmProbs; ++i) {
      GemmProb p = probs[i];
      if (p.nsplit < 1) p.nsplit = 1;
      const int nb = gemm_blocks(p);
      if (nb == 0 || p.ke <= p.kb) {
        // empty contraction: only EPI_STORE / EPI_SYM_EMA must still write; callers avoid it
        if (nb == 0) continue;
      }
      p.blk_begin = blocks;
      blocks += nb;
      b.p[n++] = p;
    }
    if (n == 0) continue;
    b.n = n;
    kfac_status_t st = dispatch(b, blocks, amode, bmode, epi, stream);
    if (st != KFAC_OK) return st;
  }
  return KFAC_OK;
}

}  // namespace kfac
