// Full K-FAC step (Osawa et al., section 3.2): per layer
//   [FACTORS] A <- eps A + (1 - eps) a_bar^T a_bar / N, G likewise (SYRK on
//             matrix cores, EMA fused into the epilogue, upper tiles mirrored;
//             convolution rows are gathered im2col-style inside the GEMM
//             loader, never materialised)
//   [INVERT]  (A + lambda I)^-1, (G + lambda I)^-1 by a blocked Cholesky
//             factorisation, a blocked triangular inverse and Z^T Z, batched
//             over all factors of the stack (section 4.2: damping)
//   [UPDATE]  T = [grad_w | grad_b] A_inv, then G_inv T with the momentum /
//             weight-decay / parameter write fused into the second GEMM's
//             epilogue.
#include <algorithm>
#include <vector>

#include "common.h"
#include "gemm.h"
#include "syrk_bf16.h"

namespace kfac {

namespace {

constexpr int kNb = kTile;   // Cholesky block size = GEMM tile

// ---------------------------------------------------------------------------
// Split-K SYRK finish, batched over factors: F[i][j] = beta F[i][j] +
// alpha * sum_s part[s][i][j] on the upper triangle, in split order, and the
// mirrored lower triangle.  One block per 32 x 32 upper tile; the mirror goes
// through LDS so both writes are row-contiguous.
constexpr int kMaxReds = 64;
struct SymRedItem {
  const float* part;
  float* F;
  int32_t d, nsplit, blk_begin, pad_;
  float alpha, beta;
};
struct SymRedTab {
  SymRedItem r[kMaxReds];
  int32_t n;
};

__global__ void __launch_bounds__(256) sym_reduce_kernel(SymRedTab tab) {
  __shared__ float t[32][33];
  int lo = 0, hi = tab.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tab.r[mid].blk_begin <= static_cast<int>(blockIdx.x)) lo = mid; else hi = mid - 1;
  }
  const SymRedItem& R = tab.r[lo];
  const int T = (R.d + 31) / 32;
  int u = blockIdx.x - R.blk_begin, I = 0;
  while (u >= T - I) { u -= T - I; ++I; }
  const int J = I + u;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t dd = static_cast<int64_t>(R.d) * R.d;
  for (int r = ty; r < 32; r += 8) {
    const int i = I * 32 + r, j = J * 32 + tx;
    float o = 0.f;
    if (i < R.d && j < R.d) {
      const int64_t e = static_cast<int64_t>(i) * R.d + j;
      float sum = 0.f;
      for (int k = 0; k < R.nsplit; ++k) sum += R.part[k * dd + e];
      o = R.beta * R.F[e] + R.alpha * sum;
      if (I != J || i <= j) R.F[e] = o;
    }
    t[r][tx] = o;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int i = J * 32 + r, j = I * 32 + tx;   // lower tile (J, I) = transpose of (I, J)
    if (i >= R.d || j >= R.d) continue;
    if (I == J && i <= j) continue;
    R.F[static_cast<int64_t>(i) * R.d + j] = t[tx][r];
  }
}

// ---------------------------------------------------------------------------
// damped Cholesky inverse, batched over matrices

constexpr int kMaxMats = 40;

struct Mat {
  const float* F;     // factor (upper triangle read)
  float* Finv;        // damped inverse (written unless the factorisation failed)
  float* L;           // working copy -> Cholesky factor (lower)
  float* Z;           // L^-1 (lower)
  float* Dinv;        // inverses of the diagonal blocks, [nblk][128][128]
  int32_t* fail;
  int32_t d;
  int32_t pad_;
};
struct MatTab {
  Mat m[kMaxMats];
  int32_t n;
  int32_t k;          // current block
  float damping;
  uint32_t* flags;
};

// Compact per-matrix view for the diagonal-block kernel (more matrices per launch).
constexpr int kMaxDiagMats = 96;
struct DMat {
  float* L;
  float* Z;
  float* Dinv;
  int32_t* fail;
  int32_t d;
  int32_t pad_;
};
struct DiagTab {
  DMat m[kMaxDiagMats];
  int32_t n;
  int32_t k;
  uint32_t* flags;
};

// L = F + damping I from F's upper triangle (both triangles of L written),
// Z = 0, fail = 0.  grid = (32 x 32 tiles, matrix); a lower tile (I > J) is
// read from F's upper tile (J, I) row by row and transposed through LDS.
__global__ void __launch_bounds__(256) chol_init_kernel(MatTab T) {
  __shared__ float t[32][33];
  const Mat& M = T.m[blockIdx.y];
  const int d = M.d;
  const int nt = (d + 31) / 32;
  if (blockIdx.x == 0 && threadIdx.x == 0) *M.fail = 0;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int tile = blockIdx.x; tile < nt * nt; tile += gridDim.x) {
    const int I = tile / nt, J = tile - (tile / nt) * nt;
    const bool lower = I > J;
    const int sr = (lower ? J : I) * 32, sc = (lower ? I : J) * 32;   // source tile in the upper triangle
    __syncthreads();
    for (int r = ty; r < 32; r += 8) {
      const int i = sr + r, j = sc + tx;
      t[r][tx] = (i < d && j < d) ? M.F[static_cast<int64_t>(i) * d + j] : 0.f;
    }
    __syncthreads();
    for (int r = ty; r < 32; r += 8) {
      const int i = I * 32 + r, j = J * 32 + tx;
      if (i >= d || j >= d) continue;
      float v;
      if (lower) v = t[tx][r];
      else if (I == J) v = t[min(r, tx)][max(r, tx)];   // diagonal tile: mirror its upper part
      else v = t[r][tx];
      if (i == j) v += T.damping;
      const int64_t e = static_cast<int64_t>(i) * d + j;
      M.L[e] = v;
      M.Z[e] = 0.f;
    }
  }
}

// Block k of every matrix with more than k blocks: Cholesky of the diagonal
// block fused with the forward substitution that inverts it (right-looking,
// column by column).  Thread (tr, tc) of a 16 x 16 grid keeps the 8 x 8
// sub-block (rows 8 tr.., columns 8 tc..) of both the factor and the inverse
// in registers; per column only the pivot, the scaled column of L and the
// finished row of the inverse go through LDS (double-buffered, two barriers
// per column).  Writes L_kk (zero above the diagonal) into L, its inverse
// into Dinv[k] and into Z's diagonal block.  A pivot that is not positive (or
// not finite) marks the matrix failed, raises KFAC_FLAG_NOT_PD and is
// replaced by 1 so the remaining steps stay finite; a failed matrix's
// inverse is not written.
__global__ void __launch_bounds__(256) chol_diag_kernel(DiagTab T) {
  __shared__ __attribute__((aligned(16))) float colj[2][kNb];
  __shared__ __attribute__((aligned(16))) float rowj[2][kNb];
  __shared__ float pivs[2];
  const DMat& M = T.m[blockIdx.x];
  const int d = M.d, k = T.k;
  const int nblk = (d + kNb - 1) / kNb;
  if (k >= nblk) return;
  const int r0 = k * kNb;
  const int bk = min(kNb, d - r0);
  const int tid = threadIdx.x;
  const int tr = tid >> 4, tc = tid & 15;
  const int R0 = tr * 8, C0 = tc * 8;
  float* Lg = M.L + static_cast<int64_t>(r0) * d + r0;
  float a[8][8], x[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = R0 + i, c = C0 + j;
      a[i][j] = (r < bk && c <= r) ? Lg[static_cast<int64_t>(r) * d + c] : 0.f;
      x[i][j] = (r < bk && r == c) ? 1.f : 0.f;
    }
  }
  const int nbk = (bk + 7) / 8;
  for (int jb = 0; jb < nbk; ++jb) {
#pragma unroll
    for (int jl = 0; jl < 8; ++jl) {
      const int j = jb * 8 + jl;
      if (j >= bk) break;
      const int p = j & 1;
      if (tr == jb && tc == jb) {
        float v = a[jl][jl];
        if (!(v > 0.f) || !isfinite(v)) {
          if (*M.fail == 0) {
            *M.fail = 1;
            raise_flag(T.flags, KFAC_FLAG_NOT_PD);
          }
          v = 1.f;
        }
        pivs[p] = sqrtf(v);
      }
      __syncthreads();
      const float s = pivs[p];
      const float inv = 1.0f / s;
      if (tc == jb) {                      // column j of L: scale below the pivot, publish all 128 rows
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = R0 + i;
          const float v = a[i][jl] * inv;
          a[i][jl] = r > j ? v : (r == j ? s : a[i][jl]);
          colj[p][r] = r > j ? v : 0.f;
        }
      }
      if (tr == jb) {                      // row j of the inverse is final once scaled
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          x[jl][c] *= inv;
          rowj[p][C0 + c] = x[jl][c];
        }
      }
      __syncthreads();
      // Rank-1 updates, branch-free: colj is zero at rows <= j, so columns <= j
      // of L and rows <= j of the inverse are left as they are; entries above
      // the diagonal of L are never read and are zeroed at write-back; row j
      // of the inverse is zero beyond column j.
      if (tr >= tc) {
        f32x4 cr0 = *reinterpret_cast<const f32x4*>(&colj[p][R0]);
        f32x4 cr1 = *reinterpret_cast<const f32x4*>(&colj[p][R0 + 4]);
        f32x4 cc0 = *reinterpret_cast<const f32x4*>(&colj[p][C0]);
        f32x4 cc1 = *reinterpret_cast<const f32x4*>(&colj[p][C0 + 4]);
        f32x4 rj0 = *reinterpret_cast<const f32x4*>(&rowj[p][C0]);
        f32x4 rj1 = *reinterpret_cast<const f32x4*>(&rowj[p][C0 + 4]);
        const float cr[8] = {cr0[0], cr0[1], cr0[2], cr0[3], cr1[0], cr1[1], cr1[2], cr1[3]};
        const float cc[8] = {cc0[0], cc0[1], cc0[2], cc0[3], cc1[0], cc1[1], cc1[2], cc1[3]};
        const float rj[8] = {rj0[0], rj0[1], rj0[2], rj0[3], rj1[0], rj1[1], rj1[2], rj1[3]};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            a[i][c] = fmaf(-cr[i], cc[c], a[i][c]);
            x[i][c] = fmaf(-cr[i], rj[c], x[i][c]);
          }
        }
      }
    }
  }
  // write back: L_kk (lower, zero above), Dinv[k] and Z_kk
  float* D = M.Dinv + static_cast<int64_t>(k) * kNb * kNb;
  float* Zg = M.Z + static_cast<int64_t>(r0) * d + r0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = R0 + i, c = C0 + j;
      const bool in = r < bk && c < bk;
      const float l = c <= r ? a[i][j] : 0.f;
      const float xv = c <= r ? x[i][j] : 0.f;
      D[r * kNb + c] = in ? xv : 0.f;
      if (in) {
        Lg[static_cast<int64_t>(r) * d + c] = l;
        Zg[static_cast<int64_t>(r) * d + c] = xv;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// planning

struct FullPlan {
  size_t ws_bytes = kFlagBytes;
  std::vector<float*> part;      // per layer and factor (2 li + which): split-K partials, or null
  std::vector<int> nsplit;       // per layer and factor
  std::vector<float*> T;         // per layer, d_out x d_a
  std::vector<Mat> mats;         // inverse work per factor
};

size_t nblk_of(int d) { return (d + kNb - 1) / kNb; }

// Row splits of an fp32 factor SYRK (128 x 128 tiles): one workgroup
// contracts about kSplitRows rows, so a launch holds many workgroups of
// similar length and tall factors (a stem convolution's 401,408 rows) do not
// serialise it; sym_reduce_kernel adds the partial products in split order.
constexpr int64_t kSplitRows = 2048;

int syrk_splits(int, int64_t rows) {
  if (rows < 2 * kSplitRows) return 1;
  return static_cast<int>(std::min<int64_t>(128, (rows + kSplitRows - 1) / kSplitRows));
}

bool fp32_factor(const kfac_layer_t& L, int which) {
  return (which == 0 ? L.act_dtype : L.grad_dtype) == KFAC_F32;
}

FullPlan plan_full(const kfac_layer_t* layers, int n, char* ws, int phases, bool refresh) {
  FullPlan P;
  size_t off = kFlagBytes;
  auto carve = [&](size_t bytes) -> char* {
    char* p = ws ? ws + off : nullptr;
    off = align_up(off + bytes, 256);
    return p;
  };
  // all regions are always carved so the size does not depend on the phases
  for (int li = 0; li < n; ++li) {
    const LayerGeom g = geom_of(layers[li]);
    for (int which = 0; which < 2; ++which) {
      const int d = which == 0 ? g.d_a : g.d_out;
      const int s = fp32_factor(layers[li], which) ? syrk_splits(d, g.rows) : 1;
      P.nsplit.push_back(s);
      P.part.push_back(s > 1 ? reinterpret_cast<float*>(carve(static_cast<size_t>(s) * d * d * 4)) : nullptr);
    }
  }
  for (int li = 0; li < n; ++li) {
    const LayerGeom g = geom_of(layers[li]);
    P.T.push_back(reinterpret_cast<float*>(carve(static_cast<size_t>(g.d_out) * g.d_a * 4)));
  }
  for (int li = 0; li < n; ++li) {
    const LayerGeom g = geom_of(layers[li]);
    for (int which = 0; which < 2; ++which) {
      const int d = which == 0 ? g.d_a : g.d_out;
      Mat m{};
      m.F = which == 0 ? layers[li].A : layers[li].G;
      m.Finv = which == 0 ? layers[li].A_inv : layers[li].G_inv;
      m.d = d;
      m.L = reinterpret_cast<float*>(carve(static_cast<size_t>(d) * d * 4));
      m.Z = reinterpret_cast<float*>(carve(static_cast<size_t>(d) * d * 4));
      m.Dinv = reinterpret_cast<float*>(carve(nblk_of(d) * kNb * kNb * 4));
      m.fail = reinterpret_cast<int32_t*>(carve(4));
      P.mats.push_back(m);
    }
  }
  (void)phases;
  (void)refresh;
  P.ws_bytes = off;
  return P;
}

kfac_status_t launch_sym_reduce(const std::vector<SymRedItem>& items, hipStream_t st) {
  for (size_t i0 = 0; i0 < items.size(); i0 += kMaxReds) {
    SymRedTab tab{};
    int blocks = 0;
    for (size_t i = i0; i < std::min(items.size(), i0 + kMaxReds); ++i) {
      SymRedItem r = items[i];
      const int T = (r.d + 31) / 32;
      r.blk_begin = blocks;
      blocks += T * (T + 1) / 2;
      tab.r[tab.n++] = r;
    }
    hipLaunchKernelGGL(sym_reduce_kernel, dim3(blocks), dim3(256), 0, st, tab);
    KFAC_HIP_TRY(hipGetLastError());
  }
  return KFAC_OK;
}

// FACTORS: every factor of the stack in a few batched launches, one per
// operand kind (row-major fp32, implicit im2col, NCHW gradient, bf16), each
// split into direct-EMA and split-K problems; then the batched split reduce.
kfac_status_t factors_phase(const kfac_layer_t* layers, int n, const kfac_hparams_t& hp, const FullPlan& P,
                            hipStream_t st) {
  const float eps = hp.ema_decay;
  enum { K_MN = 0, K_IM2COL = 1, K_NCHW = 2 };
  std::vector<GemmProb> probs[3];
  std::vector<SymRedItem> reds;
  std::vector<SyrkBf16Prob> bf16;
  for (int li = 0; li < n; ++li) {
    const kfac_layer_t& L = layers[li];
    const LayerGeom g = geom_of(L);
    for (int which = 0; which < 2; ++which) {
      const int d = which == 0 ? g.d_a : g.d_out;
      const int special = (which == 0 && g.bias) ? g.d_in : -1;
      float* F = which == 0 ? L.A : L.G;
      const void* X = which == 0 ? L.a : L.g;
      const float alpha = (1.0f - eps) / static_cast<float>(g.rows);
      if (!fp32_factor(L, which)) {
        SyrkBf16Prob q{};
        q.X = static_cast<const uint16_t*>(X);
        q.F = F;
        q.rows = g.rows;
        q.width = which == 0 ? g.d_in : g.d_out;
        q.bias = special >= 0;
        q.alpha = alpha;
        q.beta = eps;
        bf16.push_back(q);
        continue;
      }
      GemmProb p{};
      p.A = X;
      p.B = X;
      p.M = p.N = d;
      p.kb = 0;
      p.ke = static_cast<int>(g.rows);
      p.tri = TRI_UPPER;
      p.a_special = p.b_special = special;
      int kind;
      if (!g.conv) {
        kind = K_MN;
        p.lda = p.ldb = which == 0 ? g.d_in : g.d_out;
      } else if (which == 0) {
        kind = K_IM2COL;
        const int geo[8] = {g.c_in, g.h, g.w, g.kh, g.stride, g.pad, g.h_out, g.w_out};
        for (int e = 0; e < 8; ++e) p.geo[e] = geo[e];
      } else {
        kind = K_NCHW;
        p.geo[0] = g.h_out * g.w_out;
        p.geo[1] = g.d_out;
      }
      const int s = P.nsplit[2 * li + which];
      p.ldc = d;
      p.nsplit = s;
      if (s == 1) {
        p.C = F;
        p.alpha = alpha;
        p.beta = eps;
        probs[kind].push_back(p);
      } else {
        p.C = P.part[2 * li + which];
        p.split_stride = static_cast<int64_t>(d) * d;
        p.alpha = 1.0f;
        probs[kind].push_back(p);
        SymRedItem r{};
        r.part = p.C;
        r.F = F;
        r.d = d;
        r.nsplit = s;
        r.alpha = alpha;
        r.beta = eps;
        reds.push_back(r);
      }
    }
  }
  GemmScalars sc{};
  const int modes[3] = {OP_MN, OP_IM2COL, OP_NCHW};
  kfac_status_t r;
  for (int kind = 0; kind < 3; ++kind) {
    if (probs[kind].empty()) continue;
    r = launch_gemm(probs[kind], modes[kind], modes[kind], EPI_SYRK, sc, st, TILES_SMALL);
    if (r != KFAC_OK) return r;
  }
  if (!bf16.empty()) {
    r = launch_syrk_bf16(bf16, st);
    if (r != KFAC_OK) return r;
  }
  return reds.empty() ? KFAC_OK : launch_sym_reduce(reds, st);
}

kfac_status_t invert_phase(const kfac_hparams_t& hp, const FullPlan& P, uint32_t* flags, hipStream_t st) {
  const std::vector<Mat>& mats = P.mats;
  int nblk_max = 0;
  for (const Mat& m : mats) nblk_max = std::max<int>(nblk_max, static_cast<int>(nblk_of(m.d)));
  GemmScalars sc{};
  // runs `fn` on the matrices selected by `pred`, kMaxMats at a time
  auto tables = [&](auto pred, int k, auto fn) -> kfac_status_t {
    MatTab T{};
    T.damping = hp.damping;
    T.flags = flags;
    T.k = k;
    for (const Mat& m : mats) {
      if (!pred(m)) continue;
      T.m[T.n++] = m;
      if (T.n == kMaxMats) {
        kfac_status_t r = fn(T);
        if (r != KFAC_OK) return r;
        T.n = 0;
      }
    }
    return T.n > 0 ? fn(T) : KFAC_OK;
  };
  kfac_status_t r = tables([](const Mat&) { return true; }, 0, [&](MatTab& T) {
    hipLaunchKernelGGL(chol_init_kernel, dim3(2048, T.n), dim3(256), 0, st, T);
    return hipGetLastError() == hipSuccess ? KFAC_OK : KFAC_ERR_HIP;
  });
  if (r != KFAC_OK) return r;
  // blocked right-looking Cholesky
  for (int k = 0; k < nblk_max; ++k) {
    {
      DiagTab D{};
      D.k = k;
      D.flags = flags;
      for (size_t mi = 0; mi <= mats.size(); ++mi) {
        if (mi == mats.size() || D.n == kMaxDiagMats) {
          if (D.n > 0) {
            hipLaunchKernelGGL(chol_diag_kernel, dim3(D.n), dim3(256), 0, st, D);
            KFAC_HIP_TRY(hipGetLastError());
          }
          D.n = 0;
          if (mi == mats.size()) break;
        }
        const Mat& m = mats[mi];
        if (static_cast<int>(nblk_of(m.d)) <= k) continue;
        D.m[D.n++] = DMat{m.L, m.Z, m.Dinv, m.fail, m.d, 0};
      }
    }
    std::vector<GemmProb> panel, trail;
    for (const Mat& m : mats) {
      const int d = m.d;
      if (static_cast<int>(nblk_of(d)) <= k + 1) continue;
      const int r1 = (k + 1) * kNb;
      GemmProb p{};
      // L_ik = M_ik Dinv_k^T for the rows below block k
      p.A = m.L + static_cast<int64_t>(r1) * d + k * kNb;
      p.lda = d;
      p.B = m.Dinv + static_cast<int64_t>(k) * kNb * kNb;
      p.ldb = kNb;
      p.C = m.L + static_cast<int64_t>(r1) * d + k * kNb;
      p.ldc = d;
      p.M = d - r1;
      p.N = kNb;
      p.kb = 0;
      p.ke = kNb;
      p.tri = TRI_FULL;
      p.a_special = p.b_special = -1;
      p.alpha = 1.f;
      p.nsplit = 1;
      gemm_set_tiles(p);
      panel.push_back(p);
      // M_ij -= L_ik L_jk^T for k < j <= i
      GemmProb q = p;
      q.B = p.A;
      q.ldb = d;
      q.C = m.L + static_cast<int64_t>(r1) * d + r1;
      q.N = d - r1;
      q.tri = TRI_LOWER;
      gemm_set_tiles(q);
      trail.push_back(q);
    }
    if (!panel.empty()) {
      r = launch_gemm(panel, OP_K, OP_K, EPI_STORE, sc, st);
      if (r != KFAC_OK) return r;
      r = launch_gemm(trail, OP_K, OP_K, EPI_SUB, sc, st);
      if (r != KFAC_OK) return r;
    }
  }
  // Z = L^-1, block row by block row: Z_ik = Dinv_i R_ik (k < i), then
  // R_jk -= L_ji Z_ik for the rows below (R starts at zero below the diagonal)
  for (int i = 0; i < nblk_max; ++i) {
    std::vector<GemmProb> fin, upd;
    for (const Mat& m : mats) {
      const int d = m.d;
      const int nb = static_cast<int>(nblk_of(d));
      if (nb <= i) continue;
      const int r0 = i * kNb;
      const int bk = std::min(kNb, d - r0);
      if (i > 0) {
        GemmProb p{};
        p.A = m.Dinv + static_cast<int64_t>(i) * kNb * kNb;
        p.lda = kNb;
        p.B = m.Z + static_cast<int64_t>(r0) * d;
        p.ldb = d;
        p.C = m.Z + static_cast<int64_t>(r0) * d;
        p.ldc = d;
        p.M = bk;
        p.N = r0;
        p.kb = 0;
        p.ke = bk;
        p.tri = TRI_FULL;
        p.a_special = p.b_special = -1;
        p.alpha = 1.f;
        p.nsplit = 1;
        gemm_set_tiles(p);
        fin.push_back(p);
      }
      if (nb > i + 1) {
        const int r1 = r0 + kNb;
        GemmProb q{};
        q.A = m.L + static_cast<int64_t>(r1) * d + r0;
        q.lda = d;
        q.B = m.Z + static_cast<int64_t>(r0) * d;
        q.ldb = d;
        q.C = m.Z + static_cast<int64_t>(r1) * d;
        q.ldc = d;
        q.M = d - r1;
        q.N = r1;
        q.kb = 0;
        q.ke = kNb;
        q.tri = TRI_FULL;
        q.a_special = q.b_special = -1;
        q.alpha = 1.f;
        q.nsplit = 1;
        gemm_set_tiles(q);
        upd.push_back(q);
      }
    }
    if (!fin.empty()) {
      r = launch_gemm(fin, OP_K, OP_MN, EPI_STORE, sc, st);
      if (r != KFAC_OK) return r;
    }
    if (!upd.empty()) {
      r = launch_gemm(upd, OP_K, OP_MN, EPI_SUB, sc, st);
      if (r != KFAC_OK) return r;
    }
  }
  // inverse = Z^T Z (upper tiles, mirrored), written only for matrices that factored
  std::vector<GemmProb> lau;
  for (size_t mi = 0; mi < mats.size(); ++mi) {
    const Mat& m = mats[mi];
    GemmProb p{};
    p.A = m.Z;
    p.B = m.Z;
    p.lda = p.ldb = m.d;
    p.C = m.Finv;
    p.ldc = m.d;
    p.M = p.N = m.d;
    p.kb = 0;
    p.ke = m.d;
    p.tri = TRI_UPPER;
    p.k_from_diag = 1;
    p.a_special = p.b_special = -1;
    p.fail = m.fail;
    p.nsplit = 1;
    gemm_set_tiles(p);
    lau.push_back(p);
  }
  return launch_gemm(lau, OP_MN, OP_MN, EPI_SYM_IFOK, sc, st);
}

kfac_status_t update_phase(const kfac_layer_t* layers, int n, const kfac_hparams_t& hp, const FullPlan& P,
                           uint32_t* flags, hipStream_t st) {
  std::vector<GemmProb> g1, g2;
  for (int li = 0; li < n; ++li) {
    const kfac_layer_t& L = layers[li];
    const LayerGeom g = geom_of(L);
    GemmProb p{};
    // T = [grad_w | grad_b] A_inv
    p.A = L.grad_w;
    p.lda = g.d_in;
    p.A_extra = g.bias ? L.grad_b : nullptr;
    p.a_special = g.bias ? g.d_in : -1;
    p.B = L.A_inv;
    p.ldb = g.d_a;
    p.b_special = -1;
    p.C = P.T[li];
    p.ldc = g.d_a;
    p.M = g.d_out;
    p.N = g.d_a;
    p.kb = 0;
    p.ke = g.d_a;
    p.tri = TRI_FULL;
    p.alpha = 1.f;
    p.nsplit = 1;
    gemm_set_tiles(p);
    g1.push_back(p);
    // P = G_inv T (G_inv symmetric: read as its transpose), fused update
    GemmProb q{};
    q.A = L.G_inv;
    q.lda = g.d_out;
    q.a_special = -1;
    q.B = P.T[li];
    q.ldb = g.d_a;
    q.b_special = -1;
    q.M = g.d_out;
    q.N = g.d_a;
    q.kb = 0;
    q.ke = g.d_out;
    q.tri = TRI_FULL;
    q.W = L.w;
    q.Wb = L.b;
    q.V = L.mom_w;
    q.Vb = L.mom_b;
    q.d_in = g.d_in;
    q.nsplit = 1;
    gemm_set_tiles(q);
    g2.push_back(q);
  }
  GemmScalars sc{hp.lr, hp.momentum, hp.weight_decay, flags};
  kfac_status_t r = launch_gemm(g1, OP_K, OP_MN, EPI_STORE, sc, st);
  if (r != KFAC_OK) return r;
  return launch_gemm(g2, OP_MN, OP_MN, EPI_UPDATE, sc, st);
}

}  // namespace

size_t full_workspace_bytes(const kfac_layer_t* layers, int n) {
  return plan_full(layers, n, nullptr, KFAC_PHASE_ALL, true).ws_bytes;
}

kfac_status_t full_enqueue(const kfac_layer_t* layers, int n, const kfac_hparams_t& hp, char* ws, size_t ws_bytes,
                           hipStream_t st, int phases) {
  FullPlan P = plan_full(layers, n, ws, phases, hp.refresh != 0);
  if (P.ws_bytes > ws_bytes) return KFAC_ERR_WORKSPACE;
  uint32_t* flags = reinterpret_cast<uint32_t*>(ws);
  kfac_status_t r;
  if (phases & KFAC_PHASE_FACTORS) {
    r = factors_phase(layers, n, hp, P, st);
    if (r != KFAC_OK) return r;
  }
  if ((phases & KFAC_PHASE_INVERT) && hp.refresh) {
    r = invert_phase(hp, P, flags, st);
    if (r != KFAC_OK) return r;
  }
  if (phases & KFAC_PHASE_UPDATE) {
    r = update_phase(layers, n, hp, P, flags, st);
    if (r != KFAC_OK) return r;
  }
  return KFAC_OK;
}

}  // namespace kfac
