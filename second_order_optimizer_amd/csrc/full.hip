// Full K-FAC step (Osawa et al., section 3.2): per layer
//   [FACTORS] A <- eps A + (1 - eps) a_bar^T a_bar / N, G likewise (SYRK on
//             matrix cores, EMA fused into the epilogue, upper tiles mirrored;
//             fp32 convolution tensors are first laid out as rows, im2col of
//             the input and a transpose of the output gradient, in one
//             batched launch, and then take the same row-major SYRK)
//   [INVERT]  (A + lambda I)^-1, (G + lambda I)^-1 by a blocked Cholesky
//             factorisation, a blocked triangular inverse and Z^T Z, batched
//             over all factors of the stack (section 4.2: damping)
//   [UPDATE]  T = [grad_w | grad_b] A_inv, then G_inv T with the momentum /
//             weight-decay / parameter write fused into the second GEMM's
//             epilogue.
#include <algorithm>
#include <map>
#include <memory>
#include <mutex>
#include <utility>
#include <vector>

#include "common.h"
#include "gemm.h"
#include "syrk_bf16.h"

namespace kfac {

namespace {

constexpr int kNb = kTile;   // Cholesky block size = GEMM tile
constexpr int kOuter = 4;     // Cholesky blocks per outer panel

// ---------------------------------------------------------------------------
// Split-K SYRK finish, batched over factors: F[i][j] = beta F[i][j] +
// alpha * sum_s part[s][i][j] on the upper triangle, in split order, and the
// mirrored lower triangle.  One block per 32 x 32 upper tile; the mirror goes
// through LDS so both writes are row-contiguous.
constexpr int kMaxReds = 64;
struct SymRedItem {
  const float* part;
  float* F;
  const int32_t* fail;   // when set and nonzero, F is left as it is
  int32_t d, nsplit, blk_begin, packed;   // packed: F is the packed upper triangle (no mirror)
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
  if (R.fail != nullptr && *R.fail != 0) return;
  const int T = (R.d + 31) / 32;
  int u = blockIdx.x - R.blk_begin, I = 0;
  while (u >= T - I) { u -= T - I; ++I; }
  const int J = I + u;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t dd = static_cast<int64_t>(R.d) * R.d;
  for (int r = ty; r < 32; r += 8) {
    const int i = I * 32 + r, j = J * 32 + tx;
    float o = 0.f;
    const bool upper = I != J || i <= j;
    if (i < R.d && j < R.d && (upper || !R.packed)) {
      const int64_t e = static_cast<int64_t>(i) * R.d + j;
      const int64_t f = R.packed ? packed_index(i, j, R.d) : e;
      float sum = 0.f;
      for (int k = 0; k < R.nsplit; ++k) sum += R.part[k * dd + e];
      o = R.beta != 0.f ? R.beta * R.F[f] + R.alpha * sum : R.alpha * sum;
      if (upper) R.F[f] = o;
    }
    t[r][tx] = o;
  }
  if (R.packed) return;   // a packed factor holds only the upper triangle
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int i = J * 32 + r, j = I * 32 + tx;   // lower tile (J, I) = transpose of (I, J)
    if (i >= R.d || j >= R.d) continue;
    if (I == J && i <= j) continue;
    R.F[static_cast<int64_t>(i) * R.d + j] = t[tx][r];
  }
}

// ---------------------------------------------------------------------------
// im2col of convolution tensors for the factor SYRK: X[n][i] with
// n = (b, ho, wo) and i = (c, kh, kw), zero in the padding, rows of pitch ld.
// An output gradient [B, C, Ho, Wo] is the case k = 1, stride 1, pad 0 (a
// transpose to [B Ho Wo, C]).  The SYRK then reads X row-major with 16-byte
// loads instead of gathering.  One block per 64 x 64 tile of X, transposed
// through LDS: reads run along n (contiguous input for stride 1), writes
// along i.

constexpr int kMaxCols = 56;
constexpr int kColTile = 64;
struct ColItem {
  const float* x;
  float* X;
  int32_t C, H, W, k, stride, pad, Ho, Wo;
  int32_t d_in, ld, rows, blk_begin;
};
struct ColTab {
  ColItem c[kMaxCols];
  int32_t n;
};

__global__ void __launch_bounds__(256) im2col_kernel(ColTab tab) {
  __shared__ float t[kColTile][kColTile + 1];
  __shared__ int32_t coff[kColTile];   // per column of the tile: c H W + kh W + kw, or -1 past d_in
  __shared__ int32_t ckh[kColTile], ckw[kColTile];
  int lo = 0, hi = tab.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tab.c[mid].blk_begin <= static_cast<int>(blockIdx.x)) lo = mid; else hi = mid - 1;
  }
  const ColItem& It = tab.c[lo];
  const float* __restrict__ x = It.x;
  float* __restrict__ X = It.X;
  const int ti = (It.d_in + kColTile - 1) / kColTile;
  const int tile = blockIdx.x - It.blk_begin;
  const int n0 = (tile / ti) * kColTile, i0 = (tile - (tile / ti) * ti) * kColTile;
  const int H = It.H, W = It.W;
  if (threadIdx.x < kColTile) {
    const int i = i0 + threadIdx.x;
    const int kk = It.k * It.k;
    const int c = i / kk, rem = i - c * kk;
    const int kh = rem / It.k, kw = rem - kh * It.k;
    coff[threadIdx.x] = i < It.d_in ? (c * H + kh) * W + kw : -1;
    ckh[threadIdx.x] = kh;
    ckw[threadIdx.x] = kw;
  }
  __syncthreads();
  const int lx = threadIdx.x & (kColTile - 1), ly = threadIdx.x >> 6;
  // this thread reads row n0 + lx for columns i0 + ly + 4 j
  {
    const int n = n0 + lx;
    const int nc = min(n, It.rows - 1);
    const int P = It.Ho * It.Wo;
    const int b = nc / P, p = nc - b * P;
    const int ho = p / It.Wo, wo = p - ho * It.Wo;
    const int hb = ho * It.stride - It.pad, wb = wo * It.stride - It.pad;
    const float* xb = x + static_cast<int64_t>(b) * It.C * H * W + hb * W + wb;   // 32-bit offsets within one image
    const bool nin = n < It.rows;
    float v[kColTile / 4];
#pragma unroll
    for (int j = 0; j < kColTile / 4; ++j) {
      const int e = ly + 4 * j;
      const int h = hb + ckh[e], w = wb + ckw[e];
      const bool in = nin && coff[e] >= 0 && h >= 0 && h < H && w >= 0 && w < W;
      v[j] = in ? xb[coff[e]] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kColTile / 4; ++j) t[ly + 4 * j][lx] = v[j];
  }
  __syncthreads();
  // and writes 4 consecutive columns of rows n0 + 16 q + (tid / 16)
  const int i4 = (threadIdx.x & 15) * 4;
  const int i = i0 + i4;
  const bool vec = i + 4 <= It.d_in;   // rows have a pitch of 4 floats
#pragma unroll
  for (int q = 0; q < kColTile / 16; ++q) {
    const int r = 16 * q + (threadIdx.x >> 4);
    const int n = n0 + r;
    if (n >= It.rows) continue;
    float* o = X + static_cast<int64_t>(n) * It.ld + i;
    if (vec) {
      *reinterpret_cast<f32x4*>(o) = f32x4{t[i4][r], t[i4 + 1][r], t[i4 + 2][r], t[i4 + 3][r]};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i + e < It.d_in) o[e] = t[i4 + e][r];
    }
  }
}

kfac_status_t launch_im2col(const std::vector<ColItem>& items, hipStream_t st) {
  for (size_t i0 = 0; i0 < items.size(); i0 += kMaxCols) {
    ColTab tab{};
    int blocks = 0;
    for (size_t i = i0; i < items.size() && tab.n < kMaxCols; ++i) {
      ColItem c = items[i];
      c.blk_begin = blocks;
      blocks += (c.rows + kColTile - 1) / kColTile * ((c.d_in + kColTile - 1) / kColTile);
      tab.c[tab.n++] = c;
    }
    hipLaunchKernelGGL(im2col_kernel, dim3(blocks), dim3(256), 0, st, tab);
    if (hipGetLastError() != hipSuccess) return KFAC_ERR_HIP;
  }
  return KFAC_OK;
}

// ---------------------------------------------------------------------------
// damped Cholesky inverse, batched over matrices

constexpr int kMaxMats = 40;
constexpr int kLauRows = 1024;   // rows of Z per pass of the final Z^T Z

struct Mat {
  const float* F;     // factor (upper triangle read)
  float* Finv;        // damped inverse (written unless the factorisation failed)
  float* L;           // working copy -> Cholesky factor (lower)
  float* Z;           // L^-1 (lower)
  float* Dinv;        // inverses of the diagonal blocks, [nblk][128][128]
  int32_t* fail;
  int32_t d;
  int32_t packed;     // F is stored as its packed upper triangle
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

// L = F + damping I (lower triangle) from F's upper triangle, fail = 0, and
// zeros in Z's strict upper triangle within 256 of the diagonal.  Nothing
// reads L's upper triangle (the triangular inverse stages its products
// there), Z's lower triangle is written whole by the inverse, and the tiles
// of the inverse's products that straddle the diagonal (at most 256 wide)
// read Z's upper entries in that band only.  grid = (32 x 32 tiles, matrix);
// a lower tile (I > J) is read from F's upper tile (J, I) row by row and
// transposed through LDS.  T.k selects the tiles: 0 all, 1 the columns of the
// first outer panel of L (what the first inner steps need), 2 the rest.
constexpr int kInitSplit = kOuter * kNb;   // the first outer panel's columns
__global__ void __launch_bounds__(256) chol_init_kernel(MatTab T) {
  __shared__ float t[32][33];
  const Mat& M = T.m[blockIdx.y];
  const int d = M.d;
  const int nt = (d + 31) / 32;
  if (T.k != 2 && blockIdx.x == 0 && threadIdx.x == 0) *M.fail = 0;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int tile = blockIdx.x; tile < nt * nt; tile += gridDim.x) {
    const int I = tile / nt, J = tile - (tile / nt) * nt;
    const bool first = J * 32 < kInitSplit;
    const bool fill_l = I >= J && (T.k == 0 || (T.k == 1) == first);
    const bool zero_z = I <= J && I / 8 == J / 8 && T.k != 1;   // (same 256-block)
    if (!fill_l && !zero_z) continue;   // (uniform across the workgroup)
    if (fill_l) {
      const bool lower = I > J;
      const int sr = (lower ? J : I) * 32, sc = (lower ? I : J) * 32;   // source tile in the upper triangle
      __syncthreads();
      for (int r = ty; r < 32; r += 8) {
        const int i = sr + r, j = sc + tx;
        // only upper entries are used (a diagonal tile mirrors its upper part)
        float v = 0.f;
        if (i < d && j < d && i <= j) v = M.F[M.packed ? packed_index(i, j, d) : static_cast<int64_t>(i) * d + j];
        t[r][tx] = v;
      }
      __syncthreads();
    }
    for (int r = ty; r < 32; r += 8) {
      const int i = I * 32 + r, j = J * 32 + tx;
      if (i >= d || j >= d) continue;
      const int64_t e = static_cast<int64_t>(i) * d + j;
      if (i >= j) {
        if (fill_l) {
          float v = I > J ? t[tx][r] : t[min(r, tx)][max(r, tx)];   // diagonal tile: mirror its upper part
          if (i == j) v += T.damping;
          M.L[e] = v;
        }
      } else if (zero_z) {
        M.Z[e] = 0.f;
      }
    }
  }
}

// Block k of every matrix with more than k blocks: Cholesky factor of the
// diagonal block and its inverse, one workgroup (4 wavefronts) per block,
// blocked by 32 columns with the whole block in LDS.  Per 32-column panel:
//  - wavefront 0 factors the 32 x 32 diagonal sub-block in registers: lane c
//    holds column c of the sub-block, lane 32 + c column c of an identity;
//    elimination is sqrt-free (row r -= (B_rj / B_jj) row j), which yields
//    D^-1/2-scaled forms of both L (columns) and L^-1 (rows);
//  - the sub-diagonal panel L_qp = M_qp Z_pp^T and the trailing update
//    M_ij -= L_ip L_jp^T run on MFMA, one 32 x 32 tile per wavefront.
// The off-diagonal blocks of the inverse follow by rows,
// Z_ij = -Z_ii sum_{j<=m<i} L_im Z_mj, also on MFMA.  One 128 x 128 array
// holds everything (66 KB of LDS, so that the workgroup fits on a CU beside a
// 128 x 128 GEMM workgroup): L's off-diagonal blocks below the diagonal, Z's
// diagonal blocks in place of L's (which no later step reads: the panel below
// a block is formed with its inverse), and Z's off-diagonal blocks transposed
// above the diagonal.  The inverse goes to Dinv[k] and to Z's diagonal block;
// L_kk is not written back.  A pivot that is not positive (or not finite)
// marks the matrix failed, raises KFAC_FLAG_NOT_PD and is replaced by 1 so the
// remaining steps stay finite; a failed matrix's inverse is not written.
// Rows and columns beyond a partial last block are an identity.
constexpr int kLd = kNb + 1;   // LDS pitch: row and column walks hit distinct banks

__device__ inline f32x16 mfma32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// acc += sign * A B^T with A = X[ar.., ac..], B = Y[br.., bc..] (32 x 32 each, pitch kLd)
__device__ inline void mma_nt(f32x16& acc, const float* X, int ar, int ac, const float* Y, int br, int bc, float sign,
                              int lane) {
#pragma unroll
  for (int kk = 0; kk < 32; kk += 2) {
    const int k = kk + (lane >> 5);
    acc = mfma32(sign * X[(ar + (lane & 31)) * kLd + ac + k], Y[(br + (lane & 31)) * kLd + bc + k], acc);
  }
}

// acc += A B with A = X[ar.., ac..] (pitch kLd), B = Y[br.., bc..] (pitch ldy)
__device__ inline void mma_nn(f32x16& acc, const float* X, int ar, int ac, const float* Y, int ldy, int br, int bc,
                              int lane) {
#pragma unroll
  for (int kk = 0; kk < 32; kk += 2) {
    const int k = kk + (lane >> 5);
    acc = mfma32(X[(ar + (lane & 31)) * kLd + ac + k], Y[(br + k) * ldy + bc + (lane & 31)], acc);
  }
}

// acc += A^T B with A = X[ar.., ac..], B = Y[br.., bc..] (32 x 32 each, pitch kLd)
__device__ inline void mma_tn(f32x16& acc, const float* X, int ar, int ac, const float* Y, int br, int bc, int lane) {
#pragma unroll
  for (int kk = 0; kk < 32; kk += 2) {
    const int k = kk + (lane >> 5);
    acc = mfma32(X[(ar + k) * kLd + ac + (lane & 31)], Y[(br + k) * kLd + bc + (lane & 31)], acc);
  }
}

// accumulator r of lane l is element (8 (r/4) + 4 (l/32) + r%4, l%32) of the tile
__device__ inline int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

__device__ inline void tile_load(f32x16& acc, const float* S, int ld, int r0, int c0, int lane) {
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = S[(r0 + acc_row(r, lane)) * ld + c0 + (lane & 31)];
}

__device__ inline void tile_store(float* S, int ld, int r0, int c0, const f32x16& acc, float sign, int lane) {
#pragma unroll
  for (int r = 0; r < 16; ++r) S[(r0 + acc_row(r, lane)) * ld + c0 + (lane & 31)] = sign * acc[r];
}

// the tile transposed: element (i, j) to S[(r0 + j) * ld + c0 + i]
__device__ inline void tile_store_t(float* S, int ld, int r0, int c0, const f32x16& acc, float sign, int lane) {
#pragma unroll
  for (int r = 0; r < 16; ++r) S[(r0 + (lane & 31)) * ld + c0 + acc_row(r, lane)] = sign * acc[r];
}

// Wavefront-level factorization of the 32 x 32 diagonal sub-block at (c0, c0)
// of Ms; writes its inverse over it (the factor itself is not kept).
// Step j is a rank-1 update by u = column j of the (symmetric) remaining
// block, which every lane needs whole.  Lane r holds row j of column r, which
// is u_r by symmetry, so the lanes exchange u through the 64 floats at Us:
// each writes its entry, then all read it back with broadcast 16-byte reads
// (no cross-lane register moves).
__device__ __attribute__((always_inline)) inline bool factor_diag32(float* Ms, float* Us, int c0, int32_t* fail,
                                                                   uint32_t* flags, int lane) {
  const int c = lane & 31;
  const bool xl = lane >= 32;
  float v[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) v[r] = xl ? (r == c ? 1.f : 0.f) : Ms[(c0 + r) * kLd + c0 + c];
  Us[lane] = v[0];   // (the X lanes' entries, Us[32..63], are never read)
  __builtin_amdgcn_wave_barrier();
  // u_q .. u_31 (the aligned quads from q on) as last written
  auto gather = [&](float* u, int q0) {
#pragma unroll
    for (int q = q0 / 4; q < 8; ++q) {
      const f32x4 t4 = *reinterpret_cast<const f32x4*>(Us + 4 * q);
      u[4 * q] = t4.x;
      u[4 * q + 1] = t4.y;
      u[4 * q + 2] = t4.z;
      u[4 * q + 3] = t4.w;
    }
  };
  float dmine = 1.f;   // this lane's pivot (lane c: d_c)
  bool bad = false;
  float ua[32], ub[32];
  gather(ua, 0);
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    float* u = (j & 1) ? ub : ua;    // this step's u (the pivot is u_j)
    float* un = (j & 1) ? ua : ub;   // the next step's
    float piv = u[j];
    const bool ok = piv > 0.f && isfinite(piv);
    bad = bad || !ok;
    piv = ok ? piv : 1.f;
    if (c == j) dmine = piv;
    const float inv = __builtin_amdgcn_rcpf(piv);
    // u_j's quad also brought the entries before it, which are not needed:
    // held until here (their load has landed with u_j), their registers are
    // not handed to this step's updates while the load is still in flight
    // (which would make the updates wait for it)
#pragma unroll
    for (int r = 4 * (j / 4); r < j; ++r) asm volatile("" ::"v"(u[r]));
    // A lanes: columns c > j take the update (row j of column c is
    // B_jc = u_c); finished columns keep their multipliers.  X lanes: row
    // operation on the whole row.
    const float t = (xl || c > j) ? v[j] * inv : 0.f;
    if (j + 1 < 32) {
      // the next step's u first, so that its round trip through LDS
      // overlaps the rest of this step
      v[j + 1] = fmaf(-u[j + 1], t, v[j + 1]);
      Us[lane] = v[j + 1];
      __builtin_amdgcn_wave_barrier();
      gather(un, j + 1);
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    // the rest of the step's updates, each held to this step: left to
    // itself, the compiler defers every update to its first use and keeps
    // all earlier steps' u in registers
#pragma unroll
    for (int r = j + 2; r < 32; ++r) {
      v[r] = fmaf(-u[r], t, v[r]);
      asm volatile("" : "+v"(v[r]));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (bad && lane == 0 && *fail == 0) {
    *fail = 1;
    raise_flag(flags, KFAC_FLAG_NOT_PD);
  }
  // row scales 1 / sqrt(d_r): lane c computes its own pivot's (dmine) and
  // shares it through Us, one division per lane instead of 32 in a row
  Us[lane] = 1.0f / sqrtf(dmine);
  __builtin_amdgcn_wave_barrier();
  float rs[32];
  gather(rs, 0);
  __builtin_amdgcn_wave_barrier();
  if (xl) {
    // (L^-1)_rc = X_rc / sqrt(d_r)
#pragma unroll
    for (int r = 0; r < 32; ++r) Ms[(c0 + r) * kLd + c0 + c] = r >= c ? v[r] * rs[r] : 0.f;
  }
  return bad;   // (the same in every lane: all of them read the same pivots)
}

// Cholesky and inverse of the symmetric working block in Ms (pitch kLd; bk
// rows and columns hold the matrix, the rest an identity), by 32-column
// sub-blocks; on return Ms holds Z = L^-1 with its diagonal blocks in place
// (zero above their diagonal) and its off-diagonal blocks transposed above
// the diagonal.  A failed pivot also sets *sbad (in LDS; when not null).
// Returns with the workgroup synchronised.
__device__ __forceinline__ void factor_invert_block(float* Ms, float* Us, int bk, int32_t* fail, uint32_t* flags,
                                                    int* sbad, int lane, int wid) {
  // Only the first np 32-column sub-blocks hold the factor (bk rows); the
  // rest of the working block is identity, is never read by them and is not
  // written out, so a ragged last block skips it.
  const int np = (bk + 31) / 32;
  for (int p = 0; p < np; ++p) {
    const int c0 = 32 * p;
    if (wid == 0) {
      const bool bad = factor_diag32(Ms, Us, c0, fail, flags, lane);
      if (bad && sbad != nullptr && lane == 0) *sbad = 1;
    }
    __syncthreads();
    // panel below the diagonal sub-block: L_qp = M_qp Z_pp^T
    if (wid < np - 1 - p) {
      const int q = p + 1 + wid;
      f32x16 acc = {};
      mma_nt(acc, Ms, 32 * q, c0, Ms, c0, c0, 1.f, lane);
      tile_store(Ms, kLd, 32 * q, c0, acc, 1.f, lane);
    }
    __syncthreads();
    // trailing lower tiles (ib, jb), p < jb <= ib: M_ij -= L_ip L_jp^T
    const int nr = np - 1 - p;
    for (int t = wid; t < nr * (nr + 1) / 2; t += 4) {
      int ib = 0, u = t;
      while (u > ib) { u -= ib + 1; ++ib; }
      const int I = 32 * (p + 1 + ib), J = 32 * (p + 1 + u);
      f32x16 acc;
      tile_load(acc, Ms, kLd, I, J, lane);
      mma_nt(acc, Ms, I, c0, Ms, J, c0, -1.f, lane);
      tile_store(Ms, kLd, I, J, acc, 1.f, lane);
    }
    __syncthreads();
  }

  // inverse by block rows: Z_ij = -Z_ii sum_{j <= m < i} L_im Z_mj, with
  // Z_mj (m > j) held transposed at block (j, m); the sum is staged, also
  // transposed, at block (j, i), where Z_ij then goes (wavefront j alone
  // touches that block in this row)
  for (int i = 1; i < np; ++i) {
    if (wid < i) {
      const int j = wid;
      f32x16 acc = {};
      mma_nn(acc, Ms, 32 * i, 32 * j, Ms, kLd, 32 * j, 32 * j, lane);
      for (int m = j + 1; m < i; ++m) mma_nt(acc, Ms, 32 * i, 32 * m, Ms, 32 * j, 32 * m, 1.f, lane);
      tile_store_t(Ms, kLd, 32 * j, 32 * i, acc, 1.f, lane);
      f32x16 z = {};
      mma_nt(z, Ms, 32 * i, 32 * i, Ms, 32 * j, 32 * i, 1.f, lane);
      tile_store_t(Ms, kLd, 32 * j, 32 * i, z, -1.f, lane);
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) chol_diag_kernel(DiagTab T) {
  // (the Cholesky chain shares CUs with the assembly's products: its
  // wavefronts issue first)
  __builtin_amdgcn_s_setprio(3);
  __shared__ __attribute__((aligned(16))) float Ms[kNb * kLd];
  __shared__ __attribute__((aligned(16))) float Us[64];
  const DMat& M = T.m[blockIdx.x];
  const int d = M.d, k = T.k;
  const int nblk = (d + kNb - 1) / kNb;
  if (k >= nblk) return;
  const int r0 = k * kNb;
  const int bk = min(kNb, d - r0);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  float* Lg = M.L + static_cast<int64_t>(r0) * d + r0;

  // symmetric working block from the lower triangle; identity beyond bk.
  // With d a multiple of 4 (16-byte rows), thread t reads quad t % 32 of
  // rows t / 32 + 8 i, all 16 loads in flight; otherwise column t % 128 of
  // rows t / 128 + 2 i, 32 loads at a time.
  const bool vec = (d & 3) == 0;
  auto put = [&](int r, int c, float v) {   // (r, c), c <= r, and its mirror
    const float x = r < bk ? v : (r == c ? 1.f : 0.f);
    Ms[r * kLd + c] = x;
    Ms[c * kLd + r] = x;
  };
  if (vec) {
    const int q = tid & 31, rr = tid >> 5;
    f32x4 vals[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = rr + 8 * i;
      vals[i] = (r < bk && 4 * q <= r) ? *reinterpret_cast<const f32x4*>(Lg + static_cast<int64_t>(r) * d + 4 * q)
                                       : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = rr + 8 * i;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * q + e <= r) put(r, 4 * q + e, vals[i][e]);
    }
  } else {
    const int lc = tid & (kNb - 1), lr = tid >> 7;
    for (int i0 = 0; i0 < kNb / 2; i0 += 32) {
      float vals[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int r = lr + 2 * (i0 + u);
        vals[u] = (r < bk && lc <= r) ? Lg[static_cast<int64_t>(r) * d + lc] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int r = lr + 2 * (i0 + u);
        if (lc <= r) put(r, lc, vals[u]);
      }
    }
  }
  __syncthreads();

  factor_invert_block(Ms, Us, bk, M.fail, T.flags, nullptr, lane, wid);

  // write back Dinv[k] and Z_kk (L_kk itself is not read again: the panel
  // below it is formed with Dinv[k]); thread t writes quad t % 32 of rows
  // t / 32 + 8 i (bk is a multiple of 4 when d is)
  float* D = M.Dinv + static_cast<int64_t>(k) * kNb * kNb;
  float* Zg = M.Z + static_cast<int64_t>(r0) * d + r0;
  {
    const int q = tid & 31, rr = tid >> 5;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = rr + 8 * i;
      f32x4 z;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 4 * q + e;
        // (an off-diagonal 32-block of Z is held transposed)
        z[e] = (c <= r && r < bk && c < bk) ? Ms[(r >> 5) == (c >> 5) ? r * kLd + c : c * kLd + r] : 0.f;
      }
      *reinterpret_cast<f32x4*>(D + r * kNb + 4 * q) = z;
      if (r < bk) {
        float* zr = Zg + static_cast<int64_t>(r) * d + 4 * q;
        if (vec) {
          if (4 * q < bk) *reinterpret_cast<f32x4*>(zr) = z;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * q + e < bk) zr[e] = z[e];
        }
      }
    }
  }
}

// A factor of at most 128 rows and columns in one launch: the working block
// is F's upper triangle plus the damping on the diagonal (read directly, no
// separate initialisation), factored and inverted as above, and the damped
// inverse (L L^T)^-1 = Z^T Z formed on MFMA from Ms's Z and written whole
// (both triangles) unless a pivot failed.  One workgroup per factor.  With
// 32-blocks Z_ab of Z (block row a, block column b) and m >= max(a, b):
// W_ab = sum_m Z_ma^T Z_mb, where for a <= b the term m = b is Z_ab'^T Z_bb
// (a < b: Z_ba^T is the stored block (a, b); a = b: the diagonal block
// itself, transposed) and every m > b is (stored (a, m)) (stored (b, m))^T.
__global__ void __launch_bounds__(256) chol_small_kernel(MatTab T) {
  __shared__ __attribute__((aligned(16))) float Ms[kNb * kLd];
  __shared__ __attribute__((aligned(16))) float Us[64];
  __shared__ int sbad;
  const Mat& M = T.m[blockIdx.x];
  const int d = M.d;   // <= kNb
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid == 0) {
    *M.fail = 0;
    sbad = 0;
  }
  for (int e = tid; e < kNb * kLd; e += 256) Ms[e] = (e / kLd == e % kLd) ? 1.f : 0.f;
  __syncthreads();
  // upper elements (r, c), c >= r, mirrored; 32 loads in flight per thread
  const int ne = d * d;
  for (int e0 = 0; e0 < ne; e0 += 32 * 256) {
    float v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int e = e0 + u * 256 + tid;
      const int r = e / d, c = e - r * d;
      const bool up = e < ne && c >= r;
      v[u] = up ? M.F[M.packed ? packed_index(r, c, d) : static_cast<int64_t>(e)] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int e = e0 + u * 256 + tid;
      const int r = e / d, c = e - r * d;
      if (e < ne && c >= r) {
        const float x = r == c ? v[u] + T.damping : v[u];
        Ms[r * kLd + c] = x;
        Ms[c * kLd + r] = x;
      }
    }
  }
  __syncthreads();
  factor_invert_block(Ms, Us, d, M.fail, T.flags, &sbad, lane, wid);

  // W's upper 32-blocks (a, b), b-major: at most 10, so 3 per wavefront
  const int np = (d + 31) / 32;
  const int nw = np * (np + 1) / 2;
  f32x16 w[3];
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int t = wid + 4 * s;
    w[s] = f32x16{};
    if (t >= nw) continue;
    int b = 0, a = t;
    while (a > b) { a -= b + 1; ++b; }
    if (a == b) mma_tn(w[s], Ms, 32 * b, 32 * b, Ms, 32 * b, 32 * b, lane);
    else mma_nn(w[s], Ms, 32 * a, 32 * b, Ms, kLd, 32 * b, 32 * b, lane);
    for (int m = b + 1; m < np; ++m) mma_nt(w[s], Ms, 32 * a, 32 * m, Ms, 32 * b, 32 * m, 1.f, lane);
  }
  __syncthreads();   // every read of Z done: W replaces it in Ms
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int t = wid + 4 * s;
    if (t >= nw) continue;
    int b = 0, a = t;
    while (a > b) { a -= b + 1; ++b; }
    tile_store(Ms, kLd, 32 * a, 32 * b, w[s], 1.f, lane);
    if (a != b) tile_store_t(Ms, kLd, 32 * b, 32 * a, w[s], 1.f, lane);
  }
  __syncthreads();
  if (sbad != 0) return;   // a failed factor keeps its previous inverse
  for (int e = tid; e < ne; e += 256) {
    const int r = e / d, c = e - r * d;
    M.Finv[e] = Ms[r * kLd + c];
  }
}

// ---------------------------------------------------------------------------
// planning

// ---------------------------------------------------------------------------
// Bias column of the preconditioned gradient.  With a bias, d_a = d_in + 1;
// when d_in is a whole number of GEMM tiles, a (d_in + 1)-wide tile grid would
// end in a column of tiles with one valid column, which costs as much as a
// full one.  Those layers run both preconditioning GEMMs over the first d_in
// columns, and the last column as two matrix-vector products, batched over
// layers (HBM-bound: every matrix entry is read once):
//   stage 0: t[i] = sum_k [grad_w | grad_b][i][k] A_inv[k][d_in]
//   stage 1: p[i] = sum_k G_inv[i][k] t[k]; D = p + wd b; V = mu V + D; b -= lr V
// A_inv and G_inv are symmetric, so contiguous rows stand in for columns.
bool bias_column_split(const LayerGeom& g) { return g.bias && g.d_in % kTile == 0; }

constexpr int kBcThreads = 256;
constexpr int kBcRowsPerWave = 2;
constexpr int kBcRowsPerBlock = kBcThreads / kWave * kBcRowsPerWave;
constexpr int kMaxBcProbs = 48;   // kernel arguments stay within 4 KB

struct BcProb {
  const float* M;       // row i at M + i * ld, kmain entries
  const float* extra;   // stage 0: entry kmain of row i is extra[i]; stage 1: null
  const float* x;       // kmain (+1 with extra) entries
  float* y;             // stage 0: t
  float* b;             // stage 1: bias and its momentum, updated in place
  float* mb;
  int32_t rows, ld, kmain, blk_begin, vec, pad_;
};
struct BcTab {
  BcProb p[kMaxBcProbs];
  int32_t n, stage;
  float lr, momentum, weight_decay;
  uint32_t* flags;
};

__device__ inline float bc_wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Kept small (two rows per wavefront, one 16-byte load per row in flight,
// about two dozen VGPRs) so that its wavefronts fit beside the 256 x 256 GEMM
// workgroups, which leave 32-48 VGPRs per SIMD lane, and run alongside them.
__global__ void __launch_bounds__(kBcThreads) bias_col_kernel(BcTab tab) {
  int lo = 0, hi = tab.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tab.p[mid].blk_begin <= static_cast<int>(blockIdx.x)) lo = mid; else hi = mid - 1;
  }
  const BcProb P = tab.p[lo];
  const int wid = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int row0 = (blockIdx.x - P.blk_begin) * kBcRowsPerBlock + wid * kBcRowsPerWave;
  if (row0 >= P.rows) return;
  const float* m0 = P.M + static_cast<int64_t>(row0) * P.ld;
  const float* m1 = P.M + static_cast<int64_t>(min(row0 + 1, P.rows - 1)) * P.ld;   // a clamped row is discarded
  float acc0 = 0.f, acc1 = 0.f;
  int k = 0;
  if (P.vec) {   // 16-byte loads: ld, kmain multiples of 4 and aligned bases
    const int kv = P.kmain & ~(4 * kWave - 1);
    for (k = 4 * lane; k < kv; k += 4 * kWave) {
      const f32x4 xv = *reinterpret_cast<const f32x4*>(P.x + k);
      const f32x4 a0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(m0 + k));
      const f32x4 a1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(m1 + k));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc0 = fmaf(a0[e], xv[e], acc0);
        acc1 = fmaf(a1[e], xv[e], acc1);
      }
    }
    k = kv;
  }
  for (k += lane; k < P.kmain; k += kWave) {
    const float xv = P.x[k];
    acc0 = fmaf(m0[k], xv, acc0);
    acc1 = fmaf(m1[k], xv, acc1);
  }
  bool bad = false;
#pragma unroll
  for (int r = 0; r < kBcRowsPerWave; ++r) {
    const float v = bc_wave_sum(r == 0 ? acc0 : acc1);
    const int row = row0 + r;
    if (lane != 0 || row >= P.rows) continue;
    if (tab.stage == 0) {
      P.y[row] = P.extra ? fmaf(P.extra[row], P.x[P.kmain], v) : v;
    } else {
      const float w = P.b[row];
      const float d = fmaf(tab.weight_decay, w, v);
      const float vn = fmaf(tab.momentum, P.mb[row], d);
      const float wn = fmaf(-tab.lr, vn, w);
      P.mb[row] = vn;
      P.b[row] = wn;
      bad |= !(isfinite(vn) && isfinite(wn));
    }
  }
  if (bad) raise_flag(tab.flags, KFAC_FLAG_NONFINITE);
}

// Launches one stage of the bias-column products for every listed problem.
kfac_status_t launch_bias_col(std::vector<BcProb>& probs, int stage, const kfac_hparams_t& hp, uint32_t* flags,
                              hipStream_t st) {
  for (size_t g0 = 0; g0 < probs.size(); g0 += kMaxBcProbs) {
    const size_t g1 = std::min(probs.size(), g0 + kMaxBcProbs);
    BcTab T{};
    int blocks = 0;
    for (size_t i = g0; i < g1; ++i) {
      T.p[i - g0] = probs[i];
      T.p[i - g0].blk_begin = blocks;
      blocks += (probs[i].rows + kBcRowsPerBlock - 1) / kBcRowsPerBlock;
    }
    T.n = static_cast<int>(g1 - g0);
    T.stage = stage;
    T.lr = hp.lr;
    T.momentum = hp.momentum;
    T.weight_decay = hp.weight_decay;
    T.flags = flags;
    hipLaunchKernelGGL(bias_col_kernel, dim3(blocks), dim3(kBcThreads), 0, st, T);
    KFAC_HIP_TRY(hipGetLastError());
  }
  return KFAC_OK;
}

// row length of the preconditioning intermediate T: a multiple of 4 floats,
// so that its rows can be loaded 16 bytes at a time
inline int t_ld(int d_a) { return (d_a + 3) & ~3; }

struct FullPlan {
  size_t ws_bytes = kFlagBytes;
  std::vector<RescaleSeg> rescale;   // per layer: its weight (KFAC_OPT_RESCALE)
  std::vector<float*> part;      // per layer and factor (2 li + which): split-K partials, or null
  std::vector<int> nsplit;       // per layer and factor
  std::vector<float*> T;         // per layer, d_out x d_a, rows of t_ld(d_a) floats (16-byte aligned rows)
  std::vector<float*> tb;        // per layer: column d_in of T (bias-column layers), else null
  std::vector<float*> xcol;      // per layer and factor: fp32 convolution tensor as [rows, width], or null
  std::vector<int> xcol_ld;      // their row pitch (floats)
  std::vector<Mat> mats;         // inverse work per factor (2 layer + which)
  std::vector<float*> W;         // per factor: Z^T Z, assembled while the Cholesky runs (upper triangle)
  // runs of equal-size factors whose work areas sit at a constant stride
  struct Group {
    int first;                   // index into mats of the lowest address
    int count;
    int64_t stride;              // floats between neighbouring work areas
    std::vector<int> members;    // indices into mats, by address
  };
  std::vector<Group> groups;
};

size_t nblk_of(int d) { return (d + kNb - 1) / kNb; }

// Row splits of an fp32 factor SYRK (128 x 128 tiles): one workgroup
// contracts about kSplitRows rows, so a launch holds many workgroups of
// similar length and tall factors (a stem convolution's 401,408 rows) do not
// serialise it; sym_reduce_kernel adds the partial products in split order.
// A factor of at most 4 tiles is split into pieces of 32 or more rows (up to
// 8): its few workgroups would otherwise each run the whole contraction as
// one serial chain of stages (FC 64 -> 32 at batch 128: factor phase 37 ->
// 23-31 us).
constexpr int64_t kSplitRows = 2048;

int syrk_splits(int d, int64_t rows) {
  if (rows < 2 * kSplitRows) {
    const int64_t t = (d + 127) / 128;
    if (t * (t + 1) / 2 <= 4 && rows >= 64) return static_cast<int>(std::min<int64_t>(8, rows / 32));
    return 1;
  }
  return static_cast<int>(std::min<int64_t>(128, (rows + kSplitRows - 1) / kSplitRows));
}

bool fp32_factor(const kfac_layer_t& L, int which) {
  return (which == 0 ? L.act_dtype : L.grad_dtype) == KFAC_F32;
}

// an fp32 convolution factor whose rows the SYRK reads from the tensor in
// place: the output gradient, and the input of a 1 x 1, stride-1, unpadded
// convolution without a bias column (in both, row n is pixel n % HW of image
// n / HW, the tensor being [B][d][HW])
bool nchw_factor(const kfac_layer_t& L, int which) {
  const LayerGeom g = geom_of(L);
  if (!g.conv || !fp32_factor(L, which)) return false;
  if (which == 0) {
    if (g.bias || g.kh != 1 || g.kw != 1 || g.stride != 1 || g.pad != 0) return false;
    return gemm_nchw_syrk_ok(L.a, g.rows, g.h * g.w, g.d_in);
  }
  return gemm_nchw_syrk_ok(L.g, g.rows, g.h_out * g.w_out, g.d_out);
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
    RescaleSeg rs{};
    rs.w = layers[li].w;
    rs.n = static_cast<int64_t>(g.d_out) * g.d_in;
    rs.d_out = g.d_out;
    rs.part = reinterpret_cast<float*>(carve(static_cast<size_t>(rescale_blocks(rs.n)) * 4));
    P.rescale.push_back(rs);
  }
  for (int li = 0; li < n; ++li) {
    const LayerGeom g = geom_of(layers[li]);
    P.T.push_back(reinterpret_cast<float*>(carve(static_cast<size_t>(g.d_out) * t_ld(g.d_a) * 4)));
    P.tb.push_back(bias_column_split(g) ? reinterpret_cast<float*>(carve(static_cast<size_t>(g.d_out) * 4)) : nullptr);
  }
  for (int li = 0; li < n; ++li) {
    const LayerGeom g = geom_of(layers[li]);
    for (int which = 0; which < 2; ++which) {
      const bool col = g.conv && fp32_factor(layers[li], which) && !nchw_factor(layers[li], which);
      const int w = which == 0 ? g.d_in : g.d_out;
      const int ld = (w + 3) / 4 * 4;
      P.xcol_ld.push_back(col ? ld : 0);
      P.xcol.push_back(col ? reinterpret_cast<float*>(carve(static_cast<size_t>(g.rows) * ld * 4)) : nullptr);
    }
  }
  // Cholesky work areas: one contiguous chunk per factor (L, Z, W, Dinv, fail),
  // factors of equal size side by side, so that the chunks of one size lie
  // at a constant stride and every size is one batched GEMM problem
  P.mats.resize(2 * static_cast<size_t>(n));
  P.W.resize(P.mats.size());
  std::vector<int> order(P.mats.size());
  for (int li = 0; li < n; ++li) {
    const LayerGeom g = geom_of(layers[li]);
    for (int which = 0; which < 2; ++which) {
      Mat& m = P.mats[2 * li + which];
      m.F = which == 0 ? layers[li].A : layers[li].G;
      m.Finv = which == 0 ? layers[li].A_inv : layers[li].G_inv;
      m.d = which == 0 ? g.d_a : g.d_out;
      m.packed = g.packed ? 1 : 0;
      order[2 * li + which] = 2 * li + which;
    }
  }
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return P.mats[a].d > P.mats[b].d; });
  std::vector<size_t> start(order.size());
  for (size_t i = 0; i < order.size(); ++i) {
    Mat& m = P.mats[order[i]];
    const int d = m.d;
    start[i] = off;
    m.L = reinterpret_cast<float*>(carve(static_cast<size_t>(d) * d * 4));
    m.Z = reinterpret_cast<float*>(carve(static_cast<size_t>(d) * d * 4));
    P.W[order[i]] = reinterpret_cast<float*>(carve(static_cast<size_t>(d) * d * 4));
    m.Dinv = reinterpret_cast<float*>(carve(nblk_of(d) * kNb * kNb * 4));
    m.fail = reinterpret_cast<int32_t*>(carve(4));
  }
  for (size_t i = 0; i < order.size();) {
    size_t j = i + 1;
    while (j < order.size() && P.mats[order[j]].d == P.mats[order[i]].d) ++j;
    FullPlan::Group gr{order[i], static_cast<int>(j - i), 0, {}};
    if (j - i > 1) gr.stride = static_cast<int64_t>((start[i + 1] - start[i]) / 4);
    for (size_t q = i; q < j; ++q) gr.members.push_back(order[q]);
    P.groups.push_back(gr);
    i = j;
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

// FACTORS: convolution tensors laid out as rows (one batched im2col
// launch), then every fp32 factor of the stack in batched row-major SYRK
// launches (direct EMA, or split rows summed by the batched reduce
// afterwards), and the bf16 factors on the bf16 SYRK.
// Factor and EMA of fp32 linear-layer factors at most 128 wide, one
// workgroup per factor: X (plus the bias layer's constant-1 column, 1 on real
// rows only) goes through LDS in chunks of kSmallRows rows, the loads of the
// next two chunks in flight while one is contracted; each wavefront owns
// whole upper 32-blocks of X^T X (at most 10, so 3 each) and runs every row
// for them, so no partial sums are combined; then F <- beta F + alpha X^T X
// on the upper triangle (mirrored, or packed).  Used when every factor of the
// step qualifies: the general path's split SYRK and reduction are two
// launches whose workgroups each walk a chain of stages.
constexpr int kMaxSmallSyrk = 48;
constexpr int kSmallRows = 64;                // rows of X per chunk
constexpr int kSmallPitch = kNb + 4;          // LDS row of a chunk (floats)
constexpr int64_t kSmallMaxRows = 8192;       // one workgroup contracts every row
struct SmallSyrk {
  const float* X;    // [rows][w] row-major
  float* F;          // d x d (d = w + bias), whole or packed upper triangle
  int32_t rows, w, bias, packed;
  float alpha, beta;
};
struct SmallSyrkTab {
  SmallSyrk s[kMaxSmallSyrk];
  int32_t n;
};
static_assert(sizeof(SmallSyrkTab) <= 4096, "kernel arguments");

__global__ void __launch_bounds__(256) syrk_small_kernel(SmallSyrkTab T) {
  __shared__ __attribute__((aligned(16))) float Xs[kSmallRows * kSmallPitch];
  // the table entry read once, kept in registers
  const SmallSyrk& S = T.s[blockIdx.x];
  const float* X = arg_reg(S.X);
  float* F = arg_reg(S.F);
  const int w = arg_reg(S.w), bias = arg_reg(S.bias), rows = arg_reg(S.rows), packed = arg_reg(S.packed);
  const float alpha = arg_reg(S.alpha), beta = arg_reg(S.beta);
  const int d = w + bias;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nb = (d + 31) / 32, nu = nb * (nb + 1) / 2;
  // this wavefront's blocks (a, b), a <= b, b-major: t = wid, wid + 4, wid + 8
  int ba[3], bb[3];
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    int b = 0, a = wid + 4 * s;
    while (a > b) { a -= b + 1; ++b; }
    ba[s] = a;
    bb[s] = b;
  }
  f32x16 acc[3];
#pragma unroll
  for (int s = 0; s < 3; ++s) acc[s] = f32x16{};
  // A lone workgroup waits out every dependent memory round trip (several
  // microseconds each), so everything that does not depend on the contraction
  // is requested at the start: the old factor entries of this wavefront's
  // blocks (for the EMA) and the first two chunks of X, into two register
  // sets that then alternate.
  const bool rd = beta != 0.f;
  float o[3][16];
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int col = 32 * bb[s] + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * ba[s] + acc_row(r, lane);
      const bool up = wid + 4 * s < nu && row <= col && col < d;
      const int64_t f = !up ? 0 : packed ? packed_index(row, col, d) : static_cast<int64_t>(row) * d + col;
      o[s][r] = rd ? F[f] : 0.f;
    }
  }
  // chunk loads: thread t takes column t % 128 of chunk rows t / 128 + 2 u
  constexpr int kPer = kSmallRows / 2;   // 32
  const int cc = tid & (kNb - 1), rr = tid >> 7;
  auto load = [&](float (&v)[kPer], int r0) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int r = r0 + rr + 2 * u;
      v[u] = (cc < w && r < rows) ? X[static_cast<int64_t>(r) * w + cc] : 0.f;
    }
  };
  const int nch = (rows + kSmallRows - 1) / kSmallRows;
  // chunk ch from register set v: into LDS, the set refilled with chunk ch + 2,
  // then every row pair of the chunk (rows past the end are zero)
  auto step = [&](float (&v)[kPer], int ch) {
    const int r0 = ch * kSmallRows;
    __syncthreads();   // the previous chunk is no longer read
    // columns up to the last 32-block: X, the bias column (1 on real rows), zeros
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int r = rr + 2 * u;
      const float one = (bias && cc == w && r0 + r < rows) ? 1.f : 0.f;
      if (cc < 32 * nb) Xs[r * kSmallPitch + cc] = cc < w ? v[u] : one;
    }
    __syncthreads();
    if (ch + 2 < nch) load(v, r0 + 2 * kSmallRows);
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      if (wid + 4 * s >= nu) continue;
      const int ca = 32 * ba[s] + (lane & 31), cb = 32 * bb[s] + (lane & 31);
#pragma unroll
      for (int kk = 0; kk < kSmallRows; kk += 2) {
        const int k = kk + (lane >> 5);
        acc[s] = mfma32(Xs[k * kSmallPitch + ca], Xs[k * kSmallPitch + cb], acc[s]);
      }
    }
  };
  float va[kPer], vb[kPer];
  load(va, 0);
  if (nch > 1) load(vb, kSmallRows);
  for (int ch = 0; ch < nch; ch += 2) {
    step(va, ch);
    if (ch + 1 < nch) step(vb, ch + 1);
  }
  // F <- beta F + alpha acc on the upper triangle
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    if (wid + 4 * s >= nu) continue;
    const int col = 32 * bb[s] + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * ba[s] + acc_row(r, lane);
      if (row > col || col >= d) continue;
      const float x = rd ? beta * o[s][r] + alpha * acc[s][r] : alpha * acc[s][r];
      if (packed) {
        F[packed_index(row, col, d)] = x;
      } else {
        F[static_cast<int64_t>(row) * d + col] = x;
        if (row != col) F[static_cast<int64_t>(col) * d + row] = x;
      }
    }
  }
}

kfac_status_t factors_phase(const kfac_layer_t* layers, int n, const kfac_hparams_t& hp, const FullPlan& P,
                            hipStream_t st) {
  const float eps = hp.ema_decay;
  // every factor fp32, of a linear layer and at most 128 wide: one workgroup per factor
  bool small = n > 0;
  for (int li = 0; li < n && small; ++li) {
    const LayerGeom g = geom_of(layers[li]);
    small = !g.conv && g.d_a <= kNb && g.d_out <= kNb && g.rows <= kSmallMaxRows &&
            fp32_factor(layers[li], 0) && fp32_factor(layers[li], 1);
  }
  if (small) {
    SmallSyrkTab T{};
    for (int li = 0; li < n; ++li) {
      const kfac_layer_t& L = layers[li];
      const LayerGeom g = geom_of(L);
      for (int which = 0; which < 2; ++which) {
        if (T.n == kMaxSmallSyrk) {
          hipLaunchKernelGGL(syrk_small_kernel, dim3(T.n), dim3(256), 0, st, T);
          KFAC_HIP_TRY(hipGetLastError());
          T.n = 0;
        }
        SmallSyrk& q = T.s[T.n++];
        q.X = static_cast<const float*>(which == 0 ? L.a : L.g);
        q.F = which == 0 ? L.A : L.G;
        q.rows = static_cast<int32_t>(g.rows);
        q.w = which == 0 ? g.d_in : g.d_out;
        q.bias = which == 0 && g.bias ? 1 : 0;
        q.packed = g.packed ? 1 : 0;
        q.alpha = (1.0f - eps) / static_cast<float>(g.rows);
        q.beta = eps;
      }
    }
    if (T.n > 0) {
      hipLaunchKernelGGL(syrk_small_kernel, dim3(T.n), dim3(256), 0, st, T);
      KFAC_HIP_TRY(hipGetLastError());
    }
    return KFAC_OK;
  }
  std::vector<GemmProb> probs;
  std::vector<SymRedItem> reds;
  std::vector<SyrkBf16Prob> bf16;
  std::vector<ColItem> cols;
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
        q.packed = g.packed ? 1 : 0;
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
      if (!g.conv) {
        p.lda = p.ldb = which == 0 ? g.d_in : g.d_out;
      } else if (nchw_factor(L, which)) {
        p.lda = p.ldb = which == 0 ? g.h * g.w : g.h_out * g.w_out;
        p.nchw = 1;
      } else {
        // the convolution tensor as rows first (im2col of the input; the
        // output gradient transposed), then the same SYRK as a linear layer's
        const int f = 2 * li + which;
        ColItem c{};
        c.x = static_cast<const float*>(X);
        c.X = P.xcol[f];
        if (which == 0) {
          c.C = g.c_in; c.H = g.h; c.W = g.w; c.k = g.kh; c.stride = g.stride; c.pad = g.pad;
          c.d_in = g.d_in;
        } else {
          c.C = g.d_out; c.H = g.h_out; c.W = g.w_out; c.k = 1; c.stride = 1; c.pad = 0;
          c.d_in = g.d_out;
        }
        c.Ho = g.h_out; c.Wo = g.w_out;
        c.ld = P.xcol_ld[f];
        c.rows = static_cast<int32_t>(g.rows);
        cols.push_back(c);
        p.A = p.B = P.xcol[f];
        p.lda = p.ldb = P.xcol_ld[f];
      }
      const int s = P.nsplit[2 * li + which];
      p.ldc = d;
      p.nsplit = s;
      if (s == 1) {
        p.C = F;
        p.alpha = alpha;
        p.beta = eps;
        p.c_packed = g.packed ? 1 : 0;
        probs.push_back(p);
      } else {
        p.C = P.part[2 * li + which];
        p.split_stride = static_cast<int64_t>(d) * d;
        p.alpha = 1.0f;
        probs.push_back(p);
        SymRedItem r{};
        r.part = p.C;
        r.F = F;
        r.d = d;
        r.nsplit = s;
        r.alpha = alpha;
        r.beta = eps;
        r.packed = g.packed ? 1 : 0;
        reds.push_back(r);
      }
    }
  }
  GemmScalars sc{};
  kfac_status_t r;
  if (!cols.empty()) {
    r = launch_im2col(cols, st);
    if (r != KFAC_OK) return r;
  }
  if (!probs.empty()) {
    r = launch_gemm(probs, OP_MN, OP_MN, EPI_SYRK, sc, st, TILES_SMALL);
    if (r != KFAC_OK) return r;
  }
  if (!bf16.empty()) {
    r = launch_syrk_bf16(bf16, st);
    if (r != KFAC_OK) return r;
  }
  return reds.empty() ? KFAC_OK : launch_sym_reduce(reds, st);
}

// The library's side streams for one caller stream on one device: the
// Cholesky chain (s) and the inverse assembly beside it (f), with their
// events, at default priority, created at the first full step on that caller
// stream and kept for the process.  Keying them by the caller's stream keeps
// a step captured into a graph from pulling another stream's work into the
// capture: the capture reaches only the side streams of the captured stream,
// while steps on other streams (other host threads) run on their own.  A
// whole step is enqueued under the set's lock, so that every event wait names
// the record of the same call even when several host threads share a caller
// stream.
struct SideStream {
  std::mutex mu;
  hipStream_t s = nullptr;   // Cholesky inner chain
  hipStream_t f = nullptr;   // inverse assembly, as far as the chain allows
  hipEvent_t fork = nullptr, join = nullptr, fjoin = nullptr, main_done[2] = {nullptr, nullptr},
             side_done[2] = {nullptr, nullptr}, ufork = nullptr, ujoin = nullptr;
};

kfac_status_t side_streams_for(hipStream_t caller, SideStream** out) {
  static std::mutex mu;
  static std::map<std::pair<int, uintptr_t>, std::unique_ptr<SideStream>> sets;
  int dev = 0;
  KFAC_HIP_TRY(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(mu);
  std::unique_ptr<SideStream>& slot = sets[{dev, reinterpret_cast<uintptr_t>(caller)}];
  if (!slot) {
    // streams and events are not created inside an open capture: the first
    // full step on a stream has to run outside one
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
      sets.erase({dev, reinterpret_cast<uintptr_t>(caller)});
      return KFAC_ERR_UNSUPPORTED;
    }
    auto S = std::make_unique<SideStream>();
    bool ok = hipStreamCreateWithFlags(&S->s, hipStreamNonBlocking) == hipSuccess &&
              hipStreamCreateWithFlags(&S->f, hipStreamNonBlocking) == hipSuccess;
    hipEvent_t* evs[9] = {&S->fork,          &S->join,          &S->fjoin, &S->main_done[0], &S->main_done[1],
                          &S->side_done[0], &S->side_done[1], &S->ufork, &S->ujoin};
    for (hipEvent_t* e : evs) ok = ok && hipEventCreateWithFlags(e, hipEventDisableTiming) == hipSuccess;
    if (!ok) {
      for (hipEvent_t* e : evs)
        if (*e) (void)hipEventDestroy(*e);
      if (S->s) (void)hipStreamDestroy(S->s);
      if (S->f) (void)hipStreamDestroy(S->f);
      sets.erase({dev, reinterpret_cast<uintptr_t>(caller)});
      return KFAC_ERR_HIP;
    }
    slot = std::move(S);
  }
  *out = slot.get();
  return KFAC_OK;
}

kfac_status_t invert_phase(const kfac_hparams_t& hp, const FullPlan& P, uint32_t* flags, hipStream_t st,
                           SideStream* side) {
  const std::vector<Mat>& mats = P.mats;
  // the factors this step inverts: A (even entries) and / or G (odd entries)
  std::vector<char> on(mats.size());
  for (size_t mi = 0; mi < mats.size(); ++mi)
    on[mi] = (hp.refresh & (mi % 2 == 0 ? KFAC_REFRESH_A : KFAC_REFRESH_G)) != 0;
  int nblk_max = 0, d_max = 0;
  for (size_t mi = 0; mi < mats.size(); ++mi) {
    if (!on[mi]) continue;
    nblk_max = std::max<int>(nblk_max, static_cast<int>(nblk_of(mats[mi].d)));
    d_max = std::max(d_max, mats[mi].d);
  }
  if (nblk_max == 0) return KFAC_OK;
  // runs of equal-size factors of this step whose work areas lie at a
  // constant stride (a plan group with some members left out splits into runs)
  std::vector<FullPlan::Group> groups;
  for (const FullPlan::Group& g : P.groups) {
    FullPlan::Group run{-1, 0, g.stride, {}};
    for (int mi : g.members) {
      if (on[mi]) {
        if (run.count == 0) run.first = mi;
        run.members.push_back(mi);
        ++run.count;
      } else if (run.count > 0) {
        groups.push_back(run);
        run = FullPlan::Group{-1, 0, g.stride, {}};
      }
    }
    if (run.count > 0) groups.push_back(run);
  }
  GemmScalars sc{};
  // runs `fn` on the matrices of this step selected by `pred`, kMaxMats at a time
  auto tables = [&](auto pred, int k, auto fn) -> kfac_status_t {
    MatTab T{};
    T.damping = hp.damping;
    T.flags = flags;
    T.k = k;
    for (size_t mi = 0; mi < mats.size(); ++mi) {
      const Mat& m = mats[mi];
      if (!on[mi] || !pred(m)) continue;
      T.m[T.n++] = m;
      if (T.n == kMaxMats) {
        kfac_status_t r = fn(T);
        if (r != KFAC_OK) return r;
        T.n = 0;
      }
    }
    return T.n > 0 ? fn(T) : KFAC_OK;
  };
  // L = F + damping I (part 0: all of it; 1: the first outer panel's
  // columns; 2: the rest)
  auto init = [&](int part) {
    return tables([](const Mat&) { return true; }, part, [&](MatTab& T) {
      hipLaunchKernelGGL(chol_init_kernel, dim3(2048, T.n), dim3(256), 0, st, T);
      return hipGetLastError() == hipSuccess ? KFAC_OK : KFAC_ERR_HIP;
    });
  };
  kfac_status_t r;
  // Blocked right-looking Cholesky in two levels.  Inner step k factors
  // diagonal block k (chol_diag) and forms the panel L_ik = M_ik Dinv_k^T
  // below it.  Blocks are grouped kOuter at a time into outer panels; the
  // inner steps of an outer panel apply their rank-128 updates only to the
  // panel's own remaining columns (U_in), and the rest of the trailing matrix
  // takes the whole outer panel at once, a 512-deep product instead of four
  // 128-deep ones.  That far update is split: the columns of the next outer
  // panel (F_next) run on a second stream ahead of that panel's inner steps,
  // the remainder (F_rest) on the caller's stream beside them, so the
  // latency-bound inner chain overlaps the large update.  F_next(K) waits for
  // F_rest(K - 1) (both subtract into outer panel K + 1); F_rest(K) waits for
  // the last panel of outer panel K.  Events alternate between two per
  // direction so that each wait names the right step; the second stream forks
  // from and joins the caller's stream, which keeps the whole step
  // capturable in a graph.
  hipStream_t ss = side->s;
  // the chain's products raise their wavefronts' issue priority: they share CUs
  // with the assembly's products and are the latency-bound path (ResNet-50's
  // inverse 8.91 -> 8.79 ms)
  GemmScalars scp = sc;
  scp.prio = 1;
  auto diag_step = [&](int k, hipStream_t ds) -> kfac_status_t {
    DiagTab D{};
    D.k = k;
    D.flags = flags;
    for (size_t mi = 0; mi <= mats.size(); ++mi) {
      if (mi == mats.size() || D.n == kMaxDiagMats) {
        if (D.n > 0) {
          hipLaunchKernelGGL(chol_diag_kernel, dim3(D.n), dim3(256), 0, ds, D);
          KFAC_HIP_TRY(hipGetLastError());
        }
        D.n = 0;
        if (mi == mats.size()) break;
      }
      const Mat& m = mats[mi];
      if (!on[mi] || static_cast<int>(nblk_of(m.d)) <= k) continue;
      D.m[D.n++] = DMat{m.L, m.Z, m.Dinv, m.fail, m.d, 0};
    }
    return KFAC_OK;
  };
  // panel k, and the update of column block c (c = k + 1) or of everything
  // from column block k + 2 on (c < 0)
  auto panel_of = [&](const Mat& m, int k) {
    const int d = m.d, r1 = (k + 1) * kNb;
    GemmProb p{};
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
    return p;
  };
  // lower part of the trailing matrix from row and column r0 on, ncols
  // columns wide, minus the product of L's columns c .. c + depth with their
  // own transpose (rows r0..)
  auto update_of = [&](const Mat& m, int r0, int ncols, int c, int depth, uint8_t tri) {
    const int d = m.d;
    GemmProb q{};
    q.A = m.L + static_cast<int64_t>(r0) * d + c;   // L_ik, rows r0..
    q.lda = d;
    q.B = q.A;                                      // L_jk^T
    q.ldb = d;
    q.C = m.L + static_cast<int64_t>(r0) * d + r0;
    q.ldc = d;
    q.M = d - r0;
    q.N = ncols;
    q.kb = 0;
    q.ke = depth;
    q.tri = tri;
    q.a_special = q.b_special = -1;
    q.alpha = 1.f;
    q.nsplit = 1;
    gemm_set_tiles(q);
    return q;
  };
  // one problem for a run of equal-size factors (their work areas lie at a
  // constant stride)
  auto batched = [](GemmProb p, const FullPlan::Group& g) {
    if (g.count > 1) {
      p.nbatch = static_cast<int16_t>(g.count);
      p.split_stride = g.stride;
    }
    return p;
  };
  // panel k (side stream) for every matrix with a block below k
  auto panel_step = [&](int k) -> kfac_status_t {
    std::vector<GemmProb> v;
    for (const FullPlan::Group& g : groups)
      if (static_cast<int>(nblk_of(mats[g.first].d)) > k + 1) v.push_back(batched(panel_of(mats[g.first], k), g));
    return v.empty() ? KFAC_OK : launch_gemm(v, OP_K, OP_K, EPI_STORE, scp, ss);
  };
  // The inverse of each factor is assembled on stream fs as far as its
  // Cholesky factor allows: after outer panel K, rows and columns below
  // R = 512 (K + 1) of L are final (later steps touch only rows and columns
  // from R on), so every part of Z = L^-1 and of Z^T Z that needs nothing
  // beyond them can run beside the remaining steps.
  //
  // Z = L^-1 by recursive doubling.  The diagonal 128-blocks of Z are the
  // inverted diagonal blocks; at level s (128, 256, ...) each pair of
  // neighbouring inverted s-blocks of a matrix, Z11 at (c0, c0) and Z22 at
  // (r0, r0) with r0 = c0 + s, gives the block between them:
  //   Z21 = -Z22 (L21 Z11)   (L21 = rows r0.., columns c0.. of L).
  // T^T = Z11^T L21^T is staged in L's strict upper triangle at (c0, r0),
  // which no step of the Cholesky reads or writes.  Z11 is lower triangular,
  // so a tile of T^T needs rows k >= its first row of Z11; Z22 is lower
  // triangular, so a tile of Z21 needs k up to its last row.  A pair needs
  // L up to its end min(r0 + s, d): the pairs of a level become ready in
  // order, and the ready ones not yet done form one strided problem (all
  // three operands move by 2 s (d + 1) floats from pair to pair; the last,
  // shorter pair is a problem of its own).  Levels run in increasing s, so a
  // pair's own lower levels are done first.
  //
  // inverse = Z^T Z into W.  Z is lower triangular, so element (i, j) sums
  // over rows k >= max(i, j).  Rows below P = 128 * 2^m <= R of Z are
  // complete once R is reached (every pair that writes into them ends by P),
  // so, when the total Z^T Z work is small against d_max, W takes Z's rows
  // kLauRows at a time as they complete (no workgroup then runs the whole
  // height, and the passes run beside the Cholesky); otherwise it takes all
  // rows in one pass once the factor is complete (a pass of few rows would
  // read and write the whole triangle for little work).
  // Finally sym_reduce_kernel writes W's upper triangle, mirrored, into the
  // inverse unless the factorisation failed.
  struct Progress {
    std::vector<int> pairs;   // per level: pairs done
    int rows = 0;             // rows of Z already in W
    bool out = false;         // the inverse has been written
  };
  std::vector<Progress> prog(groups.size());
  double lau_flops = 0.0;
  int d_all = 0;
  for (const FullPlan::Group& g : groups) {
    const int d = mats[g.first].d;
    lau_flops += static_cast<double>(g.count) * d * d * d / 3.0;
    d_all = std::max(d_all, d);
  }
  const bool by_rows = lau_flops < 67108864.0 * d_all;
  // end of the next Z^T Z pass of a factor of size d whose rows below `done`
  // are in W, once L is final below R (done itself when there is none)
  auto lau_next = [&](int done, int R, int d) -> int {
    if (done >= d) return done;
    if (R >= d) return by_rows ? std::min(d, done + kLauRows) : d;
    if (!by_rows) return done;                   // one pass once the factor is complete
    int P2 = 0;                                  // rows of Z complete: 128 * 2^m <= R
    for (int q = kNb; q <= R; q *= 2) P2 = q;
    return done + kLauRows <= P2 ? done + kLauRows : done;
  };
  auto assemble = [&](int R, hipStream_t fs) -> kfac_status_t {
    // every level's newly ready pairs, matrix by matrix
    for (int s = kNb, lv = 0; s < d_all; s *= 2, ++lv) {
      std::vector<GemmProb> g1, g2;
      for (size_t gi = 0; gi < groups.size(); ++gi) {
        const FullPlan::Group& g = groups[gi];
        const int d = mats[g.first].d;
        if (d <= s || R <= 0) continue;
        Progress& pr = prog[gi];
        if (static_cast<int>(pr.pairs.size()) <= lv) pr.pairs.resize(lv + 1, 0);
        const int Rm = std::min(R, d);
        const int npairs = (d - s + 2 * s - 1) / (2 * s);       // pairs with r0 = 2 p s + s < d
        int ready = 0;
        while (ready < npairs && std::min((2 * ready + 2) * s, d) <= Rm) ++ready;
        const int nfull = (d - 2 * s) >= 0 ? (d - 2 * s) / (2 * s) + 1 : 0;   // pairs with r0 + s <= d
        const int p_lo = pr.pairs[lv];
        if (ready <= p_lo) continue;
        pr.pairs[lv] = ready;
        for (int mi : g.members) {
          const Mat& m = mats[mi];
          for (int part = 0; part < 2; ++part) {
            const int p0 = part == 0 ? p_lo : std::max(p_lo, nfull);
            const int p1 = part == 0 ? std::min(ready, nfull) : ready;
            const int cnt = p1 - p0;
            if (cnt <= 0) continue;
            const int c0 = 2 * p0 * s, r0 = c0 + s;
            const int m2 = part == 0 ? s : d - r0;
            GemmProb p{};
            p.A = m.Z + static_cast<int64_t>(c0) * d + c0;        // Z11, read as A[i][k] = Z11[k][i]
            p.lda = d;
            p.B = m.L + static_cast<int64_t>(r0) * d + c0;        // L21, read as B[k][j] = L21[j][k]
            p.ldb = d;
            p.C = m.L + static_cast<int64_t>(c0) * d + r0;        // T^T (s x m2) in L's upper triangle
            p.ldc = d;
            p.M = s;
            p.N = m2;
            p.kb = 0;
            p.ke = s;
            p.tri = TRI_FULL;
            p.krange = KR_FROM_ROW;
            p.a_special = p.b_special = -1;
            p.alpha = 1.f;
            p.nsplit = 1;
            p.nbatch = static_cast<int16_t>(cnt);
            p.split_stride = static_cast<int64_t>(2 * s) * (d + 1);
            gemm_set_tiles(p);
            g1.push_back(p);
            GemmProb q = p;
            q.A = m.Z + static_cast<int64_t>(r0) * d + r0;        // Z22
            q.B = m.L + static_cast<int64_t>(c0) * d + r0;        // T[k][j] = T^T[j][k]
            q.C = m.Z + static_cast<int64_t>(r0) * d + c0;        // Z21
            q.M = m2;
            q.N = s;
            q.ke = m2;
            q.krange = KR_TO_ROW;
            q.alpha = -1.f;
            gemm_set_tiles(q);
            g2.push_back(q);
          }
        }
      }
      if (g1.empty()) continue;
      kfac_status_t r = launch_gemm(g1, OP_MN, OP_K, EPI_STORE, sc, fs);
      if (r != KFAC_OK) return r;
      r = launch_gemm(g2, OP_K, OP_K, EPI_STORE, sc, fs);
      if (r != KFAC_OK) return r;
    }
    // Z^T Z passes over the rows of Z that are complete (the first stores,
    // later ones add); factors of different groups share the launches
    for (;;) {
      std::vector<GemmProb> first, later;
      for (size_t gi = 0; gi < groups.size(); ++gi) {
        const FullPlan::Group& g = groups[gi];
        const Mat& m = mats[g.first];
        const int d = m.d;
        Progress& pr = prog[gi];
        const int k1 = lau_next(pr.rows, R, d);
        if (k1 <= pr.rows) continue;
        GemmProb p{};
        p.A = m.Z;
        p.B = m.Z;
        p.lda = p.ldb = d;
        p.C = P.W[g.first];
        p.ldc = d;
        // the first pass stores every tile of W (zero where its rows add
        // nothing); a later pass adds only into the leading k1 x k1 block
        p.M = p.N = pr.rows == 0 ? d : k1;
        p.kb = pr.rows;
        p.ke = k1;
        p.tri = TRI_UPPER;
        p.krange = KR_FROM_DIAG;
        p.a_special = p.b_special = -1;
        p.nsplit = 1;
        p.alpha = pr.rows == 0 ? 1.f : -1.f;
        gemm_set_tiles(p);
        (pr.rows == 0 ? first : later).push_back(batched(p, g));
        pr.rows = k1;
      }
      if (first.empty() && later.empty()) break;
      // (128 x 128 tiles for the passes of kLauRows rows: they run beside the
      // Cholesky chain, whose kernels need room on the CUs)
      const int policy = by_rows ? TILES_SMALL : TILES_AUTO;
      kfac_status_t r = first.empty() ? KFAC_OK : launch_gemm(first, OP_MN, OP_MN, EPI_STORE, sc, fs, policy);
      if (r == KFAC_OK && !later.empty()) r = launch_gemm(later, OP_MN, OP_MN, EPI_SUB, sc, fs, policy);
      if (r != KFAC_OK) return r;
    }
    // output of the factors complete at R (not yet written)
    std::vector<SymRedItem> out;
    for (size_t gi = 0; gi < groups.size(); ++gi) {
      const FullPlan::Group& g = groups[gi];
      const int d = mats[g.first].d;
      if (R < d || prog[gi].out) continue;
      prog[gi].out = true;
      for (int mi : g.members) {
        SymRedItem it{};
        it.part = P.W[mi];
        it.F = mats[mi].Finv;
        it.fail = mats[mi].fail;
        it.d = d;
        it.nsplit = 1;
        it.alpha = 1.f;
        it.beta = 0.f;
        out.push_back(it);
      }
    }
    return out.empty() ? KFAC_OK : launch_sym_reduce(out, fs);
  };
  if (nblk_max == 1) {
    // every factor is one diagonal block: one launch per kMaxMats factors
    // reads, factors, inverts and writes them (no chain, no fork, no events)
    return tables([](const Mat&) { return true; }, 0, [&](MatTab& T) {
      hipLaunchKernelGGL(chol_small_kernel, dim3(T.n), dim3(256), 0, st, T);
      return hipGetLastError() == hipSuccess ? KFAC_OK : KFAC_ERR_HIP;
    });
  }
  hipStream_t fs = side->f;
  // the chain starts once the first outer panel is initialised; the rest of
  // L (and Z's band) follows on the caller's stream beside it, ahead of the
  // first far update there (main_done[1] for the first F_next and the
  // assembly)
  r = init(1);
  if (r != KFAC_OK) return r;
  KFAC_HIP_TRY(hipEventRecord(side->fork, st));
  const int nouter = (nblk_max + kOuter - 1) / kOuter;
  // everything between the fork and the join; an error inside still reaches
  // the join below, so the caller's stream never runs ahead of work already
  // enqueued on the side streams (and an open capture stays joined)
  auto chain = [&]() -> kfac_status_t {
  KFAC_HIP_TRY(hipStreamWaitEvent(ss, side->fork, 0));
  KFAC_HIP_TRY(hipStreamWaitEvent(fs, side->fork, 0));
  kfac_status_t r = init(2);
  if (r != KFAC_OK) return r;
  KFAC_HIP_TRY(hipEventRecord(side->main_done[1], st));
  KFAC_HIP_TRY(hipStreamWaitEvent(fs, side->main_done[1], 0));   // Z's band, before any assembly
  for (int K = 0; K < nouter; ++K) {
    const int k0 = K * kOuter, k1 = k0 + kOuter;   // blocks of outer panel K
    // second stream: F_next(K - 1) after F_rest(K - 2), then the inner steps
    if (K > 0) {
      // (K = 1: the initialisation of the rest; later: F_rest(K - 2))
      KFAC_HIP_TRY(hipStreamWaitEvent(ss, side->main_done[K & 1], 0));
      std::vector<GemmProb> fn;
      for (const FullPlan::Group& g : groups) {
        const Mat& m = mats[g.first];
        if (static_cast<int>(nblk_of(m.d)) > k0) {
          const int r0 = k0 * kNb;
          fn.push_back(batched(
              update_of(m, r0, std::min(k1 * kNb, m.d) - r0, (k0 - kOuter) * kNb, kOuter * kNb, TRI_FULL), g));
        }
      }
      if (!fn.empty()) {
        r = launch_gemm(fn, OP_K, OP_K, EPI_SUB, scp, ss);
        if (r != KFAC_OK) return r;
      }
    }
    for (int k = k0; k < k1 && k < nblk_max; ++k) {
      r = diag_step(k, ss);
      if (r != KFAC_OK) return r;
      r = panel_step(k);
      if (r != KFAC_OK) return r;
      if (k + 1 < k1) {
        std::vector<GemmProb> ui;
        for (const FullPlan::Group& g : groups) {
          const Mat& m = mats[g.first];
          if (static_cast<int>(nblk_of(m.d)) > k + 1) {
            const int r0 = (k + 1) * kNb;
            ui.push_back(batched(update_of(m, r0, std::min(k1 * kNb, m.d) - r0, k * kNb, kNb, TRI_FULL), g));
          }
        }
        if (!ui.empty()) {
          r = launch_gemm(ui, OP_K, OP_K, EPI_SUB, scp, ss);
          if (r != KFAC_OK) return r;
        }
      }
    }
    KFAC_HIP_TRY(hipEventRecord(side->side_done[K & 1], ss));
    // caller's stream: F_rest(K), after the last panel of outer panel K
    std::vector<GemmProb> fr;
    for (const FullPlan::Group& g : groups) {
      const Mat& m = mats[g.first];
      if (static_cast<int>(nblk_of(m.d)) > k1 + kOuter) {
        const int r0 = (k1 + kOuter) * kNb;
        fr.push_back(batched(update_of(m, r0, m.d - r0, k0 * kNb, kOuter * kNb, TRI_LOWER), g));
      }
    }
    KFAC_HIP_TRY(hipStreamWaitEvent(st, side->side_done[K & 1], 0));
    if (!fr.empty()) {
      r = launch_gemm(fr, OP_K, OP_K, EPI_SUB, sc, st);
      if (r != KFAC_OK) return r;
    }
    KFAC_HIP_TRY(hipEventRecord(side->main_done[K & 1], st));
    // rows and columns of L below 512 (K + 1) are final: the inverse
    // assembly of every factor still in progress goes as far as they allow,
    // on a third stream beside the remaining steps, every second outer panel
    // (fewer, larger launches: that stream is the last to finish, and its
    // small launches cost their latency whatever their size)
    bool active = false;
    for (const FullPlan::Group& g : groups) active = active || static_cast<int>(nblk_of(mats[g.first].d)) > k0;
    if (active && (K % 2 == 1 || K == nouter - 1)) {
      KFAC_HIP_TRY(hipStreamWaitEvent(fs, side->side_done[K & 1], 0));
      r = assemble(k1 * kNb, fs);
      if (r != KFAC_OK) return r;
    }
  }
  return KFAC_OK;
  };
  r = chain();
  // join: everything on the side streams before anything after it here
  const bool joined = hipEventRecord(side->join, ss) == hipSuccess && hipStreamWaitEvent(st, side->join, 0) == hipSuccess &&
                      hipEventRecord(side->fjoin, fs) == hipSuccess && hipStreamWaitEvent(st, side->fjoin, 0) == hipSuccess;
  if (r != KFAC_OK) return r;
  return joined ? KFAC_OK : KFAC_ERR_HIP;
}

// Preconditioning and update of layers with d_out <= 128 and d_a <= 128, one
// workgroup per layer: [grad_w | grad_b] and A_inv into LDS together, T =
// their product on MFMA (kept in LDS), G_inv in, P = G_inv T on MFMA, then the
// update of the GEMM path's fused epilogue (D = P + wd W; V = mu V + D;
// W -= lr V, the bias column included; a non-finite result raises
// KFAC_FLAG_NONFINITE).  Used when every layer of the step is that small: the
// two GEMM launches would otherwise each run a serial chain of stages per
// layer.  Both LDS arrays are zero outside the matrices, so the 32-blocks
// that straddle d_out or d_a contract over zeros.
constexpr int kMaxSmallUpd = 40;
struct SmallUpd {
  const float* gw;     // grad_w [d_out][d_in]
  const float* gb;     // grad_b [d_out], null without a bias
  const float* Ainv;   // [d_a][d_a]
  const float* Ginv;   // [d_out][d_out]
  float* W;
  float* b;
  float* V;
  float* Vb;
  int32_t d_out, d_in;
};
struct SmallUpdTab {
  SmallUpd u[kMaxSmallUpd];
  int32_t n;
  float lr, momentum, weight_decay;
  uint32_t* flags;
};
static_assert(sizeof(SmallUpdTab) <= 4096, "kernel arguments");

__global__ void __launch_bounds__(256) precond_small_kernel(SmallUpdTab T) {
  __shared__ __attribute__((aligned(16))) float X[kNb * kLd];   // [grad_w | grad_b], then T
  __shared__ __attribute__((aligned(16))) float Y[kNb * kLd];   // A_inv, then G_inv
  const SmallUpd& U = T.u[blockIdx.x];
  const int mo = U.d_out, di = U.d_in, da = di + (U.gb != nullptr ? 1 : 0);
  if (mo <= 0 || da <= 0) return;   // (uniform: nothing to update)
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nbi = (mo + 31) / 32, nbj = (da + 31) / 32;
  for (int e = tid; e < kNb * kLd; e += 256) {
    X[e] = 0.f;
    Y[e] = 0.f;
  }
  __syncthreads();
  // [grad_w | grad_b] (mo x da) and A_inv (da x da), 32 loads in flight per thread
  const int n1 = mo * da, n12 = n1 + da * da;
  for (int e0 = 0; e0 < n12; e0 += 32 * 256) {
    float v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int e = e0 + u * 256 + tid;
      const int f = e < n1 ? e : e - n1;
      const int r = f / da, c = f - r * da;
      const float* src = e < n1 ? (c < di ? U.gw + static_cast<int64_t>(r) * di + c : U.gb + r) : U.Ainv + f;
      v[u] = e < n12 ? *src : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int e = e0 + u * 256 + tid;
      const int f = e < n1 ? e : e - n1;
      const int r = f / da, c = f - r * da;
      if (e < n12) (e < n1 ? X : Y)[r * kLd + c] = v[u];
    }
  }
  __syncthreads();
  // T = [grad_w | grad_b] A_inv: (mo x da) blocks, at most 16, 4 per wavefront
  const int nt = nbi * nbj;
  f32x16 acc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int t = wid + 4 * s;
    acc[s] = f32x16{};
    if (t >= nt) continue;
    const int i = t / nbj, j = t - (t / nbj) * nbj;
    for (int kb = 0; kb < nbj; ++kb) mma_nn(acc[s], X, 32 * i, 32 * kb, Y, kLd, 32 * kb, 32 * j, lane);
  }
  __syncthreads();   // every read of X and Y done
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int t = wid + 4 * s;
    if (t >= nt) continue;
    const int i = t / nbj, j = t - (t / nbj) * nbj;
    tile_store(X, kLd, 32 * i, 32 * j, acc[s], 1.f, lane);
  }
  // G_inv over the blocks that P reads (rows and columns below 32 nbi; zero
  // beyond mo, where A_inv's entries were)
  const int gw = 32 * nbi, ng = gw * gw;
  for (int e0 = 0; e0 < ng; e0 += 32 * 256) {
    float v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int e = e0 + u * 256 + tid;
      const int r = e / gw, c = e - r * gw;
      v[u] = (e < ng && r < mo && c < mo) ? U.Ginv[r * mo + c] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int e = e0 + u * 256 + tid;
      const int r = e / gw, c = e - r * gw;
      if (e < ng) Y[r * kLd + c] = v[u];
    }
  }
  __syncthreads();
  // P = G_inv T, then the update, block by block (reads of a block issued together)
  bool bad = false;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int t = wid + 4 * s;
    if (t >= nt) continue;
    const int i = t / nbj, j = t - (t / nbj) * nbj;
    f32x16 pacc = {};
    for (int kb = 0; kb < nbi; ++kb) mma_nn(pacc, Y, 32 * i, 32 * kb, X, kLd, 32 * kb, 32 * j, lane);
    const int col = 32 * j + (lane & 31);
    float w0[16], v0[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * i + acc_row(r, lane);
      const bool in = row < mo && col < da;
      const int64_t e = static_cast<int64_t>(row) * di + col;
      // (outside the layer: the first weight, or the first bias when d_in = 0)
      const bool wsel = in ? col < di : di > 0;
      const int64_t off = in ? (col < di ? e : row) : 0;
      w0[r] = (wsel ? U.W : U.b)[off];
      v0[r] = (wsel ? U.V : U.Vb)[off];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * i + acc_row(r, lane);
      if (row >= mo || col >= da) continue;
      const float d = fmaf(T.weight_decay, w0[r], pacc[r]);
      const float vn = fmaf(T.momentum, v0[r], d);
      const float wn = fmaf(-T.lr, vn, w0[r]);
      if (col < di) {
        U.V[static_cast<int64_t>(row) * di + col] = vn;
        U.W[static_cast<int64_t>(row) * di + col] = wn;
      } else {
        U.Vb[row] = vn;
        U.b[row] = wn;
      }
      bad |= !(isfinite(vn) && isfinite(wn));
    }
  }
  if (__any(bad) && lane == 0) raise_flag(T.flags, KFAC_FLAG_NONFINITE);
}

kfac_status_t update_phase(const kfac_layer_t* layers, int n, const kfac_hparams_t& hp, const FullPlan& P,
                           uint32_t* flags, hipStream_t st, SideStream* side) {
  // every layer within one 128 x 128 block: one workgroup per layer
  bool small = n > 0;
  for (int li = 0; li < n && small; ++li) {
    const LayerGeom g = geom_of(layers[li]);
    small = g.d_out <= kNb && g.d_a <= kNb;
  }
  if (small) {
    SmallUpdTab T{};
    T.lr = hp.lr;
    T.momentum = hp.momentum;
    T.weight_decay = hp.weight_decay;
    T.flags = flags;
    for (int li = 0; li <= n; ++li) {
      if (li == n || T.n == kMaxSmallUpd) {
        if (T.n > 0) {
          hipLaunchKernelGGL(precond_small_kernel, dim3(T.n), dim3(256), 0, st, T);
          KFAC_HIP_TRY(hipGetLastError());
        }
        T.n = 0;
        if (li == n) break;
      }
      const kfac_layer_t& L = layers[li];
      const LayerGeom g = geom_of(L);
      SmallUpd& u = T.u[T.n++];
      u.gw = L.grad_w;
      u.gb = g.bias ? L.grad_b : nullptr;
      u.Ainv = L.A_inv;
      u.Ginv = L.G_inv;
      u.W = L.w;
      u.b = L.b;
      u.V = L.mom_w;
      u.Vb = L.mom_b;
      u.d_out = g.d_out;
      u.d_in = g.d_in;
    }
    return KFAC_OK;
  }
  std::vector<GemmProb> g1, g2;
  std::vector<BcProb> b0, b1;
  auto aligned16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  for (int li = 0; li < n; ++li) {
    const kfac_layer_t& L = layers[li];
    const LayerGeom g = geom_of(L);
    const bool split = bias_column_split(g);
    const int ncols = split ? g.d_in : g.d_a;   // columns the GEMMs produce
    if (split) {
      BcProb s0{};
      s0.M = static_cast<const float*>(L.grad_w);
      s0.extra = L.grad_b;
      s0.x = L.A_inv + static_cast<int64_t>(g.d_in) * g.d_a;
      s0.y = P.tb[li];
      s0.rows = g.d_out;
      s0.ld = g.d_in;
      s0.kmain = g.d_in;
      s0.vec = g.d_in % 4 == 0 && aligned16(s0.M) && aligned16(s0.x);
      b0.push_back(s0);
      BcProb s1{};
      s1.M = L.G_inv;
      s1.x = P.tb[li];
      s1.b = L.b;
      s1.mb = L.mom_b;
      s1.rows = g.d_out;
      s1.ld = g.d_out;
      s1.kmain = g.d_out;
      s1.vec = g.d_out % 4 == 0 && aligned16(s1.M) && aligned16(s1.x);
      b1.push_back(s1);
    }
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
    p.ldc = t_ld(g.d_a);
    p.M = g.d_out;
    p.N = ncols;
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
    q.ldb = t_ld(g.d_a);
    q.b_special = -1;
    q.M = g.d_out;
    q.N = ncols;
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
  GemmScalars sc{hp.lr, hp.momentum, hp.weight_decay, 0, flags};
  // The bias-column products (HBM-bound) run on the side stream beside the
  // two GEMMs (MFMA-bound): they read what the GEMMs read and write only t,
  // b and mom_b, which the GEMMs do not touch.
  const bool fork = !b0.empty();
  if (fork) KFAC_HIP_TRY(hipEventRecord(side->ufork, st));
  kfac_status_t r = KFAC_OK;
  if (fork) {
    if (hipStreamWaitEvent(side->s, side->ufork, 0) != hipSuccess) r = KFAC_ERR_HIP;
    if (r == KFAC_OK) r = launch_bias_col(b0, 0, hp, flags, side->s);
    if (r == KFAC_OK) r = launch_bias_col(b1, 1, hp, flags, side->s);
  }
  if (r == KFAC_OK) r = launch_gemm(g1, OP_K, OP_MN, EPI_STORE, sc, st);
  if (r == KFAC_OK) r = launch_gemm(g2, OP_MN, OP_MN, EPI_UPDATE, sc, st);
  // the join is enqueued after an error too (see invert_phase)
  if (fork && (hipEventRecord(side->ujoin, side->s) != hipSuccess || hipStreamWaitEvent(st, side->ujoin, 0) != hipSuccess))
    return r != KFAC_OK ? r : KFAC_ERR_HIP;
  return r;
}

}  // namespace

namespace {

// conv / linear layers take the Kronecker-factored path; batch-norm layers
// (a diagonal Fisher, Osawa et al. sections 1 and 5.4) the diagonal one
void split_layers(const kfac_layer_t* layers, int n, std::vector<kfac_layer_t>& kf, std::vector<kfac_layer_t>& bn) {
  for (int i = 0; i < n; ++i) (layers[i].kind == KFAC_BATCHNORM ? bn : kf).push_back(layers[i]);
}

// the batch-norm layers' diagonal workspace follows the Kronecker-factored plan
size_t bn_region_bytes(const std::vector<kfac_layer_t>& bn) {
  return bn.empty() ? 0 : diag_workspace_bytes(bn.data(), static_cast<int>(bn.size())) - kFlagBytes;
}

}  // namespace

size_t full_workspace_bytes(const kfac_layer_t* layers, int n) {
  std::vector<kfac_layer_t> kf, bn;
  split_layers(layers, n, kf, bn);
  return plan_full(kf.data(), static_cast<int>(kf.size()), nullptr, KFAC_PHASE_ALL, true).ws_bytes +
         bn_region_bytes(bn);
}

kfac_status_t full_enqueue(const kfac_layer_t* layers, int n, const kfac_hparams_t& hp, char* ws, size_t ws_bytes,
                           hipStream_t st, int phases) {
  std::vector<kfac_layer_t> kf, bn;
  split_layers(layers, n, kf, bn);
  const int nk = static_cast<int>(kf.size());
  FullPlan P = plan_full(kf.data(), nk, ws, phases, hp.refresh != 0);
  if (P.ws_bytes + bn_region_bytes(bn) > ws_bytes) return KFAC_ERR_WORKSPACE;
  uint32_t* flags = reinterpret_cast<uint32_t*>(ws);
  kfac_status_t r = KFAC_OK;
  if (nk > 0) {
    SideStream* side = nullptr;
    r = side_streams_for(st, &side);
    if (r != KFAC_OK) return r;
    std::lock_guard<std::mutex> lock(side->mu);
    if (phases & KFAC_PHASE_FACTORS) {
      r = factors_phase(kf.data(), nk, hp, P, st);
      if (r != KFAC_OK) return r;
    }
    if ((phases & KFAC_PHASE_INVERT) && hp.refresh) {
      r = invert_phase(hp, P, flags, st, side);
      if (r != KFAC_OK) return r;
    }
    if (phases & KFAC_PHASE_UPDATE) {
      r = update_phase(kf.data(), nk, hp, P, flags, st, side);
      if (r != KFAC_OK) return r;
    }
    if ((phases & KFAC_PHASE_RESCALE) && (hp.options & KFAC_OPT_RESCALE)) {
      r = launch_rescale(P.rescale, hp.rescale_eps, st);
      if (r != KFAC_OK) return r;
    }
  }
  if (!bn.empty() && (phases & (KFAC_PHASE_FACTORS | KFAC_PHASE_UPDATE))) {
    // carved from kFlagBytes past its base: right after the plan's regions
    char* base = ws + P.ws_bytes - kFlagBytes;
    r = diag_enqueue_into(bn.data(), static_cast<int>(bn.size()), hp, base, bn_region_bytes(bn) + kFlagBytes, flags,
                          st, phases & (KFAC_PHASE_FACTORS | KFAC_PHASE_UPDATE));
  }
  return r;
}

}  // namespace kfac
