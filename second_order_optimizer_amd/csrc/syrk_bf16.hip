// Factor SYRK for bfloat16 inputs on CDNA4 bf16 matrix cores.
//
// C[i][j] = sum_n X[n][i] X[n][j] over upper 128 x 128 tiles.  256 threads
// (4 wavefronts, 2 x 2), each wavefront a 64 x 64 quarter as 2 x 2
// v_mfma_f32_32x32x16_bf16 blocks.  K (the row index n) advances 32 per
// stage.  The MFMA wants, per lane, 8 consecutive k of one column, so the
// slab is stored in LDS column-major ([m][k], k contiguous): each thread
// reads a 4 (rows) x 8 (columns) bf16 block with four 16-byte loads and
// writes it transposed as eight 8-byte LDS stores.  Threads 0-127 stage the
// row-tile operand, 128-255 the column-tile operand.
#include "syrk_bf16.h"

#include <algorithm>

namespace kfac {

namespace {

constexpr int kT = 128;        // output tile
constexpr int kK = 32;         // rows of X per stage
constexpr int kRow = kK + 8;   // LDS row (bf16 elements) of one column, padded
constexpr unsigned short kOne = 0x3F80;   // bf16 1.0

struct SyrkArgs {
  const uint16_t* X;
  float* C;
  int64_t split_stride;
  int64_t rows;
  int32_t width, d, special, tiles, nsplit, ldc;
  float alpha, beta;
};

template <bool VEC>
__device__ inline void load_block(u16x8 (&v)[4], const uint16_t* __restrict__ X, int64_t rows, int width,
                                  int special, int64_t k, int m) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t r = k + q;
    u16x8 x;
    if (VEC && r < rows && m + 8 <= width) {
      x = *reinterpret_cast<const u16x8*>(X + r * width + m);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        unsigned short s = 0;
        if (r < rows && m + e < width) s = X[r * width + m + e];
        x[e] = s;
      }
    }
    if (special >= m && special < m + 8 && r < rows) x[special - m] = kOne;
    v[q] = x;
  }
}

__device__ inline void store_block(unsigned short* __restrict__ s, const u16x8 (&v)[4], int kk, int mm) {
  // element (k = kk + q, m = mm + e) -> s[(mm + e) * kRow + kk + q]
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    u16x4 c = {v[0][e], v[1][e], v[2][e], v[3][e]};
    *reinterpret_cast<u16x4*>(s + (mm + e) * kRow + kk) = c;
  }
}

template <bool VEC, bool SPLIT>
__global__ void __launch_bounds__(256) syrk_bf16_kernel(SyrkArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned short sX[2][2][kT * kRow];
  const int per = a.tiles * (a.tiles + 1) / 2;
  int t = blockIdx.x;
  const int split = t / per;
  t -= split * per;
  int ti = 0;
  while (t >= a.tiles - ti) { t -= a.tiles - ti; ++ti; }
  const int tj = ti + t;
  const int i0 = ti * kT, j0 = tj * kT;
  int64_t kb = 0, ke = a.rows;
  if (SPLIT) {
    const int64_t len = ((a.rows + a.nsplit - 1) / a.nsplit + kK - 1) / kK * kK;
    kb = split * len;
    ke = min(a.rows, kb + len);
  }
  float* C = a.C + (SPLIT ? split * a.split_stride : 0);

  const int tid = threadIdx.x;
  const int half = tid >> 7;               // 0: row-tile operand, 1: column-tile operand
  const int lt = tid & 127;
  const int kk = (lt >> 4) * 4;            // 8 k-quads
  const int mm = (lt & 15) * 8;            // 16 m-octets
  const int m_base = half ? j0 : i0;

  const int lane = tid & 63, wid = tid >> 6;
  const int wm = (wid >> 1) * 64, wn = (wid & 1) * 64;

  f32x16 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;

  u16x8 v[4];
  int buf = 0;
  if (kb < ke) {
    load_block<VEC>(v, a.X, ke, a.width, a.special, kb + kk, m_base + mm);
    store_block(sX[0][half], v, kk, mm);
  }
  __syncthreads();
  for (int64_t k0 = kb; k0 < ke; k0 += kK) {
    const bool more = k0 + kK < ke;
    if (more) load_block<VEC>(v, a.X, ke, a.width, a.special, k0 + kK + kk, m_base + mm);
    const unsigned short* sa = sX[buf][0];
    const unsigned short* sb = sX[buf][1];
#pragma unroll
    for (int ks = 0; ks < kK; ks += 16) {
      const int ko = ks + 8 * (lane >> 5);
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(sa + (wm + (lane & 31)) * kRow + ko);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(sa + (wm + 32 + (lane & 31)) * kRow + ko);
      const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(sb + (wn + (lane & 31)) * kRow + ko);
      const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(sb + (wn + 32 + (lane & 31)) * kRow + ko);
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
    }
    if (more) store_block(sX[buf ^ 1][half], v, kk, mm);
    __syncthreads();
    buf ^= 1;
  }

#pragma unroll
  for (int si = 0; si < 2; ++si) {
#pragma unroll
    for (int sj = 0; sj < 2; ++sj) {
      const int col = j0 + wn + 32 * sj + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i0 + wm + 32 * si + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= a.d || col >= a.d || row > col) continue;
        const int64_t idx = static_cast<int64_t>(row) * a.ldc + col;
        const float val = acc[si][sj][r];
        if (SPLIT) {
          C[idx] = val;
        } else {
          const float o = a.beta * C[idx] + a.alpha * val;
          C[idx] = o;
          if (row != col) C[static_cast<int64_t>(col) * a.ldc + row] = o;
        }
      }
    }
  }
}

}  // namespace

kfac_status_t launch_syrk_bf16(const uint16_t* X, int width, int64_t rows, int d, int special, float* C,
                               float alpha, float beta, int nsplit, int64_t split_stride, hipStream_t st) {
  SyrkArgs a{};
  a.X = X;
  a.C = C;
  a.split_stride = split_stride;
  a.rows = rows;
  a.width = width;
  a.d = d;
  a.special = special;
  a.tiles = (d + kT - 1) / kT;
  a.nsplit = std::max(1, nsplit);
  a.ldc = d;
  a.alpha = alpha;
  a.beta = beta;
  const int blocks = a.tiles * (a.tiles + 1) / 2 * a.nsplit;
  const bool vec = (width % 8) == 0 && (reinterpret_cast<uintptr_t>(X) % 16) == 0;
  if (a.nsplit > 1) {
    if (vec) hipLaunchKernelGGL((syrk_bf16_kernel<true, true>), dim3(blocks), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((syrk_bf16_kernel<false, true>), dim3(blocks), dim3(256), 0, st, a);
  } else {
    if (vec) hipLaunchKernelGGL((syrk_bf16_kernel<true, false>), dim3(blocks), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((syrk_bf16_kernel<false, false>), dim3(blocks), dim3(256), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? KFAC_OK : KFAC_ERR_HIP;
}

}  // namespace kfac
