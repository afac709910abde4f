// Batched fp32 MFMA GEMM used by every dense contraction of the full K-FAC
// step (factor SYRK, preconditioning, blocked Cholesky inverse).
#pragma once

#include <vector>

#include "common.h"

namespace kfac {

constexpr int kTile = 128;     // output tile (both dimensions)
constexpr int kMaxGemmProbs = 27;   // problem table of one launch (kernel arguments stay within 4 KB)

// Operand layouts.  For A (M x K): OP_MN stores element (i, k) at
// A[k * lda + i] (i contiguous), OP_K at A[i * lda + k] (k contiguous).
// For B (K x N): OP_MN stores (k, j) at B[k * ldb + j], OP_K at B[j * ldb + k].
enum GemmOp : int { OP_MN = 0, OP_K = 1 };

// Epilogues.
enum GemmEpi : int {
  EPI_STORE = 0,      // C = alpha * acc
  EPI_SUB = 1,        // C -= alpha * acc
  EPI_UPDATE = 2,     // P = acc; D = P + wd W; V = mu V + D; W -= lr V  (columns >= d_in go to b / mom_b)
  EPI_SYRK = 3,       // upper tiles; nsplit == 1: C = beta * C + alpha * acc (C not read when beta == 0),
                      // mirrored to the lower triangle (packed C: upper entries only);
                      // else C + split * split_stride = alpha * acc
};

// Tile grids.
enum GemmTri : int { TRI_FULL = 0, TRI_UPPER = 1, TRI_LOWER = 2 };

// Contraction range of one tile (i0, j0 = its first row and column).
enum GemmKRange : int {
  KR_ALL = 0,        // [kb, ke)
  KR_FROM_DIAG = 1,  // from max(i0, j0): A[i][k] = 0 for k < i and B[k][j] = 0 for k < j
  KR_FROM_ROW = 2,   // from i0: A[i][k] = 0 for k < i
  KR_TO_ROW = 3,     // up to i0 + tile: A[i][k] = 0 for k > i
};

struct GemmProb {
  const void* A;
  const void* B;
  float* C;
  const float* A_extra;   // OP_K A: column `a_special` of A is A_extra[i]
  float* W;               // EPI_UPDATE targets
  float* Wb;
  float* V;
  float* Vb;
  int64_t split_stride;   // nsplit > 1: C offset between K splits; nbatch > 1: A, B and C offset between entries (floats)
  int32_t lda, ldb, ldc;
  int32_t M, N;
  int32_t kb, ke;         // contraction range [kb, ke)
  int32_t tiles_m, tiles_n;
  int32_t a_special;      // OP_MN: element i == a_special is 1.0 (bias column); OP_K: see A_extra; -1 none
  int32_t b_special;      // OP_MN: element j == b_special is 1.0; -1 none
  int32_t d_in;           // EPI_UPDATE: columns < d_in go to W / V
  int32_t nsplit;         // K splits (each writes C + s * split_stride)
  int32_t blk_begin;
  int16_t nbatch;         // identical problems at A, B, C + b * split_stride (b < nbatch; nsplit must be 1)
  uint8_t tri;            // GemmTri
  uint8_t krange;         // GemmKRange
  uint8_t a_vec, b_vec;   // set by the launcher: 16-byte loads allowed (ld % 4 == 0, aligned base)
  uint8_t c_packed;       // EPI_SYRK with nsplit == 1: C is a packed upper triangle of an M x M matrix
  uint8_t nchw;           // EPI_SYRK with A == B: X is a convolution tensor [K / lda][M][lda] read in
                          // place (row k of X: pixel k % lda of image k / lda); see gemm_nchw_syrk_ok
  float alpha, beta;
};

struct GemmScalars {
  float lr, momentum, weight_decay;
  int32_t prio;   // nonzero: the launch's wavefronts raise their issue priority
  uint32_t* flags;
};

// Whether the factor SYRK can read X = the convolution tensor [rows / hw][d][hw]
// at `X` in place (as rows of d pixels values, GemmProb::nchw) instead of as
// materialised rows.
bool gemm_nchw_syrk_ok(const void* X, int64_t rows, int hw, int d);

// Number of workgroups one problem needs.
int gemm_blocks(const GemmProb& p);

// Fills tiles_m / tiles_n from M / N.
void gemm_set_tiles(GemmProb& p);

// Tile-size policy of a launch: AUTO picks 256 x 256 tiles for the whole
// launch when it has at least two such tiles per CU; PER_PROBLEM gives
// problems with both sides >= kBigMin the 256 x 256 tiles and the rest
// 128 x 128 tiles (two launches); SMALL uses 128 x 128 tiles throughout.
enum TilePolicy : int { TILES_AUTO = 0, TILES_PER_PROBLEM = 1, TILES_SMALL = 2 };
constexpr int kBigMin = 384;

// Launches the problems (any count; grouped internally) with operand layouts
// (amode, bmode) and epilogue `epi` on `stream`.  Problems must be
// independent: within a launch they are ordered by the contraction length of
// one workgroup, longest first, and spread over launches of similar work.
kfac_status_t launch_gemm(std::vector<GemmProb>& probs, int amode, int bmode, int epi, const GemmScalars& sc,
                          hipStream_t stream, int policy = TILES_AUTO);

}  // namespace kfac
