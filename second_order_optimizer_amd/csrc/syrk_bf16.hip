// Factor SYRK for bfloat16 inputs on CDNA4 bf16 matrix cores, batched over
// all bf16 factors of the stack.
//
// F <- beta F + alpha X^T X over upper 256 x 256 tiles, X = [rows, width]
// row-major bf16.  512 threads (8 wavefronts, 2 x 4); each wavefront owns a
// 128 x 64 part as 4 x 2 v_mfma_f32_32x32x16_bf16 blocks (128 accumulators
// per lane; two wavefronts per SIMD).  Each stage consumes 64 rows of X.  The MFMA wants 8 consecutive rows of one column per lane, so a
// slab is kept in LDS column-major ([m][k], k contiguous, rows padded to 144
// bytes, which makes both the 16-byte stores and the 16-byte MFMA operand
// reads bank-conflict free): each thread reads an 8 x 8 bf16 block with
// eight 16-byte loads (the next stage's, issued before this stage's MFMAs)
// and writes it transposed with eight 16-byte LDS stores; threads 0-255
// stage the row-tile operand, 256-511 the column-tile operand.  Diagonal
// tiles stage one operand and skip their strictly-lower region.  With a bias
// the constant-1 column is not materialised: the two otherwise idle
// wavefronts of each diagonal tile multiply the slab by a ones operand,
// which yields the column sums of X (the factor's last row and column).
#include "syrk_bf16.h"

#include <algorithm>

namespace kfac {

namespace {

constexpr int kBT = 256;        // block tile
constexpr int kBK = 64;         // rows of X per stage
constexpr int kLR = kBK + 8;    // LDS column length in bf16 (144 bytes)
constexpr int kMaxProbs = 56;
constexpr int kXcdRun = 16;           // tiles per XCD run (xcd_tile)
constexpr int kBand = 4;              // tile rows per band (band_tile)
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

struct Prob {
  const uint16_t* X;
  float* F;
  int64_t rows;
  int32_t width, bias, ldf, tiles, blk_begin, packed;   // packed: F is the packed upper triangle
  float alpha, beta;
};

// position of F's element (row, col), row <= col
__device__ inline int64_t f_index(const Prob& P, int row, int col) {
  return P.packed ? packed_index(row, col, P.ldf) : static_cast<int64_t>(row) * P.ldf + col;
}
struct Batch {
  Prob p[kMaxProbs];
  int32_t n;
  int32_t xcd_run;   // > 1: runs of this many consecutive tiles per XCD (see xcd_tile)
  int32_t band;      // > 0: tiles ordered in bands of this many tile rows (see band_tile)
};
static_assert(sizeof(Batch) <= 4096, "kernel arguments");

// Workgroups go to the 8 XCDs round-robin (workgroup w on XCD w % 8), so
// consecutive tiles would each load their panels of X into a different XCD's
// L2.  With runs of R, XCD x takes logical tiles [x R, x R + R) of every
// group of 8 R (the groups advance together, keeping the launch's order); a
// final partial group keeps the identity.  Together with the band order
// below (bands of 4 tile rows), the R = 16 tiles an XCD runs together form a
// 4 x 4 block of a factor's tile grid: 4 row panels and 4 column panels of X
// instead of 1 and 16.  Measured factor phases (random inputs): transformer
// stack 7.32 -> 7.24 ms, 16k pair 9.15 -> 8.87 ms.
__device__ inline int xcd_tile(int w, int n, int R) {
  if (R <= 1) return w;
  const int base = n / (8 * R) * (8 * R);
  if (w >= base) return w;
  return (w / 8 / R) * (8 * R) + (w % 8) * R + (w / 8) % R;
}

// Upper tile t of a T x T tile grid in band order: bands of H tile rows;
// inside a band, column after column, the band's rows of each column.  A
// run of consecutive tiles then spans a few row panels and a few column
// panels of X (a 2-D block of the grid) instead of one row panel and many
// column panels.
__device__ inline void band_tile(int t, int T, int H, int& ti, int& tj) {
  int r0 = 0;
  for (;;) {
    const int h = min(H, T - r0);
    const int tri = h * (h + 1) / 2;
    const int n = tri + (T - r0 - h) * h;
    if (t < n) {
      if (t < tri) {
        int u = 0;
        while ((u + 1) * (u + 2) / 2 <= t) ++u;
        tj = r0 + u;
        ti = r0 + t - u * (u + 1) / 2;
      } else {
        const int q = t - tri;
        tj = r0 + h + q / h;
        ti = r0 + q % h;
      }
      return;
    }
    t -= n;
    r0 += h;
  }
}

// A problem entry read once from the kernel arguments and kept in scalar
// registers (see arg_reg).
__device__ inline Prob prob_regs(const Prob& P) {
  Prob q;
  q.X = arg_reg(P.X);
  q.F = arg_reg(P.F);
  q.rows = arg_reg(P.rows);
  q.width = arg_reg(P.width);
  q.bias = arg_reg(P.bias);
  q.ldf = arg_reg(P.ldf);
  q.tiles = arg_reg(P.tiles);
  q.blk_begin = arg_reg(P.blk_begin);
  q.packed = arg_reg(P.packed);
  q.alpha = arg_reg(P.alpha);
  q.beta = arg_reg(P.beta);
  return q;
}

__device__ inline int find_prob(const Batch& b, int blk) {
  int lo = 0, hi = b.n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (b.p[mid].blk_begin <= blk) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// rows k .. k+7 of columns m .. m+7 (zero outside X)
__device__ inline void load8(u16x8 (&v)[8], const uint16_t* __restrict__ X, int64_t rows, int width, int64_t k,
                             int m) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int64_t row = k + r;
    u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
    if (row < rows) {
      const uint16_t* p = X + row * width + m;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (m + e < width) x[e] = p[e];
    }
    v[r] = x;
  }
}

// element (k = kc*8 + r, m = mo*8 + e) -> s[(mo*8 + e) * kLR + kc*8 + r]
__device__ inline void store_t(unsigned short* __restrict__ s, const u16x8 (&v)[8], int mo, int kc) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    u16x8 w;
#pragma unroll
    for (int r = 0; r < 8; ++r) w[r] = v[r][e];
    *reinterpret_cast<u16x8*>(s + (mo * 8 + e) * kLR + kc * 8) = w;
  }
}

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
syrk_bf16_kernel(Batch batch) {
  __shared__ __attribute__((aligned(16))) unsigned short sX[2][2][kBT * kLR];
  const Prob P = prob_regs(batch.p[find_prob(batch, blockIdx.x)]);
  int t = blockIdx.x - P.blk_begin;
  int ti = 0;
  while (t >= P.tiles - ti) { t -= P.tiles - ti; ++ti; }
  const int tj = ti + t;
  const bool diag = ti == tj;
  const int i0 = ti * kBT, j0 = tj * kBT;
  const int tid = threadIdx.x;
  const int half = tid >> 8;                      // operand this thread stages
  const int kc = tid & 7, mo = (tid & 255) >> 3;
  const bool stager = !(diag && half == 1);       // a diagonal tile has one operand
  const int lane = tid & 63, wid = tid >> 6;
  const int wm = (wid >> 2) * 128, wn = (wid & 3) * 64;
  // In a diagonal tile the wavefronts over the strictly-lower region (rows
  // 128.., columns ..127) have no output; with a bias they compute the column
  // sums of the tile's columns instead (wave 4: columns 0..127, wave 5:
  // 128..255, as acc[i][0]).
  const bool work = !(diag && wm > wn + 63);
  const bool colsum = P.bias && diag && !work;
  const int cs0 = (wid & 1) * 128;
  const int width = P.width;
  const int64_t rows = P.rows;
  const uint16_t* X = P.X;
  const int mcol = (half ? j0 : i0) + mo * 8;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.0f);

  u16x8 v[8];
  const int64_t nst = (rows + kBK - 1) / kBK;
  if (stager) {
    load8(v, X, rows, width, kc * 8, mcol);
    store_t(sX[0][half], v, mo, kc);
  }
  __syncthreads();
  int buf = 0;
  for (int64_t s = 0; s < nst; ++s) {
    const bool more = s + 1 < nst;
    if (more && stager) load8(v, X, rows, width, (s + 1) * kBK + kc * 8, mcol);
    const unsigned short* sa = sX[buf][0];
    const unsigned short* sb = diag ? sa : sX[buf][1];
    if (work) {
      // fragments of k-step ks + 16 are read while the MFMAs of ks run
      bf16x8 fa[2][4], fb[2][2];
      auto frag = [&](int ks, bf16x8 (&a)[4], bf16x8 (&b)[2]) {
        const int ko = ks + 8 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a[i] = *reinterpret_cast<const bf16x8*>(sa + (wm + 32 * i + (lane & 31)) * kLR + ko);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          b[j] = *reinterpret_cast<const bf16x8*>(sb + (wn + 32 * j + (lane & 31)) * kLR + ko);
      };
      frag(0, fa[0], fb[0]);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 6, 0);
#pragma unroll
      for (int ks = 0; ks < kBK; ks += 16) {
        const int cur = (ks >> 4) & 1;
        if (ks + 16 < kBK) frag(ks + 16, fa[cur ^ 1], fb[cur ^ 1]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
        // keep the next reads ahead of this k-step's MFMAs
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 6, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 8, 0);
      }
    } else if (colsum) {
#pragma unroll
      for (int ks = 0; ks < kBK; ks += 16) {
        const int ko = ks + 8 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8 x = *reinterpret_cast<const bf16x8*>(sa + (cs0 + 32 * i + (lane & 31)) * kLR + ko);
          acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, ones, acc[i][0], 0, 0, 0);
        }
      }
    }
    if (more && stager) store_t(sX[buf ^ 1][half], v, mo, kc);
    __syncthreads();
    buf ^= 1;
  }

  // accumulator r of block (i, j): row i0 + wm + 32 i + 8 (r/4) + 4 (lane/32) + r%4,
  // column j0 + wn + 32 j + lane%32
  float* F = P.F;
  const int ldf = P.ldf;
  if (work) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = j0 + wn + 32 * j + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row >= width || col >= width || row > col) continue;
          const int64_t idx = f_index(P, row, col);
          const float o = P.beta * F[idx] + P.alpha * acc[i][j][r];
          F[idx] = o;
          if (row != col && !P.packed) F[static_cast<int64_t>(col) * ldf + row] = o;
        }
      }
    }
  }
  if (colsum && (lane & 31) == 0) {
    // every column of a ones-product block holds the same column sums of X
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = i0 + cs0 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m >= width) continue;
        const int64_t idx = f_index(P, m, width);
        const float o = P.beta * F[idx] + P.alpha * acc[i][0][r];
        F[idx] = o;
        if (!P.packed) F[static_cast<int64_t>(width) * ldf + m] = o;
      }
    }
    if (ti == 0 && cs0 == 0 && lane == 0) {
      const int64_t c = f_index(P, width, width);
      F[c] = P.beta * F[c] + P.alpha * static_cast<float>(rows);
    }
  }
}

// ---------------------------------------------------------------------------
// The same SYRK for rows of a multiple of 8 elements (16-byte aligned), with
// CDNA4's direct-to-LDS loads and transposing LDS reads.  X is staged
// row-major, 32 rows per stage, in a 4-stage LDS ring filled by
// buffer_load_dwordx4 ... lds (no registers; rows past the end read as zero
// through the buffer's range check).  Stages go in pairs: one wait and one
// barrier cover two stages, whose MFMAs run while the next pair loads into
// the other half of the 4-slot ring; inside a pair the fragments of each
// 16-row half-step are read while the MFMAs of the previous one run.  An MFMA operand wants 8 consecutive rows of one column per lane:
// two ds_read_b64_tr_b16 give it from the row-major tile (within 16 lanes,
// lane i receives column c + i of the 4 rows the group addresses).  Each
// row's 16-byte chunks are XOR-swizzled by 4 (row mod 4): the 4 rows of a
// transposing read then fall in distinct 64-byte windows of the 256-byte
// bank cycle (no bank conflicts, by the SQ_LDS_BANK_CONFLICT counter).  The workgroup
// barrier carries no memory fence (a fence is not needed for LDS the
// loads write directly); each wavefront waits for its own loads of the pair
// (vmcnt) before the barrier instead.

constexpr int kRBK = 32;                  // rows of X per stage
constexpr int kNS = 4;                    // stages in the LDS ring
constexpr int kOpElems = kRBK * kBT;      // one operand of one stage (bf16 elements, 16 KB)

// XOR swizzle of a row's 16-byte chunks
__device__ inline int kSwz(int row) { return (row & 3) << 2; }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

__device__ inline bf16x8 tr_frag(const unsigned short* base, int off0, int off1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + off0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + off1));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// element offset of this lane's first transposing read for the MFMA block
// whose 32 columns start at cb0 (multiple of 32), k-step base ks (0 or 16);
// the second read is 4 rows further (same swizzle: ks and 8 (g / 2) are
// multiples of 8)
__device__ inline int tr_off(int cb0, int ks, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int row = ks + 8 * (g >> 1) + (s >> 2);
  const int chunk = (cb0 >> 3) + 2 * (g & 1) + ((s & 3) >> 1);
  const int phys = chunk ^ kSwz(row);
  return row * kBT + phys * 8 + 4 * (s & 1);
}

// s_waitcnt with only the vector-memory counter limited to n (n < 16)
#define KFAC_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8))

// PACKED: F holds the packed upper triangle (a separate instantiation, so
// that the whole-storage epilogue keeps its registers).
template <bool PACKED>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
syrk_bf16_dma_kernel(Batch batch) {
  __shared__ __attribute__((aligned(16))) unsigned short ring[kNS][2][kOpElems];
  const int blk = xcd_tile(blockIdx.x, gridDim.x, batch.xcd_run);
  const Prob P = prob_regs(batch.p[find_prob(batch, blk)]);
  int t = blk - P.blk_begin;
  int ti = 0, tj;
  if (batch.band > 0) {
    band_tile(t, P.tiles, batch.band, ti, tj);
  } else {
    while (t >= P.tiles - ti) { t -= P.tiles - ti; ++ti; }
    tj = ti + t;
  }
  const bool diag = ti == tj;
  const int i0 = ti * kBT, j0 = tj * kBT;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int wm = (wid >> 2) * 128, wn = (wid & 3) * 64;
  const bool work = !(diag && wm > wn + 63);
  const bool colsum = P.bias && diag && !work;
  const int cs0 = (wid & 1) * 128;
  const int width = P.width;
  const int64_t rows = P.rows;
  const int nops = diag ? 1 : 2;
  // buffer resource: base, stride 0, num_records = the bytes of X (reads
  // past them return 0), raw 32-bit data
  const uint64_t xa = reinterpret_cast<uint64_t>(P.X);
  const i32x4 rsrc = {static_cast<int>(xa & 0xffffffffu), static_cast<int>((xa >> 32) & 0xffffu),
                      static_cast<int>(rows * width * 2), 0x00020000};

  // this lane's chunk of each load: chunk p of the operand-stage buffer holds
  // row p / 32, logical 16-byte chunk (p % 32) ^ 2 (row % 4)
  uint32_t ld_off[2][2];
#pragma unroll
  for (int op = 0; op < 2; ++op)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int p = (wid * 2 + u) * 64 + lane;
      const int k = p >> 5, c = (p & 31) ^ kSwz(k);
      ld_off[op][u] = static_cast<uint32_t>((static_cast<int64_t>(k) * width + (op ? j0 : i0) + 8 * c) * 2);
    }
  const uint32_t stage_bytes = static_cast<uint32_t>(kRBK) * width * 2;
  const int64_t nst = (rows + kRBK - 1) / kRBK;
  // loads of stage s into its ring slot: 16 bytes per lane straight into LDS
  // at M0 + 16 lane.  Issued as assembly so that the compiler does not wait
  // for them before every LDS read (it cannot tell ring slots apart); the
  // vmcnt waits and the barrier below order them instead.
  // stages are consumed in pairs; an odd count gets one more stage past the
  // end of X, which the range check fills with zeros
  const int64_t nst2 = (nst + 1) & ~int64_t(1);
  auto issue = [&](int64_t s) {
    if (s >= nst2) return;
    const int slot = static_cast<int>(s % kNS);
    const uint32_t so = static_cast<uint32_t>(s) * stage_bytes;
#pragma unroll
    for (int op = 0; op < 2; ++op) {
      if (op >= nops) break;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
            (__attribute__((address_space(3))) void*)(&ring[slot][op][(wid * 2 + u) * 512])));
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :
                     : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(so + ld_off[op][u]), "s"(rsrc)
                     : "memory", "m0");
      }
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.0f);

  // per-lane operand offsets (element offsets inside an operand-stage buffer)
  int oa[2][4], ob[2][2], oc[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      oa[h][i] = tr_off(wm + 32 * i, 16 * h, lane);
      oc[h][i] = tr_off(cs0 + 32 * i, 16 * h, lane);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) ob[h][j] = tr_off(wn + 32 * j, 16 * h, lane);
  }

  // two stages per barrier: stages s, s + 1 (slots s % 4, s % 4 + 1) are
  // waited for together; the slots of s - 2, s - 1 are then refilled with
  // s + 2, s + 3
  issue(0);
  issue(1);
  for (int64_t s = 0; s < nst2; s += 2) {
    KFAC_WAIT_VM(0);
    __builtin_amdgcn_s_barrier();
    issue(s + 2);
    issue(s + 3);
    const int slot0 = static_cast<int>(s & 3);
    if (work) {
      // four half-steps t (stage s + t / 2, k half t % 2); the fragments of
      // t + 1 are read while the MFMAs of t run
      auto frags = [&](int t, bf16x8 (&fa)[4], bf16x8 (&fb)[2]) {
        const unsigned short* sa = ring[slot0 + (t >> 1)][0];
        const unsigned short* sb = diag ? sa : ring[slot0 + (t >> 1)][1];
        const int h = t & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = tr_frag(sa, oa[h][i], oa[h][i] + 4 * kBT);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[j] = tr_frag(sb, ob[h][j], ob[h][j] + 4 * kBT);
      };
      bf16x8 fa[2][4], fb[2][2];
      frags(0, fa[0], fb[0]);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 12, 0);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int cur = t & 1;
        if (t < 3) frags(t + 1, fa[cur ^ 1], fb[cur ^ 1]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
        if (t < 3) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
          }
        } else {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 8, 0);
        }
      }
    } else if (colsum) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const unsigned short* sa = ring[slot0 + (t >> 1)][0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8 x = tr_frag(sa, oc[t & 1][i], oc[t & 1][i] + 4 * kBT);
          acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, ones, acc[i][0], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  }

  // accumulator r of block (i, j): row i0 + wm + 32 i + 8 (r/4) + 4 (lane/32) + r%4,
  // column j0 + wn + 32 j + lane%32.  Per 32 x 32 block: the 16 reads of F
  // issue together, the EMA result goes to the upper triangle row-wise and,
  // transposed through a 32 x 33 LDS staging tile of this wavefront (the ring
  // is idle once every wavefront has left the loop), to the lower triangle
  // in 128-byte row pieces.
  float* F = P.F;
  const int ldf = P.ldf;
  __syncthreads();
  float* stg = reinterpret_cast<float*>(&ring[0][0][0]) + wid * (32 * 33);
  if (work) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r0 = i0 + wm + 32 * i, c0 = j0 + wn + 32 * j;
        if (r0 > c0 + 31 || r0 >= width || c0 >= width) continue;   // no upper element in the block
        const int col = c0 + (lane & 31);
        // unconditional loads (an element outside the upper triangle reads the
        // block's first element, which is inside it) keep them in one batch
        float o[16];
        if constexpr (PACKED) {
          // packed row starts relative to this lane's first row rb: element
          // (rb + k, col) lies at B(rb) + k (ldf - 1) - k (2 rb + k - 1) / 2 + col,
          // with B(i) = i (ldf - 1) - i (i - 1) / 2 (one 64-bit base per lane,
          // 32-bit offsets)
          const int rb = r0 + 4 * (lane >> 5);
          float* Fb = F + (static_cast<int64_t>(rb) * (ldf - 1) - static_cast<int64_t>(rb) * (rb - 1) / 2);
          const int fb0 = static_cast<int>(packed_index(r0, c0, ldf) - (static_cast<int64_t>(rb) * (ldf - 1) -
                                                                         static_cast<int64_t>(rb) * (rb - 1) / 2));
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int k = 8 * (r >> 2) + (r & 3);
            const int row = rb + k;
            const bool in = row < width && col < width && row <= col;
            o[r] = Fb[in ? k * (ldf - 1) - k * (2 * rb + k - 1) / 2 + col : fb0];
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int k = 8 * (r >> 2) + (r & 3);
            const int row = rb + k;
            const bool in = row < width && col < width && row <= col;
            const float v = P.beta * o[r] + P.alpha * acc[i][j][r];
            if (in) Fb[k * (ldf - 1) - k * (2 * rb + k - 1) / 2 + col] = v;
          }
          continue;   // the upper triangle is all a packed factor holds
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = r0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const bool in = row < width && col < width && row <= col;
          o[r] = F[in ? static_cast<int64_t>(row) * ldf + col : static_cast<int64_t>(r0) * ldf + c0];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int row = r0 + rr;
          const bool in = row < width && col < width && row <= col;
          const float v = P.beta * o[r] + P.alpha * acc[i][j][r];
          if (in) F[static_cast<int64_t>(row) * ldf + col] = v;
          stg[(lane & 31) * 33 + rr] = v;
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int cc = 2 * q + (lane >> 5), rr = lane & 31;
          const int row = r0 + rr, mcol = c0 + cc;
          if (row < mcol && mcol < width) F[static_cast<int64_t>(mcol) * ldf + row] = stg[cc * 33 + rr];
        }
      }
    }
  }
  if (colsum && (lane & 31) == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = i0 + cs0 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m >= width) continue;
        const int64_t idx = PACKED ? packed_index(m, width, ldf) : static_cast<int64_t>(m) * ldf + width;
        const float o = P.beta * F[idx] + P.alpha * acc[i][0][r];
        F[idx] = o;
        if (!PACKED) F[static_cast<int64_t>(width) * ldf + m] = o;
      }
    }
    if (ti == 0 && cs0 == 0 && lane == 0) {
      const int64_t c = PACKED ? packed_index(width, width, ldf) : static_cast<int64_t>(width) * ldf + width;
      F[c] = P.beta * F[c] + P.alpha * static_cast<float>(rows);
    }
  }
}

}  // namespace

kfac_status_t launch_syrk_bf16(const std::vector<SyrkBf16Prob>& probs, hipStream_t st) {
  // Rows whose width is a multiple of 8 (16-byte aligned) go to the
  // direct-to-LDS kernel, in row chunks whose byte offsets fit its 32-bit
  // buffer range (chunk 0 applies the EMA, later chunks add: beta = 1);
  // chunks of one factor run in successive launches.  Other widths go to the
  // register-staged kernel with scalar loads.
  struct Piece {
    Prob p;
    int pass;
  };
  std::vector<Piece> dma, dma_packed, ragged;   // one kernel instantiation per launch
  for (const SyrkBf16Prob& q : probs) {
    Prob p{};
    p.X = q.X;
    p.F = q.F;
    p.rows = q.rows;
    p.width = q.width;
    p.bias = q.bias;
    p.ldf = q.width + (q.bias ? 1 : 0);
    p.tiles = (q.width + kBT - 1) / kBT;
    p.alpha = q.alpha;
    p.beta = q.beta;
    p.packed = q.packed;
    const bool aligned = (q.width % 8) == 0 && (reinterpret_cast<uintptr_t>(q.X) % 16) == 0;
    if (!aligned) {
      ragged.push_back({p, 0});
      continue;
    }
    const int64_t limit = ((int64_t(1) << 31) - 1) / (static_cast<int64_t>(q.width) * 2) - 2 * kRBK;
    const int64_t chunk = std::max<int64_t>(kRBK, limit / kRBK * kRBK);
    int pass = 0;
    for (int64_t r0 = 0; r0 < q.rows; r0 += chunk, ++pass) {
      Prob c = p;
      c.X = q.X + r0 * q.width;
      c.rows = std::min<int64_t>(chunk, q.rows - r0);
      c.beta = pass == 0 ? q.beta : 1.0f;
      (q.packed ? dma_packed : dma).push_back({c, pass});
    }
  }
  auto launch = [&](const std::vector<Piece>& pieces, bool use_dma) -> kfac_status_t {
    int passes = 0;
    for (const Piece& x : pieces) passes = std::max(passes, x.pass + 1);
    for (int pass = 0; pass < passes; ++pass) {
      size_t i = 0;
      while (i < pieces.size()) {
        Batch b{};
        int blocks = 0;
        for (; i < pieces.size() && b.n < kMaxProbs; ++i) {
          if (pieces[i].pass != pass) continue;
          Prob p = pieces[i].p;
          p.blk_begin = blocks;
          blocks += p.tiles * (p.tiles + 1) / 2;
          b.p[b.n++] = p;
        }
        if (b.n == 0) continue;
        b.xcd_run = kXcdRun;
        b.band = kBand;
        if (use_dma && b.p[0].packed) hipLaunchKernelGGL(syrk_bf16_dma_kernel<true>, dim3(blocks), dim3(512), 0, st, b);
        else if (use_dma) hipLaunchKernelGGL(syrk_bf16_dma_kernel<false>, dim3(blocks), dim3(512), 0, st, b);
        else hipLaunchKernelGGL(syrk_bf16_kernel, dim3(blocks), dim3(512), 0, st, b);
        if (hipGetLastError() != hipSuccess) return KFAC_ERR_HIP;
      }
    }
    return KFAC_OK;
  };
  kfac_status_t r = launch(dma, true);
  if (r == KFAC_OK) r = launch(dma_packed, true);
  return r != KFAC_OK ? r : launch(ragged, false);
}

}  // namespace kfac
