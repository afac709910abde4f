// Batched fp32 GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x2_f32), fp32 in,
// fp32 accumulate, fp32 out.  Three kernels:
//   gemm_f32_kernel           register-staged: the next stage's A/B slabs are
//                             fetched into registers while the current ones,
//                             staged in LDS, feed the MFMAs; 128 x 128 tiles on
//                             256 threads (4 wavefronts of 2 x 2 MFMA 32 x 32
//                             blocks) or 256 x 256 tiles on 512 threads (8
//                             wavefronts of 4 x 2 blocks) when a launch has at
//                             least two such tiles per CU; every problem kind;
//   gemm_f32_dma_kernel       256 x 256 tiles with direct-to-LDS loads
//                             (buffer_load ... lds into a 4-slot ring), for the
//                             large launches whose problems it can load;
//   gemm_f32_dma_syrk_kernel  the factor SYRK on 128 x 128 tiles with the same
//                             loader, from row-major X or from a convolution
//                             tensor read in place.
// One launch runs a table of independent problems (layers, matrices, K
// splits, batches); each workgroup finds its problem by binary search over
// the table's block offsets.
#include "gemm.h"

#include <algorithm>
#include <type_traits>

namespace kfac {

namespace {

constexpr int kLdsPad = 4;

// Two shapes: SMALL = 128 x 128 tile, 4 wavefronts (2 x 2) of 64 x 64;
// BIG = 256 x 256 tile, 8 wavefronts (2 x 4) of 128 x 64.
// f(std::integral_constant<int, i>) for i = B .. E - 1
template <int B, int E, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// K depth of one LDS stage: 32 (fewer barriers per MFMA), except for the
// factor SYRK, whose 128 x 128 tiles keep more workgroups per CU with 16
// (both measured).
constexpr int kTileKDeep = 32;
constexpr int kTileKSyrk = 16;

template <bool BIG, int TK>
struct Cfg {
  static constexpr int kTK = TK;
  static constexpr int kThreads = BIG ? 512 : 256;
  static constexpr int kBT = BIG ? 256 : 128;          // output tile
  static constexpr int kRow = kBT + kLdsPad;           // MN operand: LDS row of one k (floats)
  static constexpr int kKRow = TK + 1;             // K operand: LDS row of one m (odd: conflict-free reads)
  static constexpr int kSlab = (TK * kRow > kBT * kKRow) ? TK * kRow : kBT * kKRow;
  static constexpr int kWavesN = BIG ? 4 : 2;
  static constexpr int kWM = BIG ? 128 : 64;           // wavefront tile rows
  static constexpr int kWN = 64;                       // wavefront tile cols
  static constexpr int kBI = kWM / 32, kBJ = kWN / 32; // MFMA blocks per wavefront
  static constexpr int kItems = TK * kBT / 4 / kThreads;   // float4 groups per thread per operand
};

// LDS layout of an operand mode: [k][m] rows for i-contiguous operands,
// [m][k] rows for k-contiguous ones.
__host__ __device__ constexpr bool k_major(int mode) { return mode == OP_K; }

// A launch's problem table, passed as kernel arguments.  Launches of at most
// kSmallCap problems (most launches of the Cholesky chain) take the small
// table: HIP copies the whole argument block per launch into a kernel
// argument pool of bounded size, and a refresh step of the 16k pair, with
// about a thousand launches of 4 KB tables, exhausted it, so that the host
// waited for the GPU to drain it (34.7 ms to enqueue one step).
template <int CAP>
struct GemmBatchT {
  GemmProb p[CAP];
  int32_t n;
  GemmScalars sc;
};
using GemmBatch = GemmBatchT<kMaxGemmProbs>;
constexpr int kSmallCap = 4;
using GemmBatchSmall = GemmBatchT<kSmallCap>;
static_assert(sizeof(GemmBatch) <= 4096, "kernel arguments");

template <typename Batch>
__device__ inline int find_prob(const Batch& b, int blk) {
  int lo = 0, hi = b.n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (b.p[mid].blk_begin <= blk) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// registers of one thread's share of a slab
template <bool BIG, int TK>
using SlabRegs = float[Cfg<BIG, TK>::kItems * 4];

// This thread's share of a TK x BT operand slab (kItems groups of 4 floats).
// MN layout: group g covers row kk = g / (BT/4), columns 4 (g % (BT/4)) .. +3.
// K layout : group g covers column mm = g / (TK/4), k = 4 (g % (TK/4)) .. +3.
template <bool BIG, int TK, int MODE, bool EXTRA>
__device__ inline void load_slab(SlabRegs<BIG, TK>& r, const float* __restrict__ base, int ld, int m0, int mlim,
                                  int k0, int klim, int special, const float* __restrict__ extra, bool vec) {
  using C = Cfg<BIG, TK>;
#pragma unroll
  for (int h = 0; h < C::kItems; ++h) {
    const int g = threadIdx.x + h * C::kThreads;
    if (MODE == OP_MN) {
      const int k = k0 + g / (C::kBT / 4);
      const int m = m0 + (g % (C::kBT / 4)) * 4;
      const bool kin = k < klim;
      const float* p = base + static_cast<int64_t>(k) * ld + m;
      if (vec && kin && m + 3 < mlim && (special < m || special > m + 3)) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(p);
        r[4 * h] = v[0]; r[4 * h + 1] = v[1]; r[4 * h + 2] = v[2]; r[4 * h + 3] = v[3];
        continue;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v = 0.f;
        if (kin) {
          if (m + q == special) v = 1.0f;          // virtual constant-1 (bias) column
          else if (m + q < mlim) v = p[q];
        }
        r[4 * h + q] = v;
      }
    } else {
      const int m = m0 + g / (TK / 4);
      const int k = k0 + (g % (TK / 4)) * 4;
      const bool min_ = m < mlim;
      const float* p = base + static_cast<int64_t>(m) * ld + k;
      if (vec && min_ && k + 3 < klim && (!EXTRA || special < k || special > k + 3)) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(p);
        r[4 * h] = v[0]; r[4 * h + 1] = v[1]; r[4 * h + 2] = v[2]; r[4 * h + 3] = v[3];
        continue;
      }
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

template <bool BIG, int TK, int MODE>
__device__ inline void store_slab(float* __restrict__ s, const SlabRegs<BIG, TK>& r) {
  using C = Cfg<BIG, TK>;
#pragma unroll
  for (int h = 0; h < C::kItems; ++h) {
    const int g = threadIdx.x + h * C::kThreads;
    if (!k_major(MODE)) {
      const int kk = g / (C::kBT / 4);
      const int mm = (g % (C::kBT / 4)) * 4;
      f32x4 v = {r[4 * h], r[4 * h + 1], r[4 * h + 2], r[4 * h + 3]};
      *reinterpret_cast<f32x4*>(s + kk * C::kRow + mm) = v;
    } else {
      const int mm = g / (TK / 4);
      const int kq = (g % (TK / 4)) * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) s[mm * C::kKRow + kq + q] = r[4 * h + q];
    }
  }
}

// The problem entry a workgroup works on, read once from the kernel arguments
// and kept in scalar registers (see arg_reg).  The fused-update kernels read
// it in place: any copy of the entry pushes their 256 x 256 instantiation past
// 256 VGPRs (68 bytes of scratch per lane).
template <int EPI>
__device__ inline std::conditional_t<EPI == EPI_UPDATE, const GemmProb&, GemmProb> prob_regs(const GemmProb& P) {
  if constexpr (EPI == EPI_UPDATE) return P;
  else {
  GemmProb q;
  q.A = arg_reg(P.A);
  q.B = arg_reg(P.B);
  q.C = arg_reg(P.C);
  q.A_extra = arg_reg(P.A_extra);
  q.W = arg_reg(P.W);
  q.Wb = arg_reg(P.Wb);
  q.V = arg_reg(P.V);
  q.Vb = arg_reg(P.Vb);
  q.split_stride = arg_reg(P.split_stride);
  q.lda = arg_reg(P.lda);
  q.ldb = arg_reg(P.ldb);
  q.ldc = arg_reg(P.ldc);
  q.M = arg_reg(P.M);
  q.N = arg_reg(P.N);
  q.kb = arg_reg(P.kb);
  q.ke = arg_reg(P.ke);
  q.tiles_m = arg_reg(P.tiles_m);
  q.tiles_n = arg_reg(P.tiles_n);
  q.a_special = arg_reg(P.a_special);
  q.b_special = arg_reg(P.b_special);
  q.d_in = arg_reg(P.d_in);
  q.nsplit = arg_reg(P.nsplit);
  q.blk_begin = arg_reg(P.blk_begin);
  q.nbatch = static_cast<int16_t>(arg_reg(static_cast<int32_t>(P.nbatch)));
  q.tri = static_cast<uint8_t>(arg_reg(static_cast<uint32_t>(P.tri)));
  q.krange = static_cast<uint8_t>(arg_reg(static_cast<uint32_t>(P.krange)));
  q.a_vec = static_cast<uint8_t>(arg_reg(static_cast<uint32_t>(P.a_vec)));
  q.b_vec = static_cast<uint8_t>(arg_reg(static_cast<uint32_t>(P.b_vec)));
  q.c_packed = static_cast<uint8_t>(arg_reg(static_cast<uint32_t>(P.c_packed)));
  q.nchw = static_cast<uint8_t>(arg_reg(static_cast<uint32_t>(P.nchw)));
  q.alpha = arg_reg(P.alpha);
  q.beta = arg_reg(P.beta);
  return q;
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

// Epilogue: accumulator r of block (si, sj) is C[row][col] with
// row = i0 + wm + 32 si + 8 (r / 4) + 4 (lane / 32) + r % 4, col = j0 + wn + 32 sj + lane % 32.
// r1a / r1b (EPI_STORE only, may be null): a rank-one term r1a[row] r1b[col]
// added to the product before scaling (the bias column of A taken out of the
// contraction).
template <int EPI, typename C, typename Batch>
__device__ __forceinline__ void gemm_epilogue(const Batch& batch, const GemmProb& P, float* Cp,
                                              f32x16 (&acc)[C::kBI][C::kBJ], int i0, int j0, int wm, int wn,
                                              int lane, const float* __restrict__ r1a,
                                              const float* __restrict__ r1b) {
  // Read-modify-write epilogues first issue every read of a block row (from a
  // clamped, always valid address), then compute and store: one memory round
  // trip per block row instead of one per element (a read after a store to
  // the same array is not moved ahead of it, so reads issued element by
  // element would each wait a full round trip).  The factor SYRK reads the
  // old factor only for its EMA (one row split, beta != 0): upper elements,
  // at their packed or whole position.
  const bool ema = EPI == EPI_SYRK && P.nsplit == 1;
  const bool ema_read = ema && P.beta != 0.f;
  const float wd = batch.sc.weight_decay, mom = batch.sc.momentum, lr = batch.sc.lr;
  // the update's targets and extent, read once here (after the main loop, so
  // that they hold no registers there)
  float* const uW = EPI == EPI_UPDATE ? arg_reg(P.W) : nullptr;
  float* const uWb = EPI == EPI_UPDATE ? arg_reg(P.Wb) : nullptr;
  float* const uV = EPI == EPI_UPDATE ? arg_reg(P.V) : nullptr;
  float* const uVb = EPI == EPI_UPDATE ? arg_reg(P.Vb) : nullptr;
  const int ud_in = EPI == EPI_UPDATE ? arg_reg(P.d_in) : 0;
  const int uM = EPI == EPI_UPDATE ? arg_reg(P.M) : P.M;
  const int uN = EPI == EPI_UPDATE ? arg_reg(P.N) : P.N;
  constexpr bool kReads = EPI == EPI_SUB || EPI == EPI_UPDATE || EPI == EPI_SYRK;
  bool bad = false;
  if constexpr (EPI == EPI_UPDATE) {
    // one 32 x 32 block at a time (its 32 reads together): staging a whole
    // block row would take this epilogue past 256 VGPRs
    static_for<0, C::kBI>([&](auto si_c) {
      constexpr int si = decltype(si_c)::value;
#pragma unroll
      for (int sj = 0; sj < C::kBJ; ++sj) {
        const int col = j0 + wn + 32 * sj + (lane & 31);
        float w0[16], v0[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i0 + wm + 32 * si + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const bool in = row < uM && col < uN;
          const bool wcol = !in || col < ud_in;
          const int64_t e = in ? static_cast<int64_t>(row) * ud_in + col : 0;
          w0[r] = wcol ? uW[e] : uWb[row];
          v0[r] = wcol ? uV[e] : uVb[row];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i0 + wm + 32 * si + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row >= uM || col >= uN) continue;
          const bool wcol = col < ud_in;
          float* wp = wcol ? uW + static_cast<int64_t>(row) * ud_in + col : uWb + row;
          float* vp = wcol ? uV + static_cast<int64_t>(row) * ud_in + col : uVb + row;
          const float d = fmaf(wd, w0[r], acc[si][sj][r]);
          const float vn = fmaf(mom, v0[r], d);
          const float wn2 = fmaf(-lr, vn, w0[r]);
          *vp = vn;
          *wp = wn2;
          bad |= !(isfinite(vn) && isfinite(wn2));
        }
      }
    });
    if (__any(bad) && lane == 0) raise_flag(batch.sc.flags, KFAC_FLAG_NONFINITE);
    return;
  }
  // block rows by a compile-time index: a runtime one would place acc in scratch
  static_for<0, C::kBI>([&](auto si_c) {
    constexpr int si = decltype(si_c)::value;
    float c0v[C::kBJ][16], c1v[C::kBJ][16];
    if (kReads && (EPI != EPI_SYRK || ema_read)) {
#pragma unroll
      for (int sj = 0; sj < C::kBJ; ++sj) {
        const int col = j0 + wn + 32 * sj + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i0 + wm + 32 * si + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const bool in = row < uM && col < uN;
          const int64_t idx = in ? static_cast<int64_t>(row) * P.ldc + col : 0;
          if (EPI == EPI_UPDATE) {
            const bool wcol = !in || col < ud_in;
            const int64_t e = in ? static_cast<int64_t>(row) * ud_in + col : 0;
            c0v[sj][r] = wcol ? uW[e] : uWb[row];
            c1v[sj][r] = wcol ? uV[e] : uVb[row];
          } else if (EPI == EPI_SYRK) {
            const bool up = in && row <= col;
            c0v[sj][r] = Cp[!up ? 0 : P.c_packed ? packed_index(row, col, P.M) : idx];
          } else {
            c0v[sj][r] = Cp[idx];
          }
        }
      }
    }
#pragma unroll
    for (int sj = 0; sj < C::kBJ; ++sj) {
      const int col = j0 + wn + 32 * sj + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i0 + wm + 32 * si + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= uM || col >= uN) continue;
        float v = acc[si][sj][r];
        if (EPI == EPI_STORE && r1a != nullptr) v = fmaf(r1a[row], r1b[col], v);
        const int64_t idx = static_cast<int64_t>(row) * P.ldc + col;
        if (EPI == EPI_STORE) {
          Cp[idx] = P.alpha * v;
        } else if (EPI == EPI_SUB) {
          Cp[idx] = c0v[sj][r] - P.alpha * v;
        } else if (EPI == EPI_SYRK && !ema) {
          Cp[idx] = P.alpha * v;
        } else if (EPI == EPI_SYRK) {
          if (row <= col) {
            const int64_t u = P.c_packed ? packed_index(row, col, P.M) : idx;
            const float o = ema_read ? P.beta * c0v[sj][r] + P.alpha * v : P.alpha * v;
            Cp[u] = o;
            if (row != col && !P.c_packed) Cp[static_cast<int64_t>(col) * P.ldc + row] = o;
          }
        } else if (EPI == EPI_UPDATE) {
          const bool wcol = col < ud_in;
          float* wp = wcol ? uW + static_cast<int64_t>(row) * ud_in + col : uWb + row;
          float* vp = wcol ? uV + static_cast<int64_t>(row) * ud_in + col : uVb + row;
          const float w = c0v[sj][r];
          const float d = fmaf(wd, w, v);
          const float vn = fmaf(mom, c1v[sj][r], d);
          const float wn2 = fmaf(-lr, vn, w);
          *vp = vn;
          *wp = wn2;
          bad |= !(isfinite(vn) && isfinite(wn2));
        }
      }
    }
  });
  if (EPI == EPI_UPDATE) {
    if (__any(bad) && lane == 0) raise_flag(batch.sc.flags, KFAC_FLAG_NONFINITE);
  }
}

template <int AMODE, int BMODE, int EPI, bool BIG, typename Batch>
__device__ __forceinline__ void gemm_f32_body(const Batch& batch) {
  if (batch.sc.prio) __builtin_amdgcn_s_setprio(3);
  constexpr int TK = EPI == EPI_SYRK ? kTileKSyrk : kTileKDeep;
  using C = Cfg<BIG, TK>;
  __shared__ __attribute__((aligned(16))) float sA[2][C::kSlab];
  __shared__ __attribute__((aligned(16))) float sB[2][C::kSlab];
  const auto& P = prob_regs<EPI>(batch.p[find_prob(batch, blockIdx.x)]);
  int split, ti, tj;
  tile_coords(P, blockIdx.x - P.blk_begin, split, ti, tj);
  const int i0 = ti * C::kBT, j0 = tj * C::kBT;
  int kb = P.kb, ke = P.ke;
  if (P.krange == KR_FROM_DIAG) kb = max(kb, max(i0, j0));
  else if (P.krange == KR_FROM_ROW) kb = max(kb, i0);
  else if (P.krange == KR_TO_ROW) ke = min(ke, i0 + C::kBT);
  const float* Ab = static_cast<const float*>(P.A);
  const float* Bb = static_cast<const float*>(P.B);
  float* Cp = P.C;
  if (P.nbatch > 1) {
    // the tile grid index past one problem counts batch entries
    const int64_t off = static_cast<int64_t>(split) * P.split_stride;
    Ab += off;
    Bb += off;
    Cp += off;
  } else {
    if (P.nsplit > 1) {
      const int len = ((ke - kb + P.nsplit - 1) / P.nsplit + TK - 1) / TK * TK;
      const int s0 = kb + split * len;
      ke = min(ke, s0 + len);
      kb = s0;
    }
    Cp += static_cast<int64_t>(split) * P.split_stride;
  }

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int wm = (wid / C::kWavesN) * C::kWM, wn = (wid % C::kWavesN) * C::kWN;

  // A wavefront whose part of the tile lies outside C, or strictly below the
  // diagonal of a diagonal tile of an upper-triangle grid, has no output to
  // produce and skips its MFMAs (it still stages its share of the slabs).
  const bool live = i0 + wm < P.M && j0 + wn < P.N && !(P.tri == TRI_UPPER && ti == tj && wm >= wn + C::kWN);

  f32x16 acc[C::kBI][C::kBJ];
#pragma unroll
  for (int a = 0; a < C::kBI; ++a)
#pragma unroll
    for (int b = 0; b < C::kBJ; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  float ra[C::kItems * 4], rb[C::kItems * 4];
  int buf = 0;
  if (kb < ke) {
    load_slab<BIG, TK, AMODE, true>(ra, Ab, P.lda, i0, P.M, kb, ke, P.a_special, P.A_extra, P.a_vec);
    load_slab<BIG, TK, BMODE, false>(rb, Bb, P.ldb, j0, P.N, kb, ke, P.b_special, Bb, P.b_vec);
    store_slab<BIG, TK, AMODE>(sA[0], ra);
    store_slab<BIG, TK, BMODE>(sB[0], rb);
  }
  __syncthreads();
  // The main loop is instantiated twice: wavefronts without output run it
  // without MFMAs (a branch inside one loop costs the others registers).
  auto main_loop = [&](auto compute) {
  for (int k0 = kb; k0 < ke; k0 += TK) {
    const bool more = k0 + TK < ke;
    if (more) {
      load_slab<BIG, TK, AMODE, true>(ra, Ab, P.lda, i0, P.M, k0 + TK, ke, P.a_special, P.A_extra, P.a_vec);
      load_slab<BIG, TK, BMODE, false>(rb, Bb, P.ldb, j0, P.N, k0 + TK, ke, P.b_special, Bb, P.b_vec);
    }
    if constexpr (decltype(compute)::value) {
    const float* a = sA[buf];
    const float* b = sB[buf];
    // fragments of k-substep kk + 2 are read while the MFMAs of kk run
    float af[2][C::kBI], bf[2][C::kBJ];
    auto frag = [&](int kk, float (&fa)[C::kBI], float (&fb)[C::kBJ]) {
      const int kl = kk + (lane >> 5);
#pragma unroll
      for (int i = 0; i < C::kBI; ++i) {
        const int m = wm + 32 * i + (lane & 31);
        fa[i] = !k_major(AMODE) ? a[kl * C::kRow + m] : a[m * C::kKRow + kl];
      }
#pragma unroll
      for (int j = 0; j < C::kBJ; ++j) {
        const int n = wn + 32 * j + (lane & 31);
        fb[j] = !k_major(BMODE) ? b[kl * C::kRow + n] : b[n * C::kKRow + kl];
      }
    };
    frag(0, af[0], bf[0]);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, C::kBI + C::kBJ, 0);
#pragma unroll
    for (int kk = 0; kk < TK; kk += 2) {
      const int cur = (kk >> 1) & 1;
      if (kk + 2 < TK) frag(kk + 2, af[cur ^ 1], bf[cur ^ 1]);
#pragma unroll
      for (int i = 0; i < C::kBI; ++i)
#pragma unroll
        for (int j = 0; j < C::kBJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[cur][i], bf[cur][j], acc[i][j], 0, 0, 0);
      // the scheduler would otherwise sink the reads next to their MFMAs
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, C::kBI + C::kBJ, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, C::kBI * C::kBJ, 0);
    }
    }
    if (more) {
      store_slab<BIG, TK, AMODE>(sA[buf ^ 1], ra);
      store_slab<BIG, TK, BMODE>(sB[buf ^ 1], rb);
    }
    __syncthreads();
    buf ^= 1;
  }
  };
  if (live) main_loop(std::true_type{});
  else main_loop(std::false_type{});

  gemm_epilogue<EPI, C>(batch, P, Cp, acc, i0, j0, wm, wn, lane, nullptr, nullptr);
}

template <int AMODE, int BMODE, int EPI, bool BIG, int CAP>
__global__ void __launch_bounds__((Cfg<BIG, kTileKDeep>::kThreads)) gemm_f32_kernel(GemmBatchT<CAP> batch) {
  gemm_f32_body<AMODE, BMODE, EPI, BIG>(batch);
}

// The factor SYRK on 128 x 128 tiles with the register budget of at least two
// wavefronts per SIMD: the compiler then keeps the accumulators in VGPRs and
// fits four wavefronts per SIMD (three otherwise); ResNet-50's factor phase
// measured 10.38 -> 10.04 ms.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 8)))
gemm_f32_syrk_kernel(GemmBatch batch) {
  gemm_f32_body<OP_MN, OP_MN, EPI_SYRK, false>(batch);
}

// ---------------------------------------------------------------------------
// The 256 x 256 kernel with direct-to-LDS operand loads.  Each stage holds
// 16 of K for both operands; a 4-slot LDS ring is filled by
// buffer_load_dwordx4 ... lds (no registers, no LDS stores by the
// wavefronts), three stages ahead of the one being multiplied, with one
// barrier per stage.  It takes the problems whose contraction range of every
// tile is whole stages (K bounds multiples of 16; the bias column of an OP_K
// A, the last index of a whole-K contraction, is added in the epilogue as a
// rank-one term) and whose rows start 16-byte aligned (an OP_MN B may instead
// load 4 bytes per lane, four instructions per row).  Each operand is read
// through a buffer resource that ends at its last element, so the loads of
// tile rows or columns past M or N stay inside the operand's rows (their
// products land in outputs the epilogue drops) and loads past the end read 0.
// LDS layouts:
//   OP_MN operand  [k][256 + 4] (one load instruction per k row, the 4-float
//                  pad keeps the two half-wave rows of a fragment read apart);
//   OP_K operand   [m][16], the four 16-byte chunks of row m stored at
//                  position chunk ^ kswz(m) (the lane that loads a position
//                  fetches the chunk that belongs there), so that the 16-byte
//                  reads of 8 consecutive rows, and of the 4 rows of 16
//                  consecutive ones that share a 64-byte quarter of a
//                  256-byte line, fall on distinct banks (with (m >> 1) & 3
//                  alone the second group collided: SQ_LDS_BANK_CONFLICT).
// Contraction order: at substep s (0..7) of a stage, lane half h takes
// k = 8 h + s for both operands (any bijection is a valid order; this one
// lets an OP_K lane read its 8 values of a stage with two 16-byte reads).

typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDK = 16;                    // K per stage
constexpr int kDNS = 4;                    // ring slots
constexpr int kDRow = 256 + 4;             // OP_MN row (floats)
constexpr int kDSlot = kDK * kDRow;        // floats per operand and slot (>= 256 x 16 for OP_K)

// chunk swizzle of row m of an OP_K stage (see above)
__device__ inline int kswz(int m) { return ((m >> 1) ^ (m >> 2)) & 3; }

// buffer resource over `bytes` bytes at `base` (reads past them return 0);
// the values are workgroup-uniform, read from the first lane so that the
// resource sits in scalar registers
__device__ inline i32x4_t buf_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4_t{__builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xffffffffu)),
                 __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xffffu)),
                 __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)), 0x00020000};
}

// 16 bytes per lane from byte offset `voff` of `rsrc` to LDS at lds + 16 lane
__device__ inline void dma16(const void* lds, uint32_t voff, i32x4_t rsrc) {
  const uint32_t l = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)lds));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(l)), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// 4 bytes per lane from byte offset `voff` of `rsrc` to LDS at lds + 4 lane
__device__ inline void dma4(const void* lds, uint32_t voff, i32x4_t rsrc) {
  const uint32_t l = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)lds));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(l)), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// s_waitcnt with only the vector-memory counter limited to n (n < 64; its
// bits 3:0 and 5:4 sit at 3:0 and 15:14 of the immediate)
#define KFAC_GEMM_WAIT_VM(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | ((((n) >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8))

// Bytes from an operand's first element to the end of its last one: `rows`
// rows of `ld` floats of which the last is read up to column `cols`.
__host__ __device__ inline uint64_t operand_extent(int64_t rows, int64_t ld, int64_t cols) {
  return rows <= 0 ? 0 : static_cast<uint64_t>(((rows - 1) * ld + cols) * 4);
}

// B16: the OP_MN B loads 16 bytes per lane (rows 16-byte aligned); otherwise
// 4 bytes per lane, four instructions per row.
template <int AMODE, int BMODE, int EPI, bool B16>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_f32_dma_kernel(GemmBatch batch) {
  if (batch.sc.prio) __builtin_amdgcn_s_setprio(3);
  using C = Cfg<true, kTileKDeep>;
  __shared__ __attribute__((aligned(16))) float ring[kDNS][2][kDSlot];
  const auto& P = prob_regs<EPI>(batch.p[find_prob(batch, blockIdx.x)]);
  int split, ti, tj;
  tile_coords(P, blockIdx.x - P.blk_begin, split, ti, tj);
  const int i0 = ti * 256, j0 = tj * 256;
  // the contraction of the whole problem (the bias index of A excluded) and
  // of this tile
  const int kend = P.a_special >= 0 ? P.a_special : P.ke;
  int kb = P.kb, ke = kend;
  if (P.krange == KR_FROM_DIAG) kb = max(kb, max(i0, j0));
  else if (P.krange == KR_FROM_ROW) kb = max(kb, i0);
  else if (P.krange == KR_TO_ROW) ke = min(ke, i0 + 256);
  const float* Ab = static_cast<const float*>(P.A);
  const float* Bb = static_cast<const float*>(P.B);
  float* Cp = P.C;
  if (P.nbatch > 1) {
    const int64_t off = static_cast<int64_t>(split) * P.split_stride;
    Ab += off;
    Bb += off;
    Cp += off;
  }
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int wm = (wid / C::kWavesN) * C::kWM, wn = (wid % C::kWavesN) * C::kWN;
  const bool live = i0 + wm < P.M && j0 + wn < P.N && !(P.tri == TRI_UPPER && ti == tj && wm >= wn + C::kWN);

  const i32x4_t ra = buf_rsrc(Ab, static_cast<uint32_t>(AMODE == OP_MN ? operand_extent(kend, P.lda, P.M)
                                                                       : operand_extent(P.M, P.lda, kend)));
  const i32x4_t rb = buf_rsrc(Bb, static_cast<uint32_t>(BMODE == OP_MN ? operand_extent(kend, P.ldb, P.N)
                                                                       : operand_extent(P.N, P.ldb, kend)));
  // this wavefront's load instructions of a stage: q = 2 wid + u (0..15) of
  // each operand; an OP_MN instruction is row q of the stage, an OP_K one
  // rows 16 q .. 16 q + 15 of the tile
  auto op_off = [&](int mode, int ld, int t0, int q, int vec) -> uint32_t {
    if (mode == OP_MN)
      return static_cast<uint32_t>((static_cast<int64_t>(kb + q) * ld + t0 + vec * lane) * 4);
    const int m = 16 * q + (lane >> 2);
    const int c = (lane & 3) ^ kswz(m);
    return static_cast<uint32_t>((static_cast<int64_t>(t0 + m) * ld + kb + 4 * c) * 4);
  };
  uint32_t a_off[2], b_off[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    a_off[u] = op_off(AMODE, P.lda, i0, 2 * wid + u, 4);
    b_off[u] = op_off(BMODE, P.ldb, j0, 2 * wid + u, B16 ? 4 : 1);
  }
  const uint32_t a_step = AMODE == OP_MN ? static_cast<uint32_t>(kDK * P.lda * 4) : kDK * 4;
  const uint32_t b_step = BMODE == OP_MN ? static_cast<uint32_t>(kDK * P.ldb * 4) : kDK * 4;
  const int nst = ke > kb ? (ke - kb) / kDK : 0;
  auto issue = [&](int s, int slot) {
    if (s >= nst) return;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = 2 * wid + u;
      dma16(&ring[slot][0][AMODE == OP_MN ? q * kDRow : q * 256], a_off[u] + static_cast<uint32_t>(s) * a_step, ra);
      if (BMODE == OP_K) {
        dma16(&ring[slot][1][q * 256], b_off[u] + static_cast<uint32_t>(s) * b_step, rb);
      } else if (B16) {
        dma16(&ring[slot][1][q * kDRow], b_off[u] + static_cast<uint32_t>(s) * b_step, rb);
      } else {
#pragma unroll
        for (int part = 0; part < 4; ++part)
          dma4(&ring[slot][1][q * kDRow + 64 * part], b_off[u] + static_cast<uint32_t>(s) * b_step + 256 * part, rb);
      }
    }
  };
  constexpr int kLoads = (BMODE == OP_MN && !B16) ? 10 : 4;   // load instructions per lane and stage

  f32x16 acc[C::kBI][C::kBJ];
#pragma unroll
  for (int a = 0; a < C::kBI; ++a)
#pragma unroll
    for (int b = 0; b < C::kBJ; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int s = 0; s < kDNS - 1; ++s) issue(s, s);
  int slot = 0;
  for (int s = 0; s < nst; ++s) {
    // this lane's loads of stage s have landed once at most those of the
    // later stages already issued (kLoads per stage) remain
    const int later = min(nst - 1 - s, kDNS - 2);
    if (later >= 2) KFAC_GEMM_WAIT_VM(2 * kLoads);
    else if (later == 1) KFAC_GEMM_WAIT_VM(kLoads);
    else KFAC_GEMM_WAIT_VM(0);
    __builtin_amdgcn_s_barrier();
    issue(s + kDNS - 1, slot == 0 ? kDNS - 1 : slot - 1);
    if (live) {
      const float* sa = ring[slot][0];
      const float* sb = ring[slot][1];
      // OP_K operands: rows wm + 32 i + l32 (wn + 32 j + l32); chunks 2 h and
      // 2 h + 1 hold k = 8 h .. 8 h + 7
      float ak[8][C::kBI], bk[8][C::kBJ];
      if (AMODE == OP_K) {
#pragma unroll
        for (int i = 0; i < C::kBI; ++i) {
          const int m = wm + 32 * i + l32;
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(sa + m * kDK + 4 * ((2 * h + cc) ^ kswz(m)));
#pragma unroll
            for (int e = 0; e < 4; ++e) ak[4 * cc + e][i] = v[e];
          }
        }
      }
      if (BMODE == OP_K) {
#pragma unroll
        for (int j = 0; j < C::kBJ; ++j) {
          const int n = wn + 32 * j + l32;
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(sb + n * kDK + 4 * ((2 * h + cc) ^ kswz(n)));
#pragma unroll
            for (int e = 0; e < 4; ++e) bk[4 * cc + e][j] = v[e];
          }
        }
      }
      // OP_MN operands: one float per block and substep, read a substep ahead
      float bfr[2][C::kBJ], afr[2][C::kBI];
      auto frag = [&](int st, float (&fa)[C::kBI], float (&fb)[C::kBJ]) {
        const int kr = 8 * h + st;
        if (BMODE == OP_MN) {
#pragma unroll
          for (int j = 0; j < C::kBJ; ++j) fb[j] = sb[kr * kDRow + wn + 32 * j + l32];
        }
        if (AMODE == OP_MN) {
#pragma unroll
          for (int i = 0; i < C::kBI; ++i) fa[i] = sa[kr * kDRow + wm + 32 * i + l32];
        }
      };
      constexpr int kReads = (AMODE == OP_MN ? C::kBI : 0) + (BMODE == OP_MN ? C::kBJ : 0);
      frag(0, afr[0], bfr[0]);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const int cur = st & 1;
        if (st < 7) frag(st + 1, afr[cur ^ 1], bfr[cur ^ 1]);
#pragma unroll
        for (int i = 0; i < C::kBI; ++i)
#pragma unroll
          for (int j = 0; j < C::kBJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(AMODE == OP_K ? ak[st][i] : afr[cur][i],
                                                            BMODE == OP_K ? bk[st][j] : bfr[cur][j], acc[i][j], 0, 0,
                                                            0);
        if (kReads > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kReads, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, C::kBI * C::kBJ, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this stage's reads are done before the next barrier
    slot = slot == kDNS - 1 ? 0 : slot + 1;
  }

  const float* r1a = nullptr;
  const float* r1b = nullptr;
  if (EPI == EPI_STORE && P.a_special >= 0) {
    r1a = P.A_extra;
    r1b = Bb + static_cast<int64_t>(P.a_special) * P.ldb;
  }
  gemm_epilogue<EPI, C>(batch, P, Cp, acc, i0, j0, wm, wn, lane, r1a, r1b);
}

template <int AM, int BM, int EPI>
kfac_status_t launch_group(const GemmBatch& b, int blocks, bool big, hipStream_t s) {
  if (big) {
    hipLaunchKernelGGL((gemm_f32_kernel<AM, BM, EPI, true, kMaxGemmProbs>), dim3(blocks), dim3(512), 0, s, b);
  } else if constexpr (AM == OP_MN && BM == OP_MN && EPI == EPI_SYRK) {
    hipLaunchKernelGGL(gemm_f32_syrk_kernel, dim3(blocks), dim3(256), 0, s, b);
  } else if (b.n <= kSmallCap) {
    GemmBatchSmall t{};
    for (int i = 0; i < b.n; ++i) t.p[i] = b.p[i];
    t.n = b.n;
    t.sc = b.sc;
    hipLaunchKernelGGL((gemm_f32_kernel<AM, BM, EPI, false, kSmallCap>), dim3(blocks), dim3(256), 0, s, t);
  } else {
    hipLaunchKernelGGL((gemm_f32_kernel<AM, BM, EPI, false, kMaxGemmProbs>), dim3(blocks), dim3(256), 0, s, b);
  }
  return hipGetLastError() == hipSuccess ? KFAC_OK : KFAC_ERR_HIP;
}

kfac_status_t dispatch(const GemmBatch& b, int blocks, bool big, int am, int bm, int epi, hipStream_t s) {
#define KFAC_GEMM_CASE(A_, B_, E_) \
  if (am == A_ && bm == B_ && epi == E_) return launch_group<A_, B_, E_>(b, blocks, big, s);
  KFAC_GEMM_CASE(OP_MN, OP_MN, EPI_STORE)
  KFAC_GEMM_CASE(OP_MN, OP_MN, EPI_SUB)
  KFAC_GEMM_CASE(OP_MN, OP_MN, EPI_UPDATE)
  KFAC_GEMM_CASE(OP_MN, OP_K, EPI_STORE)
  KFAC_GEMM_CASE(OP_K, OP_MN, EPI_STORE)
  KFAC_GEMM_CASE(OP_K, OP_MN, EPI_SUB)
  KFAC_GEMM_CASE(OP_K, OP_K, EPI_STORE)
  KFAC_GEMM_CASE(OP_K, OP_K, EPI_SUB)
  KFAC_GEMM_CASE(OP_MN, OP_MN, EPI_SYRK)
#undef KFAC_GEMM_CASE
  return KFAC_ERR_UNSUPPORTED;
}

// ---------------------------------------------------------------------------
// The factor SYRK (upper 128 x 128 tiles of X^T X, X = [rows, d] row-major,
// no virtual bias column) with direct-to-LDS loads: 4 wavefronts of 64 x 64,

// ---------------------------------------------------------------------------
// The factor SYRK (upper 128 x 128 tiles of X^T X, X = [rows, d] row-major,
// no virtual bias column) with direct-to-LDS loads: 4 wavefronts of 64 x 64,
// 16 rows of X per stage, a 3-slot ring filled two stages ahead, one
// barrier per stage; three workgroups per CU (ResNet-50's factor phase:
// 10.15 ms with the register-staged kernel, 10.61 ms with a 4-slot ring and
// two workgroups per CU, 9.94 ms with this).  A stage holds each operand as 8
// row pairs ([2][128] floats, written by one 16-byte-per-lane load each)
// with 4 floats of padding after each pair; a diagonal tile loads one
// operand.  Rows of a K split past the end of X read as zero (buffer range).
// Contraction order as in the kernel above: substep s, lane half h -> row
// 8 h + s of the stage.

constexpr int kSK = 16;                    // rows of X per stage
constexpr int kSNS = 3;                    // ring slots (three workgroups per CU)
constexpr int kSPair = 2 * 128 + 4;        // a row pair (floats)
constexpr int kSSlot = (kSK / 2) * kSPair; // floats per operand and slot

// NCHW: X is a convolution tensor [B][d][HW] read in place (row k of X is
// pixel k % HW of image k / HW: X[k][i] at (k / HW) d HW + i HW + k % HW,
// lda = HW, a multiple of 16 so that no stage spans two images); its stages
// sit in LDS as the OP_K operand of the 256 x 256 kernel ([m][16], swizzled).
template <bool NCHW>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
gemm_f32_dma_syrk_kernel(GemmBatch batch) {
  using C = Cfg<false, kTileKSyrk>;
  __shared__ __attribute__((aligned(16))) float ring[kSNS][2][kSSlot];
  const auto& P = prob_regs<EPI_SYRK>(batch.p[find_prob(batch, blockIdx.x)]);
  int split, ti, tj;
  tile_coords(P, blockIdx.x - P.blk_begin, split, ti, tj);
  const int i0 = ti * 128, j0 = tj * 128;
  const bool diag = ti == tj;
  int kb = P.kb, ke = P.ke;
  if (P.nsplit > 1) {
    const int len = ((ke - kb + P.nsplit - 1) / P.nsplit + kTileKSyrk - 1) / kTileKSyrk * kTileKSyrk;
    const int s0 = kb + split * len;
    ke = min(ke, s0 + len);
    kb = s0;
  }
  float* Cp = P.C + static_cast<int64_t>(split) * P.split_stride;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int wm = (wid / C::kWavesN) * C::kWM, wn = (wid % C::kWavesN) * C::kWN;
  const bool live = i0 + wm < P.M && j0 + wn < P.N && !(diag && wm >= wn + C::kWN);

  // X: rows [0, P.ke) of lda floats (NCHW: ke / HW images of d HW floats);
  // reads past them return zero
  const i32x4_t rx = buf_rsrc(P.A, static_cast<uint32_t>(static_cast<uint64_t>(P.ke) * (NCHW ? P.M : P.lda) * 4));
  const int nops = diag ? 1 : 2;
  // load instruction q = 2 wid + u (0..7) of an operand: rows 2 q, 2 q + 1 of
  // the stage (NCHW: tile rows 16 q .. 16 q + 15, 16 pixels each)
  uint32_t off[2][2];
#pragma unroll
  for (int op = 0; op < 2; ++op)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = 2 * wid + u;
      if (NCHW) {
        const int m = 16 * q + (lane >> 2);
        const int c = (lane & 3) ^ kswz(m);
        off[op][u] = static_cast<uint32_t>((static_cast<int64_t>((op ? j0 : i0) + m) * P.lda + 4 * c) * 4);
      } else {
        const int row = 2 * q + (lane >> 5);
        off[op][u] = static_cast<uint32_t>(
            (static_cast<int64_t>(kb + row) * P.lda + (op ? j0 : i0) + 4 * (lane & 31)) * 4);
      }
    }
  const uint32_t step = static_cast<uint32_t>(kSK * P.lda * 4);
  const int nst = (ke - kb + kSK - 1) / kSK;
  // byte offset of stage s (NCHW: image and first pixel of its rows)
  auto stage_off = [&](int s) -> uint32_t {
    if (!NCHW) return static_cast<uint32_t>(s) * step;
    const int k0 = kb + s * kSK;
    const int img = k0 / P.lda;
    return static_cast<uint32_t>((static_cast<int64_t>(img) * P.M * P.lda + (k0 - img * P.lda)) * 4);
  };
  auto issue = [&](int s, int slot) {
    if (s >= nst) return;
    const uint32_t so = stage_off(s);
#pragma unroll
    for (int op = 0; op < 2; ++op) {
      if (op >= nops) break;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        dma16(&ring[slot][op][(2 * wid + u) * (NCHW ? 256 : kSPair)], off[op][u] + so, rx);
    }
  };

  f32x16 acc[C::kBI][C::kBJ];
#pragma unroll
  for (int a = 0; a < C::kBI; ++a)
#pragma unroll
    for (int b = 0; b < C::kBJ; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int h = lane >> 5, l32 = lane & 31;
  const int per_stage = 2 * nops;
#pragma unroll
  for (int s = 0; s < kSNS - 1; ++s) issue(s, s);
  int slot = 0;
  for (int s = 0; s < nst; ++s) {
    const int later = min(nst - 1 - s, kSNS - 2) * per_stage;
    switch (later) {
      case 0: KFAC_GEMM_WAIT_VM(0); break;
      case 2: KFAC_GEMM_WAIT_VM(2); break;
      case 4: KFAC_GEMM_WAIT_VM(4); break;
      default: KFAC_GEMM_WAIT_VM(8); break;
    }
    __builtin_amdgcn_s_barrier();
    issue(s + kSNS - 1, slot == 0 ? kSNS - 1 : slot - 1);
    if (live && NCHW) {
      const float* sa = ring[slot][0];
      const float* sb = diag ? sa : ring[slot][1];
      // rows wm + 32 i + l32 (wn + 32 j + l32): chunks 2 h and 2 h + 1 hold
      // the stage's k = 8 h .. 8 h + 7
      float ak[8][C::kBI], bk[8][C::kBJ];
#pragma unroll
      for (int i = 0; i < C::kBI; ++i) {
        const int m = wm + 32 * i + l32;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(sa + m * kSK + 4 * ((2 * h + cc) ^ kswz(m)));
#pragma unroll
          for (int e = 0; e < 4; ++e) ak[4 * cc + e][i] = v[e];
        }
      }
#pragma unroll
      for (int j = 0; j < C::kBJ; ++j) {
        const int n = wn + 32 * j + l32;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(sb + n * kSK + 4 * ((2 * h + cc) ^ kswz(n)));
#pragma unroll
          for (int e = 0; e < 4; ++e) bk[4 * cc + e][j] = v[e];
        }
      }
#pragma unroll
      for (int st = 0; st < 8; ++st) {
#pragma unroll
        for (int i = 0; i < C::kBI; ++i)
#pragma unroll
          for (int j = 0; j < C::kBJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(ak[st][i], bk[st][j], acc[i][j], 0, 0, 0);
      }
    } else if (live) {
      const float* sa = ring[slot][0];
      const float* sb = diag ? sa : ring[slot][1];
      float afr[2][C::kBI], bfr[2][C::kBJ];
      auto frag = [&](int st, float (&fa)[C::kBI], float (&fb)[C::kBJ]) {
        const int kr = 8 * h + st;
        const int base = (kr >> 1) * kSPair + (kr & 1) * 128 + l32;
#pragma unroll
        for (int i = 0; i < C::kBI; ++i) fa[i] = sa[base + wm + 32 * i];
#pragma unroll
        for (int j = 0; j < C::kBJ; ++j) fb[j] = sb[base + wn + 32 * j];
      };
      frag(0, afr[0], bfr[0]);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const int cur = st & 1;
        if (st < 7) frag(st + 1, afr[cur ^ 1], bfr[cur ^ 1]);
#pragma unroll
        for (int i = 0; i < C::kBI; ++i)
#pragma unroll
          for (int j = 0; j < C::kBJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(afr[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, C::kBI + C::kBJ, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, C::kBI * C::kBJ, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    slot = slot == kSNS - 1 ? 0 : slot + 1;
  }
  gemm_epilogue<EPI_SYRK, C>(batch, P, Cp, acc, i0, j0, wm, wn, lane, nullptr, nullptr);
}

kfac_status_t dispatch_dma(const GemmBatch& b, int blocks, int am, int bm, int epi, bool b16, hipStream_t s) {
  if (epi == EPI_SYRK) {
    if (b.p[0].nchw) hipLaunchKernelGGL(gemm_f32_dma_syrk_kernel<true>, dim3(blocks), dim3(256), 0, s, b);
    else hipLaunchKernelGGL(gemm_f32_dma_syrk_kernel<false>, dim3(blocks), dim3(256), 0, s, b);
    return hipGetLastError() == hipSuccess ? KFAC_OK : KFAC_ERR_HIP;
  }
#define KFAC_DMA_CASE(A_, B_, E_, W_)                                                        \
  if (am == A_ && bm == B_ && epi == E_ && b16 == W_) {                                      \
    hipLaunchKernelGGL((gemm_f32_dma_kernel<A_, B_, E_, W_>), dim3(blocks), dim3(512), 0, s, b); \
    return hipGetLastError() == hipSuccess ? KFAC_OK : KFAC_ERR_HIP;                         \
  }
  KFAC_DMA_CASE(OP_K, OP_MN, EPI_STORE, true)      // preconditioning, [grad_w | grad_b] A_inv
  KFAC_DMA_CASE(OP_K, OP_MN, EPI_STORE, false)
  KFAC_DMA_CASE(OP_MN, OP_MN, EPI_UPDATE, true)    // preconditioning, G_inv T + update
  KFAC_DMA_CASE(OP_K, OP_K, EPI_SUB, true)         // Cholesky trailing updates
  KFAC_DMA_CASE(OP_MN, OP_K, EPI_STORE, true)      // triangular inverse
  KFAC_DMA_CASE(OP_K, OP_K, EPI_STORE, true)
  KFAC_DMA_CASE(OP_MN, OP_MN, EPI_STORE, true)     // Z^T Z
  KFAC_DMA_CASE(OP_MN, OP_MN, EPI_SUB, true)
#undef KFAC_DMA_CASE
  return KFAC_ERR_UNSUPPORTED;
}

// the direct-to-LDS factor SYRK: no virtual bias column, 16-byte aligned rows,
// enough rows to fill its ring (a short problem stays in the launch of the
// others: one launch instead of two)
constexpr int kDmaSyrkMinRows = 512;
bool dma_syrk_eligible(const GemmProb& p) {
  if (p.nchw) return true;   // planned with gemm_nchw_syrk_ok
  if (p.ke - p.kb < kDmaSyrkMinRows) return false;
  if (p.A != p.B || p.lda != p.ldb || p.a_special >= 0 || p.b_special >= 0 || p.nbatch > 1 || p.tri != TRI_UPPER ||
      p.krange != KR_ALL || p.kb != 0 || p.M != p.N)
    return false;
  if (p.lda % 4 != 0 || (reinterpret_cast<uintptr_t>(p.A) & 15) != 0) return false;
  return static_cast<uint64_t>(p.ke) * p.lda * 4 < (uint64_t(1) << 32);
}

// Whether the 256 x 256 direct-to-LDS kernel takes problem `p` (see the
// kernel's comment); b16 is set to the OP_MN B load width it needs.
bool dma_eligible(const GemmProb& p, int am, int bm, int epi, bool& b16) {
  const bool combo = (am == OP_K && bm == OP_MN && epi == EPI_STORE) ||
                     (am == OP_MN && bm == OP_MN && (epi == EPI_UPDATE || epi == EPI_STORE || epi == EPI_SUB)) ||
                     (am == OP_K && bm == OP_K && (epi == EPI_SUB || epi == EPI_STORE)) ||
                     (am == OP_MN && bm == OP_K && epi == EPI_STORE);
  if (!combo || p.nsplit > 1 || p.b_special >= 0) return false;
  if (p.a_special >= 0 && !(am == OP_K && epi == EPI_STORE && p.krange == KR_ALL && p.a_special == p.ke - 1 &&
                            p.A_extra != nullptr))
    return false;
  const int kend = p.a_special >= 0 ? p.a_special : p.ke;
  if (p.kb < 0 || p.kb % kDK != 0 || kend % kDK != 0 || kend <= p.kb) return false;
  if (p.nbatch > 1 && p.split_stride % 4 != 0) return false;
  const auto al = [](const void* q, uintptr_t a) { return (reinterpret_cast<uintptr_t>(q) & (a - 1)) == 0; };
  // 16-byte loads: aligned rows, and an operand's last element ends a 16-byte chunk
  if (p.lda % 4 != 0 || !al(p.A, 16) || (am == OP_MN && p.M % 4 != 0)) return false;
  if (bm == OP_K) {
    if (p.ldb % 4 != 0 || !al(p.B, 16)) return false;
    b16 = true;
  } else if (p.ldb % 4 == 0 && al(p.B, 16) && p.N % 4 == 0) {
    b16 = true;
  } else if (am == OP_K && epi == EPI_STORE && al(p.B, 4)) {
    b16 = false;
  } else {
    return false;
  }
  const uint64_t ea = am == OP_MN ? operand_extent(kend, p.lda, p.M) : operand_extent(p.M, p.lda, kend);
  const uint64_t eb = bm == OP_MN ? operand_extent(kend, p.ldb, p.N) : operand_extent(p.N, p.ldb, kend);
  return ea < (uint64_t(1) << 32) && eb < (uint64_t(1) << 32);
}

int tiles_for(const GemmProb& p, int bt) {
  const int tm = (p.M + bt - 1) / bt, tn = (p.N + bt - 1) / bt;
  const int per = p.tri == TRI_FULL ? tm * tn : tm * (tm + 1) / 2;
  return per * std::max(1, p.nsplit) * std::max<int>(1, p.nbatch);
}

}  // namespace

bool gemm_nchw_syrk_ok(const void* X, int64_t rows, int hw, int d) {
  return hw > 0 && hw % kSK == 0 && rows % hw == 0 && rows >= kDmaSyrkMinRows && d > 0 &&
         (reinterpret_cast<uintptr_t>(X) & 15) == 0 &&
         (static_cast<uint64_t>(rows) * d + static_cast<uint64_t>(128) * hw) * 4 < (uint64_t(1) << 32);
}

void gemm_set_tiles(GemmProb& p) {
  p.tiles_m = (p.M + kTile - 1) / kTile;
  p.tiles_n = (p.N + kTile - 1) / kTile;
}

int gemm_blocks(const GemmProb& p) { return tiles_for(p, kTile); }

namespace {

// contraction length of one workgroup of `p`
int64_t block_k(const GemmProb& p) {
  const int64_t k = std::max(0, p.ke - p.kb);
  return (k + std::max(1, p.nsplit) - 1) / std::max(1, p.nsplit);
}

kfac_status_t launch_with(std::vector<GemmProb>& probs, int amode, int bmode, int epi, const GemmScalars& sc,
                          hipStream_t stream, bool big, bool dma = false, bool b16 = false) {
  const int bt = big ? 2 * kTile : kTile;
  std::vector<GemmProb> ps;
  for (GemmProb p : probs) {
    if (p.nsplit < 1) p.nsplit = 1;
    if (p.nbatch < 1) p.nbatch = 1;
    p.tiles_m = (p.M + bt - 1) / bt;
    p.tiles_n = (p.N + bt - 1) / bt;
    p.a_vec = (p.lda % 4) == 0 && (reinterpret_cast<uintptr_t>(p.A) % 16) == 0 && (p.kb % 4) == 0;
    p.b_vec = (p.ldb % 4) == 0 && (reinterpret_cast<uintptr_t>(p.B) % 16) == 0 && (p.kb % 4) == 0;
    if (tiles_for(p, bt) > 0) ps.push_back(p);
  }
  // longest workgroups first, so a launch ends on short ones
  std::stable_sort(ps.begin(), ps.end(),
                   [](const GemmProb& a, const GemmProb& b) { return block_k(a) > block_k(b); });
  // greedy balance of the work over the fewest launches the table size allows
  const size_t nl = (ps.size() + kMaxGemmProbs - 1) / kMaxGemmProbs;
  std::vector<GemmBatch> batches(nl);
  std::vector<double> work(nl, 0.0);
  std::vector<int> blocks(nl, 0);
  for (const GemmProb& p : ps) {
    size_t best = nl;
    for (size_t l = 0; l < nl; ++l)
      if (batches[l].n < kMaxGemmProbs && (best == nl || work[l] < work[best])) best = l;
    GemmBatch& b = batches[best];
    GemmProb q = p;
    const int nb = tiles_for(q, bt);
    q.blk_begin = blocks[best];
    blocks[best] += nb;
    work[best] += static_cast<double>(nb) * static_cast<double>(block_k(q));
    b.p[b.n++] = q;
  }
  for (size_t l = 0; l < nl; ++l) {
    batches[l].sc = sc;
    kfac_status_t st = dma ? dispatch_dma(batches[l], blocks[l], amode, bmode, epi, b16, stream)
                           : dispatch(batches[l], blocks[l], big, amode, bmode, epi, stream);
    if (st != KFAC_OK) return st;
  }
  return KFAC_OK;
}

}  // namespace

kfac_status_t launch_gemm(std::vector<GemmProb>& probs, int amode, int bmode, int epi, const GemmScalars& sc,
                          hipStream_t stream, int policy) {
  if (policy == TILES_SMALL && epi == EPI_SYRK && amode == OP_MN && bmode == OP_MN) {
    std::vector<GemmProb> dma, nchw, rest;
    for (const GemmProb& p : probs) (p.nchw ? nchw : dma_syrk_eligible(p) ? dma : rest).push_back(p);
    kfac_status_t st = dma.empty() ? KFAC_OK : launch_with(dma, amode, bmode, epi, sc, stream, false, true);
    if (st == KFAC_OK && !nchw.empty()) st = launch_with(nchw, amode, bmode, epi, sc, stream, false, true);
    if (st != KFAC_OK) return st;
    return rest.empty() ? KFAC_OK : launch_with(rest, amode, bmode, epi, sc, stream, false);
  }
  if (policy == TILES_SMALL) return launch_with(probs, amode, bmode, epi, sc, stream, false);
  if (policy == TILES_PER_PROBLEM) {
    std::vector<GemmProb> big, small;
    // 256 x 256 tiles only where they add no padding over 128 x 128 tiles
    auto pad = [](int x, int t) { return (x + t - 1) / t * t; };
    for (const GemmProb& p : probs) {
      const bool b = p.M >= kBigMin && p.N >= kBigMin && pad(p.M, 2 * kTile) == pad(p.M, kTile) &&
                     pad(p.N, 2 * kTile) == pad(p.N, kTile);
      (b ? big : small).push_back(p);
    }
    kfac_status_t st = big.empty() ? KFAC_OK : launch_with(big, amode, bmode, epi, sc, stream, true);
    if (st != KFAC_OK) return st;
    return small.empty() ? KFAC_OK : launch_with(small, amode, bmode, epi, sc, stream, false);
  }
  // 256 x 256 tiles when the launch still has at least two tiles per CU;
  // then the problems the direct-to-LDS kernel can load go to it
  int big_tiles = 0;
  for (const GemmProb& p : probs) big_tiles += tiles_for(p, 2 * kTile);
  if (big_tiles < 512) return launch_with(probs, amode, bmode, epi, sc, stream, false);
  std::vector<GemmProb> dma16, dma4, rest;
  for (const GemmProb& p : probs) {
    bool b16 = true;
    (dma_eligible(p, amode, bmode, epi, b16) ? (b16 ? dma16 : dma4) : rest).push_back(p);
  }
  kfac_status_t st = dma16.empty() ? KFAC_OK : launch_with(dma16, amode, bmode, epi, sc, stream, true, true, true);
  if (st == KFAC_OK && !dma4.empty()) st = launch_with(dma4, amode, bmode, epi, sc, stream, true, true, false);
  if (st != KFAC_OK) return st;
  return rest.empty() ? KFAC_OK : launch_with(rest, amode, bmode, epi, sc, stream, true);
}

}  // namespace kfac
