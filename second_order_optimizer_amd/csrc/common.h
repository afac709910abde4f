// Internal declarations shared by the library's translation units.
// Everything here is gfx950 (CDNA4) code: 64-lane wavefronts, MFMA, 160 KB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <vector>

#include "../../include/kfac.h"

namespace kfac {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

// Workspace layout: [0, 256) flag word (+ padding); then regions carved by the
// planner, each 256-byte aligned.
constexpr size_t kFlagBytes = 256;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Sets `bits` in the workspace flag word.  Called by one lane.
__device__ inline void raise_flag(uint32_t* flags, uint32_t bits) { atomicOr(flags, bits); }

// A (workgroup-uniform) kernel-argument value held in a scalar register for
// the rest of the kernel.  The compiler otherwise treats argument loads as
// free to repeat and re-reads a table entry's fields at each use, each read
// waited for on its own: a serial chain of scalar-memory round trips, most
// costly in epilogues, where every wavefront of a workgroup runs it at once.
template <typename T>
__device__ inline T arg_reg(T v) {
  asm volatile("" : "+s"(v));
  return v;
}
// Pointers come from global-memory arguments: that is restated after the
// register pin (which hides it), so that accesses through them stay global
// loads and stores rather than flat ones (a flat load also holds up every
// wait for LDS reads until it returns).
template <typename T>
__device__ inline T* arg_reg(T* v) {
  uint64_t u = reinterpret_cast<uint64_t>(v);
  asm volatile("" : "+s"(u));
  return (T*)reinterpret_cast<__attribute__((address_space(1))) T*>(u);
}

// Packed upper-triangle storage of a symmetric d x d factor: element (i, j),
// i <= j, at i d - i (i - 1) / 2 + (j - i) (rows of the upper triangle one
// after the other).
__host__ __device__ inline int64_t packed_index(int64_t i, int64_t j, int64_t d) {
  return i * (2 * d - i + 1) / 2 + (j - i);
}

__device__ inline float bf16_bits_to_float(unsigned short u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

#define KFAC_HIP_TRY(expr)                                  \
  do {                                                      \
    hipError_t _e = (expr);                                 \
    if (_e != hipSuccess) return KFAC_ERR_HIP;              \
  } while (0)

// ---------------------------------------------------------------------------
// host-side helpers shared by the launchers

struct LayerGeom {
  int64_t rows;
  int d_in, d_out, d_a;
  bool conv, bias, bn, packed;
  int batch, c_in, h, w, kh, kw, stride, pad, h_out, w_out;
};

LayerGeom geom_of(const kfac_layer_t& L);

// weight rescaling (rescale.hip): W <- W sqrt(2 d_out) / (||W||_F + eps) for
// every listed weight; `part` holds rescale_blocks(n) floats of workspace.
struct RescaleSeg {
  float* w;
  float* part;
  int64_t n;
  int32_t d_out;
};
int64_t rescale_blocks(int64_t n);
kfac_status_t launch_rescale(const std::vector<RescaleSeg>& segs, float eps, hipStream_t st);

// diag method (diag.hip)
size_t diag_workspace_bytes(const kfac_layer_t* layers, int n);
kfac_status_t diag_enqueue(const kfac_layer_t* layers, int n, const kfac_hparams_t& hp, char* ws,
                           size_t ws_bytes, hipStream_t stream, int phases);
// The diagonal step with its scratch in a device array of the library (at most
// kNoAllocScratchBytes; larger stacks get KFAC_ERR_WORKSPACE) and the flag
// word at `flags`; allocates no device memory.
constexpr size_t kNoAllocScratchBytes = KFAC_NOALLOC_SCRATCH_BYTES;
kfac_status_t diag_enqueue_noalloc(const kfac_layer_t* layers, int n, const kfac_hparams_t& hp, uint32_t* flags,
                                   hipStream_t stream, int phases);
// The diagonal step with its workspace regions carved from `ws` (the first
// kFlagBytes of it unused) and the flag word at `flags` (the full method runs
// its batch-norm layers through this).
kfac_status_t diag_enqueue_into(const kfac_layer_t* layers, int n, const kfac_hparams_t& hp, char* ws,
                                size_t ws_bytes, uint32_t* flags, hipStream_t stream, int phases);

// full method (full.hip)
size_t full_workspace_bytes(const kfac_layer_t* layers, int n);
kfac_status_t full_enqueue(const kfac_layer_t* layers, int n, const kfac_hparams_t& hp, char* ws,
                           size_t ws_bytes, hipStream_t stream, int phases);

}  // namespace kfac
