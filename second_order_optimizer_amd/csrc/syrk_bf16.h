// Factor SYRK for bfloat16 activations / gradients on bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
#pragma once

#include "common.h"

namespace kfac {

// Upper 128 x 128 tiles of X^T X over rows [0, rows), X = [rows, width]
// row-major bf16 with a virtual constant-1 column at index `special` (-1:
// none), so the result is d x d.
//   nsplit == 1: C <- beta C + alpha acc, mirrored into the lower triangle
//   nsplit  > 1: split s stores its raw sum into C + s * split_stride
kfac_status_t launch_syrk_bf16(const uint16_t* X, int width, int64_t rows, int d, int special, float* C,
                               float alpha, float beta, int nsplit, int64_t split_stride, hipStream_t st);

}  // namespace kfac
