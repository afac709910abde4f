// Factor SYRK + EMA for bfloat16 activations / gradients on bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate), batched over factors.
#pragma once

#include <vector>

#include "common.h"

namespace kfac {

// One factor: F <- beta F + alpha X^T X (both triangles written), where
// X = [rows, width] row-major bf16.  With `bias`, F is (width + 1)^2 and the
// last row / column is the EMA of the column sums (the constant-1 input), and
// F[width][width] += alpha * rows.  With `packed`, F holds only the upper
// triangle, row after row (packed_index).
struct SyrkBf16Prob {
  const uint16_t* X;
  float* F;
  int64_t rows;
  int32_t width;
  int32_t bias;
  float alpha, beta;
  int32_t packed;
  int32_t pad_;
};

kfac_status_t launch_syrk_bf16(const std::vector<SyrkBf16Prob>& probs, hipStream_t st);

}  // namespace kfac
