// Full K-FAC step launcher (placeholder until the factor, inverse and
// preconditioning kernels land).
#include "common.h"

namespace kfac {

size_t full_workspace_bytes(const kfac_layer_t*, int) { return kFlagBytes; }

kfac_status_t full_enqueue(const kfac_layer_t*, int, const kfac_hparams_t&, char*, size_t, hipStream_t, int) {
  return KFAC_ERR_UNSUPPORTED;
}

}  // namespace kfac
