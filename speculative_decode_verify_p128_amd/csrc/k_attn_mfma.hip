// Matrix-core verify attention kernels (placeholder: not yet selected).
#include "device.h"
#include "internal.h"

namespace sdv {

bool mfma_supported(const AttnArgs&) { return false; }

hipError_t launch_attn_dense_mfma(const AttnArgs&, const DenseSource&, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_attn_sparse_mfma(const AttnArgs&, const SparseSource&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace sdv
