// bf16 MFMA FlashRelation forward (placeholder until the MFMA kernel lands).
#include "rel_internal.h"

namespace rel {

bool fwd_mfma_supported(int) { return false; }

hipError_t launch_fwd_mfma_bf16(const FwdArgs&, const HeadParams&, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace rel
