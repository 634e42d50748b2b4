// Packed document-causal prefill (placeholder until the matrix-core kernel lands).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

hipError_t launch_prefill(const PrefillArgs &a, int32_t num_tiles_bound, hipStream_t stream) {
  (void)a;
  (void)num_tiles_bound;
  (void)stream;
  return hipErrorNotSupported;
}

}  // namespace pkv
