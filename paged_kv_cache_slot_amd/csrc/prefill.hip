// Varlen chunked-prefill attention (placeholder until the MFMA kernel lands).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

size_t prefill_workspace_bytes(int, int, int, int, int, int) { return 0; }

hipError_t launch_prefill(const PrefillArgs&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace pa
