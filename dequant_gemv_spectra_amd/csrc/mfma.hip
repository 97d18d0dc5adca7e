// Batched SPECTRA product (placeholder until the MFMA tile kernel lands).
#include "spectra_internal.h"

namespace spectra {

bool mfma_supports(const DeviceView&, int64_t) { return false; }

hipError_t launch_mfma(const DeviceView&, const uint16_t*, uint16_t*, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace spectra
