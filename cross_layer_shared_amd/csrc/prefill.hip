// Causal chunked prefill (placeholder until the MFMA kernel lands).
#include "common.h"

namespace yoco {
hipError_t launch_prefill(const PrefillParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace yoco
