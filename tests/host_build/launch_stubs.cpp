// Test-only stand-ins for the GPU side of libyoco.so, so that the C ABI layer
// (yoco_api.cpp) builds and runs on a host with no GPU, under AddressSanitizer
// and UndefinedBehaviorSanitizer. Every launcher records the parameters it was
// given and returns the status the test driver sets (hipSuccess, or an error
// to check the YOCO_ERR_LAUNCH mapping). Nothing here touches a device.
#include <string.h>

#include "common.h"
#include "stubs.h"

namespace stubs {
hipError_t result = hipSuccess;
int launches = 0;
yoco::ComposeParams compose;
yoco::ComposeBackwardParams backward;
float* backward_partial = nullptr;
yoco::DecodeParams decode;
bool decode_bf16 = false;
yoco::PrefillParams prefill;
struct Merge merge;
char scratch_bytes[1 << 12];   // address handed out as the noalloc scratch (never dereferenced)
}  // namespace stubs

namespace yoco {

hipError_t launch_compose(const ComposeParams& p, bool, hipStream_t) {
  stubs::compose = p;
  ++stubs::launches;
  return stubs::result;
}

hipError_t launch_compose_backward(const ComposeBackwardParams& p, bool, float* partial, hipStream_t) {
  stubs::backward = p;
  stubs::backward_partial = partial;
  ++stubs::launches;
  return stubs::result;
}

hipError_t launch_decode_partial(const DecodeParams& p, bool bf16, hipStream_t) {
  stubs::decode = p;
  stubs::decode_bf16 = bf16;
  ++stubs::launches;
  return stubs::result;
}

hipError_t launch_decode_merge(const float* part_o, const float* part_lse, int B, int Hq, int D, int S, float* out,
                               float* lse, hipStream_t) {
  stubs::merge = {part_o, part_lse, B, Hq, D, S, out, lse};
  ++stubs::launches;
  return stubs::result;
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t) {
  stubs::prefill = p;
  ++stubs::launches;
  return stubs::result;
}

hipError_t noalloc_scratch(hipStream_t, char** ptr) {
  *ptr = stubs::scratch_bytes;
  return stubs::result;
}

}  // namespace yoco

extern "C" const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub launch error"; }
