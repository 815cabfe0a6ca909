// fp32 decode split pass in append mode: one self-decoder decode step that composes
// the new token's K'_i, V'_i, writes them into the layer's cache and attends.

#include "decode_kernel.h"

namespace yoco {

hipError_t launch_decode_append(const DecodeParams& p, hipStream_t stream) {
  return launch_mode<kAppend>(p, stream);
}

}  // namespace yoco
