// fp32 decode split pass in compose-on-read mode (the comparator that caches the
// raw K_i, V_i and K_1, V_1 and forms K', V' per row).

#include "decode_kernel.h"

namespace yoco {

hipError_t launch_decode_compose_on_read(const DecodeParams& p, hipStream_t stream) {
  return launch_mode<kComposeOnRead>(p, stream);
}

}  // namespace yoco
