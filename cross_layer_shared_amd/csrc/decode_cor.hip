// Decode split pass in compose-on-read mode (the comparator that caches the
// raw K_i, V_i and K_1, V_1 and forms K', V' per row).

#include "decode_kernel.h"

namespace yoco {

hipError_t launch_decode_compose_on_read(const DecodeParams& p, bool bf16, hipStream_t stream) {
  if (bf16) return launch_decode_mfma(p, stream);   // the arithmetic of the composed-cache decode, row for row
  return launch_mode<kComposeOnRead>(p, bf16, stream);
}

}  // namespace yoco
