// Decode attention: the plain split pass (over a composed cache), the
// dispatch to the other modes and the standalone merge. The kernels are in
// decode_kernel.h.

#include "decode_kernel.h"

namespace yoco {

hipError_t launch_decode_partial(const DecodeParams& p, bool bf16, hipStream_t stream) {
  if (p.append) return launch_decode_append(p, bf16, stream);
  if (p.compose_on_read) return launch_decode_compose_on_read(p, bf16, stream);
  if (bf16) return launch_decode_mfma(p, stream);
  return launch_mode<kPlain>(p, bf16, stream);
}

hipError_t launch_decode_merge(const float* part_o, const float* part_lse, int B, int Hq, int D, int S, float* out,
                               float* lse, hipStream_t stream) {
  // heads are merged four at a time when Hq allows it (one workgroup each)
  const int G = (Hq % 4 == 0) ? 4 : 1;
  dim3 grid(B * Hq / G);
  if (D == 64) {
    if (G == 4) decode_merge_kernel<64, 4><<<grid, kThreads, 0, stream>>>(part_o, part_lse, S, out, lse);
    else decode_merge_kernel<64, 1><<<grid, kThreads, 0, stream>>>(part_o, part_lse, S, out, lse);
  } else {
    if (G == 4) decode_merge_kernel<128, 4><<<grid, kThreads, 0, stream>>>(part_o, part_lse, S, out, lse);
    else decode_merge_kernel<128, 1><<<grid, kThreads, 0, stream>>>(part_o, part_lse, S, out, lse);
  }
  return hipGetLastError();
}

}  // namespace yoco
