// Decode attention: the dispatch of the split pass (bf16 caches: the
// matrix-core kernel of decode_mfma.hip; fp32 caches: the vector-ALU kernel of
// decode_kernel.h in its three modes) and the standalone merge.

#include "decode_kernel.h"

namespace yoco {

hipError_t launch_decode_partial(const DecodeParams& p, bool bf16, hipStream_t stream) {
  if (bf16) return launch_decode_mfma(p, stream);   // every mode of a bf16 cache runs on the matrix cores
  if (p.append) return launch_mode<kAppend>(p, stream);
  if (p.compose_on_read) return launch_mode<kComposeOnRead>(p, stream);
  return launch_mode<kPlain>(p, stream);
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
