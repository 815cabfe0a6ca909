// Shared host-side definitions of the gfx950 HIP path: launch parameters and
// launcher declarations (no oracle code here). Host code only, so that the C
// ABI layer builds with any C++ compiler.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace yoco {

// Device view of a 4-D tensor: element (b, h, t, 0) at ptr + b*sb + h*sh + t*st.
struct View4 {
  const void* ptr;
  int64_t sb, sh, st;
};

// ----------------------------------------------------------------- launchers
// Each returns hipSuccess or the error of the launch (hipGetLastError).

struct ComposeParams {
  View4 k1, ki, v1, vi;  // sources, rows [0, n)
  View4 kc, vc;          // caches, rows [t0, t0 + n)
  int t0, B, n, Hkv, D;
  float cK1, cK2, cV1, cV2;  // lambda folded into the weights (fp32)
};
hipError_t launch_compose(const ComposeParams& p, bool bf16, hipStream_t stream);

// Which terms of a composition are present: 3 = both, 2 = only X_i, 1 = only
// X_1, 0 = none (a zero coefficient drops its term and its read).
inline int compose_terms(float c1, float c2) { return (c1 != 0.f ? 1 : 0) | (c2 != 0.f ? 2 : 0); }

struct ComposeBackwardParams {
  View4 gk, gv;              // upstream gradients of K', V' (rows [t0, t0 + n)), cache dtype
  View4 k1, ki, v1, vi;      // forward sources (rows [0, n)), cache dtype
  View4 dk1, dki, dv1, dvi;  // fp32 gradients (rows [0, n)): dk1, dv1 accumulated, dki, dvi written
  int t0, B, n, Hkv, D;
  float cK1, cK2, cV1, cV2;  // lambda folded into the weights (fp32)
  float lambda;
  float* dalpha;             // [4] fp32: daK1, daK2, daV1, daV2
};
// Launch shape of the backward: kBackwardThreads threads per workgroup, each
// handling kBackwardVecPerThread four-element vectors.
constexpr int kBackwardThreads = 256;
constexpr int kBackwardVecPerThread = 4;
inline int compose_backward_blocks(const ComposeBackwardParams& p) {
  const uint64_t total = (uint64_t)p.B * p.n * p.Hkv * (p.D / 4);
  return (int)((total + kBackwardThreads * kBackwardVecPerThread - 1) / (kBackwardThreads * kBackwardVecPerThread));
}
hipError_t launch_compose_backward(const ComposeBackwardParams& p, bool bf16, float* partial, hipStream_t stream);

struct DecodeParams {
  const void* q;          // [B, Hq, D]
  View4 k, v;             // caches
  const int32_t* seq_lens;
  int B, T, Hq, Hkv, D;
  float scale_log2;       // softmax scale * log2(e)
  int num_splits;
  int rows_per_split;
  int waves;              // wavefronts per workgroup: 4 or 8
  bool prefetch;          // double-buffered row loads (short splits)
  float* out;             // [B, Hq, D] (used when num_splits == 1)
  float* lse;             // [B, Hq] or null (used when num_splits == 1)
  float* part_o;          // [B, Hq, S, D]   (used when num_splits > 1)
  float* part_lse;        // [B, Hq, S]
  unsigned* tickets;      // [B, Hkv] zero-initialised counters, or null (no fused merge)
  // Compose on read (the comparator that caches the raw K_i, V_i): when set, k and
  // v are layer i's raw caches and k1, v1 layer 1's; K' and V' are formed per row.
  bool compose_on_read;
  View4 k1, v1;
  // Self-decoder step (append): the new token's source rows, read at row
  // seq_len - 1 of each view (stride_t = 0 for a one-token buffer); the composed
  // row is written into k, v at that row. Shares the folded weights below.
  bool append;
  View4 nk1, nki, nv1, nvi;
  float cK1, cK2, cV1, cV2;
  int termsK, termsV;
};
hipError_t launch_decode_partial(const DecodeParams& p, bool bf16, hipStream_t stream);
hipError_t launch_decode_merge(const float* part_o, const float* part_lse, int B, int Hq, int D, int S,
                               float* out, float* lse, hipStream_t stream);

struct PrefillParams {
  const void* q;   // [B, C, Hq, D] bf16
  View4 k, v;      // bf16 caches
  int B, C, p0, Hq, Hkv, D;
  float scale_log2;
  void* out;       // [B, C, Hq, D]
  bool out_bf16;
  float* lse;      // [B, Hq, C] or null
};
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

// Device address of the allocation-free decode's scratch array on the current
// GPU (YOCO_NOALLOC_SCRATCH_BYTES bytes, the first YOCO_NOALLOC_COUNTER_BYTES
// of them merge counters). The first call on a device looks it up and clears
// the counters with a kernel on `stream`.
hipError_t noalloc_scratch(hipStream_t stream, char** ptr);

}  // namespace yoco
