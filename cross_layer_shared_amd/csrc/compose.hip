// Composition of a lower-half layer's cached KVs, written straight into the
// cache (YOCO++ technical summary, section 2, KV composition equations; key
// technical innovation 1: the composed K', V' are what is cached). The element
// arithmetic is compose_math.h's; a zero weight also drops its read.
//
// HBM-bound (0.5 flop per byte in bf16): every thread moves 16-byte vectors,
// K and V of the same position are handled by the same thread in one launch,
// and each thread handles one position (deeper unrolling measured slower on
// MI355X: fewer, longer-lived waves keep less in flight); nontemporal loads
// and stores (temporal ones measured at about half the bandwidth). A thread's
// (b, t, h, chunk) comes from its linear index by three divisions by
// runtime-invariant sizes, each done with one high multiply (+1-2% measured
// over the compiler's generic 32-bit division).

#include <hip/hip_runtime.h>

#include "common.h"
#include "compose_math.h"
#include "fastdiv.h"

namespace yoco {
namespace {

constexpr int kThreads = 512;   // measured: 512 > 256 (+4.6%) > 1024
constexpr int kUnroll = 1;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool BF16, int TERMS>
__device__ __forceinline__ u32x4 combine(u32x4 x1, u32x4 xi, float c1, float c2) {
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = compose_dword<BF16>(x1[j], xi[j], c1, c2, TERMS);
  return out;
}

struct Args {
  ComposeParams p;
  FastDiv dc, dh, dn;
  uint32_t cpr;     // 16-byte chunks per row (D * elemsize / 16)
  uint32_t total;   // B * n * Hkv * cpr
  int esize;        // bytes per element
};

__device__ __forceinline__ const u32x4* at(const View4& v, int b, int h, int t, uint32_t c, int es) {
  const char* base = static_cast<const char*>(v.ptr);
  int64_t e = (int64_t)b * v.sb + (int64_t)h * v.sh + (int64_t)t * v.st;
  return reinterpret_cast<const u32x4*>(base + e * es) + c;
}

template <bool BF16, int TK, int TV>
__global__ __launch_bounds__(kThreads) void compose_kernel(Args a) {
  const ComposeParams& p = a.p;
  u32x4 k1[kUnroll] = {}, ki[kUnroll] = {}, v1[kUnroll] = {}, vi[kUnroll] = {};
  uint32_t idx[kUnroll];
  const uint32_t base = (uint32_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;

  // Issue every load of the UNROLL positions first, then combine and store.
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    idx[u] = base + u * kThreads;
    if (idx[u] >= a.total) continue;
    const uint32_t r0 = fdiv(idx[u], a.dc);
    const uint32_t c = idx[u] - r0 * a.cpr;
    const uint32_t r1 = fdiv(r0, a.dh);
    const int h = (int)(r0 - r1 * (uint32_t)p.Hkv);
    const uint32_t r2 = fdiv(r1, a.dn);
    const int t = (int)(r1 - r2 * (uint32_t)p.n);
    const int b = (int)r2;
    if constexpr (TK & 1) k1[u] = __builtin_nontemporal_load(at(p.k1, b, h, t, c, a.esize));
    if constexpr (TK & 2) ki[u] = __builtin_nontemporal_load(at(p.ki, b, h, t, c, a.esize));
    if constexpr (TV & 1) v1[u] = __builtin_nontemporal_load(at(p.v1, b, h, t, c, a.esize));
    if constexpr (TV & 2) vi[u] = __builtin_nontemporal_load(at(p.vi, b, h, t, c, a.esize));
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    if (idx[u] >= a.total) continue;
    const uint32_t r0 = fdiv(idx[u], a.dc);
    const uint32_t c = idx[u] - r0 * a.cpr;
    const uint32_t r1 = fdiv(r0, a.dh);
    const int h = (int)(r0 - r1 * (uint32_t)p.Hkv);
    const uint32_t r2 = fdiv(r1, a.dn);
    const int t = (int)(r1 - r2 * (uint32_t)p.n);
    const int b = (int)r2;
    u32x4 ko = combine<BF16, TK>(k1[u], ki[u], p.cK1, p.cK2);
    u32x4 vo = combine<BF16, TV>(v1[u], vi[u], p.cV1, p.cV2);
    __builtin_nontemporal_store(ko, const_cast<u32x4*>(at(p.kc, b, h, p.t0 + t, c, a.esize)));
    __builtin_nontemporal_store(vo, const_cast<u32x4*>(at(p.vc, b, h, p.t0 + t, c, a.esize)));
  }
}

template <bool BF16, int TK>
hipError_t dispatch_v(const Args& a, int tv, dim3 grid, hipStream_t s) {
  switch (tv) {
    case 0: compose_kernel<BF16, TK, 0><<<grid, kThreads, 0, s>>>(a); break;
    case 1: compose_kernel<BF16, TK, 1><<<grid, kThreads, 0, s>>>(a); break;
    case 2: compose_kernel<BF16, TK, 2><<<grid, kThreads, 0, s>>>(a); break;
    default: compose_kernel<BF16, TK, 3><<<grid, kThreads, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

template <bool BF16>
hipError_t dispatch(const Args& a, int tk, int tv, dim3 grid, hipStream_t s) {
  switch (tk) {
    case 0: return dispatch_v<BF16, 0>(a, tv, grid, s);
    case 1: return dispatch_v<BF16, 1>(a, tv, grid, s);
    case 2: return dispatch_v<BF16, 2>(a, tv, grid, s);
    default: return dispatch_v<BF16, 3>(a, tv, grid, s);
  }
}

}  // namespace

hipError_t launch_compose(const ComposeParams& p, bool bf16, hipStream_t stream) {
  Args a;
  a.p = p;
  a.esize = bf16 ? 2 : 4;
  a.cpr = (uint32_t)(p.D * a.esize / 16);
  a.dc = make_fastdiv(a.cpr);
  a.dh = make_fastdiv((uint32_t)p.Hkv);
  a.dn = make_fastdiv((uint32_t)p.n);
  a.total = (uint32_t)((uint64_t)p.B * p.n * p.Hkv * a.cpr);
  dim3 grid((a.total + kThreads * kUnroll - 1) / (kThreads * kUnroll));
  int tk = compose_terms(p.cK1, p.cK2), tv = compose_terms(p.cV1, p.cV2);
  return bf16 ? dispatch<true>(a, tk, tv, grid, stream) : dispatch<false>(a, tk, tv, grid, stream);
}

}  // namespace yoco
