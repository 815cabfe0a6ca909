// Backward of the KV composition of one lower-half layer (YOCO++ technical
// summary, section 2: the four residual weights are learnable; key technical
// innovation 2: lambda scales them so that they learn). With
// K'_i = lambda (aK1 K_1 + aK2 K_i) and upstream gradients gk = dL/dK'_i:
//
//   dK_1 += c1 * gk,  dK_i = c2 * gk   (c = fl32(lambda * a), fp32),
//   daK1 = lambda * <gk, K_1>,  daK2 = lambda * <gk, K_i>,
//
// and likewise for V. HBM-bound: per element position it reads gk, gv, K_1,
// K_i, V_1, V_i, reads-modifies-writes the two accumulated fp32 gradients and
// writes the other two, all with nontemporal accesses. A thread handles four
// consecutive elements, so that every access instruction of a wavefront
// covers one contiguous span (a store pattern that leaves holes in each
// 32-byte sector is written back sector by sector, doubling the write
// traffic). The weight gradients are dot products over all positions: each
// workgroup writes its four fp32 partial sums, and a second kernel adds the
// partials in a fixed order in fp64 (deterministic).

#include <type_traits>

#include <hip/hip_runtime.h>

#include "common.h"
#include "compose_math.h"
#include "fastdiv.h"

namespace yoco {
namespace {

constexpr int kThreads = kBackwardThreads;
constexpr int kVecPerThread = kBackwardVecPerThread;   // four-element vectors per thread, loads issued together
constexpr int kFinishThreads = 1024;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool BF16>
struct Src {
  typedef typename std::conditional<BF16, u32x2, u32x4>::type vec;   // four stored elements
  static constexpr int kES = BF16 ? 2 : 4;
  __device__ __forceinline__ static f32x4 unpack(const vec& w) {
    f32x4 x;
    if constexpr (BF16) {
      x[0] = bf16_lo(w[0]);
      x[1] = bf16_hi(w[0]);
      x[2] = bf16_lo(w[1]);
      x[3] = bf16_hi(w[1]);
    } else {
      x[0] = __uint_as_float(w[0]);
      x[1] = __uint_as_float(w[1]);
      x[2] = __uint_as_float(w[2]);
      x[3] = __uint_as_float(w[3]);
    }
    return x;
  }
};

__device__ __forceinline__ int64_t off(const View4& v, int b, int h, int t) {
  return (int64_t)b * v.sb + (int64_t)h * v.sh + (int64_t)t * v.st;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void compose_backward_kernel(ComposeBackwardParams p, uint32_t cpr,
                                                                    uint32_t total, FastDiv dc, FastDiv dh,
                                                                    FastDiv dn, float* __restrict__ partial) {
  using SV = Src<BF16>;
  using vec = typename SV::vec;
  float sk1 = 0.f, ski = 0.f, sv1 = 0.f, svi = 0.f;
  const uint32_t first = blockIdx.x * (kThreads * kVecPerThread) + threadIdx.x;
  vec gk[kVecPerThread], gv[kVecPerThread], k1[kVecPerThread], ki[kVecPerThread], v1[kVecPerThread],
      vi[kVecPerThread];
  f32x4 a1[kVecPerThread], b1[kVecPerThread];
  f32x4* dk1p[kVecPerThread];
  f32x4* dv1p[kVecPerThread];
  f32x4* dkip[kVecPerThread];
  f32x4* dvip[kVecPerThread];
  bool live[kVecPerThread];
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const uint32_t idx = first + u * kThreads;
    live[u] = idx < total;
    const uint32_t i = live[u] ? idx : total - 1;     // clamped: loads stay in bounds, results unused
    const uint32_t r0 = fdiv(i, dc);
    const uint32_t c = i - r0 * cpr;
    const uint32_t r1 = fdiv(r0, dh);
    const int h = (int)(r0 - r1 * (uint32_t)p.Hkv);
    const uint32_t r2 = fdiv(r1, dn);
    const int t = (int)(r1 - r2 * (uint32_t)p.n);
    const int b = (int)r2;
    auto ld = [&](const View4& v, int row) {
      return __builtin_nontemporal_load(reinterpret_cast<const vec*>(static_cast<const char*>(v.ptr) +
                                                                     off(v, b, h, row) * SV::kES) + c);
    };
    gk[u] = ld(p.gk, p.t0 + t);
    gv[u] = ld(p.gv, p.t0 + t);
    k1[u] = ld(p.k1, t);
    ki[u] = ld(p.ki, t);
    v1[u] = ld(p.v1, t);
    vi[u] = ld(p.vi, t);
    auto gp = [&](const View4& v) {
      return reinterpret_cast<f32x4*>(static_cast<char*>(const_cast<void*>(v.ptr)) + off(v, b, h, t) * 4) + c;
    };
    dk1p[u] = gp(p.dk1);
    dv1p[u] = gp(p.dv1);
    dkip[u] = gp(p.dki);
    dvip[u] = gp(p.dvi);
    a1[u] = __builtin_nontemporal_load(dk1p[u]);
    b1[u] = __builtin_nontemporal_load(dv1p[u]);
  }
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const f32x4 g = SV::unpack(gk[u]), h = SV::unpack(gv[u]);
    const f32x4 x1 = SV::unpack(k1[u]), xi = SV::unpack(ki[u]), y1 = SV::unpack(v1[u]), yi = SV::unpack(vi[u]);
    f32x4 ak, bv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (live[u]) {
        sk1 = __builtin_fmaf(g[e], x1[e], sk1);
        ski = __builtin_fmaf(g[e], xi[e], ski);
        sv1 = __builtin_fmaf(h[e], y1[e], sv1);
        svi = __builtin_fmaf(h[e], yi[e], svi);
      }
      a1[u][e] = __builtin_fmaf(p.cK1, g[e], a1[u][e]);
      b1[u][e] = __builtin_fmaf(p.cV1, h[e], b1[u][e]);
      ak[e] = p.cK2 * g[e];
      bv[e] = p.cV2 * h[e];
    }
    if (live[u]) {
      __builtin_nontemporal_store(a1[u], dk1p[u]);
      __builtin_nontemporal_store(b1[u], dv1p[u]);
      __builtin_nontemporal_store(ak, dkip[u]);
      __builtin_nontemporal_store(bv, dvip[u]);
    }
  }
  // workgroup sums of the four dot products
  __shared__ float red[kThreads / 64][4];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    sk1 += __shfl_xor(sk1, o);
    ski += __shfl_xor(ski, o);
    sv1 += __shfl_xor(sv1, o);
    svi += __shfl_xor(svi, o);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[wave][0] = sk1;
    red[wave][1] = ski;
    red[wave][2] = sv1;
    red[wave][3] = svi;
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) s += red[w][threadIdx.x];
    partial[blockIdx.x * 4 + threadIdx.x] = s;
  }
}

// dalpha[k] = lambda * sum over workgroups of partial[wg][k], summed in fp64 in a fixed order.
__global__ __launch_bounds__(kFinishThreads) void compose_backward_finish(const float* __restrict__ partial,
                                                                         int nblocks, float lambda,
                                                                         float* __restrict__ dalpha) {
  __shared__ double red[kFinishThreads / 64][4];
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  for (int i = threadIdx.x; i < nblocks; i += kFinishThreads) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(partial + 4 * (size_t)i);
#pragma unroll
    for (int k = 0; k < 4; ++k) s[k] += (double)v[k];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s[k] += __shfl_xor(s[k], o);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0)
#pragma unroll
    for (int k = 0; k < 4; ++k) red[wave][k] = s[k];
  __syncthreads();
  if (threadIdx.x < 4) {
    double t = 0.0;
    for (int w = 0; w < kFinishThreads / 64; ++w) t += red[w][threadIdx.x];
    dalpha[threadIdx.x] = (float)((double)lambda * t);
  }
}

}  // namespace

hipError_t launch_compose_backward(const ComposeBackwardParams& p, bool bf16, float* partial, hipStream_t stream) {
  const uint32_t cpr = (uint32_t)(p.D / 4);
  const uint32_t total = (uint32_t)((uint64_t)p.B * p.n * p.Hkv * cpr);
  const int nb = compose_backward_blocks(p);
  const FastDiv dc = make_fastdiv(cpr), dh = make_fastdiv((uint32_t)p.Hkv), dn = make_fastdiv((uint32_t)p.n);
  if (bf16)
    compose_backward_kernel<true><<<nb, kThreads, 0, stream>>>(p, cpr, total, dc, dh, dn, partial);
  else
    compose_backward_kernel<false><<<nb, kThreads, 0, stream>>>(p, cpr, total, dc, dh, dn, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  compose_backward_finish<<<1, kFinishThreads, 0, stream>>>(partial, nb, p.lambda, p.dalpha);
  return hipGetLastError();
}

}  // namespace yoco
