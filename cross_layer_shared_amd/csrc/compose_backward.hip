// Backward of the KV composition of one lower-half layer (YOCO++ technical
// summary, section 2: the four residual weights are learnable; key technical
// innovation 2: lambda scales them so that they learn). With
// K'_i = lambda (aK1 K_1 + aK2 K_i) and upstream gradients gk = dL/dK'_i:
//
//   dK_1 += c1 * gk,  dK_i = c2 * gk   (c = fl32(lambda * a), fp32),
//   daK1 = lambda * <gk, K_1>,  daK2 = lambda * <gk, K_i>,
//
// and likewise for V. HBM-bound: per element position it reads gk, gv, K_1,
// K_i, V_1, V_i (nontemporal), reads-modifies-writes the two accumulated fp32
// gradients (temporal: a nontemporal read-modify-write measured slower on
// MI355X) and writes the other two (nontemporal). The weight gradients are
// dot products over all positions: each workgroup
// writes its four fp32 partial sums, and a second kernel adds the partials in
// a fixed order in fp64 (deterministic).

#include "common.h"
#include "compose_math.h"

namespace yoco {
namespace {

constexpr int kThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ const char* elem(const View4& v, int b, int h, int t, int es) {
  return static_cast<const char*>(v.ptr) + ((int64_t)b * v.sb + (int64_t)h * v.sh + (int64_t)t * v.st) * es;
}

// Unpack one 16-byte vector of stored values into fp32.
template <bool BF16>
__device__ __forceinline__ void unpack(const u32x4& w, float (&x)[BF16 ? 8 : 4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (BF16) {
      x[2 * j] = bf16_lo(w[j]);
      x[2 * j + 1] = bf16_hi(w[j]);
    } else {
      x[j] = __uint_as_float(w[j]);
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void compose_backward_kernel(ComposeBackwardParams p, uint32_t cpr,
                                                                    uint32_t total, float* __restrict__ partial) {
  constexpr int E = BF16 ? 8 : 4;      // elements per 16-byte source vector
  constexpr int ES = BF16 ? 2 : 4;
  float sk1 = 0.f, ski = 0.f, sv1 = 0.f, svi = 0.f;
  const uint32_t idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx < total) {
    const uint32_t c = idx % cpr;
    uint32_t r = idx / cpr;
    const int h = (int)(r % (uint32_t)p.Hkv);
    r /= (uint32_t)p.Hkv;
    const int t = (int)(r % (uint32_t)p.n);
    const int b = (int)(r / (uint32_t)p.n);
    auto ld = [&](const View4& v, int row) {
      return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(elem(v, b, h, row, ES)) + c);
    };
    float gk[E], gv[E], k1[E], ki[E], v1[E], vi[E];
    unpack<BF16>(ld(p.gk, p.t0 + t), gk);
    unpack<BF16>(ld(p.gv, p.t0 + t), gv);
    unpack<BF16>(ld(p.k1, t), k1);
    unpack<BF16>(ld(p.ki, t), ki);
    unpack<BF16>(ld(p.v1, t), v1);
    unpack<BF16>(ld(p.vi, t), vi);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      sk1 = __builtin_fmaf(gk[e], k1[e], sk1);
      ski = __builtin_fmaf(gk[e], ki[e], ski);
      sv1 = __builtin_fmaf(gv[e], v1[e], sv1);
      svi = __builtin_fmaf(gv[e], vi[e], svi);
    }
    // fp32 gradients: E elements = E/4 vectors of 4 floats
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
      f32x4* dk1 = reinterpret_cast<f32x4*>(const_cast<char*>(elem(p.dk1, b, h, t, 4))) + c * (E / 4) + q;
      f32x4* dki = reinterpret_cast<f32x4*>(const_cast<char*>(elem(p.dki, b, h, t, 4))) + c * (E / 4) + q;
      f32x4* dv1 = reinterpret_cast<f32x4*>(const_cast<char*>(elem(p.dv1, b, h, t, 4))) + c * (E / 4) + q;
      f32x4* dvi = reinterpret_cast<f32x4*>(const_cast<char*>(elem(p.dvi, b, h, t, 4))) + c * (E / 4) + q;
      f32x4 a1 = *dk1, b1 = *dv1, ak, bv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a1[e] = __builtin_fmaf(p.cK1, gk[4 * q + e], a1[e]);
        b1[e] = __builtin_fmaf(p.cV1, gv[4 * q + e], b1[e]);
        ak[e] = p.cK2 * gk[4 * q + e];
        bv[e] = p.cV2 * gv[4 * q + e];
      }
      *dk1 = a1;
      *dv1 = b1;
      __builtin_nontemporal_store(ak, dki);
      __builtin_nontemporal_store(bv, dvi);
    }
  }
  // workgroup sums of the four dot products
  __shared__ float red[kThreads / 64][4];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    sk1 += __shfl_xor(sk1, off);
    ski += __shfl_xor(ski, off);
    sv1 += __shfl_xor(sv1, off);
    svi += __shfl_xor(svi, off);
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
__global__ __launch_bounds__(kThreads) void compose_backward_finish(const float* __restrict__ partial, int nblocks,
                                                                    float lambda, float* __restrict__ dalpha) {
  __shared__ double red[kThreads][4];
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  for (int i = threadIdx.x; i < nblocks; i += kThreads)
#pragma unroll
    for (int k = 0; k < 4; ++k) s[k] += (double)partial[i * 4 + k];
#pragma unroll
  for (int k = 0; k < 4; ++k) red[threadIdx.x][k] = s[k];
  __syncthreads();
  for (int stride = kThreads / 2; stride > 0; stride >>= 1) {
    if ((int)threadIdx.x < stride)
#pragma unroll
      for (int k = 0; k < 4; ++k) red[threadIdx.x][k] += red[threadIdx.x + stride][k];
    __syncthreads();
  }
  if (threadIdx.x < 4) dalpha[threadIdx.x] = (float)((double)lambda * red[0][threadIdx.x]);
}

}  // namespace

int compose_backward_blocks(const ComposeBackwardParams& p, bool bf16) {
  const uint64_t cpr = (uint64_t)p.D * (bf16 ? 2 : 4) / 16;
  const uint64_t total = (uint64_t)p.B * p.n * p.Hkv * cpr;
  return (int)((total + kThreads - 1) / kThreads);
}

hipError_t launch_compose_backward(const ComposeBackwardParams& p, bool bf16, float* partial, hipStream_t stream) {
  const uint32_t cpr = (uint32_t)(p.D * (bf16 ? 2 : 4) / 16);
  const uint32_t total = (uint32_t)((uint64_t)p.B * p.n * p.Hkv * cpr);
  const int nb = compose_backward_blocks(p, bf16);
  if (bf16)
    compose_backward_kernel<true><<<nb, kThreads, 0, stream>>>(p, cpr, total, partial);
  else
    compose_backward_kernel<false><<<nb, kThreads, 0, stream>>>(p, cpr, total, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  compose_backward_finish<<<1, kThreads, 0, stream>>>(partial, nb, p.lambda, p.dalpha);
  return hipGetLastError();
}

}  // namespace yoco
