// Causal chunked prefill of a cross-decoder layer over the global cache
// (YOCO summary, abstract: the model behaves like a decoder-only
// Transformer, so the query at absolute position p attends to cache rows
// [0, p]; YOCO++ summary, section 3: prefill is compute-bound).
//
// Dense contraction on bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
// A workgroup of 4 wavefronts serves 4 (head, 32-query block) slots that share
// one kv head; it streams the cache in 64-key tiles staged through LDS, K
// row-major and V transposed, so that all four wavefronts read each tile
// from LDS instead of from memory.
//
// Per wavefront and tile:
//   S^T = K Q^T   (2 x 32 keys by 32 queries; D = 128 in 8 MFMA k-steps)
//   online softmax per query column, log2 domain, fp32
//   O^T += V^T P^T (4 x 32 dims by 32 queries; 64 keys in 4 MFMA k-steps)
// Computing the transposed products keeps every softmax statistic of a query
// inside one lane pair (lane j and j+32), and the S^T accumulator registers
// become the P^T operand of the PV product without leaving the lane: the key
// rows of each 32-key block are fed to the MFMA in the order that swaps bits 2
// and 3 of the key index, which makes the 8 P values a lane holds for one PV
// k-step 8 consecutive keys, i.e. one 16-byte read of the transposed V tile.
// Probabilities are rounded to bf16 for the PV product; the normaliser sums
// the same fp32 values.

#include <math.h>

#include "common.h"

namespace yoco {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQB = 32;               // queries per wavefront
constexpr int kKT = 64;               // keys per tile
constexpr int kKPad = kD + 8;         // K tile row stride (bf16 elements)
constexpr int kVPad = kKT + 8;        // transposed V tile row stride (bf16 elements)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Row of a 32-key block that MFMA row i carries: bits 2 and 3 swapped.
__device__ __forceinline__ int perm_key(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// max / sum with the partner lane (lane ^ 32)
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int HPW, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
  constexpr int WQ = kWaves / HPW;  // query blocks per workgroup
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[kKT * kKPad];
  __shared__ __attribute__((aligned(16))) __bf16 vt_lds[kD * kVPad];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 5;          // lane half
  const int j = lane & 31;          // query column of this lane
  const int n_qgroups = gridDim.x;
  const int qg = n_qgroups - 1 - (int)blockIdx.x;   // heaviest (latest) query blocks first
  const int h = blockIdx.y * HPW + (wave % HPW);
  const int g = (blockIdx.y * HPW) / (p.Hq / p.Hkv);
  const int b = blockIdx.z;
  const int c_wg = qg * (WQ * kQB);                 // first chunk row of the workgroup
  const int c_w = c_wg + (wave / HPW) * kQB;        // first chunk row of this wavefront
  const int c_hi = min(c_wg + WQ * kQB, p.C);       // workgroup rows end
  const int kv_len = p.p0 + c_hi;                   // keys any query of the workgroup can see
  const int n_tiles = (kv_len + kKT - 1) / kKT;

  // Q^T operand: lane (q, j) holds query row c_w + j, dims 16c + 8q .. +8.
  const int c_me = min(c_w + j, p.C - 1);
  const int pos = p.p0 + c_w + j;                   // absolute position of this lane's query
  bf16x8 qf[8];
  {
    const __bf16* qrow = static_cast<const __bf16*>(p.q) + (((size_t)b * p.C + c_me) * p.Hq + h) * kD + 8 * q;
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qrow + 16 * c);
  }

  // cooperative tile loads: thread t covers dims 8*(t%16) .. +8 of keys 4*(t/16) .. +4
  const int ld_d = 8 * (tid & 15);
  const int ld_k = 4 * (tid >> 4);
  const char* kbase = static_cast<const char*>(p.k.ptr) + ((int64_t)b * p.k.sb + (int64_t)g * p.k.sh + ld_d) * 2;
  const char* vbase = static_cast<const char*>(p.v.ptr) + ((int64_t)b * p.v.sb + (int64_t)g * p.v.sh + ld_d) * 2;
  const int64_t kst = p.k.st * 2, vst = p.v.st * 2;
  u32x4 kreg[4], vreg[4];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = min(t * kKT + ld_k + i, kv_len - 1);
      kreg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + row * kst));
      vreg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + row * vst));
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&k_lds[(ld_k + i) * kKPad + ld_d]) = kreg[i];
    // transpose: for each of the 8 dims, the 4 keys ld_k..ld_k+3 as one 8-byte write
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo01 = __builtin_amdgcn_perm(vreg[1][e], vreg[0][e], 0x05040100u);  // dim 2e:   k0 | k1
      const uint32_t lo23 = __builtin_amdgcn_perm(vreg[3][e], vreg[2][e], 0x05040100u);  //          k2 | k3
      const uint32_t hi01 = __builtin_amdgcn_perm(vreg[1][e], vreg[0][e], 0x07060302u);  // dim 2e+1
      const uint32_t hi23 = __builtin_amdgcn_perm(vreg[3][e], vreg[2][e], 0x07060302u);
      u32x2 lo = {lo01, lo23}, hi = {hi01, hi23};
      *reinterpret_cast<u32x2*>(&vt_lds[(ld_d + 2 * e) * kVPad + ld_k]) = lo;
      *reinterpret_cast<u32x2*>(&vt_lds[(ld_d + 2 * e + 1) * kVPad + ld_k]) = hi;
    }
  };

  f32x16 o_acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o_acc[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl = p.scale_log2;
  const int first_masked_tile = (p.p0 + c_wg) / kKT;  // tiles before it are fully visible to every query

  load_tile(0);
  for (int t = 0; t < n_tiles; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < n_tiles) load_tile(t + 1);

    // ---- S^T = K Q^T for 2 blocks of 32 keys ----
    f32x16 s[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[hb][r] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&k_lds[(32 * hb + perm_key(j)) * kKPad + 16 * c + 8 * q]);
        s[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[hb], 0, 0, 0);
      }
    }

    // ---- mask, scale, tile max ----
    const int key0 = t * kKT;
    const bool masked = t >= first_masked_tile;
    float mt = -INFINITY;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = s[hb][r] * sl;
        if (masked) {
          const int key = key0 + 32 * hb + perm_key(8 * (r >> 2) + 4 * q + (r & 3));
          if (key > pos) v = -INFINITY;
        }
        s[hb][r] = v;
        mt = fmaxf(mt, v);
      }
    }
    mt = xor32_max(mt);
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    if (__builtin_amdgcn_ballot_w64(m_new > m_run)) {
      const float alpha = fast_exp2(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o_acc[db][r] *= alpha;
    }
    m_run = m_new;

    // ---- P = exp2(S - m), row sums, bf16 P^T operands ----
    bf16x8 pb[2][2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0v = fast_exp2(s[hb][8 * hs + 2 * e] - m_use);
          const float p1v = fast_exp2(s[hb][8 * hs + 2 * e + 1] - m_use);
          l_run += p0v + p1v;
          w[e] = pack2(p0v, p1v);
        }
        u32x4 wv = {w[0], w[1], w[2], w[3]};
        pb[hb][hs] = __builtin_bit_cast(bf16x8, wv);
      }
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(&vt_lds[(32 * db + j) * kVPad + 32 * hb + 16 * hs + 8 * q]);
          o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[hb][hs], o_acc[db], 0, 0, 0);
        }
      }
    }
  }

  // ---- normalise and write ----
  const float l_tot = xor32_sum(l_run);
  const float inv = 1.0f / l_tot;
  const int c_out = c_w + j;
  if (c_out < p.C) {
    const size_t row = (((size_t)b * p.C + c_out) * p.Hq + h) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int d = 32 * db + 8 * rb + 4 * q;
        const float o0 = o_acc[db][4 * rb] * inv, o1 = o_acc[db][4 * rb + 1] * inv;
        const float o2 = o_acc[db][4 * rb + 2] * inv, o3 = o_acc[db][4 * rb + 3] * inv;
        if constexpr (OUT_BF16) {
          u32x2 w = {pack2(o0, o1), pack2(o2, o3)};
          *reinterpret_cast<u32x2*>(static_cast<__bf16*>(p.out) + row + d) = w;
        } else {
          float4 w = make_float4(o0, o1, o2, o3);
          *reinterpret_cast<float4*>(static_cast<float*>(p.out) + row + d) = w;
        }
      }
    }
    if (p.lse && q == 0) p.lse[((size_t)b * p.Hq + h) * p.C + c_out] = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
  }
}

template <int HPW>
hipError_t launch_hpw(const PrefillParams& p, hipStream_t s) {
  constexpr int WQ = kWaves / HPW;
  dim3 grid((p.C + WQ * kQB - 1) / (WQ * kQB), p.Hq / HPW, p.B);
  if (p.out_bf16)
    prefill_kernel<HPW, true><<<grid, kThreads, 0, s>>>(p);
  else
    prefill_kernel<HPW, false><<<grid, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  if (p.D != kD) return hipErrorInvalidValue;
  const int G = p.Hq / p.Hkv;
  if (G >= 4) return launch_hpw<4>(p, stream);
  if (G == 2) return launch_hpw<2>(p, stream);
  return launch_hpw<1>(p, stream);
}

}  // namespace yoco
