// Causal chunked prefill of a cross-decoder layer over the global cache
// (YOCO summary, abstract: end to end the model works as a decoder-only
// Transformer does, so the query at absolute position p attends to cache rows
// [0, p]; YOCO++ summary, section 3: prefill is compute-bound).
//
// Dense contraction on bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
// A workgroup of 8 wavefronts serves 8 (head, 32-query block) slots that share
// one kv head (4 heads x 2 consecutive query blocks); it streams the cache in
// 128-key tiles staged through LDS (two stages, one barrier per tile), so that
// all eight wavefronts read each tile from LDS instead of from memory. K and V
// are both stored row-major; the V operand of the PV product is read with the
// gfx950 transposing LDS read (ds_read_b64_tr_b16), which hands each lane 4
// consecutive keys of one dim.
//
// Per wavefront and tile:
//   S^T = K Q^T   (4 x 32 keys by 32 queries; D = 128 in 8 MFMA k-steps)
//   online softmax per query column, log2 domain, fp32
//   O^T += V^T P^T (4 x 32 dims by 32 queries; 128 keys in 8 MFMA k-steps)
// Computing the transposed products keeps every softmax statistic of a query
// inside one lane pair (lane j and j+32), and the S^T accumulator registers
// become the P^T operand of the PV product without leaving the lane: the key
// rows of each 32-key block are fed to the MFMA in the order that swaps bits 2
// and 3 of the key index, which makes the 8 P values a lane holds for one PV
// k-step 8 consecutive keys: two transposing reads of 4 keys each.
// Probabilities are rounded to bf16 for the PV product; the normaliser sums
// the same fp32 values.
//
// Every workgroup of one (sequence, kv head) streams the same K and V tiles,
// so the tiles are loaded through the L2 (temporal loads), and the 1-D grid is
// mapped so that all workgroups of one (sequence, head group) run on the same
// XCD (workgroups are dealt round-robin to the 8 XCDs, each with its own L2):
// the workgroups resident on an XCD walk one kv head's tiles nearly in step
// and share each fetch.

#include <math.h>

#include "common.h"

namespace yoco {
namespace {

constexpr int kWaves = 8;             // 4 heads x 2 query blocks; one workgroup per CU
constexpr int kThreads = 64 * kWaves;
constexpr int kQB = 32;               // queries per wavefront
constexpr int kKT = 128;              // keys per tile (two LDS stages: 148 KiB at D = 128)
constexpr int kNB = kKT / 32;         // 32-key MFMA blocks per tile

// Sizes that follow the head dimension (D = 64 or 128).
template <int D>
struct Dim {
  static constexpr int kNQ = D / 16;            // MFMA k-steps of the score product (Q fragments)
  static constexpr int kNDB = D / 32;           // 32-dim blocks of the output (O accumulators)
  static constexpr int kTPR = D / 8;            // threads per tile row in the cooperative loads
  static constexpr int kKPT = kKT / (kThreads / kTPR);   // keys per thread in the cooperative loads
  static constexpr int kKPad = D + 8;           // K tile row stride (bf16): 16-lane b128 reads hit distinct banks
  static constexpr int kVPad = D + 32;          // V tile row stride (bf16); no LDS bank conflicts at D = 128
  static constexpr int kStage = kKT * kKPad + kKT * kVPad;   // bf16 elements per LDS stage
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing LDS read: within each 16-lane group, lane i receives element
// (i % 4) of the 8-byte rows addressed by lanes 4e + i/4, e = 0..3.
__device__ __forceinline__ s16x4 read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) void*)(const_cast<__bf16*>(p)));
}

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

template <int D, int HPW, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(PrefillParams p) {
  constexpr int WQ = kWaves / HPW;  // query blocks per workgroup
  constexpr int kNQ = Dim<D>::kNQ, kNDB = Dim<D>::kNDB, kTPR = Dim<D>::kTPR, kKPT = Dim<D>::kKPT;
  constexpr int kKPad = Dim<D>::kKPad, kVPad = Dim<D>::kVPad, kStage = Dim<D>::kStage;
  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 5;          // lane half
  const int j = lane & 31;          // query column of this lane
  const int ngrp = p.Hq / HPW;
  const int npair = ngrp * p.B;
  const int n_qgroups = (int)gridDim.x / npair;
  int pair, qlin;
  {
    const int L = blockIdx.x;
    if (npair % 8 == 0) {   // workgroup L runs on XCD L % 8: keep each (b, head group) on one XCD
      const int x = L % 8, i = L / 8, ppx = npair / 8;
      pair = x + 8 * (i % ppx);
      qlin = i / ppx;
    } else {
      pair = L % npair;
      qlin = L / npair;
    }
  }
  const int qg = n_qgroups - 1 - qlin;   // heaviest (latest) query blocks first
  const int hgrp = pair % ngrp;
  const int h = hgrp * HPW + (wave % HPW);
  const int g = (hgrp * HPW) / (p.Hq / p.Hkv);
  const int b = pair / ngrp;
  const int c_wg = qg * (WQ * kQB);                 // first chunk row of the workgroup
  const int c_w = c_wg + (wave / HPW) * kQB;        // first chunk row of this wavefront
  const int c_hi = min(c_wg + WQ * kQB, p.C);       // workgroup rows end
  const int kv_len = p.p0 + c_hi;                   // keys any query of the workgroup can see
  const int n_tiles = (kv_len + kKT - 1) / kKT;

  // Q^T operand: lane (q, j) holds query row c_w + j, dims 16c + 8q .. +8.
  const int c_me = min(c_w + j, p.C - 1);
  const int pos = p.p0 + c_w + j;                   // absolute position of this lane's query
  bf16x8 qf[kNQ];
  {
    const __bf16* qrow = static_cast<const __bf16*>(p.q) + (((size_t)b * p.C + c_me) * p.Hq + h) * D + 8 * q;
#pragma unroll
    for (int c = 0; c < kNQ; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qrow + 16 * c);
  }

  // cooperative tile loads: thread t covers dims 8*(t%kTPR) .. +8 of keys kKPT*(t/kTPR) .. +kKPT
  const int ld_d = 8 * (tid % kTPR);
  const int ld_k = kKPT * (tid / kTPR);
  const int64_t kst = p.k.st * 2, vst = p.v.st * 2;
  const char* kbase = static_cast<const char*>(p.k.ptr) + ((int64_t)b * p.k.sb + (int64_t)g * p.k.sh + ld_d) * 2;
  const char* vbase = static_cast<const char*>(p.v.ptr) + ((int64_t)b * p.v.sb + (int64_t)g * p.v.sh + ld_d) * 2;
  u32x4 kreg[kKPT], vreg[kKPT];
  auto load_tile = [&](int t) {
    const int row0 = t * kKT + ld_k;
    if (t * kKT + kKT <= kv_len) {          // whole tile inside the cache prefix: no clamping
      const char* kp = kbase + row0 * kst;
      const char* vp = vbase + row0 * vst;
#pragma unroll
      for (int i = 0; i < kKPT; ++i) {
        kreg[i] = *reinterpret_cast<const u32x4*>(kp + i * kst);
        vreg[i] = *reinterpret_cast<const u32x4*>(vp + i * vst);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kKPT; ++i) {
        const int row = min(row0 + i, kv_len - 1);
        kreg[i] = *reinterpret_cast<const u32x4*>(kbase + row * kst);
        vreg[i] = *reinterpret_cast<const u32x4*>(vbase + row * vst);
      }
    }
  };
  auto store_tile = [&](int stage) {
    __bf16* kl = lds + stage * kStage;
    __bf16* vl = kl + kKT * kKPad;
#pragma unroll
    for (int i = 0; i < kKPT; ++i) {
      *reinterpret_cast<u32x4*>(&kl[(ld_k + i) * kKPad + ld_d]) = kreg[i];
      *reinterpret_cast<u32x4*>(&vl[(ld_k + i) * kVPad + ld_d]) = vreg[i];
    }
  };

  // Lane roles of the transposing V reads: group gq = lane/16, s = lane%16 addresses
  // V[key + 8*(gq/2) + s/4][dim + 16*(gq%2) + 4*(s%4)] and receives dim (lane % 32)
  // of 4 consecutive keys.
  const int gq = lane >> 4, sl16 = lane & 15;
  const int tr_off = (8 * (gq >> 1) + (sl16 >> 2)) * kVPad + 16 * (gq & 1) + 4 * (sl16 & 3);
  const int k_off = perm_key(j) * kKPad + 8 * q;

  f32x16 o_acc[kNDB];
#pragma unroll
  for (int db = 0; db < kNDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o_acc[db][r] = 0.f;
  float m_run = -INFINITY;   // running max of scaled scores (log2 domain)
  float l_run = 0.f;         // this lane's share of the running sum
  const float sl = p.scale_log2;

  // One tile of kKT keys: scores, online softmax, PV, and the hand-over of the next tile.
  auto tile = [&]<bool MASKED>(int t) {
    const int stage = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);
    const __bf16* kl = lds + stage * kStage;
    const __bf16* vl = kl + kKT * kKPad;

    // ---- S^T = K Q^T for kNB blocks of 32 keys (raw dot products) ----
    f32x16 sc[kNB];
#pragma unroll
    for (int hb = 0; hb < kNB; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[hb][r] = 0.f;
#pragma unroll
    for (int c = 0; c < kNQ; ++c) {
#pragma unroll
      for (int hb = 0; hb < kNB; ++hb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kl[32 * hb * kKPad + k_off + 16 * c]);
        sc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], sc[hb], 0, 0, 0);
      }
    }
    // Schedule: the K fragment reads run four ahead of the MFMAs that use them
    // (the default schedule keeps one or two ahead; +1-2% measured).
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);   // 4 LDS reads
#pragma unroll
    for (int i = 0; i < kNQ * kNB - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);  // 1 LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);   // the last 4 MFMAs

    // ---- causal mask (diagonal tiles only), tile max ----
    if constexpr (MASKED) {
      const int key0 = t * kKT;
#pragma unroll
      for (int hb = 0; hb < kNB; ++hb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * hb + perm_key(8 * (r >> 2) + 4 * q + (r & 3));
          if (key > pos) sc[hb][r] = -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int hb = 0; hb < kNB; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[hb][r]);
    // the scale is positive, so the max of the scaled scores is the scaled max
    mt = xor32_max(mt) * sl;
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    if (__builtin_amdgcn_ballot_w64(m_new > m_run)) {
      const float alpha = fast_exp2(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < kNDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o_acc[db][r] *= alpha;
    }
    m_run = m_new;

    // ---- P = exp2(scale * S - m), row sums, bf16 P^T operands ----
    bf16x8 pb[kNB][2];
#pragma unroll
    for (int hb = 0; hb < kNB; ++hb) {
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0v = fast_exp2(__builtin_fmaf(sc[hb][8 * hs + 2 * e], sl, -m_use));
          const float p1v = fast_exp2(__builtin_fmaf(sc[hb][8 * hs + 2 * e + 1], sl, -m_use));
          l_run += p0v + p1v;
          w[e] = pack2(p0v, p1v);
        }
        u32x4 wv = {w[0], w[1], w[2], w[3]};
        pb[hb][hs] = __builtin_bit_cast(bf16x8, wv);
      }
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int hb = 0; hb < kNB; ++hb) {
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        const __bf16* vk = vl + (32 * hb + 16 * hs) * kVPad + tr_off;
#pragma unroll
        for (int db = 0; db < kNDB; ++db) {
          const s16x4 lo = read_tr16(vk + 32 * db);
          const s16x4 hi = read_tr16(vk + 32 * db + 4 * kVPad);
          typedef short s16x8 __attribute__((ext_vector_type(8)));
          const s16x8 a8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), pb[hb][hs], o_acc[db],
                                                              0, 0, 0);
        }
      }
    }

    if (t + 1 < n_tiles) store_tile(stage ^ 1);
    __syncthreads();
  };

  // Tiles before first_masked hold only keys <= every query position of the workgroup.
  const int first_masked = min((p.p0 + c_wg) / kKT, n_tiles);
  load_tile(0);
  store_tile(0);
  // Every load issued so far (Q and the first tile) is complete here, so the
  // loop's waits only cover the tile prefetched inside it.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  for (int t = 0; t < first_masked; ++t) tile.template operator()<false>(t);
  for (int t = first_masked; t < n_tiles; ++t) tile.template operator()<true>(t);

  // ---- normalise and write ----
  const float l_tot = xor32_sum(l_run);
  const float inv = 1.0f / l_tot;
  const int c_out = c_w + j;
  if (c_out < p.C) {
    const size_t row = (((size_t)b * p.C + c_out) * p.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < kNDB; ++db) {
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

template <int D, int HPW>
hipError_t launch_hpw(const PrefillParams& p, hipStream_t s) {
  constexpr int WQ = kWaves / HPW;
  dim3 grid(((p.C + WQ * kQB - 1) / (WQ * kQB)) * (p.Hq / HPW) * p.B);
  if (p.out_bf16)
    prefill_kernel<D, HPW, true><<<grid, kThreads, 0, s>>>(p);
  else
    prefill_kernel<D, HPW, false><<<grid, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dim(const PrefillParams& p, hipStream_t s) {
  const int G = p.Hq / p.Hkv;
  if (G >= 4) return launch_hpw<D, 4>(p, s);
  if (G == 2) return launch_hpw<D, 2>(p, s);
  return launch_hpw<D, 1>(p, s);
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  if (p.D == 128) return launch_dim<128>(p, stream);
  if (p.D == 64) return launch_dim<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace yoco
