// Causal chunked prefill of a cross-decoder layer over the global cache
// (YOCO summary, abstract: end to end the model works as a decoder-only
// Transformer does, so the query at absolute position p attends to cache rows
// [0, p]; YOCO++ summary, section 3: prefill is compute-bound).
//
// Dense contraction on bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
// In both kernels here a workgroup of 8 wavefronts serves 8 (head, 32-query
// block) slots that share one kv head (4 heads x 2 consecutive query blocks)
// and stages the cache through LDS, so that all eight wavefronts read each
// tile from LDS instead of from memory. At D = 128 the software-pipelined
// prefill_pipe_kernel runs (its own comment below gives the step structure and
// the data movement); at D = 64 prefill_kernel, whose two wavefronts per SIMD
// take turns between an MFMA phase and a softmax phase over 128-key tiles
// (half a tile apart at D = 128, where it ran before; in step at D = 64, whose
// softmax phase dominates). The V operand of the PV product needs 4 or 8
// consecutive keys of one dim per lane: prefill_kernel reads it with the
// gfx950 transposing LDS read (ds_read_b64_tr_b16, 4 keys per read);
// prefill_pipe_kernel transposes each V tile once into LDS.
//
// Per wavefront and tile of prefill_kernel (prefill_pipe_kernel: 64-key steps):
//   S^T = K Q^T   (4 x 32 keys by 32 queries; D = 128 in 8 MFMA k-steps)
//   online softmax per query column, log2 domain, fp32
//   O^T += V^T P^T (4 x 32 dims by 32 queries; 128 keys in 8 MFMA k-steps)
// Computing the transposed products keeps every softmax statistic of a query
// inside one lane pair (lane j and j+32), and the S^T accumulator registers
// become the P^T operand of the PV product without leaving the lane: the key
// rows of each 32-key block are fed to the MFMA in the order that swaps bits 2
// and 3 of the key index, which makes the 8 P values a lane holds for one PV
// k-step 8 consecutive keys.
// Probabilities are rounded to bf16 for the PV product, and the normaliser
// sums the same rounded values.
//
// Every workgroup of one (sequence, kv head) streams the same K and V tiles,
// so the tiles are loaded through the L2, and the 1-D grid is
// mapped so that all workgroups of one (sequence, head group) run on the same
// XCD (workgroups are dealt round-robin to the 8 XCDs, each with its own L2):
// the workgroups resident on an XCD walk one kv head's tiles nearly in step
// and share each fetch.

#include <math.h>

#include <hip/hip_runtime.h>

#include "common.h"
#include "prefill_layout.h"

namespace yoco {
namespace {

constexpr int kWaves = 8;             // 4 heads x 2 query blocks; one workgroup per CU
constexpr int kThreads = 64 * kWaves;
constexpr int kQB = 32;               // queries per wavefront
constexpr int kKT = 128;              // keys per tile (two slots each of K and V: 148 KiB at D = 128)
constexpr int kNB = kKT / 32;         // 32-key MFMA blocks per tile
constexpr float kLazy = 8.f;          // rescale threshold of the running max (log2 units)

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
typedef float f32x4 __attribute__((ext_vector_type(4)));
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
// The same read through a restrict-qualified pointer. Once inlined, the read
// carries alias-scope metadata, and the compiler then no longer makes it wait
// for every direct global-to-LDS load in flight (it cannot tell which LDS
// bytes those write, and a plain transposing read carries no alias
// information). The kernel that uses it orders its direct loads and reads
// with its own waits and barriers.
__device__ __forceinline__ s16x4 read_tr16_scoped(const __bf16* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) void*)(const_cast<__bf16*>(p)));
}

// Row of a 32-key block that MFMA row i carries: bits 2 and 3 swapped.
using pipe::perm_key;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Maximum that propagates NaN (llvm.maximum). Unlike fmaxf it needs no
// quieting of its inputs first, and chains of it become three-input
// v_maximum3_f32; a NaN score yields a NaN row either way.
__device__ __forceinline__ float max_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max / sum with the partner lane (lane ^ 32)
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
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
  auto load_rows = [&](u32x4* reg, const char* base, int64_t st, int t) {
    const int row0 = t * kKT + ld_k;
    if (t * kKT + kKT <= kv_len) {          // whole tile inside the cache prefix: no clamping
      const char* ptr = base + row0 * st;
#pragma unroll
      for (int i = 0; i < kKPT; ++i) reg[i] = *reinterpret_cast<const u32x4*>(ptr + i * st);
    } else {
#pragma unroll
      for (int i = 0; i < kKPT; ++i) reg[i] = *reinterpret_cast<const u32x4*>(base + min(row0 + i, kv_len - 1) * st);
    }
  };
  // K tile t lives in K slot t % 2 and V tile t in V slot t % 2.
  auto k_slot = [&](int t) { return lds + (t & 1) * kStage; };
  auto v_slot = [&](int t) { return lds + (t & 1) * kStage + kKT * kKPad; };
  auto store_k = [&](const u32x4* reg, int t) {
    __bf16* kl = k_slot(t);
#pragma unroll
    for (int i = 0; i < kKPT; ++i) *reinterpret_cast<u32x4*>(&kl[(ld_k + i) * kKPad + ld_d]) = reg[i];
  };
  auto store_v = [&](const u32x4* reg, int t) {
    __bf16* vl = v_slot(t);
#pragma unroll
    for (int i = 0; i < kKPT; ++i) *reinterpret_cast<u32x4*>(&vl[(ld_k + i) * kVPad + ld_d]) = reg[i];
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
  f32x16 sc[kNB];            // raw scores of the current tile (S^T blocks)
  bf16x8 pb[kNB][2];         // bf16 probabilities of the current tile (P^T operands)

  // ---- S^T = K Q^T for kNB blocks of 32 keys (raw dot products) ----
  auto scores = [&](int t) {
    const __bf16* kl = k_slot(t);
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
  };
  // Schedules of the MFMA phase (0x008: MFMA, 0x100: LDS read). A wavefront
  // runs this phase while the other wavefront of its SIMD is in its softmax
  // phase, so the operand reads must run well ahead of the MFMAs that use
  // them: PV operands (two reads per MFMA) kAP MFMAs ahead, K fragments (one
  // read per MFMA) 2 kAP ahead.
  constexpr int kAP = 4;
  constexpr int kNS = kNQ * kNB;        // MFMAs of the scores
  constexpr int kNP = kNB * 2 * kNDB;   // MFMAs of the PV product
  auto sched_scores = [] {
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAP, 0);
#pragma unroll
    for (int i = 0; i < kNS - 2 * kAP; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kAP, 0);
  };
  auto sched_pv_scores = [] {
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAP, 0);
#pragma unroll
    for (int i = 0; i < kNP; ++i) {   // the last kAP of these fetch the first 2 kAP K fragments
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < kNS - 2 * kAP; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kAP, 0);
  };
  auto sched_pv = [] {
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAP, 0);
#pragma unroll
    for (int i = 0; i < kNP - kAP; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAP, 0);
  };

  // ---- causal mask (diagonal tiles only), online softmax, bf16 P^T operands ----
  auto mask = [&](int t) {
    // key offsets within the tile are constants per register (plus 8 on the
    // upper lane half: its bit 2 lands on bit 3), compared against one
    // per-tile limit
    const int lim = pos - t * kKT - 8 * q;
#pragma unroll
    for (int hb = 0; hb < kNB; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * hb + perm_key(8 * (r >> 2) + (r & 3)) > lim) sc[hb][r] = -INFINITY;
  };
  // Tile max and the lazy rescale; returns the reference max the
  // exponentials subtract.
  auto softmax_max = [&]() {
    // tile max: four chains of three-input maxima, one per 32-key block
    float mb[kNB];
#pragma unroll
    for (int hb = 0; hb < kNB; ++hb) {
      float m = max_nan(sc[hb][0], sc[hb][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) m = max_nan(max_nan(m, sc[hb][r]), sc[hb][r + 1]);
      mb[hb] = m;
    }
    // the scale is positive, so the max of the scaled scores is the scaled max
    const float mt = xor32_max(max_nan(max_nan(mb[0], mb[1]), max_nan(mb[2], mb[3]))) * sl;
    // Lazy rescaling: the reference max m_run only moves when some row's
    // tile max exceeds it by more than kLazy (log2 units), so exponentials
    // stay below 2^kLazy and the accumulators are rescaled in few tiles.
    // Numerator and normaliser share the reference, so the result is exact
    // up to rounding for any choice of it.
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazy)) {
      const float m_new = max_nan(m_run, mt);
      const float alpha = fast_exp2(m_run - ((m_new == -INFINITY) ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < kNDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o_acc[db][r] *= alpha;
      m_run = m_new;
    }
    return (m_run == -INFINITY) ? 0.f : m_run;
  };
  // P = exp2(scale * S - m) rounded to bf16 pairs; the normaliser sums the
  // rounded values (the ones the PV product uses) with dot2 against (1, 1).
  // hook(i) runs before the i-th of the 2 kNB chunks of eight exponentials.
  auto softmax_exp = [&](float m_use, auto&& hook) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float ls[kNB][2];
#pragma unroll
    for (int hb = 0; hb < kNB; ++hb) {
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        hook(2 * hb + hs);
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0v = fast_exp2(__builtin_fmaf(sc[hb][8 * hs + 2 * e], sl, -m_use));
          const float p1v = fast_exp2(__builtin_fmaf(sc[hb][8 * hs + 2 * e + 1], sl, -m_use));
          w[e] = pack2(p0v, p1v);
        }
        float a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[0]), ones, 0.f, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[1]), ones, a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[2]), ones, a, false);
        ls[hb][hs] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[3]), ones, a, false);
        u32x4 wv = {w[0], w[1], w[2], w[3]};
        pb[hb][hs] = __builtin_bit_cast(bf16x8, wv);
      }
    }
    l_run += ((ls[0][0] + ls[0][1]) + (ls[1][0] + ls[1][1])) + ((ls[2][0] + ls[2][1]) + (ls[3][0] + ls[3][1]));
  };

  // ---- O^T += V^T P^T ----
  auto pv = [&](int t) {
    const __bf16* vl = v_slot(t);
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
  };

  // Two wavefront groups (waves 0-3 and 4-7: one of each on every SIMD). Per
  // tile a wavefront has an MFMA phase (PV of the previous tile, then the
  // scores of this one) and a softmax phase (VALU and the exponential unit).
  // At D = 128 the workgroup advances in intervals separated by a barrier, and
  // in each interval one group is in its MFMA phase while the other is in its
  // softmax phase, so the two kinds of work overlap on every SIMD; group 1
  // starts one interval late. The group in its softmax phase also moves its
  // half of the key rows of K tile s+1 and V tile s (s = interval / 2) from
  // memory into their LDS slots: K slot (s+1) % 2 was last read by the scores
  // of tile s-1 and V slot s % 2 by the PV of tile s-2, both finished by the
  // end of interval 2s-1, and the first reads of the new tiles come in
  // interval 2s+2.
  const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);
  constexpr bool kStagger = (D == 128);   // the two groups half a tile apart
  const int first_masked = min((p.p0 + c_wg) / kKT, n_tiles);   // earlier tiles need no causal mask
  {
    u32x4 kr[kKPT], vr[kKPT];
    load_rows(kr, kbase, kst, 0);
    load_rows(vr, vbase, vst, 0);
    store_k(kr, 0);
    store_v(vr, 0);
    if (n_tiles > 1) {
      load_rows(kr, kbase, kst, 1);
      store_k(kr, 1);
    }
  }
  // Every load issued so far (Q and the first tiles) is complete here.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  // The softmax phase of tile t, with the copy duty s = t (+ grp when staggered).
  // One of the 2 kKPT row loads goes out before each chunk of eight
  // exponentials (spread out like this the phase ran faster than with all
  // loads issued at its start). Rows past the cache prefix are clamped, so
  // every request is valid; outside the duty the rows are not stored.
  auto softmax_phase = [&](int t) {
    const int s = t + (kStagger ? grp : 0);
    const bool mk = s >= 1 && s + 1 < n_tiles;
    const bool mv = s >= 1 && s < n_tiles;
    if (t >= first_masked) mask(t);
    const float m_use = softmax_max();
    u32x4 kr[kKPT], vr[kKPT];   // this thread's rows of the tiles in flight
    const int krow0 = (s + 1) * kKT + ld_k, vrow0 = s * kKT + ld_k;
    softmax_exp(m_use, [&](int i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i < kKPT)
        kr[i] = *reinterpret_cast<const u32x4*>(kbase + min(krow0 + i, kv_len - 1) * kst);
      else if (i < 2 * kKPT)
        vr[i - kKPT] = *reinterpret_cast<const u32x4*>(vbase + min(vrow0 + i - kKPT, kv_len - 1) * vst);
      __builtin_amdgcn_sched_barrier(0);
    });
    // The probabilities are only read in the next phase; without this the
    // compiler sinks their computation below the LDS stores, whose wait for
    // the tile loads would then stall the wavefront with nothing to overlap.
#pragma unroll
    for (int hb = 0; hb < kNB; ++hb)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) asm volatile("" : "+v"(pb[hb][hs]));
    if (mk) store_k(kr, s + 1);
    if (mv) store_v(vr, s);
  };
  // Staggered (D = 128): group 0 runs MFMA(t) in interval 2t, softmax(t) in
  // 2t+1 and the last PV in 2n; group 1 runs one interval later; both pass
  // 2n+1 barriers. In step (D = 64, where the softmax phase outweighs the
  // MFMA phase so much that two softmax phases side by side hide each
  // other's latency better): both groups run the same phase, and one barrier
  // per tile, after the softmax phase, is enough, since the copy duty of
  // interval 2t+1 writes slots last read in interval 2t-2. The scheduling
  // fences keep every MFMA and exponential inside its own phase: the compiler
  // would otherwise sink the last MFMAs of a phase past the barrier.
  auto interval_end = [] {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto phase_end = [&] {
    if constexpr (kStagger)
      interval_end();
    else
      __builtin_amdgcn_sched_barrier(0);
  };
  if (kStagger && grp) interval_end();
  scores(0);
  sched_scores();
  phase_end();
  softmax_phase(0);
  interval_end();
  for (int t = 1; t < n_tiles; ++t) {
    pv(t - 1);
    scores(t);
    sched_pv_scores();
    phase_end();
    softmax_phase(t);
    interval_end();
  }
  pv(n_tiles - 1);
  sched_pv();
  if (kStagger && !grp) interval_end();

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

// ---------------------------------------------------------------------------
// Software-pipelined kernel (D = 128). A SIMD's matrix core and its vector
// ALU overlap well only when one wavefront interleaves both kinds of
// instruction: a wavefront issuing MFMAs back to back leaves the other
// wavefront of its SIMD few VALU issue slots (and of two wavefronts with an
// MFMA ready, the older always gets the matrix core), whereas VALU
// instructions placed between a wavefront's own MFMAs run in their shadow. So every
// wavefront runs the whole pipeline itself, in 64-key steps. Step u, with the
// scores S(u) and the probabilities P(u - 1) in registers, is 36 MFMA slots,
// each an MFMA and the VALU work it shadows, fenced so the compiler keeps the
// order:
//   slots  0-19  PV of P(u - 1), per 16-key slice four O MFMAs and a half-size
//                one that adds the slice's probabilities into the normaliser
//                (ones rows times P) | slots 0-1 maxima of S(u) keys 32-63, slot 2
//                the reference decision, slots 3-13 scale and shift S(u),
//                slots 10-17 exponentials of S(u) keys 0-31
//   slots 20-35  scores S(u + 1) (keys 0-31, then 32-63) | slots 20-27
//                exponentials of S(u) keys 32-63, slots 29-35 row maxima of
//                S(u + 1) keys 0-31
// Each register block is overwritten right after its last reader, so S and P
// need one buffer each. The normaliser on the matrix core costs half an MFMA
// per slice and saves the row sums' adds on the vector ALU, which is the busier
// unit: with the MFMAs taken out, a step's remaining instructions still take
// longer than its MFMAs.
//
// Lazy rescaling with the deferred PV product: the reference max may move
// early in step u, once the maxima of S(u) are known and before S(u) is
// exponentiated. O and the normaliser receive P(u - 1), computed against the
// old reference, during step u, so both take the factor at the end of step u.
//
// Data movement. K and V tiles reach LDS by direct loads (buffer_load ...
// lds) three steps ahead, into three K slots and three V slots (unpadded
// 256-byte rows; chunk c of row r at position c ^ (r % 16) in K, c ^ 4 (r % 4)
// in V, so the 16-lane K operand reads and the 32-lane transposing V reads
// each touch every bank once). The PV operand needs 8 consecutive keys of one
// dim per lane; the transposing LDS read delivers 4 per 8-byte read at a
// quarter of the rate of 16-byte reads, so instead of every wavefront
// transposing every tile, the workgroup transposes each V tile once (each
// wavefront 8 keys by 128 dims) into a V^T slot (rows of 64 keys, 144-byte
// stride), from which the PV operands are single 16-byte reads. Step u issues
// the loads of K and V step u + 3 into slots u % 3 (last read in step u - 1),
// transposes V step u + 1 into V^T slot (u + 1) % 3 (last read by PV in step
// u - 1), reads K slot (u + 1) % 3 and V^T slot (u - 1) % 3. Before the
// barrier that ends step u each wavefront waits for all its loads but the four
// just issued; the LDS reads it may still have in flight are the next step's
// first operands, from a V^T slot not rewritten before step u + 2. Rows past
// the cache prefix lie outside the buffer range and load as zeros.
// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (vmcnt is split over bits 3:0 and 15:14) and leaves the other
// counters unconstrained.
constexpr int vm_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

template <int HPW, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_pipe_kernel(PrefillParams p) {
  // LDS layout and per-lane addresses: prefill_layout.h (checked by a host build)
  constexpr int D = pipe::kD;
  constexpr int WQ = kWaves / HPW;
  constexpr int kSK = pipe::kSK;           // keys per step
  constexpr int kSB = kSK / 32;            // 32-key MFMA blocks per step
  constexpr int kNQ = D / 16, kNDB = D / 32;
  constexpr int kNS = pipe::kNS;           // LDS slots per tensor
  constexpr int kRowB = pipe::kRowB;
  constexpr int kSlotB = pipe::kSlotB;
  constexpr int kVBase = pipe::kVBase;
  constexpr int kVTRow = pipe::kVTRow;
  constexpr int kVTSlotB = pipe::kVTSlotB;
  constexpr int kLoads = pipe::kLoads;
  constexpr int kBufWord3 = 0x00020000;    // raw buffer resource, 32-bit data format
  static_assert(kWaves == pipe::kWaves, "one wavefront count");
  __shared__ __attribute__((aligned(16))) char lds[pipe::kLdsBytes];   // 150 KiB

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 5;
  const int j = lane & 31;
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
  const int qg = n_qgroups - 1 - qlin;
  const int hgrp = pair % ngrp;
  const int h = hgrp * HPW + (wave % HPW);
  const int g = (hgrp * HPW) / (p.Hq / p.Hkv);
  const int b = pair / ngrp;
  const int c_wg = qg * (WQ * kQB);
  const int c_w = c_wg + (wave / HPW) * kQB;
  const int c_hi = min(c_wg + WQ * kQB, p.C);
  const int kv_len = p.p0 + c_hi;
  const int n = (kv_len + kSK - 1) / kSK;                 // steps
  const int fm = min((p.p0 + c_wg) / kSK, n);              // first step whose scores need the causal mask

  // no slot ever holds a non-finite leftover: zero the LDS before the first load lands
  for (int i = tid; i < (int)(sizeof(lds) / 16); i += kThreads) reinterpret_cast<u32x4*>(lds)[i] = u32x4{0u, 0u, 0u, 0u};

  const int c_me = min(c_w + j, p.C - 1);
  const int pos = p.p0 + c_w + j;
  bf16x8 qf[kNQ];
  {
    const __bf16* qrow = static_cast<const __bf16*>(p.q) + (((size_t)b * p.C + c_me) * p.Hq + h) * D + 8 * q;
#pragma unroll
    for (int c = 0; c < kNQ; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qrow + 16 * c);
  }
  __syncthreads();   // the zero fill is done before any direct load is issued

  // direct loads: load i of wavefront w writes rows 8w + 4i + lane/16 of a slot, 16 bytes at position lane % 16
  const int64_t kst_b = p.k.st * 2, vst_b = p.v.st * 2;
  const char* kb = static_cast<const char*>(p.k.ptr) + ((int64_t)b * p.k.sb + (int64_t)g * p.k.sh) * 2;
  const char* vb = static_cast<const char*>(p.v.ptr) + ((int64_t)b * p.v.sb + (int64_t)g * p.v.sh) * 2;
  uint32_t koff[kLoads], voff[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = pipe::load_row(wave, i, lane), ps = lane & 15;
    koff[i] = (uint32_t)(r * kst_b) + 16u * (uint32_t)pipe::k_load_chunk(r, ps);
    voff[i] = (uint32_t)(r * vst_b) + 16u * (uint32_t)pipe::v_load_chunk(r, ps);
  }
  auto issue = [&](const char* base, int64_t st_b, const uint32_t* off, int x, int slot_byte) {
    const int rows = min(kv_len - kSK * x, kSK);
    const uint32_t bytes = rows > 0 ? (uint32_t)((int64_t)(rows - 1) * st_b + kRowB) : 0u;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + (int64_t)x * kSK * st_b), (short)0, (int)bytes, kBufWord3);
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(lds + slot_byte + pipe::load_lds_offset(wave, i)), 16, off[i], 0,
          0, 0);
  };
  auto issue_k = [&](int x, int slot) { issue(kb, kst_b, koff, x, slot * kSlotB); };
  auto issue_v = [&](int x, int slot) { issue(vb, vst_b, voff, x, kVBase + slot * kSlotB); };

  // LDS addresses (bytes). K operand of k-step c at aK[c] (+ slot, + 32-key block).
  uint32_t aK[kNQ];
#pragma unroll
  for (int c = 0; c < kNQ; ++c) aK[c] = pipe::k_operand(lane, c);
  // Transposing reads of a V tile (wavefront w covers 8 keys of all 128 dims, one
  // read per 32-dim block), where their 4 keys land in V^T, and where lane l
  // reads its PV operand (dim l % 32, keys 8 (l / 32) .. +8).
  uint32_t aT[kNDB];
#pragma unroll
  for (int db = 0; db < kNDB; ++db) aT[db] = pipe::tr_read(wave, lane, db);
  const uint32_t aW = pipe::vt_write(wave, lane, 0);
  const uint32_t aP = pipe::pv_operand(lane, 0, 0, 0);

  f32x16 o_acc[kNDB];
#pragma unroll
  for (int db = 0; db < kNDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o_acc[db][r] = 0.f;
  // The normaliser rides on the matrix core: one 16x16x32 MFMA per PV k-step
  // takes the P^T operand register as its B operand. Read that way, lane
  // groups 0 and 2 (lanes 0-15, 32-47) hold the 16 keys of queries 0-15 in
  // their k positions, groups 1 and 3 those of queries 16-31. The A operand
  // has ones where row 0 meets groups 0 and 2 and where row 4 meets groups 1
  // and 3, zeros elsewhere, so row 0 of l_acc accumulates the sum over keys of
  // the bf16 probabilities of queries 0-15 and row 4 that of queries 16-31
  // (exact products, fp32 sums). Rows 0 and 4 land in element 0 of lanes 0-15
  // and 16-31: lane j holds query j's sum, the query whose reference and
  // rescale factor it also holds; every other element is zero. This needs
  // only that A and B spread k over lanes and elements alike.
  f32x4 l_acc = {0.f, 0.f, 0.f, 0.f};
  bf16x8 ones_row;
  {
    const int g = lane >> 4, r16 = lane & 15;
    const bool one = (r16 == 0 && (g & 1) == 0) || (r16 == 4 && (g & 1) == 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) ones_row[e] = one ? (__bf16)1.0f : (__bf16)0.0f;
  }
  // Reference max (log2 domain) the exponentials subtract. It starts at the
  // most negative finite value, so the first finite score moves it before
  // any exponential and masked (-inf) scores still give exp2(-inf) = 0.
  float m_ref = -__FLT_MAX__;
  float m_old = -__FLT_MAX__;   // the reference before the latest decision
  bool have_pend = false;       // wave-uniform: O and the normaliser owe exp2(m_old - m_ref)
  const float sl = p.scale_log2;
  f32x16 sc[kSB];            // scores of one step (raw, then scaled and shifted)
  u32x4 pw[kSB][2];          // bf16 probabilities of one step, packed in pairs (P^T operands)
  s16x4 tv[kNDB];            // this wavefront's share of a V tile, transposed

  auto transpose_read1 = [&](int vslot_byte, int db) {
    tv[db] = read_tr16_scoped(reinterpret_cast<const __bf16*>(lds + aT[db] + vslot_byte));
  };
  auto transpose_write1 = [&](int vtslot_byte, int db) {
    *reinterpret_cast<s16x4*>(lds + aW + vtslot_byte + db * 32 * kVTRow) = tv[db];
  };
  auto transpose_read = [&](int vslot_byte) {
#pragma unroll
    for (int db = 0; db < kNDB; ++db) transpose_read1(vslot_byte, db);
  };
  auto transpose_write = [&](int vtslot_byte) {
#pragma unroll
    for (int db = 0; db < kNDB; ++db) transpose_write1(vtslot_byte, db);
  };
  auto pv_operand = [&](int vtslot_byte, int hb, int hs, int db) {
    return *reinterpret_cast<const bf16x8*>(lds + aP + vtslot_byte + db * 32 * kVTRow + (32 * hb + 16 * hs) * 2);
  };
  auto k_operand = [&](int kslot_byte, int hb, int c) {
    return *reinterpret_cast<const bf16x8*>(lds + aK[c] + kslot_byte + hb * 32 * kRowB);
  };
  auto qk_block = [&](int kslot_byte, int hb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[hb][r] = 0.f;
#pragma unroll
    for (int c = 0; c < kNQ; ++c)
      sc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand(kslot_byte, hb, c), qf[c], sc[hb], 0, 0, 0);
  };
  auto pv_block = [&](int vtslot_byte, int hb) {
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
      for (int db = 0; db < kNDB; ++db)
        o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pv_operand(vtslot_byte, hb, hs, db),
                                                            __builtin_bit_cast(bf16x8, pw[hb][hs]), o_acc[db], 0, 0, 0);
      l_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_row, __builtin_bit_cast(bf16x8, pw[hb][hs]), l_acc, 0, 0, 0);
    }
  };
  auto mask_block = [&](int u, int hb) {
    const int lim = pos - u * kSK - 8 * q;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * hb + perm_key(8 * (r >> 2) + (r & 3)) > lim) sc[hb][r] = -INFINITY;
  };
  auto max_block = [&](int hb) {
    float m = max_nan(sc[hb][0], sc[hb][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) m = max_nan(max_nan(m, sc[hb][r]), sc[hb][r + 1]);
    return m;
  };
  auto scale_block = [&](int hb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[hb][r] = __builtin_fmaf(sc[hb][r], sl, -m_ref);
  };
  // exponentials of two scaled scores, rounded to a bf16 pair in pw (the
  // normaliser sums exactly these rounded values, in l_acc)
  auto exp_pair = [&](int hb, int hs, int e) {
    pw[hb][hs][e] = pack2(fast_exp2(sc[hb][8 * hs + 2 * e]), fast_exp2(sc[hb][8 * hs + 2 * e + 1]));
  };
  auto exp_block = [&](int hb) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      exp_pair(hb, 0, e);
      exp_pair(hb, 1, e);
    }
  };
  // The reference decision for S(u), at the start of step u, from m, this
  // lane's maximum of S(u) (the partner lane holds the other half of the
  // row). Branch-free; the factor itself is computed only when the
  // reference moves, at the end of the step.
  float mb0_c = -INFINITY;   // maximum of S(u) keys 0-31, taken in step u - 1
  auto decide_max = [&](float m) {
    const float mt = xor32_max(m) * sl;
    const bool need = __builtin_amdgcn_ballot_w64(mt > m_ref + kLazy) != 0;
    m_old = m_ref;
    m_ref = need ? max_nan(m_ref, mt) : m_ref;
    have_pend = need;
  };
  auto decide = [&](float mb1) { decide_max(max_nan(mb0_c, mb1)); };
  // end of step u: O, now holding PV up to step u - 1 against the old
  // reference, takes the factor decided at the start of the step
  auto step_end = [&] {
    if (have_pend) {
      const float pend = fast_exp2(m_old - m_ref);
#pragma unroll
      for (int db = 0; db < kNDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o_acc[db][r] *= pend;
      l_acc[0] *= pend;   // the other elements of l_acc stay 0
      have_pend = false;
    }
  };
  // Every direct load but the four just issued has landed in LDS, then the
  // barrier. LDS reads may still be in flight: all but the next step's first
  // PV operands were consumed by this step's MFMAs, and those read a V^T slot
  // that is not rewritten before step u + 2. This step's V^T writes complete
  // before any later LDS read of this wavefront returns (LDS operations
  // complete in order), so before the next barrier.
  auto step_barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vm_wait(2 * kLoads));
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // P(u) and the normaliser are read only in later steps; without this the
  // compiler sinks the exponentials out of the step, past its MFMAs, to just
  // before the barrier
  auto anchor = [&] {
#pragma unroll
    for (int hb = 0; hb < kSB; ++hb)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) asm volatile("" : "+v"(pw[hb][hs]));
  };
  // The first PV operands of the next step come from a V^T slot written two
  // steps before; they are read before the barrier that ends a step, so the
  // next step's first MFMA does not wait for LDS.
  constexpr int kCarry = 3;
  bf16x8 carry[kCarry];
  auto prefetch_next = [&](int vtslot_byte) {
#pragma unroll
    for (int t = 0; t < kCarry; ++t) carry[t] = pv_operand(vtslot_byte, 0, t / kNDB, t % kNDB);
  };

  // Steady step u (1 <= u, u + 1 < fm; T = u % 3): 36 fenced slots.
  //   slots  0-19  PV of P(u - 1) and the normaliser | 0-1: maxima of S(u)
  //                keys 32-63; 2: the reference decision; 3-13: scale and
  //                shift S(u) (keys 0-31 first); 10-17: exponentials of keys
  //                0-31
  //   slots 20-35  scores S(u + 1) | 20-27: exponentials of keys 32-63;
  //                29-35: maxima of S(u + 1) keys 0-31
  // The loads of step u + 3 go out in slot 3, the V tile transposition rides
  // on the score slots, whose operand reads are light.
  auto step_fast = [&]<int T>(int u) {
    constexpr int KS = ((T + 1) % kNS) * kSlotB;          // K step u + 1
    constexpr int VTR = ((T + 2) % kNS) * kVTSlotB;       // V^T step u - 1
    constexpr int VSRC = ((T + 1) % kNS) * kSlotB;        // V step u + 1, to transpose
    constexpr int VTW = ((T + 1) % kNS) * kVTSlotB;
    constexpr int VTN = T * kVTSlotB;                     // V^T step u, read by the next step
    constexpr int kOps = 2 * kSB * kNDB + kSB * kNQ;      // 16 PV + 16 score operands from LDS
    constexpr int kPVS = 2 * kSB * (kNDB + 1);            // 20 PV-phase slots (4 PV MFMAs + 1 sum per k-step)
    constexpr int kSlots = kPVS + kSB * kNQ;              // + 16 score slots
    bf16x8 opnd[kOps];
    auto fetch = [&](int o) {
      if (o < 2 * kSB * kNDB)
        opnd[o] = pv_operand(VTR, o / (2 * kNDB), (o / kNDB) % 2, o % kNDB);
      else
        opnd[o] = k_operand(KS, (o - 2 * kSB * kNDB) / kNQ, (o - 2 * kSB * kNDB) % kNQ);
    };
    // operand used at slot t (for a sum slot: the next one); operands are read
    // three PV operands or four score operands ahead
    auto op_at = [](int t) { return t < kPVS ? 4 * (t / 5) + (t % 5 == 4 ? 4 : t % 5) : 16 + (t - kPVS); };
    auto want = [&](int t) { const int o = op_at(t); return min(o < 16 ? o + kCarry : o + 4, kOps - 1); };
#pragma unroll
    for (int o = 0; o < kCarry; ++o) opnd[o] = carry[o];
    float mb0 = 0.f;
    const f32x16 zero = {};
#pragma unroll
    for (int t = 0; t < kSlots; ++t) {
#pragma unroll
      for (int o = (t == 0 ? kCarry : want(t - 1) + 1); o <= want(t); ++o) fetch(o);
      if (t == 3) {
        issue_k(u + 3, T);
        issue_v(u + 3, T);
      }
      if (t >= kPVS && t < kPVS + 4) transpose_read1(VSRC, t - kPVS);
      if (t >= kPVS + 10 && t < kPVS + 14) transpose_write1(VTW, t - kPVS - 10);
      if (t < kPVS) {
        const int gk = t / 5, hb = gk / 2, hs = gk % 2, db = t % 5;
        if (db < kNDB)
          o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[4 * gk + db], __builtin_bit_cast(bf16x8, pw[hb][hs]),
                                                              o_acc[db], 0, 0, 0);
        else
          l_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_row, __builtin_bit_cast(bf16x8, pw[hb][hs]), l_acc, 0, 0,
                                                          0);
      } else {
        const int hb = (t - kPVS) / kNQ, c = (t - kPVS) % kNQ;
        sc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[16 + (t - kPVS)], qf[c], c == 0 ? zero : sc[hb], 0, 0, 0);
      }
      // VALU in the MFMA's shadow
      if (t < 2) {
        // maxima of S(u) keys 32-63 joined to those of keys 0-31, three-input maxima
        if (t == 0) mb0 = mb0_c;
#pragma unroll
        for (int r = 8 * t; r < 8 * t + 8; r += 2) mb0 = max_nan(max_nan(mb0, sc[1][r]), sc[1][r + 1]);
      } else if (t == 2) {
        decide_max(mb0);
      } else if (t < 10) {
        // scalings: block 0 in slots 3-6, block 1 elements 0-11 in slots 7-9
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * (t - 3) + i, hb = e / 16, r = e % 16;
          sc[hb][r] = __builtin_fmaf(sc[hb][r], sl, -m_ref);
        }
      } else if (t < 18) {
        // exponentials of keys 0-31 (P(u - 1) keys 0-31 was read by slot 9);
        // block 1 elements 12-15 scaled in slots 10-13
        const int i = t - 10;
        if (i < 4) sc[1][12 + i] = __builtin_fmaf(sc[1][12 + i], sl, -m_ref);
        exp_pair(0, i / 4, i % 4);
      } else if (t >= kPVS && t < kPVS + 8) {
        // exponentials of keys 32-63 (P(u - 1) keys 32-63 was read by slot 19)
        const int i = t - kPVS;
        exp_pair(1, i / 4, i % 4);
      } else if (t == kPVS + 9) {
        mb0 = max_nan(max_nan(sc[0][0], sc[0][1]), sc[0][2]);
      } else if (t > kPVS + 9) {
        const int r = 3 + 2 * (t - kPVS - 10);   // slots 30-35: elements 3-14 in pairs, then 15
        mb0 = max_nan(max_nan(mb0, sc[0][r]), sc[0][r + 1]);
        if (r == 13) mb0 = max_nan(mb0, sc[0][15]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    mb0_c = mb0;
    anchor();
    asm volatile("" : "+v"(mb0_c));
    prefetch_next(VTN);
    step_end();
    step_barrier();
  };
  // any step, with the products and the mask as it needs them
  auto step_edge = [&](int u) {
    const int T = u % kNS;
    const int KS = ((T + 1) % kNS) * kSlotB, VTR = ((T + 2) % kNS) * kVTSlotB;
    decide(max_block(1));
    transpose_read(((T + 1) % kNS) * kSlotB);
    issue_k(u + 3, T);
    issue_v(u + 3, T);
    scale_block(0);
    scale_block(1);
    if (u >= 1) {
      pv_block(VTR, 0);
      pv_block(VTR, 1);
    }
    exp_block(0);
    exp_block(1);
    anchor();
    transpose_write(((T + 1) % kNS) * kVTSlotB);
    if (u + 1 < n) {
      qk_block(KS, 0);
      qk_block(KS, 1);
      if (u + 1 >= fm) {
        mask_block(u + 1, 0);
        mask_block(u + 1, 1);
      }
      mb0_c = max_block(0);
    }
    prefetch_next(T * kVTSlotB);
    __builtin_amdgcn_sched_barrier(0);
    step_end();
    step_barrier();
  };

  // prologue: K and V steps 0-2 in flight; V step 0 transposed, the scores of step 0
  issue_k(0, 0);
  issue_v(0, 0);
  issue_k(1, 1);
  issue_v(1, 1);
  issue_k(2, 2);
  issue_v(2, 2);
  __builtin_amdgcn_s_waitcnt(vm_wait(4 * kLoads));   // K and V step 0 landed (steps 1 and 2 may fly)
  asm volatile("s_barrier" ::: "memory");
  transpose_read(0);
  qk_block(0, 0);
  qk_block(0, 1);
  transpose_write(0);
  if (fm == 0) {
    mask_block(0, 0);
    mask_block(0, 1);
  }
  mb0_c = max_block(0);
  // K and V step 1 landed, V^T step 0 written; step 0 may overwrite K and V slot 0
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vm_wait(2 * kLoads) & ~0x0F00);   // K and V step 1 landed, and lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  step_edge(0);
  const int fast_end = fm - 1;   // steps 1 <= u < fast_end have u + 1 < fm <= n
  int u = 1;
  for (; u + 2 < fast_end; u += 3) {
    step_fast.template operator()<1>(u);
    step_fast.template operator()<2>(u + 1);
    step_fast.template operator()<0>(u + 2);
  }
  for (; u < n; ++u) step_edge(u);
  // PV of the last step (V^T written before the last barrier); O owes no factor: the last one was applied at the end of step n - 1
  pv_block(((n - 1) % kNS) * kVTSlotB, 0);
  pv_block(((n - 1) % kNS) * kVTSlotB, 1);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no direct load may land after the workgroup ends

  const float l_tot = xor32_sum(l_acc[0]);   // lanes 32-63 hold zeros in element 0
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
    if (p.lse && q == 0) p.lse[((size_t)b * p.Hq + h) * p.C + c_out] = (m_ref + __log2f(l_tot)) * 0.69314718055994530942f;
  }
}

template <int D, int HPW>
hipError_t launch_hpw(const PrefillParams& p, hipStream_t s) {
  constexpr int WQ = kWaves / HPW;
  dim3 grid(((p.C + WQ * kQB - 1) / (WQ * kQB)) * (p.Hq / HPW) * p.B);
  if constexpr (D == 128) {
    if (p.out_bf16)
      prefill_pipe_kernel<HPW, true><<<grid, kThreads, 0, s>>>(p);
    else
      prefill_pipe_kernel<HPW, false><<<grid, kThreads, 0, s>>>(p);
  } else {
    if (p.out_bf16)
      prefill_kernel<D, HPW, true><<<grid, kThreads, 0, s>>>(p);
    else
      prefill_kernel<D, HPW, false><<<grid, kThreads, 0, s>>>(p);
  }
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
