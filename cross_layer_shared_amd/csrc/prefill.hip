// Causal chunked prefill of a cross-decoder layer over the global cache
// (YOCO summary, abstract: end to end the model works as a decoder-only
// Transformer does, so the query at absolute position p attends to cache rows
// [0, p]; YOCO++ summary, section 3: prefill is compute-bound).
//
// Dense contraction on bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
// A workgroup of 8 wavefronts serves 8 (head, 32-query block) slots that share
// one kv head (4 heads x 2 consecutive query blocks); it streams the cache in
// 128-key tiles staged through LDS (two K and two V slots), so that all eight
// wavefronts read each tile from LDS instead of from memory. K and V are both
// stored row-major; the V operand of the PV product is read with the gfx950
// transposing LDS read (ds_read_b64_tr_b16), which hands each lane 4
// consecutive keys of one dim.
//
// At D = 128 the two wavefronts on each SIMD (waves w and w + 4) run half a
// tile apart: while one issues the MFMAs of a tile (PV of the previous tile,
// scores of this one) the other runs the softmax of its tile on the VALU and
// the exponential unit, and the workgroup barrier between the halves swaps
// the roles. Run in step instead, both wavefronts would wait on the matrix
// core at the same time and then both on the VALU. At D = 64 the MFMA phase
// is half as long and the softmax phase dominates; there they run in step.
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
// Probabilities are rounded to bf16 for the PV product, and the normaliser
// sums the same rounded values.
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
      float m = fmaxf(sc[hb][0], sc[hb][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) m = fmaxf(fmaxf(m, sc[hb][r]), sc[hb][r + 1]);
      mb[hb] = m;
    }
    // the scale is positive, so the max of the scaled scores is the scaled max
    const float mt = xor32_max(fmaxf(fmaxf(mb[0], mb[1]), fmaxf(mb[2], mb[3]))) * sl;
    // Lazy rescaling: the reference max m_run only moves when some row's
    // tile max exceeds it by more than kLazy (log2 units), so exponentials
    // stay below 2^kLazy and the accumulators are rescaled in few tiles.
    // Numerator and normaliser share the reference, so the result is exact
    // up to rounding for any choice of it.
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mt);
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
