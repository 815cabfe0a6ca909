// Decode attention of the cross-decoder over the one shared cache
// (YOCO summary, abstract and method details: every cross-decoder layer
// attends, by cross-attention, to the one global KV cache; YOCO++ summary, section 2:
// the cache is the middle layer's composed K'_{L/2}, V'_{L/2}; section 3:
// decoding reads exactly one KV set per layer).
//
// Split pass: one workgroup (4 or 8 wavefronts) per (sequence b, kv head g,
// split s) streams the split's rows of K' and V' exactly once, through buffer
// resources bounded at the split's end. The G = Hq/Hkv query heads that share
// kv head g are all served from the same loaded row. Short splits double-buffer
// the row loads where a register set of rows is small.
//
// Lane layout of a wavefront: the 64 lanes form four 16-lane DPP rows
// ("groups"); in one iteration group j holds cache rows base + 4u + j for
// u < U = 16/G, lane s of the group holding elements [s*D/16, (s+1)*D/16) of
// each row. A V load instruction of the wavefront reads four consecutive
// cache rows (a contiguous 1 KiB block for a bf16 D=128 cache).
//
// Scores: each lane forms 16 = U*G partial dot products over its slice, and a
// transposed butterfly over the 16 lanes of the group (DPP partners s^8, s^7,
// s^2, s^1, which span the 4 lane bits) leaves lane s holding the complete
// score of (row u, head hh) with s = u*G + hh. The butterfly keeps, at every
// stage, the same half of each lane's values and sends the other half when
// slot k of lane s holds the partial of index s ^ c(k), c(k) = k ^ (k & 4 ?
// 3 : 0) ("XOR layout"); lane s then needs K row (s / G) ^ (c(k) / G) and
// query head (s mod G) ^ (c(k) mod G) for slot k. The query heads are loaded
// in that permuted order once, and the K load of row slot r fetches row
// ((s / G) ^ r) per lane, which keeps every load segment G * D/16 elements
// long; this is used where those segments are at least 64 bytes. Otherwise
// every lane holds the rows in plain order and the butterfly selects which
// half to keep and send per lane bit. Each group keeps an
// online-softmax state (running max m and sum l per head, in the log2
// domain, and the weighted value sums of its slice); the running max only
// rescales the value sums when some lane's maximum grew. The four groups and
// wavefronts merge their states once per split.
//
// Compose on read (the comparator that caches raw K_i, V_i): layer 1's rows are
// loaded beside layer i's and every K', V' row is formed with the compose
// kernel's arithmetic before use.
//
// Self-decoder step (append mode): the sequence's last row n - 1 is the new
// token. The split that owns it composes the token's K'_i, V'_i from its
// K_1, K_i, V_1, V_i rows with the compose kernel's arithmetic, writes them
// into the cache and folds the row into its softmax state; the cache is read
// only for rows [0, n - 1).
//
// Merge: the splits' normalised outputs are combined with their log-sum-exps.
// In the combined entry point the merge is fused: every workgroup takes a
// ticket (atomic counter per (b, g)) after writing its partial, and the last
// one merges the S partials of its G heads in one pass (running maximum) and
// resets the counter to zero.

#pragma once

#include <math.h>

#include <hip/hip_runtime.h>

#include "common.h"
#include "compose_math.h"

namespace yoco {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---- DPP helpers (within 16-lane rows) ----
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kHalfMirror = 0x141;    // row_half_mirror: lane ^ 7 within 8
constexpr int kRowRor = 0x120;        // + n: rotate right by n within the row
constexpr int kRowNewBcast = 0x150;   // + n: broadcast lane n of each row

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  // every control used here reads a valid lane of the same row, so no lane keeps an old value
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Broadcast lane n (compile-time) of each 16-lane row to the whole row.
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return dpp<kRowNewBcast + N>(x);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int N>
struct DW {
  typedef uint32_t type __attribute__((ext_vector_type(N)));
};
template <>
struct DW<1> {
  typedef uint32_t type;
};

template <bool BF16, int D>
struct Layout {
  static constexpr int kEPL = D / 16;                       // elements per lane per row
  static constexpr int kNDW = BF16 ? kEPL / 2 : kEPL;       // dwords per lane per row
  static constexpr int kES = BF16 ? 2 : 4;                  // bytes per element
  typedef typename DW<kNDW>::type vec;
};

// Raw buffer resource over [base, base + bytes): loads at offsets past the end
// return zeros (dword 3 = 32-bit data format, unswizzled, as gfx950 expects).
constexpr int kBufferWord3 = 0x00020000;
constexpr int kLoadNT = 2;   // cache policy: nontemporal (streamed once)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

// N dwords (N = 2, 4 or 8) at byte offset off of a buffer, nontemporal.
template <int N>
__device__ __forceinline__ typename DW<N>::type buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  if constexpr (N == 2) {
    return __builtin_bit_cast(typename DW<2>::type, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kLoadNT));
  } else if constexpr (N == 4) {
    return __builtin_bit_cast(typename DW<4>::type, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kLoadNT));
  } else {
    static_assert(N == 8, "row slices are 2, 4 or 8 dwords");
    const i32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kLoadNT);
    const i32x4 c = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off + 16, 0, kLoadNT);
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    const i32x8 v = __builtin_shufflevector(a, c, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(typename DW<8>::type, v);
  }
}

template <int N>
__device__ __forceinline__ uint32_t dw_at(const typename DW<N>::type& v, int i) {
  if constexpr (N == 1) {
    return v;
  } else {
    return v[i];
  }
}

// Transposed butterfly: x[16] partial sums on the 16 lanes of a row ->
// the lane s returns the full sum of value index s.
__device__ __forceinline__ float reduce16_transposed(const float (&x)[16], int s) {
  float y8[8], y4[4], y2[2];
  const bool b3 = s & 8, b2 = s & 4, b1 = s & 2, b0 = s & 1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float keep = b3 ? x[i + 8] : x[i];
    float send = b3 ? x[i] : x[i + 8];
    y8[i] = keep + dpp<kRowRor + 8>(send);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float keep = b2 ? y8[i + 4] : y8[i];
    float send = b2 ? y8[i] : y8[i + 4];
    y4[i] = keep + dpp<kHalfMirror>(send);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float keep = b1 ? y4[i + 2] : y4[i];
    float send = b1 ? y4[i] : y4[i + 2];
    y2[i] = keep + dpp<kQuadSwap2>(send);
  }
  float keep = b0 ? y2[1] : y2[0];
  float send = b0 ? y2[0] : y2[1];
  return keep + dpp<kQuadSwap1>(send);
}

// The same reduction in the XOR layout: slot k of lane s holds the partial of
// value index s ^ xor_slot(k), so every stage keeps the lower half of the
// slots and sends the upper half, with no per-lane selects.
__device__ __host__ constexpr int xor_slot(int k) { return k ^ ((k & 4) ? 3 : 0); }
__device__ __forceinline__ float reduce16_xor(const float (&x)[16]) {
  float y8[8], y4[4], y2[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) y8[i] = x[i] + dpp<kRowRor + 8>(x[i + 8]);
#pragma unroll
  for (int i = 0; i < 4; ++i) y4[i] = y8[i] + dpp<kHalfMirror>(y8[i + 4]);
#pragma unroll
  for (int i = 0; i < 2; ++i) y2[i] = y4[i] + dpp<kQuadSwap2>(y4[i + 2]);
  return y2[0] + dpp<kQuadSwap1>(y2[1]);
}

// All-reduce (max or sum) over the lanes of a row that share s mod G.
template <int G, bool MAX>
__device__ __forceinline__ float reduce_same_head(float x) {
  if constexpr (G <= 1) x = MAX ? fmaxf(x, dpp<kRowRor + 1>(x)) : x + dpp<kRowRor + 1>(x);
  if constexpr (G <= 2) x = MAX ? fmaxf(x, dpp<kRowRor + 2>(x)) : x + dpp<kRowRor + 2>(x);
  if constexpr (G <= 4) x = MAX ? fmaxf(x, dpp<kRowRor + 4>(x)) : x + dpp<kRowRor + 4>(x);
  if constexpr (G <= 8) x = MAX ? fmaxf(x, dpp<kRowRor + 8>(x)) : x + dpp<kRowRor + 8>(x);
  return x;
}

template <int I, int N>
struct Unroll {
  template <typename F>
  __device__ __forceinline__ static void run(F&& f) {
    f.template operator()<I>();
    Unroll<I + 1, N>::run(f);
  }
};
template <int N>
struct Unroll<N, N> {
  template <typename F>
  __device__ __forceinline__ static void run(F&&) {}
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Agent-scope relaxed atomic accesses: on gfx950 they are performed coherently
// across the XCDs (write-through / read-through of the per-XCD L2), which is
// what the fused merge needs without an L2-wide writeback per workgroup.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LSE merge of S split partials for G consecutive heads (rows bh0 .. bh0+G-1 of
// [B*Hq]); the heads are spread over the NW wavefronts. Per head, the splits are
// taken in batches of 8 whose loads are all issued before they are used, with a
// running maximum (online rescaling) so that no separate pass finds the maximum.
template <int D, int G, int NW, bool AGENT>
__device__ __forceinline__ void merge_splits(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                                             int S, int bh0, float* __restrict__ out, float* __restrict__ lse) {
  constexpr int PER = D / 64;
  constexpr int BATCH = 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  auto ld = [](const float* p) { return AGENT ? load_agent(p) : *p; };
  for (int hh = wave; hh < G; hh += NW) {
    const size_t r0 = (size_t)(bh0 + hh) * S;
    // one pass: the running maximum M rescales the sums when a batch raises it,
    // so a split count up to BATCH costs a single round of loads
    float M = -INFINITY, L = 0.f, o[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] = 0.f;
    for (int i0 = 0; i0 < S; i0 += BATCH) {
      float li[BATCH], ov[BATCH][PER];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int i = min(i0 + u, S - 1);
        li[u] = ld(&part_lse[r0 + i]);
#pragma unroll
        for (int k = 0; k < PER; ++k) ov[u][k] = ld(&part_o[(r0 + i) * D + lane + 64 * k]);
      }
      // empty splits (lse = -inf) and the clamped tail of the last batch weigh 0
#pragma unroll
      for (int u = 0; u < BATCH; ++u)
        if (i0 + u >= S) li[u] = -INFINITY;
      float mb = -INFINITY;
#pragma unroll
      for (int u = 0; u < BATCH; ++u) mb = fmaxf(mb, li[u]);
      if (mb == -INFINITY) continue;   // the same for every lane: all lanes read the same lse values
      const float Mn = fmaxf(M, mb);
      const float keep = (M == -INFINITY) ? 0.f : __expf(M - Mn);
      L *= keep;
#pragma unroll
      for (int k = 0; k < PER; ++k) o[k] *= keep;
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const float w = (li[u] == -INFINITY) ? 0.f : __expf(li[u] - Mn);
        L += w;
#pragma unroll
        for (int k = 0; k < PER; ++k) o[k] = __builtin_fmaf(w, ov[u][k], o[k]);
      }
      M = Mn;
    }
    const float inv = 1.0f / L;
#pragma unroll
    for (int k = 0; k < PER; ++k) out[(size_t)(bh0 + hh) * D + lane + 64 * k] = o[k] * inv;
    if (lse && lane == 0) lse[bh0 + hh] = M + logf(L);
  }
}

constexpr int kPlain = 0;          // decode over a composed cache
constexpr int kComposeOnRead = 1;  // K', V' formed per row from two raw caches
constexpr int kAppend = 2;         // self-decoder step: compose and append the new row

// Merge the wavefronts' softmax states of one split (in LDS: sm_acc [NW][G][D],
// sm_m, sm_l [NW][G], log2 domain) and write the split's result: the output
// itself when there is one split, else the split's partial, and then, with
// tickets, the fused merge by the last workgroup of (b, g) to finish. Called by
// every thread of the workgroup after a barrier that follows the LDS writes.
template <int D, int G, int NW>
__device__ __forceinline__ void finish_split(const DecodeParams& p, int b, int g, int split,
                                             const float* __restrict__ sm_acc, const float* __restrict__ sm_m,
                                             const float* __restrict__ sm_l) {
  // ---- merge the wavefronts and write this split's result ----
  const int h0 = g * G;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * NW) {
    const int hh = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w * G + hh]);
    float Lsum = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      float m = sm_m[w * G + hh];
      float wt = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
      Lsum += wt * sm_l[w * G + hh];
      O += wt * sm_acc[(w * G + hh) * D + d];
    }
    const bool empty = !(Lsum > 0.f);
    const float o = empty ? 0.f : O / Lsum;
    const float lse = empty ? -INFINITY : (M + __log2f(Lsum)) * 0.69314718055994530942f;
    const int h = h0 + hh;
    if (p.num_splits == 1) {
      p.out[((size_t)b * p.Hq + h) * D + d] = o;
      if (p.lse && d == 0) p.lse[(size_t)b * p.Hq + h] = lse;
    } else {
      const size_t row = ((size_t)b * p.Hq + h) * p.num_splits + split;
      if (p.tickets) {          // published to the merging workgroup, possibly on another XCD
        store_agent(&p.part_o[row * D + d], o);
        if (d == 0) store_agent(&p.part_lse[row], lse);
      } else {
        p.part_o[row * D + d] = o;
        if (d == 0) p.part_lse[row] = lse;
      }
    }
  }
  if (p.num_splits == 1 || p.tickets == nullptr) return;

  // ---- fused merge: the last workgroup of (b, g) to finish merges all splits ----
  // Every wave drains its partial stores (acknowledged at agent scope) before
  // the barrier, so the ticket is taken only after the whole partial is visible.
  __shared__ int sm_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old =
        __hip_atomic_fetch_add(&p.tickets[b * p.Hkv + g], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm_last = old == (unsigned)(p.num_splits - 1);
  }
  __syncthreads();
  if (!sm_last) return;
  merge_splits<D, G, NW, true>(p.part_o, p.part_lse, p.num_splits, b * p.Hq + h0, p.out, p.lse);
  if (threadIdx.x == 0)   // ready for the next call
    __hip_atomic_store(&p.tickets[b * p.Hkv + g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool BF16, int D, int G, int NW, bool PREFETCH, int MODE>
__global__ __launch_bounds__(64 * NW) void decode_split_kernel(DecodeParams p) {
  constexpr bool COR = MODE == kComposeOnRead;
  constexpr bool APP = MODE == kAppend;
  using L = Layout<BF16, D>;
  using vec = typename L::vec;
  constexpr int EPL = L::kEPL;
  constexpr int NDW = L::kNDW;
  constexpr int U = 16 / G;          // rows per group per iteration
  constexpr int R = 4 * U;           // rows per wavefront per iteration
  constexpr int LG = G >= 16 ? 4 : G >= 8 ? 3 : G >= 4 ? 2 : G >= 2 ? 1 : 0;   // log2(G)
  constexpr bool XL = G >= 4 && G * EPL * L::kES >= 64;   // XOR layout: K segments of >= 64 bytes

  __shared__ float sm_acc[NW][G][D];
  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane >> 4;
  const int s = lane & 15;
  const int my_u = s / G;            // row of the score this lane owns

  int len = p.T;
  if (p.seq_lens) {
    len = p.seq_lens[b];
    len = len < 1 ? 1 : (len > p.T ? p.T : len);
  }
  const int ts = split * p.rows_per_split;
  // In append mode the cache supplies rows [0, len - 1); row len - 1 is the
  // new token, handled by the split whose range holds it.
  const int te = min(ts + p.rows_per_split, APP ? len - 1 : len);
  const bool own_new = APP && split == (len - 1) / p.rows_per_split;

  // Query slices of the G heads of this group (same dims as the lane's K
  // slice); in the XOR layout qv[m] holds head m ^ (s mod G).
  vec qv[G];
  const char* qbase = static_cast<const char*>(p.q) + ((size_t)(b * p.Hq + g * G) * D + s * EPL) * L::kES;
#pragma unroll
  for (int m = 0; m < G; ++m)
    qv[m] = *reinterpret_cast<const vec*>(qbase + (size_t)(XL ? (m ^ (s & (G - 1))) : m) * D * L::kES);

  float acc[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
  float m_run = -INFINITY;   // running max (log2 domain) of head my_h in this group
  float l_run = 0.f;         // this lane's share of the running sum

  const char* kbase = static_cast<const char*>(p.k.ptr) + ((int64_t)b * p.k.sb + (int64_t)g * p.k.sh) * L::kES +
                      s * EPL * L::kES;
  const char* vbase = static_cast<const char*>(p.v.ptr) + ((int64_t)b * p.v.sb + (int64_t)g * p.v.sh) * L::kES +
                      s * EPL * L::kES;
  const int64_t kst = p.k.st * L::kES, vst = p.v.st * L::kES;

  // The split's rows stream through buffer resources over rows [0, te) of
  // (b, g): a lane's address is one 32-bit offset (the host checks that a
  // head's rows span less than 2 GiB), and rows at or past te read as zeros,
  // so the last block needs no clamping (its scores are masked below).
  auto head_rows = [&](const View4& t, int64_t st_b) {
    return rows_rsrc(static_cast<const char*>(t.ptr) + ((int64_t)b * t.sb + (int64_t)g * t.sh) * L::kES,
                     te > 0 ? (uint32_t)te * (uint32_t)st_b : 0u);
  };
  const auto rk = head_rows(p.k, kst), rv = head_rows(p.v, vst);
  const uint32_t lane_k = (uint32_t)j * (uint32_t)kst + s * EPL * L::kES;
  // K row slot r of the lane: row base + krow(r) + j
  auto krow = [&](int r) { return XL ? 4 * ((s >> LG) ^ r) : 4 * r; };
  const uint32_t lane_v = (uint32_t)j * (uint32_t)vst + s * EPL * L::kES;

  // Compose on read: layer 1's rows are read as well and K', V' are formed per
  // row with the compose kernel's arithmetic (two KV sets read instead of one).
  __amdgpu_buffer_rsrc_t rk1 = rk, rv1 = rv;
  uint32_t k1st = 0, v1st = 0, lane_k1 = 0, lane_v1 = 0;
  if constexpr (COR) {
    k1st = (uint32_t)(p.k1.st * L::kES);
    v1st = (uint32_t)(p.v1.st * L::kES);
    rk1 = head_rows(p.k1, k1st);
    rv1 = head_rows(p.v1, v1st);
    lane_k1 = (uint32_t)j * k1st + s * EPL * L::kES;
    lane_v1 = (uint32_t)j * v1st + s * EPL * L::kES;
  }
  auto compose_vec = [&](const vec& x1, const vec& xi, float c1, float c2, int terms) {
    vec out;
    if constexpr (NDW == 1) {
      out = compose_dword<BF16>(x1, xi, c1, c2, terms);
    } else {
#pragma unroll
      for (int w = 0; w < NDW; ++w) out[w] = compose_dword<BF16>(x1[w], xi[w], c1, c2, terms);
    }
    return out;
  };

  // Append mode: the owner's first wavefront loads the new token's source rows
  // now and composes them after the stream (the loads are in flight meanwhile).
  vec nk1{}, nki{}, nv1{}, nvi{};
  if constexpr (APP) {
    if (own_new && wave == 0) {
      auto src = [&](const View4& t) {
        return *reinterpret_cast<const vec*>(static_cast<const char*>(t.ptr) +
                                             ((int64_t)b * t.sb + (int64_t)g * t.sh + (int64_t)(len - 1) * t.st +
                                              s * EPL) * L::kES);
      };
      nk1 = src(p.nk1);
      nki = src(p.nki);
      nv1 = src(p.nv1);
      nvi = src(p.nvi);
    }
  }

  auto load = [&](int base, vec (&kr)[U], vec (&vr)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) kr[u] = buffer_load<NDW>(rk, lane_k + (uint32_t)(base + krow(u)) * (uint32_t)kst);
#pragma unroll
    for (int u = 0; u < U; ++u) vr[u] = buffer_load<NDW>(rv, lane_v + (uint32_t)(base + 4 * u) * (uint32_t)vst);
    if constexpr (COR) {
      vec k1r[U], v1r[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        k1r[u] = buffer_load<NDW>(rk1, lane_k1 + (uint32_t)(base + krow(u)) * k1st);
        v1r[u] = buffer_load<NDW>(rv1, lane_v1 + (uint32_t)(base + 4 * u) * v1st);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kr[u] = compose_vec(k1r[u], kr[u], p.cK1, p.cK2, p.termsK);
        vr[u] = compose_vec(v1r[u], vr[u], p.cV1, p.cV2, p.termsV);
      }
    }
  };

  auto rows = [&](const vec (&kr)[U], const vec (&vr)[U], int base) {
    // Partial dot products over this lane's slice: slot k pairs K row slot u
    // with query register hh (plain layout: x[u*G + hh]).
    float x[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int u = XL ? (xor_slot(k) >> LG) : k / G;
      const int hh = XL ? (xor_slot(k) & (G - 1)) : k % G;
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < NDW; ++w) {
        uint32_t kw = dw_at<NDW>(kr[u], w), qw = dw_at<NDW>(qv[hh], w);
        if constexpr (BF16) {
          a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw), __builtin_bit_cast(bf16x2_t, kw), a,
                                              false);
        } else {
          a = __builtin_fmaf(__uint_as_float(qw), __uint_as_float(kw), a);
        }
      }
      x[k] = a;
    }
    float sc = (XL ? reduce16_xor(x) : reduce16_transposed(x, s)) * p.scale_log2;
    if (base + 4 * my_u + j >= te) sc = -INFINITY;

    float mt = reduce_same_head<G, true>(sc);
    float m_new = fmaxf(m_run, mt);
    float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    float pr = fast_exp2(sc - m_use);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run)) {
      float alpha = fast_exp2(m_run - m_use);
      l_run *= alpha;
      Unroll<0, G>::run([&]<int HH>() {
        float ah = row_bcast<HH>(alpha);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[HH][e] *= ah;
      });
    }
    m_run = m_new;
    l_run += pr;

    // acc[hh] += p(u, hh) * V[u] for the U rows of this group.
    Unroll<0, 16>::run([&]<int V>() {
      constexpr int u = V / G, hh = V % G;
      float pv = row_bcast<V>(pr);
#pragma unroll
      for (int w = 0; w < NDW; ++w) {
        uint32_t vw = dw_at<NDW>(vr[u], w);
        if constexpr (BF16) {
          acc[hh][2 * w] = __builtin_fmaf(pv, lo_bf16(vw), acc[hh][2 * w]);
          acc[hh][2 * w + 1] = __builtin_fmaf(pv, hi_bf16(vw), acc[hh][2 * w + 1]);
        } else {
          acc[hh][w] = __builtin_fmaf(pv, __uint_as_float(vw), acc[hh][w]);
        }
      }
    });
  };

  // Rows of this wavefront: base, base + STEP, ... With PREFETCH the next
  // block's loads are in flight while the current block is consumed (two
  // register sets); short splits need that, long ones prefer the occupancy.
  constexpr int STEP = NW * R;
  int base = ts + wave * R;
  if constexpr (PREFETCH) {
    if (base < te) {
      vec ka[U], va[U], kb[U], vb[U];
      load(base, ka, va);
      while (true) {
        const int nb = base + STEP;
        if (nb < te) load(nb, kb, vb);
        rows(ka, va, base);
        base = nb;
        if (base >= te) break;
        const int nb2 = base + STEP;
        if (nb2 < te) load(nb2, ka, va);
        rows(kb, vb, base);
        base = nb2;
        if (base >= te) break;
      }
    }
  } else {
    // one register set: fewer registers, more wavefronts resident per SIMD
    for (; base < te; base += STEP) {
      vec kr[U], vr[U];
      load(base, kr, vr);
      rows(kr, vr, base);
    }
  }

  // ---- append mode: compose the new row and write it into the cache ----
  vec kn{}, vn{};
  if constexpr (APP) {
    if (own_new && wave == 0) {
      kn = compose_vec(nk1, nki, p.cK1, p.cK2, p.termsK);
      vn = compose_vec(nv1, nvi, p.cV1, p.cV2, p.termsV);
      if (j == 0) {
        *reinterpret_cast<vec*>(const_cast<char*>(kbase) + (int64_t)(len - 1) * kst) = kn;
        *reinterpret_cast<vec*>(const_cast<char*>(vbase) + (int64_t)(len - 1) * vst) = vn;
      }
    }
  }

  // ---- merge the four groups of the wavefront ----
  float l_h = reduce_same_head<G, false>(l_run);   // group's sum for head my_h
  float mg[G], lg[G];
  Unroll<0, G>::run([&]<int HH>() {
    mg[HH] = row_bcast<HH>(m_run);
    lg[HH] = row_bcast<HH>(l_h);
  });
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float M = fmaxf(mg[hh], __shfl_xor(mg[hh], 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    float w = (mg[hh] == -INFINITY) ? 0.f : fast_exp2(mg[hh] - M);
    float lw = lg[hh] * w;
    lw += __shfl_xor(lw, 16);
    lw += __shfl_xor(lw, 32);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float a = acc[hh][e] * w;
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      acc[hh][e] = a;
    }
    if constexpr (APP) {
      // Fold the new row into the owner's first wavefront: its score (the full
      // dot product over the 16 lanes of the group) joins the state (M, lw, acc).
      if (own_new && wave == 0) {
        float x = 0.f;
        vec qh = qv[hh];   // this lane's slice of head hh's query
        if constexpr (XL) {
#pragma unroll
          for (int m = 0; m < G; ++m)
            if ((m ^ (s & (G - 1))) == hh) qh = qv[m];
        }
#pragma unroll
        for (int w2 = 0; w2 < NDW; ++w2) {
          uint32_t kw = dw_at<NDW>(kn, w2), qw = dw_at<NDW>(qh, w2);
          if constexpr (BF16) {
            x = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw), __builtin_bit_cast(bf16x2_t, kw),
                                                x, false);
          } else {
            x = __builtin_fmaf(__uint_as_float(qw), __uint_as_float(kw), x);
          }
        }
        x = reduce_same_head<1, false>(x) * p.scale_log2;
        const float M2 = fmaxf(M, x);
        const float wo = (M == -INFINITY) ? 0.f : fast_exp2(M - M2);
        const float wn = fast_exp2(x - M2);
        lw = lw * wo + wn;
#pragma unroll
        for (int w2 = 0; w2 < NDW; ++w2) {
          uint32_t vw = dw_at<NDW>(vn, w2);
          if constexpr (BF16) {
            acc[hh][2 * w2] = __builtin_fmaf(wn, lo_bf16(vw), acc[hh][2 * w2] * wo);
            acc[hh][2 * w2 + 1] = __builtin_fmaf(wn, hi_bf16(vw), acc[hh][2 * w2 + 1] * wo);
          } else {
            acc[hh][w2] = __builtin_fmaf(wn, __uint_as_float(vw), acc[hh][w2] * wo);
          }
        }
        M = M2;
      }
    }
    if (j == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[wave][hh][s * EPL + e] = acc[hh][e];
      if (s == 0) {
        sm_m[wave][hh] = M;
        sm_l[wave][hh] = lw;
      }
    }
  }
  __syncthreads();

  finish_split<D, G, NW>(p, b, g, split, &sm_acc[0][0][0], &sm_m[0][0], &sm_l[0][0]);
}

// Standalone merge: one workgroup of 4 wavefronts per (b, group of 4 heads), one head per wavefront.
template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(const float* __restrict__ part_o,
                                                                const float* __restrict__ part_lse, int S,
                                                                float* __restrict__ out, float* __restrict__ lse) {
  merge_splits<D, G, kWaves, false>(part_o, part_lse, S, blockIdx.x * G, out, lse);
}

// One launch. Two register sets of rows (prefetch) only where a set is small:
// a set holds 2 * (16 / G) row slices of NDW dwords (more with compose on
// read), and the small-G or fp32 D = 128 shapes would spill with two. The
// wavefront count, and with it the order of every sum, stays as chosen.
template <bool BF16, int D, int G, int NW, bool PF, int MODE>
hipError_t launch_one(const DecodeParams& p, dim3 grid, hipStream_t s) {
  constexpr int set_regs = (MODE == kComposeOnRead ? 4 : 2) * (16 / G) * Layout<BF16, D>::kNDW;
  if constexpr (PF && set_regs > 32) {
    decode_split_kernel<BF16, D, G, NW, false, MODE><<<grid, 64 * NW, 0, s>>>(p);
  } else {
    decode_split_kernel<BF16, D, G, NW, PF, MODE><<<grid, 64 * NW, 0, s>>>(p);
  }
  return hipGetLastError();
}

template <bool BF16, int D, int NW, bool PF, int MODE>
hipError_t launch_gc(const DecodeParams& p, hipStream_t s) {
  dim3 grid(p.num_splits, p.Hkv, p.B);
  switch (p.Hq / p.Hkv) {
    case 1: return launch_one<BF16, D, 1, NW, PF, MODE>(p, grid, s);
    case 2: return launch_one<BF16, D, 2, NW, PF, MODE>(p, grid, s);
    case 4: return launch_one<BF16, D, 4, NW, PF, MODE>(p, grid, s);
    case 8: return launch_one<BF16, D, 8, NW, PF, MODE>(p, grid, s);
    case 16: return launch_one<BF16, D, 16, NW, PF, MODE>(p, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16, int D, int MODE>
hipError_t launch_nw(const DecodeParams& p, hipStream_t s) {
  if (!p.prefetch) return p.waves == 8 ? launch_gc<BF16, D, 8, false, MODE>(p, s) : launch_gc<BF16, D, 4, false, MODE>(p, s);
  if (p.waves == 8) return launch_gc<BF16, D, 8, true, MODE>(p, s);
  return launch_gc<BF16, D, 4, true, MODE>(p, s);
}

// The split pass in one mode, for every supported dtype, D, G and launch shape.
// The vector-ALU split pass serves fp32 caches (bf16 caches take the
// matrix-core kernel of decode_mfma.hip in every mode).
template <int MODE>
hipError_t launch_mode(const DecodeParams& p, hipStream_t s) {
  return p.D == 64 ? launch_nw<false, 64, MODE>(p, s) : launch_nw<false, 128, MODE>(p, s);
}

}  // namespace

// The split pass of a bf16 decode over a composed cache on the matrix cores (decode_mfma.hip).
hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream);

}  // namespace yoco
