// Decode split pass on the matrix cores: bf16 caches, decode over a composed
// cache (YOCO summary, abstract and method details: every cross-decoder layer
// attends to the one global KV cache; YOCO++ summary, section 2: that cache is
// the middle layer's composed K'_{L/2}, V'_{L/2}; section 3: decoding reads
// one KV set per layer).
//
// The split pass does, per cache row, 4 G D flops against 4 D bytes: far
// below any ridge, so the time is the stream of K' and V'. On the vector ALU
// those flops still cost about 270 instructions per 16 rows per wavefront,
// which delay each wavefront's next loads; here both contractions run on
// v_mfma_f32_16x16x32_bf16 and the vector ALU keeps only the softmax.
//
// One workgroup per (sequence b, kv head g, split), as in the vector kernel,
// whose merge of the wavefronts, split partials and fused log-sum-exp merge
// it shares (finish_split). A wavefront takes blocks of 32 cache rows:
//   K and V rows arrive by 16-byte loads of whole rows (four rows of 256
//     bytes per instruction at D = 128), the access pattern that streams
//     fastest: a load instruction that gathers 64-byte pieces of 16 rows, as
//     an MFMA operand taken straight from memory would, moves 128 MiB about
//     17% slower. Both go through the wavefront's own LDS buffers.
//   S^T = K Q^T: two 16-row MFMA blocks by 16 query columns (the G heads of
//     kv head g; columns G..15 are zero), D/32 k-steps each, the K operand
//     one 16-byte LDS read (K rows stored with their 16-byte chunks XOR-
//     swizzled so that the 16 rows one read instruction serves sit in
//     distinct banks). Row r of block bb carries cache row
//     8 (r / 4) + 4 bb + (r % 4), so that lane (lg, q)
//     ends up with the scores of query q for the 8 consecutive rows
//     8 lg .. 8 lg + 7 of the block: exactly the P^T operand it supplies to
//   O^T += V^T P^T: one MFMA per 16 dims, V^T read from LDS with the gfx950
//     transposing read (each lane gets 4 consecutive rows of one dim).
// The probabilities stay fp32-accurate: each is split into a bf16 head and a
// bf16 remainder (p - head, exact in fp32, rounded once more), and both go
// through the PV product, so the weights carry about 16 significant bits.
// The softmax is online in the log2 domain with a lazily moved reference
// (rescaled only when a block's maximum exceeds it by more than 2^8).

#include <math.h>

#include <hip/hip_runtime.h>

#include "decode_kernel.h"
#include "decode_layout.h"

namespace yoco {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kBlock = 32;       // cache rows per block (one k-step of the PV product)
constexpr float kLazy = 8.f;     // rescale threshold of the running max (log2 units)

// Transposing LDS read: within each 16-lane group, lane i receives element
// (i % 4) of the 8-byte rows addressed by lanes 4e + i/4, e = 0..3.
__device__ __forceinline__ s16x4_t read_tr16(const __bf16* ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4_t*)(__attribute__((address_space(3))) void*)(const_cast<__bf16*>(ptr)));
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};   // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// max / sum over the four 16-lane rows that hold the same query (lanes q, q+16, q+32, q+48)
__device__ __forceinline__ float rows_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int G, int NW, int MODE>
__global__ __launch_bounds__(64 * NW) void decode_mfma_kernel(DecodeParams p) {
  constexpr bool COR = MODE == kComposeOnRead;   // K', V' formed per row from two raw caches
  constexpr bool APP = MODE == kAppend;          // self-decoder step: compose and append the new row
  constexpr int NQK = D / 32;          // k-steps of the score product
  constexpr int NDB = D / 16;          // 16-dim blocks of O^T
  // per-wavefront LDS buffers and their addresses: decode_layout.h (checked by a host build)
  using L = dlay::Shape<D>;
  constexpr int RPI = L::RPI;          // cache rows per load instruction (L::LPR lanes per row, 16 bytes each)
  constexpr int NVI = L::NLI;          // load instructions per block and tensor
  constexpr int SV = NW * L::kVElems * 2;             // bytes of the per-wavefront V buffers
  constexpr int SK = NW * L::kKElems * 2;             // bytes of the per-wavefront K buffers
  constexpr int SM = NW * G * (D + 2) * 4;            // bytes of the wavefront merge
  __shared__ __attribute__((aligned(16))) unsigned char smem[SV + SK > SM ? SV + SK : SM];

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  // Kernel arguments in one batch: the query pointer and the cache views the
  // first row loads need are held in registers here, ahead of the branches
  // below; left to the compiler they are fetched in a second round trip after
  // the first batch, and every launch pays it before its stream starts.
  asm volatile("" ::"s"(p.q), "s"(p.k.ptr), "s"(p.k.sb), "s"(p.k.sh), "s"(p.k.st), "s"(p.v.ptr), "s"(p.v.sb),
               "s"(p.v.sh), "s"(p.v.st));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lg = lane >> 4;            // 16-lane row of the MFMA operands
  const int lr = lane & 15;            // lane within the row: query column / key row / dim

  int len = p.T;
  if (p.seq_lens) {
    len = p.seq_lens[b];
    len = len < 1 ? 1 : (len > p.T ? p.T : len);
  }
  const int ts = split * p.rows_per_split;
  // In append mode the cache supplies rows [0, len - 1); row len - 1 is the
  // new token, composed and folded in by the split whose range holds it.
  const int te = min(ts + p.rows_per_split, APP ? len - 1 : len);
  const bool own_new = APP && split == (len - 1) / p.rows_per_split;

  // Append mode: the owner's first wavefront loads the new token's K_1, K_i,
  // V_1, V_i rows now (lanes 0 .. D/8 - 1, 8 elements each) and composes them
  // after its stream.
  __shared__ __attribute__((aligned(16))) __bf16 s_new[2][D];   // the composed new row: K', V'
  u32x4_t nsrc[4] = {};
  const bool new_lane = own_new && threadIdx.x < D / 8;
  if constexpr (APP) {
    if (new_lane) {
      const View4* views[4] = {&p.nk1, &p.nki, &p.nv1, &p.nvi};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        nsrc[i] = *reinterpret_cast<const u32x4_t*>(static_cast<const __bf16*>(views[i]->ptr) + (int64_t)b * views[i]->sb +
                                                    (int64_t)g * views[i]->sh + (int64_t)(len - 1) * views[i]->st +
                                                    8 * threadIdx.x);
    }
  }

  // Q^T operand: lane (lg, lr) holds query head g G + lr (zero for lr >= G),
  // dims 32 j + 8 lg .. + 8 of k-step j.
  bf16x8_t qf[NQK];
  {
    const __bf16* qrow = static_cast<const __bf16*>(p.q) + ((size_t)(b * p.Hq + g * G + min(lr, G - 1)) * D + 8 * lg);
#pragma unroll
    for (int j = 0; j < NQK; ++j) {
      const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * j);
      qf[j] = lr < G ? v : bf16x8_t{};
    }
  }

  // The split's rows of (b, g) through buffer resources bounded at te: rows at
  // or past te read as zeros (and their scores are masked), so a block that
  // crosses the end needs no clamping.
  const uint32_t kst = (uint32_t)(p.k.st * 2), vst = (uint32_t)(p.v.st * 2);
  const auto rk = rows_rsrc(static_cast<const char*>(p.k.ptr) + ((int64_t)b * p.k.sb + (int64_t)g * p.k.sh) * 2,
                            te > 0 ? (uint32_t)te * kst : 0u);
  const auto rv = rows_rsrc(static_cast<const char*>(p.v.ptr) + ((int64_t)b * p.v.sb + (int64_t)g * p.v.sh) * 2,
                            te > 0 ? (uint32_t)te * vst : 0u);
  // Block loads: instruction i brings rows RPI i .. + RPI, lane -> row lane / L::LPR, dims 8 (lane % L::LPR).
  const uint32_t koff = (uint32_t)dlay::load_row<D>(0, lane) * kst + 16u * dlay::load_chunk<D>(lane);
  const uint32_t voff = (uint32_t)dlay::load_row<D>(0, lane) * vst + 16u * dlay::load_chunk<D>(lane);

  auto load = [&](int base, u32x4_t (&kr)[NVI], u32x4_t (&vr)[NVI]) {
#pragma unroll
    for (int i = 0; i < NVI; ++i) kr[i] = buffer_load<4>(rk, (uint32_t)(base + RPI * i) * kst + koff);
#pragma unroll
    for (int i = 0; i < NVI; ++i) vr[i] = buffer_load<4>(rv, (uint32_t)(base + RPI * i) * vst + voff);
  };

  // Compose on read (the comparator that caches the raw K_i, V_i): layer 1's
  // rows are loaded at the same places and every K', V' element is formed with
  // the compose kernel's arithmetic, so the products see exactly the values a
  // composed cache would hold.
  __amdgpu_buffer_rsrc_t rk1 = rk, rv1 = rv;
  uint32_t k1st = kst, v1st = vst, koff1 = koff, voff1 = voff;
  if constexpr (COR) {
    k1st = (uint32_t)(p.k1.st * 2);
    v1st = (uint32_t)(p.v1.st * 2);
    rk1 = rows_rsrc(static_cast<const char*>(p.k1.ptr) + ((int64_t)b * p.k1.sb + (int64_t)g * p.k1.sh) * 2,
                    te > 0 ? (uint32_t)te * k1st : 0u);
    rv1 = rows_rsrc(static_cast<const char*>(p.v1.ptr) + ((int64_t)b * p.v1.sb + (int64_t)g * p.v1.sh) * 2,
                    te > 0 ? (uint32_t)te * v1st : 0u);
    koff1 = (uint32_t)dlay::load_row<D>(0, lane) * k1st + 16u * dlay::load_chunk<D>(lane);
    voff1 = (uint32_t)dlay::load_row<D>(0, lane) * v1st + 16u * dlay::load_chunk<D>(lane);
  }
  auto compose4 = [&](u32x4_t x1, u32x4_t xi, float c1, float c2, int terms) {
    u32x4_t r;
#pragma unroll
    for (int w = 0; w < 4; ++w) r[w] = compose_dword<true>(x1[w], xi[w], c1, c2, terms);
    return r;
  };
  auto load_composed = [&](int base, u32x4_t (&kr)[NVI], u32x4_t (&vr)[NVI]) {
    u32x4_t k1r[NVI], v1r[NVI];
    load(base, kr, vr);
#pragma unroll
    for (int i = 0; i < NVI; ++i) k1r[i] = buffer_load<4>(rk1, (uint32_t)(base + RPI * i) * k1st + koff1);
#pragma unroll
    for (int i = 0; i < NVI; ++i) v1r[i] = buffer_load<4>(rv1, (uint32_t)(base + RPI * i) * v1st + voff1);
#pragma unroll
    for (int i = 0; i < NVI; ++i) kr[i] = compose4(k1r[i], kr[i], p.cK1, p.cK2, p.termsK);
#pragma unroll
    for (int i = 0; i < NVI; ++i) vr[i] = compose4(v1r[i], vr[i], p.cV1, p.cV2, p.termsV);
  };

  __bf16* sv = reinterpret_cast<__bf16*>(smem) + wave * L::kVElems;
  // this wavefront's K buffer: kBlock rows of D, chunk c of row r at position c ^ k_swizzle(r)
  __bf16* sk = reinterpret_cast<__bf16*>(smem + SV) + wave * L::kKElems;
  f32x4_t o[NDB];
#pragma unroll
  for (int n = 0; n < NDB; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // reference max of query lr (log2 domain), the same in all four rows
  float l_run = 0.f;         // this lane's share of the running sum of query lr
  const float sl = p.scale_log2;

  auto block = [&](const u32x4_t (&kr)[NVI], const u32x4_t (&vr)[NVI], int base) {
    // K and V rows into this wavefront's LDS buffers (K swizzled, V padded rows)
#pragma unroll
    for (int i = 0; i < NVI; ++i) *reinterpret_cast<u32x4_t*>(sk + dlay::k_write<D>(i, lane)) = kr[i];
#pragma unroll
    for (int i = 0; i < NVI; ++i) *reinterpret_cast<u32x4_t*>(sv + dlay::v_write<D>(i, lane)) = vr[i];
    __builtin_amdgcn_wave_barrier();
    // S^T: lane (lg, q) gets the raw scores of query q for rows 8 lg + 4 bb + i
    f32x4_t sc[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      sc[bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NQK; ++j) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(sk + dlay::k_read<D>(lane, bb, j));
        sc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[j], sc[bb], 0, 0, 0);
      }
    }
    if (base + kBlock > te) {   // rows past the split's end
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (base + 8 * lg + 4 * bb + i >= te) sc[bb][i] = -INFINITY;
    }
    // block max of the query (the scale is positive, so the max of the scaled
    // scores is the scaled max), lazy move of the reference
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    const float mt = rows_max(mx) * sl;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < NDB; ++n) o[n] *= alpha;
      m_run = m_new;
    }
    const float mu = (m_run == -INFINITY) ? 0.f : m_run;
    // probabilities of rows 8 lg + e, e = 4 bb + i; split into bf16 head and remainder
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float p0 = fast_exp2(__builtin_fmaf(sc[w >> 1][2 * (w & 1)], sl, -mu));
      const float p1 = fast_exp2(__builtin_fmaf(sc[w >> 1][2 * (w & 1) + 1], sl, -mu));
      l_run += p0 + p1;
      hi[w] = pack_bf16(p0, p1);
      lo[w] = pack_bf16(p0 - lo_bf16(hi[w]), p1 - hi_bf16(hi[w]));
    }
    const bf16x8_t phi = __builtin_bit_cast(bf16x8_t, u32x4_t{hi[0], hi[1], hi[2], hi[3]});
    const bf16x8_t plo = __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], lo[2], lo[3]});
    // O^T += V^T P^T, V^T from the transposing reads: lane (lg, r) gets dim 16 n + r
    // of rows 8 lg .. 8 lg + 7 (two reads of four rows)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int n = 0; n < NDB; ++n) {
      const s16x4_t r0 = read_tr16(sv + dlay::v_tr_read<D>(lane, n, 0));
      const s16x4_t r1 = read_tr16(sv + dlay::v_tr_read<D>(lane, n, 1));
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi, o[n], 0, 0, 0);
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo, o[n], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  };

  // Blocks of this wavefront: base, base + NW 32, ...; the next block's loads
  // are in flight while the current one is consumed (two register sets).
  constexpr int STEP = NW * kBlock;
  int base = ts + wave * kBlock;
  if constexpr (COR) {
    // one register set (four raw streams per block), composed as it arrives
    for (; base < te; base += STEP) {
      u32x4_t kr[NVI], vr[NVI];
      load_composed(base, kr, vr);
      block(kr, vr, base);
    }
  } else if (base < te) {
    u32x4_t ka[NVI], kb[NVI], va[NVI], vb[NVI];
    load(base, ka, va);
    while (true) {
      const int nb = base + STEP;
      if (nb < te) load(nb, kb, vb);
      block(ka, va, base);
      base = nb;
      if (base >= te) break;
      const int nb2 = base + STEP;
      if (nb2 < te) load(nb2, ka, va);
      block(kb, vb, base);
      base = nb2;
      if (base >= te) break;
    }
  }

  // ---- append mode: compose the new row, write it into the cache and fold it
  // into the first wavefront's state ----
  if constexpr (APP) {
    if (own_new && wave == 0) {
      if (new_lane) {
        u32x4_t kn, vn;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          kn[w] = compose_dword<true>(nsrc[0][w], nsrc[1][w], p.cK1, p.cK2, p.termsK);
          vn[w] = compose_dword<true>(nsrc[2][w], nsrc[3][w], p.cV1, p.cV2, p.termsV);
        }
        *reinterpret_cast<u32x4_t*>(const_cast<__bf16*>(static_cast<const __bf16*>(p.k.ptr)) + (int64_t)b * p.k.sb +
                                    (int64_t)g * p.k.sh + (int64_t)(len - 1) * p.k.st + 8 * threadIdx.x) = kn;
        *reinterpret_cast<u32x4_t*>(const_cast<__bf16*>(static_cast<const __bf16*>(p.v.ptr)) + (int64_t)b * p.v.sb +
                                    (int64_t)g * p.v.sh + (int64_t)(len - 1) * p.v.st + 8 * threadIdx.x) = vn;
        *reinterpret_cast<u32x4_t*>(&s_new[0][8 * threadIdx.x]) = kn;
        *reinterpret_cast<u32x4_t*>(&s_new[1][8 * threadIdx.x]) = vn;
      }
      __builtin_amdgcn_wave_barrier();
      // score of the new row for query lr: this lane's dims 32 j + 8 lg .. + 8, summed over the four rows
      float x = 0.f;
#pragma unroll
      for (int j = 0; j < NQK; ++j) {
        const u32x4_t kw = *reinterpret_cast<const u32x4_t*>(&s_new[0][32 * j + 8 * lg]);
        const u32x4_t qw = __builtin_bit_cast(u32x4_t, qf[j]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // element through a scalar first: a bit-cast straight from a vector
          // element compiles to the first element only (all four times)
          const uint32_t qe = qw[w], ke = kw[w];
          x = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qe), __builtin_bit_cast(bf16x2_t, ke), x,
                                              false);
        }
      }
      x = rows_sum(x) * sl;
      const float m2 = fmaxf(m_run, x);
      const float wo = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m2);
      const float wn = fast_exp2(x - m2);
      l_run = l_run * wo + (lg == 0 ? wn : 0.f);   // the new row's weight counted once per query
#pragma unroll
      for (int n = 0; n < NDB; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[n][i] = __builtin_fmaf(wn, (float)s_new[1][16 * n + 4 * lg + i], o[n][i] * wo);
      m_run = m2;
    }
  }

  // ---- this wavefront's state into LDS: lane (lg, q) holds dims 16 n + 4 lg + i of query q ----
  const float l_q = rows_sum(l_run);
  __syncthreads();   // every wavefront is done with its V buffer
  float* sm_acc = reinterpret_cast<float*>(smem);          // [NW][G][D]
  float* sm_m = sm_acc + NW * G * D;                        // [NW][G]
  float* sm_l = sm_m + NW * G;                              // [NW][G]
  if (lr < G) {
#pragma unroll
    for (int n = 0; n < NDB; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_acc[(wave * G + lr) * D + 16 * n + 4 * lg + i] = o[n][i];
    if (lg == 0) {
      sm_m[wave * G + lr] = m_run;
      sm_l[wave * G + lr] = l_q;
    }
  }
  __syncthreads();
  finish_split<D, G, NW>(p, b, g, split, sm_acc, sm_m, sm_l);
}

template <int D, int NW, int MODE>
hipError_t launch_g(const DecodeParams& p, hipStream_t s) {
  const dim3 grid(p.num_splits, p.Hkv, p.B);
  switch (p.Hq / p.Hkv) {
    case 1: decode_mfma_kernel<D, 1, NW, MODE><<<grid, 64 * NW, 0, s>>>(p); break;
    case 2: decode_mfma_kernel<D, 2, NW, MODE><<<grid, 64 * NW, 0, s>>>(p); break;
    case 4: decode_mfma_kernel<D, 4, NW, MODE><<<grid, 64 * NW, 0, s>>>(p); break;
    case 8: decode_mfma_kernel<D, 8, NW, MODE><<<grid, 64 * NW, 0, s>>>(p); break;
    case 16: decode_mfma_kernel<D, 16, NW, MODE><<<grid, 64 * NW, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode_mfma(const DecodeParams& p, hipStream_t s) {
  if (p.D == 128) return p.waves == 8 ? launch_g<128, 8, MODE>(p, s) : launch_g<128, 4, MODE>(p, s);
  if (p.D == 64) return p.waves == 8 ? launch_g<64, 8, MODE>(p, s) : launch_g<64, 4, MODE>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream) {
  if (p.append) return launch_mode_mfma<kAppend>(p, stream);
  return p.compose_on_read ? launch_mode_mfma<kComposeOnRead>(p, stream) : launch_mode_mfma<kPlain>(p, stream);
}

}  // namespace yoco
