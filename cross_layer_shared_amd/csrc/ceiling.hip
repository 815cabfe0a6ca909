// Achievable-rate probes (libyoco_ceiling.so): plain streaming kernels
// with the traffic pattern of the decode (one read of a buffer, 16-byte loads,
// several in flight per thread) and of the compose (four input streams, two
// output streams, one 16-byte vector of each per thread), and none of the
// method's arithmetic. The YOCO++ technical summary, section 3, prices decode
// and composition in bytes moved; these kernels give the time those bytes take
// on this chip when nothing else is done with them. A matrix-core probe does the
// same for the compute-bound prefill: back-to-back bf16 MFMAs on caller data.

#include <stdarg.h>
#include <stdio.h>

#include <hip/hip_runtime.h>

#include "../../include/yoco_ceiling.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStrideWorkgroups = 2048;
constexpr uint32_t kSinkKey = 0x9E3779B9u;

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT) {
    return __builtin_nontemporal_load(p);
  } else {
    return *p;
  }
}

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Workgroup w reads vectors [w * per_wg, min((w + 1) * per_wg, n)), or, with
// per_wg = 0, every thread strides over all n vectors; UNROLL loads of each
// thread are in flight together.
template <bool NT, int UNROLL>
__global__ __launch_bounds__(1024) void read_kernel(const u32x4* __restrict__ src, uint64_t n, uint64_t per_wg,
                                                    uint32_t* __restrict__ sink) {
  const uint64_t nt = blockDim.x;
  uint64_t lo, hi, step;
  if (per_wg) {
    lo = (uint64_t)blockIdx.x * per_wg + threadIdx.x;
    hi = min((uint64_t)(blockIdx.x + 1) * per_wg, n);
    step = nt;
  } else {
    lo = (uint64_t)blockIdx.x * nt + threadIdx.x;
    hi = n;
    step = (uint64_t)gridDim.x * nt;
  }
  uint32_t acc = 0;
  for (uint64_t i = lo; i < hi; i += UNROLL * step) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint64_t k = i + u * step;
      v[u] = k < hi ? load16<NT>(src + k) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= fold(v[u]);
  }
  if (acc == kSinkKey) sink[0] = acc;
}

// Workgroup w reads vectors [w * per_wg, min((w + 1) * per_wg, n)) in blocks of
// 64 UNROLL vectors (UNROLL KiB), dealt to its wavefronts in turn; a
// wavefront's UNROLL loads of a block are in flight together, each a
// contiguous 1 KiB, as the decode's wavefronts stream their row blocks.
template <int UNROLL>
__global__ __launch_bounds__(1024) void read_blocks_kernel(const u32x4* __restrict__ src, uint64_t n, uint64_t per_wg,
                                                           uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
  const uint64_t lo = (uint64_t)blockIdx.x * per_wg, hi = min(lo + per_wg, n);
  uint32_t acc = 0;
  for (uint64_t blk = lo + (uint64_t)wave * 64 * UNROLL; blk < hi; blk += (uint64_t)waves * 64 * UNROLL) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint64_t k = blk + 64 * u + lane;
      v[u] = k < hi ? __builtin_nontemporal_load(src + k) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= fold(v[u]);
  }
  if (acc == kSinkKey) sink[0] = acc;
}

// U positions per thread, blockDim apart (each load and store instruction of a
// wavefront stays one contiguous 1 KiB); every load is issued before any store.
template <int U>
__global__ __launch_bounds__(1024) void read4_write2_kernel(const u32x4* __restrict__ a, const u32x4* __restrict__ b,
                                                            const u32x4* __restrict__ c, const u32x4* __restrict__ d,
                                                            u32x4* __restrict__ e, u32x4* __restrict__ f, uint64_t n) {
  const uint64_t base = (uint64_t)blockIdx.x * blockDim.x * U + threadIdx.x;
  u32x4 va[U], vb[U], vc[U], vd[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t i = base + (uint64_t)u * blockDim.x;
    if (i < n) {
      va[u] = __builtin_nontemporal_load(a + i);
      vb[u] = __builtin_nontemporal_load(b + i);
      vc[u] = __builtin_nontemporal_load(c + i);
      vd[u] = __builtin_nontemporal_load(d + i);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t i = base + (uint64_t)u * blockDim.x;
    if (i < n) {
      __builtin_nontemporal_store(va[u] + vb[u], e + i);
      __builtin_nontemporal_store(vc[u] + vd[u], f + i);
    }
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kMfmaThreads = 512;     // 8 wavefronts: two per SIMD
constexpr float kMfmaSinkKey = 1234.5f;

// Matrix-core probe: two accumulators, each MFMA with a different (A, B) pair
// from the 8 + 8 operand registers (A index r or r + 4, B index 3r + 1 or
// 5r + 2, mod 8), so the operands change at every instruction as they do in
// the prefill. A chain of 32x32x16 MFMAs on one accumulator issues at the
// full rate, so two chains keep the matrix core busy.
__global__ __launch_bounds__(kMfmaThreads) void mfma_kernel(const bf16x8* __restrict__ pool, uint32_t pool_vecs,
                                                            int iters, float* __restrict__ sink) {
  const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t base = (uint32_t)((16 * t) % pool_vecs);   // pool_vecs >= 16: one wrap at most
  bf16x8 a[8], b[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint32_t ia = base + r, ib = base + 8 + r;
    a[r] = pool[ia >= pool_vecs ? ia - pool_vecs : ia];
    b[r] = pool[ib >= pool_vecs ? ib - pool_vecs : ib];
  }
  f32x16 c0 = {}, c1 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r], b[(3 * r + 1) & 7], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(r + 4) & 7], b[(5 * r + 2) & 7], c1, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e];
  if (s == kMfmaSinkKey) sink[0] = s;
}

thread_local char g_err[256] = "";

yoco_status fail(yoco_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

yoco_status launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(YOCO_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  g_err[0] = '\0';
  return YOCO_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_threads(int t) { return t >= 64 && t <= 1024 && t % 64 == 0; }

bool overlap(const void* x, const void* y, size_t n) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
  return a < b + n && b < a + n;
}

template <int U>
void launch_read(dim3 grid, int threads, hipStream_t stream, bool nt, const u32x4* s, uint64_t n, uint64_t per_wg,
                 uint32_t* sink) {
  if (nt)
    read_kernel<true, U><<<grid, threads, 0, stream>>>(s, n, per_wg, sink);
  else
    read_kernel<false, U><<<grid, threads, 0, stream>>>(s, n, per_wg, sink);
}

template <int U>
void launch_read_blocks(dim3 grid, int threads, hipStream_t stream, const u32x4* s, uint64_t n, uint64_t per_wg,
                        uint32_t* sink) {
  read_blocks_kernel<U><<<grid, threads, 0, stream>>>(s, n, per_wg, sink);
}

}  // namespace

extern "C" {

const char* yoco_ceiling_last_error(void) { return g_err; }

yoco_status yoco_ceiling_read(const void* src, size_t bytes, int workgroups, int threads, int loads_per_thread,
                              int nontemporal, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink) return fail(YOCO_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(src)) return fail(YOCO_ERR_ALIGNMENT, "src not 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(sink) & 3u)) return fail(YOCO_ERR_ALIGNMENT, "sink not 4-byte aligned");
  if (bytes == 0 || bytes % 16) return fail(YOCO_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if (workgroups < 0 || workgroups > (1 << 20)) return fail(YOCO_ERR_INVALID_ARG, "workgroups out of range");
  if (!valid_threads(threads)) return fail(YOCO_ERR_INVALID_ARG, "threads must be 64..1024, a multiple of 64");
  const int u = loads_per_thread;
  if (u != 1 && u != 2 && u != 4 && u != 8 && u != 16)
    return fail(YOCO_ERR_INVALID_ARG, "loads_per_thread must be 1, 2, 4, 8 or 16");
  const uint64_t n = bytes / 16;
  const uint64_t per_wg = workgroups ? (n + workgroups - 1) / workgroups : 0;
  const dim3 grid(workgroups ? workgroups : kStrideWorkgroups);
  const u32x4* s = static_cast<const u32x4*>(src);
  const bool nt = nontemporal != 0;
  switch (u) {
    case 1: launch_read<1>(grid, threads, stream, nt, s, n, per_wg, sink); break;
    case 2: launch_read<2>(grid, threads, stream, nt, s, n, per_wg, sink); break;
    case 4: launch_read<4>(grid, threads, stream, nt, s, n, per_wg, sink); break;
    case 8: launch_read<8>(grid, threads, stream, nt, s, n, per_wg, sink); break;
    default: launch_read<16>(grid, threads, stream, nt, s, n, per_wg, sink); break;
  }
  return launched("ceiling read");
}

yoco_status yoco_ceiling_read_blocks(const void* src, size_t bytes, int workgroups, int threads, int loads_per_thread,
                                     uint32_t* sink, hipStream_t stream) {
  if (!src || !sink) return fail(YOCO_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(src)) return fail(YOCO_ERR_ALIGNMENT, "src not 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(sink) & 3u)) return fail(YOCO_ERR_ALIGNMENT, "sink not 4-byte aligned");
  if (bytes == 0 || bytes % 16) return fail(YOCO_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if (workgroups < 1 || workgroups > (1 << 20)) return fail(YOCO_ERR_INVALID_ARG, "workgroups out of range");
  if (!valid_threads(threads)) return fail(YOCO_ERR_INVALID_ARG, "threads must be 64..1024, a multiple of 64");
  const int u = loads_per_thread;
  if (u != 1 && u != 2 && u != 4 && u != 8 && u != 16)
    return fail(YOCO_ERR_INVALID_ARG, "loads_per_thread must be 1, 2, 4, 8 or 16");
  const uint64_t n = bytes / 16;
  const uint64_t per_wg = (n + workgroups - 1) / workgroups;
  const dim3 grid(workgroups);
  const u32x4* s = static_cast<const u32x4*>(src);
  switch (u) {
    case 1: launch_read_blocks<1>(grid, threads, stream, s, n, per_wg, sink); break;
    case 2: launch_read_blocks<2>(grid, threads, stream, s, n, per_wg, sink); break;
    case 4: launch_read_blocks<4>(grid, threads, stream, s, n, per_wg, sink); break;
    case 8: launch_read_blocks<8>(grid, threads, stream, s, n, per_wg, sink); break;
    default: launch_read_blocks<16>(grid, threads, stream, s, n, per_wg, sink); break;
  }
  return launched("ceiling read_blocks");
}

yoco_status yoco_ceiling_read4_write2(const void* a, const void* b, const void* c, const void* d, void* e, void* f,
                                      size_t bytes, int threads, int positions_per_thread, hipStream_t stream) {
  const void* ins[4] = {a, b, c, d};
  void* outs[2] = {e, f};
  for (const void* p : ins)
    if (!p) return fail(YOCO_ERR_INVALID_ARG, "null pointer");
  for (void* p : outs)
    if (!p) return fail(YOCO_ERR_INVALID_ARG, "null pointer");
  for (const void* p : ins)
    if (!aligned16(p)) return fail(YOCO_ERR_ALIGNMENT, "a source is not 16-byte aligned");
  for (void* p : outs)
    if (!aligned16(p)) return fail(YOCO_ERR_ALIGNMENT, "a destination is not 16-byte aligned");
  if (bytes == 0 || bytes % 16 || bytes >= (1ull << 35))
    return fail(YOCO_ERR_INVALID_ARG, "bytes must be a positive multiple of 16 below 2^35");
  if (!valid_threads(threads)) return fail(YOCO_ERR_INVALID_ARG, "threads must be 64..1024, a multiple of 64");
  const int u = positions_per_thread;
  if (u != 1 && u != 2 && u != 4) return fail(YOCO_ERR_INVALID_ARG, "positions_per_thread must be 1, 2 or 4");
  for (void* o : outs)
    for (const void* p : ins)
      if (overlap(o, p, bytes)) return fail(YOCO_ERR_INVALID_ARG, "a destination overlaps a source");
  if (overlap(e, f, bytes)) return fail(YOCO_ERR_INVALID_ARG, "the destinations overlap");
  const uint64_t n = bytes / 16;
  const uint64_t per_wg = (uint64_t)threads * u;
  const dim3 grid((unsigned)((n + per_wg - 1) / per_wg));
  const u32x4 *pa = static_cast<const u32x4*>(a), *pb = static_cast<const u32x4*>(b);
  const u32x4 *pc = static_cast<const u32x4*>(c), *pd = static_cast<const u32x4*>(d);
  u32x4 *pe = static_cast<u32x4*>(e), *pf = static_cast<u32x4*>(f);
  if (u == 1)
    read4_write2_kernel<1><<<grid, threads, 0, stream>>>(pa, pb, pc, pd, pe, pf, n);
  else if (u == 2)
    read4_write2_kernel<2><<<grid, threads, 0, stream>>>(pa, pb, pc, pd, pe, pf, n);
  else
    read4_write2_kernel<4><<<grid, threads, 0, stream>>>(pa, pb, pc, pd, pe, pf, n);
  return launched("ceiling read4_write2");
}

yoco_status yoco_ceiling_mfma_bf16(const void* operands, size_t operand_bytes, int workgroups, int iters,
                                   float* sink, hipStream_t stream) {
  if (!operands || !sink) return fail(YOCO_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(operands)) return fail(YOCO_ERR_ALIGNMENT, "operands not 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(sink) & 3u)) return fail(YOCO_ERR_ALIGNMENT, "sink not 4-byte aligned");
  if (operand_bytes < 256 || operand_bytes % 16 || operand_bytes / 16 > 0xFFFFFFF0ull)
    return fail(YOCO_ERR_INVALID_ARG, "operand_bytes must be a multiple of 16, at least 256 and below 2^36");
  if (workgroups < 1 || workgroups > 65536) return fail(YOCO_ERR_INVALID_ARG, "workgroups must be 1..65536");
  if (iters < 1 || iters > (1 << 24)) return fail(YOCO_ERR_INVALID_ARG, "iters must be 1..2^24");
  mfma_kernel<<<dim3(workgroups), kMfmaThreads, 0, stream>>>(static_cast<const bf16x8*>(operands),
                                                             (uint32_t)(operand_bytes / 16), iters, sink);
  return launched("ceiling mfma_bf16");
}

}  // extern "C"
