// Per-wavefront LDS buffers of the matrix-core decode (decode_mfma_kernel):
// sizes and per-lane addresses, in bf16 elements from the start of the
// wavefront's buffer. Kept apart from the kernel, and usable on the host, so
// that a host build can check every address: that the block loads fill each
// buffer exactly once, that each MFMA operand read finds the cache row and
// dims its lane supplies, and that the reads and writes the kernel issues
// touch distinct LDS banks within each group of lanes served together.
//
// A wavefront streams blocks of 32 cache rows. Its loads bring whole rows:
// load instruction i carries rows RPI i .. + RPI, lane l holding the 16 bytes
// (8 dims) at chunk l % LPR of row RPI i + l / LPR. K rows are stored unpadded
// with chunk c of row r at position c ^ k_swizzle(r); V rows are stored with a
// padded stride of D + 32 elements. The score MFMA (v_mfma_f32_16x16x32_bf16,
// lane (lg = l / 16, lr = l % 16) supplying A[lr][8 lg .. + 8]) takes block bb's
// row lr from cache row 8 (lr / 4) + 4 bb + lr % 4, dims 32 j + 8 lg for k-step j;
// the value MFMA's A operand (V^T) is read with the transposing LDS read, lane
// (lg, r) receiving dim 16 n + r of rows 8 lg .. 8 lg + 7 in two reads.

#pragma once

#include <hip/hip_runtime.h>

namespace yoco {
namespace dlay {

constexpr int kBlock = 32;   // cache rows per block

template <int D>
struct Shape {
  static constexpr int LPR = D / 8;             // lanes per cache row in a block load
  static constexpr int RPI = 64 / LPR;          // cache rows per load instruction
  static constexpr int NLI = kBlock / RPI;      // load instructions per block and tensor
  static constexpr int NQK = D / 32;            // k-steps of the score product
  static constexpr int NDB = D / 16;            // 16-dim blocks of O^T
  static constexpr int VPAD = D + 32;           // V row stride (elements)
  static constexpr int kVElems = kBlock * VPAD; // one wavefront's V buffer
  static constexpr int kKElems = kBlock * D;    // one wavefront's K buffer
};

// Chunk c of K row r (r < 32) sits at position c ^ k_swizzle(r): the 16 rows a
// score operand read serves then land in distinct banks (distinct chunk
// positions of a 256-byte row at D = 128; distinct (row parity, chunk) pairs
// at D = 64), and so do the 16 lanes of a row-contiguous write.
template <int D>
__host__ __device__ constexpr int k_swizzle(int r) {
  return D == 128 ? ((r & 3) | ((r >> 1) & 12)) : (((r >> 1) & 1) | ((r >> 2) & 6));
}

// Block load i, lane l: the cache row (within the block) and the chunk it carries.
template <int D>
__host__ __device__ constexpr int load_row(int i, int lane) {
  return Shape<D>::RPI * i + lane / Shape<D>::LPR;
}
template <int D>
__host__ __device__ constexpr int load_chunk(int lane) {
  return lane % Shape<D>::LPR;
}

// Where load i's 16 bytes go in the K and V buffers.
template <int D>
__host__ __device__ constexpr int k_write(int i, int lane) {
  return load_row<D>(i, lane) * D + 8 * (load_chunk<D>(lane) ^ k_swizzle<D>(load_row<D>(i, lane)));
}
template <int D>
__host__ __device__ constexpr int v_write(int i, int lane) {
  return load_row<D>(i, lane) * Shape<D>::VPAD + 8 * load_chunk<D>(lane);
}

// Score operand of block bb, k-step j: row and 16-byte read.
template <int D>
__host__ __device__ constexpr int k_row(int lane, int bb) {
  return 8 * ((lane & 15) >> 2) + 4 * bb + (lane & 3);
}
template <int D>
__host__ __device__ constexpr int k_read(int lane, int bb, int j) {
  return k_row<D>(lane, bb) * D + 8 * ((4 * j + (lane >> 4)) ^ k_swizzle<D>(k_row<D>(lane, bb)));
}

// Transposing read h (rows 8 lg + 4 h .. + 4) of dim block n: the 8 bytes lane
// (lg, r) addresses, row 8 lg + 4 h + r / 4, dims 16 n + 4 (r % 4) .. + 4.
template <int D>
__host__ __device__ constexpr int v_tr_read(int lane, int n, int h) {
  return (8 * (lane >> 4) + 4 * h + ((lane & 15) >> 2)) * Shape<D>::VPAD + 4 * (lane & 3) + 16 * n;
}

}  // namespace dlay
}  // namespace yoco
