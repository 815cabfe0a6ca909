// LDS layout and per-lane addresses of the software-pipelined D = 128 causal
// prefill (prefill_pipe_kernel). Kept apart from the kernel, and usable on the
// host, so that a host build can check every address the kernel forms: the
// bounds of the 150 KiB LDS array, that the direct loads fill each tile
// exactly once, that each MFMA operand read finds the key rows and dims its
// lane must supply, and which reads touch every LDS bank once.
//
// Products (YOCO summary, abstract: the cross-decoder attends causally to the
// one global cache): S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16.
// Lane l of such an MFMA supplies A[m = l % 32][k = 8 (l / 32) .. + 8] and
// B[k = 8 (l / 32) .. + 8][n = l % 32].
//
// One step covers 64 keys. K and V tiles sit in three slots each of 64
// unpadded 256-byte rows (128 bf16 dims); chunk c (16 bytes, dims 8c .. 8c+7)
// of row r is stored at position c ^ (r % 16) in K and c ^ 4 (r % 4) in V. The
// workgroup transposes each V tile once into a V^T slot: 128 rows (dims) of
// 64 keys, 144 bytes apart.

#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace yoco {
namespace pipe {

constexpr int kD = 128;
constexpr int kWaves = 8;                 // wavefronts per workgroup
constexpr int kSK = 64;                   // keys per step
constexpr int kNS = 3;                    // LDS slots per tensor
constexpr int kRowB = kD * 2;             // bytes per stored K or V row
constexpr int kSlotB = kSK * kRowB;       // 16 KiB
constexpr int kVBase = kNS * kSlotB;      // V slots follow the K slots
constexpr int kVTRow = kSK * 2 + 16;      // bytes per V^T row (64 keys + pad)
constexpr int kVTSlotB = kD * kVTRow;     // 18 KiB
constexpr int kVTBase = 2 * kNS * kSlotB;
constexpr int kLdsBytes = kVTBase + kNS * kVTSlotB;   // 150 KiB
constexpr int kLoads = kSK / 4 / kWaves;  // direct loads (4 rows each) per wavefront, tensor and step

// Row i of each 32-key block is fed to the score MFMA as row perm_key(i):
// index bits 2 and 3 swapped, so that the 8 probabilities a lane holds for one
// PV k-step are 8 consecutive keys.
__host__ __device__ constexpr int perm_key(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// Direct loads: load i of wavefront w brings tile rows 8w + 4i .. + 4, lane l
// writing the 16 bytes at position l % 16 of row 8w + 4i + l / 16 (LDS
// destination slot + (8w + 4i) * kRowB + 16 l). The lane fetches the global
// chunk that belongs at that position.
__host__ __device__ constexpr int load_row(int wave, int i, int lane) { return 8 * wave + 4 * i + (lane >> 4); }
__host__ __device__ constexpr int load_lds_offset(int wave, int i) { return (8 * wave + 4 * i) * kRowB; }
__host__ __device__ constexpr int k_load_chunk(int row, int pos) { return pos ^ (row & 15); }
__host__ __device__ constexpr int v_load_chunk(int row, int pos) { return pos ^ (4 * (row & 3)); }

// K operand of score k-step c (dims 16c .. 16c+15) for the 32-key block at
// row 0 of a K slot: lane (j = l % 32, q = l / 32) reads chunk 2c + q of key
// row perm_key(j). Add the slot's byte offset and 32 * kRowB per later block.
__host__ __device__ constexpr uint32_t k_operand(int lane, int c) {
  const int j = lane & 31, q = lane >> 5, pk = perm_key(j);
  return (uint32_t)(pk * kRowB + 16 * (q ^ (pk & 15))) ^ (32u * c);
}

// Transposing V reads (ds_read_b64_tr_b16: within each 16-lane group the lanes
// address 4 rows of 16 dims, 4 lanes per row, and lane i receives dim i of the
// 4 rows). Wavefront w covers keys kb_w .. + 4 and kb_w + 8 .. + 4
// (kb_w = 16 (w / 2) + 4 (w % 2)) of all 128 dims, one read per 32-dim block
// db; lane (gq = l / 16, i) receives dim 32 db + 16 (gq % 2) + i of keys
// kb_w + 8 (gq / 2) .. + 4. Byte address within V slot 0.
__host__ __device__ constexpr int tr_first_key(int wave, int lane) {
  return 16 * (wave >> 1) + 4 * (wave & 1) + 8 * ((lane >> 4) >> 1);
}
__host__ __device__ constexpr int tr_dim(int lane, int db) { return 32 * db + 16 * ((lane >> 4) & 1) + (lane & 15); }
__host__ __device__ constexpr uint32_t tr_read(int wave, int lane, int db) {
  const int gq = lane >> 4, sl16 = lane & 15, r4 = sl16 >> 2;
  const int kb_w = 16 * (wave >> 1) + 4 * (wave & 1);
  return (uint32_t)(kVBase + (kb_w + 8 * (gq >> 1) + r4) * kRowB + 64 * r4 + 32 * (gq & 1) + 16 * ((sl16 >> 1) & 1) +
                    8 * (sl16 & 1)) ^
         (64u * db);
}
// Where those 4 keys of that dim land in V^T slot 0 (8 bytes).
__host__ __device__ constexpr uint32_t vt_write(int wave, int lane, int db) {
  return (uint32_t)(kVTBase + tr_dim(lane, db) * kVTRow + 2 * tr_first_key(wave, lane));
}

// PV operand of 16-key k-step hs of 32-key block hb, dims 32 db .. + 32: lane
// (j, q) reads V^T row 32 db + j, keys 32 hb + 16 hs + 8 q .. + 8 (16 bytes).
// Byte address within V^T slot 0.
__host__ __device__ constexpr uint32_t pv_operand(int lane, int hb, int hs, int db) {
  const int j = lane & 31, q = lane >> 5;
  return (uint32_t)(kVTBase + j * kVTRow + 16 * q + db * 32 * kVTRow + (32 * hb + 16 * hs) * 2);
}

static_assert(kLdsBytes == 150 * 1024, "the pipelined prefill holds 150 KiB of LDS");
static_assert(kLoads * 4 * kWaves == kSK, "the direct loads cover a tile");

}  // namespace pipe
}  // namespace yoco
