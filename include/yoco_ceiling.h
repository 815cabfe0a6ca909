/*
 * yoco_ceiling.h - achievable-rate probes of MI355X (gfx950), the yardsticks
 * the kernels of libyoco.so are measured against: bandwidth for the HBM-bound
 * ones, matrix-core throughput for the prefill.
 *
 * The YOCO++ technical summary, section 3 (efficiency analysis), states the
 * method's cost in memory traffic: decoding reads exactly one KV set per layer,
 * and the composition adds only I/O. How close a kernel comes to those bytes'
 * time is read against two peaks: the published 8 TB/s of HBM3E, and what a
 * plain kernel with the same traffic pattern and no arithmetic achieves on
 * the same chip. These probes are that plain kernel. They carry none of the
 * method's arithmetic and are built into a library of their own,
 * libyoco_ceiling.so.
 *
 * Conventions are those of yoco.h: device pointers on the current HIP device,
 * caller-owned buffers, asynchronous launches on `stream`, no allocation, every
 * argument checked before anything is enqueued (a yoco_status is returned and
 * the message is readable with yoco_ceiling_last_error() on the same thread).
 */
#ifndef YOCO_CEILING_H
#define YOCO_CEILING_H

#include <stddef.h>
#include <stdint.h>

#include "yoco.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * yoco_ceiling_read - stream `bytes` bytes from `src` once, as the decode
 * streams its cache: 16-byte loads, several in flight per thread.
 *   src          16-byte aligned; bytes a positive multiple of 16.
 *   workgroups   > 0: workgroup w reads the w-th of `workgroups` contiguous,
 *                equal ranges (the decode's split layout); 0: every thread
 *                strides over the whole buffer (grid of 2048 workgroups).
 *   threads      threads per workgroup: 64, 128, ..., 1024.
 *   loads_per_thread  1, 2, 4, 8 or 16: the 16-byte loads of a thread issued
 *                together before their data is used (consecutive thread
 *                strides of the workgroup's range).
 *   nontemporal  1: nontemporal loads (the decode's policy); 0: ordinary loads
 *                (these allocate in the caches: a read of a buffer larger than
 *                the 256 MB Infinity Cache evicts what it held).
 *   sink         device uint32 [1]: written only if the XOR of all loaded
 *                words equals a fixed 32-bit constant (keeps the loads live).
 */
yoco_status yoco_ceiling_read(const void* src, size_t bytes, int workgroups, int threads, int loads_per_thread,
                              int nontemporal, uint32_t* sink, hipStream_t stream);

/*
 * yoco_ceiling_read_blocks - the same single read with the decode's per-
 * wavefront access: workgroup w reads the w-th of `workgroups` contiguous,
 * equal ranges, dealt to its wavefronts in blocks of loads_per_thread KiB;
 * the loads of one block (each a contiguous 1 KiB: 64 lanes x 16 bytes) are
 * in flight together. Nontemporal loads.
 *   workgroups   >= 1; threads and loads_per_thread as for yoco_ceiling_read.
 */
yoco_status yoco_ceiling_read_blocks(const void* src, size_t bytes, int workgroups, int threads, int loads_per_thread,
                                     uint32_t* sink, hipStream_t stream);

/*
 * yoco_ceiling_read4_write2 - the compose kernel's traffic with no arithmetic:
 * e = a + b and f = c + d as 32-bit integers over `bytes` bytes per stream,
 * 16-byte vectors, nontemporal loads and stores.
 *   a, b, c, d   sources; e, f destinations (must not overlap the sources).
 *   bytes        bytes per stream, a positive multiple of 16, below 2^35.
 *   threads      threads per workgroup: 64, 128, ..., 1024.
 *   positions_per_thread  1, 2 or 4 vectors of each stream per thread, a
 *                workgroup's width apart; all loads before the stores.
 */
yoco_status yoco_ceiling_read4_write2(const void* a, const void* b, const void* c, const void* d, void* e, void* f,
                                      size_t bytes, int threads, int positions_per_thread, hipStream_t stream);

/*
 * yoco_ceiling_mfma_bf16 - the matrix cores' achievable rate on given operand
 * data, the yardstick of the MFMA-bound prefill (the YOCO++ technical summary,
 * section 3, calls prefill compute-bound). Every wavefront of `workgroups`
 * workgroups of 8 wavefronts (two per SIMD, as the prefill runs) issues
 * 16 * iters v_mfma_f32_32x32x16_bf16 (32,768 flop each) back to back on two
 * fp32 accumulators, taking its operands from 8 A and 8 B registers per lane
 * in a rotation that gives every MFMA a different operand pair; the matrix
 * core's power, and with it the rate the chip sustains, depends on those
 * values, so the caller supplies them.
 *   operands        device bf16 pool, 16-byte aligned, a multiple of 16
 *                   bytes, at least 256; lane t of the grid loads its 16
 *                   registers from 16-byte vectors (16 t + r) mod
 *                   (operand_bytes / 16), r = 0 .. 15.
 *   workgroups      1 .. 65536 (256 fills each CU of an MI355X once).
 *   iters           1 .. 2^24.
 *   sink            device float [1]: written only if the accumulators sum to
 *                   a fixed value (keeps the products live).
 * Work per call: workgroups * 8 * iters * 16 * 32768 flop.
 */
yoco_status yoco_ceiling_mfma_bf16(const void* operands, size_t operand_bytes, int workgroups, int iters,
                                   float* sink, hipStream_t stream);

/* Message of the last failing call on this host thread ("" if none). */
const char* yoco_ceiling_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* YOCO_CEILING_H */
