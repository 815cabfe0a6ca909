/*
 * yoco.h - C ABI of the cross-layer KV-sharing hot path (YOCO / YOCO++) on
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [YOCO++] "YOCO++: Enhancing YOCO with KV Residual Connections for
 *            Efficient LLM Inference", section 2 (methodology: the KV
 *            composition equations; reuse of the middle layer's composed KVs
 *            by every upper-half layer; key technical innovations 1-3) and
 *            section 3 (efficiency: decode reads one KV set per layer).
 *   [YOCO]   "You Only Cache Once: Decoder-Decoder Architectures for Language
 *            Models", abstract and method details (the cross-decoder reuses
 *            the global KV cache through cross-attention; the model behaves
 *            like a decoder-only Transformer; 1M-token contexts).
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers on the calling thread's current HIP
 *     device, unless stated otherwise. The caller owns every buffer (inputs,
 *     caches, outputs, workspace). The library never allocates, frees or
 *     synchronises; kernels are enqueued asynchronously on `stream` (NULL is
 *     the null stream). Functions keep no state between calls (the one
 *     exception is the per-GPU scratch array of yoco_cross_attn_decode_noalloc)
 *     and may be called from several host threads.
 *   - Every argument is checked before anything is enqueued. On error the
 *     function returns a non-zero yoco_status, enqueues nothing and records
 *     a message readable with yoco_last_error() on the same host thread.
 *     No C++ exception crosses this interface.
 *   - A 4-D tensor is described by yoco_tensor4: element strides for the
 *     batch, head and token axes; the head-dimension axis (D) is contiguous.
 *     Base pointers must be 16-byte aligned and every stride times the
 *     element size a multiple of 16 bytes (YOCO_ERR_ALIGNMENT). Strides are
 *     non-negative. A cache that attention reads row by row needs
 *     stride_t >= D; a tensor the library writes must give each of its
 *     elements an address of its own (no stride 0 over an axis longer than
 *     one, no overlapping rows); both are YOCO_ERR_INVALID_ARG otherwise.
 *     Sources that are only read (compose inputs, the one-token rows of
 *     yoco_self_attn_decode) may use any strides, including 0.
 *   - bf16 values are IEEE binary32 values truncated to their upper 16 bits;
 *     every result written as bf16 is rounded to nearest, ties to even.
 *   - Grouped-query attention: query head h reads kv head h / (Hq / Hkv).
 *   - The softmax scale defaults (scale <= 0) to 1 / sqrt(D).
 */
#ifndef YOCO_H
#define YOCO_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define YOCO_VERSION 100 /* major * 100 + minor */

typedef enum {
  YOCO_OK = 0,
  YOCO_ERR_INVALID_ARG = 1, /* a size, pointer, range or overlap is invalid          */
  YOCO_ERR_UNSUPPORTED = 2, /* valid, but this dtype / head size is not implemented  */
  YOCO_ERR_ALIGNMENT = 3,   /* a pointer or stride breaks the 16-byte rule           */
  YOCO_ERR_WORKSPACE = 4,   /* the workspace is missing or smaller than required     */
  YOCO_ERR_LAUNCH = 5       /* the HIP runtime refused the launch                    */
} yoco_status;

typedef enum { YOCO_F32 = 0, YOCO_BF16 = 1 } yoco_dtype;

typedef struct yoco_tensor4 {
  void* ptr;        /* element (b, h, t, 0) is at ptr + b*stride_b + h*stride_h + t*stride_t */
  int64_t stride_b; /* element strides                                                       */
  int64_t stride_h;
  int64_t stride_t;
  int64_t rows;     /* extent of the token axis (capacity of a cache)                        */
} yoco_tensor4;

/*
 * yoco_compose_kv - composition of one lower-half layer's cached KVs.
 *
 * [YOCO++] section 2, KV composition: for a self-decoder layer i >= 2,
 *     K'_i = lambda * (aK1 * K_1 + aK2 * K_i),   V'_i = lambda * (aV1 * V_1 + aV2 * V_i),
 * with four scalar residual weights per layer and lambda = 35 ([YOCO++]
 * key technical innovations 2). Per [YOCO++] innovation 1 the composed pair
 * is what is cached, so it is written straight into the cache.
 *
 *   k1, ki, v1, vi  sources, rows [0, n) of each are read ([B, n, Hkv, D] token-major
 *                   from a QKV projection is the usual layout; any strides work).
 *   k_cache, v_cache  destinations: rows [t0, t0 + n) are written.
 *   B, n, Hkv, D    sizes; n >= 1, D * elemsize a multiple of 16 bytes, D <= 1024.
 *   lambda, aK1..aV2  fp32 scalars. The kernel folds the scale into the weights
 *                   once per call: c1 = fl32(lambda * a1), c2 = fl32(lambda * a2)
 *                   (products formed in double), then computes fma(c2, X_i, c1 * X_1)
 *                   in fp32. With the initialisation a1 = 0, a2 = fl32(1/lambda)
 *                   ([YOCO++] innovation 3) this returns X_i bit for bit.
 *   dtype           YOCO_F32 or YOCO_BF16 (sources and caches share it).
 * Aliasing: ki / vi (or k1 / v1) may alias their destination exactly (same pointer
 * and strides, t0 = 0: in-place); any other overlap between a source and a
 * destination is YOCO_ERR_INVALID_ARG. k_cache and v_cache must not overlap
 * element-wise.
 */
yoco_status yoco_compose_kv(yoco_tensor4 k1, yoco_tensor4 ki, yoco_tensor4 v1, yoco_tensor4 vi,
                            yoco_tensor4 k_cache, yoco_tensor4 v_cache, int t0, int B, int n, int Hkv,
                            int D, float lambda, float aK1, float aK2, float aV1, float aV2,
                            yoco_dtype dtype, hipStream_t stream);

/*
 * yoco_compose_backward_workspace_size - bytes of workspace yoco_compose_kv_backward
 * needs (fp32 partial sums, four per workgroup). Host-only; 0 on bad sizes.
 */
size_t yoco_compose_backward_workspace_size(int B, int n, int Hkv, int D, yoco_dtype dtype);

/*
 * yoco_compose_kv_backward - gradients of one layer's composition.
 *
 * [YOCO++] section 2: the four residual weights are learnable; innovation 2:
 * lambda scales them. With K'_i = lambda (aK1 K_1 + aK2 K_i) and the upstream
 * gradient gk = dL/dK'_i (likewise V):
 *     dK_1 += c1 * gk,   dK_i = c2 * gk       (c = fl32(lambda * a), fp32),
 *     daK1 = lambda * <gk, K_1>,   daK2 = lambda * <gk, K_i>   (and aV1, aV2).
 *   gk, gv          upstream gradients, cache layout and dtype; rows [t0, t0+n) read.
 *   k1, ki, v1, vi  the forward sources; rows [0, n) read.
 *   dk1, dv1        fp32 gradients of layer 1's K, V, rows [0, n): ACCUMULATED (+=),
 *                   so one buffer collects the contributions of every layer i.
 *   dki, dvi        fp32 gradients of layer i's K, V, rows [0, n): written.
 *   dalpha          device fp32 [4]: (daK1, daK2, daV1, daV2), written. The dot
 *                   products are summed per workgroup in fp32 and across
 *                   workgroups in fp64 in a fixed order (deterministic).
 *   workspace       >= yoco_compose_backward_workspace_size(B, n, Hkv, D, dtype)
 *                   bytes, 16-byte aligned; contents on entry do not matter.
 *   dtype           YOCO_F32 or YOCO_BF16 (inputs); D * elemsize a multiple of 16.
 * The four gradient outputs must not overlap each other or any input
 * (YOCO_ERR_INVALID_ARG). Two kernels are enqueued on `stream`.
 */
yoco_status yoco_compose_kv_backward(yoco_tensor4 gk, yoco_tensor4 gv, int t0, yoco_tensor4 k1, yoco_tensor4 ki,
                                     yoco_tensor4 v1, yoco_tensor4 vi, yoco_tensor4 dk1, yoco_tensor4 dki,
                                     yoco_tensor4 dv1, yoco_tensor4 dvi, int B, int n, int Hkv, int D, float lambda,
                                     float aK1, float aK2, float aV1, float aV2, float* dalpha, void* workspace,
                                     size_t workspace_bytes, yoco_dtype dtype, hipStream_t stream);

/*
 * yoco_decode_num_splits - the split count the decode picks when given 0.
 * Host-only; returns >= 1, or 0 if a size is not positive.
 */
int yoco_decode_num_splits(int B, int T, int Hq, int Hkv, int D);

/*
 * yoco_decode_workspace_size - bytes of workspace the decode needs.
 * num_splits = 0 means the automatic choice. The workspace holds one 32-bit
 * counter per (b, kv head) [B, Hkv] first, then the per-split partial outputs
 * [B, Hq, S, D] fp32 and their log-sum-exps [B, Hq, S] fp32, each section
 * starting on a 16-byte boundary. The counters lead so that their place
 * depends on B * Hkv only, not on T or the split count.
 * Host-only; returns 0 if a size is not positive or no workspace is needed.
 */
size_t yoco_decode_workspace_size(int B, int T, int Hq, int Hkv, int D, int num_splits);

/*
 * yoco_cross_attn_decode - one cross-decoder layer's decode attention over the
 * shared cache.
 *
 * [YOCO] method details / abstract: every cross-decoder layer reuses the one
 * global KV cache through cross-attention; [YOCO++] section 2: that cache is
 * the middle layer's composed K'_{L/2}, V'_{L/2}; section 3: decoding reads
 * exactly one KV set per layer. For query head h of sequence b, over cache
 * rows t in [0, T_b):
 *     s_t = scale * <q[b,h,:], K'[b,g,t,:]>,  o = sum_t softmax(s)_t V'[b,g,t,:],
 *     lse = ln sum_t exp(s_t),                g = h / (Hq / Hkv).
 * The key axis is cut into S contiguous splits that run in parallel; each
 * keeps a running (max, sum, weighted value) state and the splits are merged
 * with their log-sum-exps (an exact regrouping of the same sums). The merge is
 * fused into the same launch: the last workgroup of each (b, kv head) to
 * finish, found with an atomic counter in the workspace, merges the splits.
 *
 *   q          [B, Hq, D] contiguous, dtype kv_dtype.
 *   k_cache, v_cache  rows [0, T) are read.
 *   seq_lens   device int32 [B] or NULL (all T). Values are clamped to [1, T] on
 *              the device (they are not read on the host).
 *   scale      softmax scale; <= 0 selects 1 / sqrt(D).
 *   out        [B, Hq, D] fp32, written.   lse  [B, Hq] fp32 natural log, or NULL.
 *   workspace  device buffer of at least yoco_decode_workspace_size(...) bytes,
 *              16-byte aligned; ignored (may be NULL) when the effective split
 *              count is 1. Its counter section (the first 4 * B * Hkv bytes)
 *              must be zero when a call starts. Zero-fill a new workspace once:
 *              every completed call leaves its own counter section zero again,
 *              whatever T and the split count are, but the bytes after it hold
 *              that call's partials. So a workspace reused for a call with a
 *              larger B * Hkv than the call before needs bytes
 *              [4 * B_prev * Hkv_prev, 4 * B * Hkv) zeroed first (or keep one
 *              workspace per B * Hkv). One workspace serves one call at a time:
 *              calls that share a workspace must be ordered (same stream, or
 *              synchronised).
 *   num_splits 0 = automatic; otherwise the split count S >= 1.
 *   kv_dtype   YOCO_F32 or YOCO_BF16; D in {64, 128}; Hq a multiple of Hkv,
 *              Hq / Hkv in {1, 2, 4, 8, 16}.
 * The rows of one (sequence, kv head) are addressed with 32-bit offsets:
 * (T + 64) * stride_t * element size must stay below 2 GiB for each cache
 * (YOCO_ERR_UNSUPPORTED otherwise; a head-major 1M-token bf16 D = 128 cache
 * spans 256 MiB).
 */
yoco_status yoco_cross_attn_decode(const void* q, yoco_tensor4 k_cache, yoco_tensor4 v_cache,
                                   const int32_t* seq_lens, int B, int T, int Hq, int Hkv, int D,
                                   float scale, float* out, float* lse, void* workspace,
                                   size_t workspace_bytes, int num_splits, yoco_dtype kv_dtype,
                                   hipStream_t stream);

/*
 * yoco_cross_attn_decode_noalloc - yoco_cross_attn_decode with no workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The split partials and the merge counters live in a scratch array inside
 * the library: YOCO_NOALLOC_SCRATCH_BYTES bytes of device memory per GPU that
 * runs it, held until the process ends; the first YOCO_NOALLOC_COUNTER_BYTES
 * hold the counters (so B * Hkv <= YOCO_NOALLOC_COUNTER_BYTES / 4), the rest
 * the partials, 4 * B * Hq * S * (D + 1) bytes (16-byte aligned sections). A
 * call that needs more returns YOCO_ERR_WORKSPACE and enqueues nothing; a call
 * whose effective split count is 1 uses no scratch. Nothing is allocated or
 * freed. The first call on a device looks up the array's address and clears
 * its counters with a kernel on `stream`: make that call outside graph capture.
 * Every call on one GPU shares that GPU's array, and every completed call
 * leaves the counters at zero: calls that overlap on one GPU (other streams,
 * other host threads) race and must be ordered by the caller.
 * Arguments, results and the other errors as for yoco_cross_attn_decode.
 */
#define YOCO_NOALLOC_SCRATCH_BYTES (8u << 20)
#define YOCO_NOALLOC_COUNTER_BYTES (64u << 10)
yoco_status yoco_cross_attn_decode_noalloc(const void* q, yoco_tensor4 k_cache, yoco_tensor4 v_cache,
                                           const int32_t* seq_lens, int B, int T, int Hq, int Hkv, int D,
                                           float scale, float* out, float* lse, int num_splits,
                                           yoco_dtype kv_dtype, hipStream_t stream);

/*
 * yoco_cross_attn_decode_compose_on_read - the same decode when the cache holds
 * the raw K_i, V_i and K_1, V_1 instead of the composed pair.
 *
 * The comparator for [YOCO++] key technical innovation 1 and section 3: a
 * design that combines layers at read time (as FusedKV does, [YOCO++] section
 * 1) must fetch two KV sets per decode step, while YOCO++ caches the composed
 * pair and fetches one. Each row is composed on read with exactly the
 * arithmetic of yoco_compose_kv (fl32-folded weights, one fma, one rounding),
 * so the result equals yoco_compose_kv followed by yoco_cross_attn_decode bit
 * for bit, at twice the cache traffic.
 *
 *   k1_cache, v1_cache  layer 1's K_1, V_1 (rows [0, T) read).
 *   ki_cache, vi_cache  layer i's raw K_i, V_i (rows [0, T) read).
 *   lambda, aK1..aV2    as for yoco_compose_kv.
 * Other arguments, the workspace rules and the errors as for
 * yoco_cross_attn_decode.
 */
yoco_status yoco_cross_attn_decode_compose_on_read(const void* q, yoco_tensor4 k1_cache, yoco_tensor4 ki_cache,
                                                   yoco_tensor4 v1_cache, yoco_tensor4 vi_cache,
                                                   const int32_t* seq_lens, int B, int T, int Hq, int Hkv, int D,
                                                   float lambda, float aK1, float aK2, float aV1, float aV2,
                                                   float scale, float* out, float* lse, void* workspace,
                                                   size_t workspace_bytes, int num_splits, yoco_dtype kv_dtype,
                                                   hipStream_t stream);

/*
 * yoco_self_attn_decode - one decode step of a lower-half (self-decoder) layer i:
 * compose the new token's K'_i, V'_i, append them to the layer's own cache and
 * attend over the whole sequence.
 *
 * [YOCO++] section 2 (KV composition; the composed pair is what layer i caches)
 * and section 3 (the lower half keeps L/2 caches, one per layer). For each
 * sequence b with n = seq_lens[b] (T when seq_lens is NULL; clamped to [1, T]):
 *     K'_new = fl(c_K1 K_1,new + c_K2 K_i,new),  V'_new likewise
 * (fl32-folded weights and one rounding, bit for bit yoco_compose_kv), written
 * into k_cache, v_cache at row n - 1; then the query attends over cache rows
 * [0, n - 1) and the new row, as yoco_cross_attn_decode does over n rows.
 * The cache's old contents at row n - 1 are never read.
 *
 *   k1_new, ki_new, v1_new, vi_new
 *              the new token's K_1, K_i, V_1, V_i, element (b, g, :) read at
 *              row n - 1 of each view. A buffer holding only the new token
 *              ([B, Hkv, D] or [B, 1, Hkv, D]) is passed with stride_t = 0 and
 *              rows >= 1; otherwise rows >= T. K_1's row is usually layer 1's
 *              own cache, which holds K_1 unchanged. A source may be the very
 *              same view as its destination cache (in-place compose of a row
 *              already written there raw); any other overlap with either
 *              cache is YOCO_ERR_INVALID_ARG.
 *   k_cache, v_cache  layer i's composed caches: rows [0, n - 1) read, row
 *              n - 1 written.
 *   lambda, aK1..aV2  as for yoco_compose_kv.
 * Other arguments, the workspace rules and the errors as for
 * yoco_cross_attn_decode. Launches on stream; the written rows are visible to
 * later work on that stream.
 */
yoco_status yoco_self_attn_decode(const void* q, yoco_tensor4 k1_new, yoco_tensor4 ki_new, yoco_tensor4 v1_new,
                                  yoco_tensor4 vi_new, yoco_tensor4 k_cache, yoco_tensor4 v_cache,
                                  const int32_t* seq_lens, int B, int T, int Hq, int Hkv, int D, float lambda,
                                  float aK1, float aK2, float aV1, float aV2, float scale, float* out, float* lse,
                                  void* workspace, size_t workspace_bytes, int num_splits, yoco_dtype kv_dtype,
                                  hipStream_t stream);

/*
 * yoco_cross_attn_decode_partial - the split pass of yoco_cross_attn_decode alone.
 * Writes, for every (b, h, split), the split's normalised output and its
 * log-sum-exp into the workspace (an empty split gets o = 0, lse = -inf); the
 * counter section is neither read nor written. Arguments as for
 * yoco_cross_attn_decode; num_splits must be >= 2 here.
 */
yoco_status yoco_cross_attn_decode_partial(const void* q, yoco_tensor4 k_cache, yoco_tensor4 v_cache,
                                           const int32_t* seq_lens, int B, int T, int Hq, int Hkv,
                                           int D, float scale, void* workspace, size_t workspace_bytes,
                                           int num_splits, yoco_dtype kv_dtype, hipStream_t stream);

/*
 * yoco_decode_merge - the log-sum-exp merge of S split partials.
 * For each (b, h): M = max_s lse_s, w_s = exp(lse_s - M),
 *     o = sum_s w_s o_s / sum_s w_s,  lse = M + ln sum_s w_s.
 *   workspace  the partials written by yoco_cross_attn_decode_partial with the
 *              same B, Hq, Hkv, D and num_splits (the workspace layout above).
 *   out        [B, Hq, D] fp32.   lse  [B, Hq] fp32 or NULL.
 */
yoco_status yoco_decode_merge(const void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int D,
                              int num_splits, float* out, float* lse, hipStream_t stream);

/*
 * yoco_cross_attn_prefill - causal chunked prefill of a cross-decoder layer
 * over the global cache.
 *
 * [YOCO] abstract: end to end the model works as a decoder-only Transformer
 * does, so the query at absolute position p attends to cache rows [0, p]
 * (inclusive: its own composed KV is already in the cache); [YOCO++] section
 * 3: prefill is compute-bound. A chunk holds C query rows at positions [p0, p0 + C).
 * QK^T and PV run on bf16 MFMA with fp32 accumulation; the softmax is fp32,
 * the probabilities are rounded to bf16 for the PV product and the normaliser
 * sums those rounded values.
 *
 *   q          [B, C, Hq, D] contiguous bf16.
 *   k_cache, v_cache  bf16; rows [0, p0 + C) are read; p0 + C <= rows.
 *   out        [B, C, Hq, D] contiguous, out_dtype YOCO_F32 or YOCO_BF16.
 *   lse        [B, Hq, C] fp32 natural log, or NULL.
 *   dtype      must be YOCO_BF16; D in {64, 128}; Hq / Hkv in {1, 2, 4, 8, 16}.
 */
yoco_status yoco_cross_attn_prefill(const void* q, yoco_tensor4 k_cache, yoco_tensor4 v_cache, int B,
                                    int C, int p0, int Hq, int Hkv, int D, float scale, void* out,
                                    yoco_dtype out_dtype, float* lse, yoco_dtype dtype,
                                    hipStream_t stream);

/* Static text for a status code. */
const char* yoco_status_string(yoco_status s);
/* Message of the last failing call on this host thread ("" if none). */
const char* yoco_last_error(void);
/* YOCO_VERSION of the built library. */
int yoco_version(void);

#ifdef __cplusplus
}
#endif

#endif /* YOCO_H */
