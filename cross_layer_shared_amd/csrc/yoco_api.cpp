// C ABI of the cross-layer KV-sharing hot path: argument checks, launch
// configuration and status codes. Nothing here allocates, frees or
// synchronises; every check runs before anything is enqueued.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "../../include/yoco.h"
#include "common.h"

namespace {

thread_local char g_err[512] = "";

yoco_status fail(yoco_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

yoco_status ok() {
  g_err[0] = '\0';
  return YOCO_OK;
}

size_t esize(yoco_dtype dt) { return dt == YOCO_BF16 ? 2 : 4; }

bool valid_dtype(yoco_dtype dt) { return dt == YOCO_F32 || dt == YOCO_BF16; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte span [lo, hi) touched by rows [r0, r1) of a tensor with H heads, B batches.
struct Span {
  uintptr_t lo, hi;
};

Span span_of(const yoco_tensor4& t, int B, int H, int64_t r0, int64_t r1, int D, size_t es) {
  // Strides are non-negative (checked), so the extremes are the first and last elements.
  int64_t first = r0 * t.stride_t;
  int64_t last = (int64_t)(B - 1) * t.stride_b + (int64_t)(H - 1) * t.stride_h + (r1 - 1) * t.stride_t + D;
  uintptr_t base = reinterpret_cast<uintptr_t>(t.ptr);
  return {base + (uintptr_t)(first * (int64_t)es), base + (uintptr_t)(last * (int64_t)es)};
}

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

yoco_status check_tensor(const char* name, const yoco_tensor4& t, int64_t rows_needed, size_t es) {
  if (!t.ptr) return fail(YOCO_ERR_INVALID_ARG, "%s: null pointer", name);
  if (t.stride_b < 0 || t.stride_h < 0 || t.stride_t < 0)
    return fail(YOCO_ERR_INVALID_ARG, "%s: negative stride", name);
  if (t.rows < rows_needed)
    return fail(YOCO_ERR_INVALID_ARG, "%s: %lld rows, %lld needed", name, (long long)t.rows,
                (long long)rows_needed);
  if (!aligned16(t.ptr)) return fail(YOCO_ERR_ALIGNMENT, "%s: base pointer not 16-byte aligned", name);
  if ((t.stride_b * (int64_t)es) % 16 || (t.stride_h * (int64_t)es) % 16 || (t.stride_t * (int64_t)es) % 16)
    return fail(YOCO_ERR_ALIGNMENT, "%s: a stride is not a multiple of 16 bytes", name);
  return YOCO_OK;
}

// Rows of one (sequence, head) must not overlap: a cache read row by row, or a
// tensor written row by row, needs stride_t >= D (a stride of 0 would make
// every row the same memory).
yoco_status check_row_stride(const char* name, const yoco_tensor4& t, int D) {
  if (t.stride_t < D)
    return fail(YOCO_ERR_INVALID_ARG, "%s: stride_t = %lld is below D = %d (rows overlap)", name,
                (long long)t.stride_t, D);
  return YOCO_OK;
}

// A tensor the kernels write must give every element (b, h, t, d) of its B x H x
// rows x D extent an address of its own: sorted by stride, each axis of extent
// above one must step past the whole span of the axes below it.
yoco_status check_distinct(const char* name, const yoco_tensor4& t, int B, int H, int64_t rows, int D) {
  struct Axis {
    int64_t stride, extent;
  } ax[4] = {{1, D}, {t.stride_t, rows}, {t.stride_h, H}, {t.stride_b, B}};
  std::sort(ax, ax + 4, [](const Axis& a, const Axis& b) { return a.stride < b.stride; });
  int64_t span = 0;   // elements spanned by the axes taken so far, minus one
  for (const Axis& a : ax) {
    if (a.extent <= 1) continue;
    if (a.stride <= span)
      return fail(YOCO_ERR_INVALID_ARG, "%s: strides map two elements to one address", name);
    span += a.stride * (a.extent - 1);
  }
  return YOCO_OK;
}

// The decode kernels address one (sequence, head)'s rows with 32-bit byte
// offsets: rows [0, T) plus one block of overrun must span less than 2 GiB.
yoco_status check_head_span(const char* name, const yoco_tensor4& t, int64_t T, size_t es) {
  if ((T + 64) * t.stride_t * (int64_t)es >= (int64_t)1 << 31)
    return fail(YOCO_ERR_UNSUPPORTED, "%s: the rows of one (sequence, head) span 2 GiB or more", name);
  return YOCO_OK;
}

yoco::View4 view(const yoco_tensor4& t) { return {t.ptr, t.stride_b, t.stride_h, t.stride_t}; }

yoco_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(YOCO_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

float fold(float lambda, float a) { return (float)((double)lambda * (double)a); }

bool supported_group(int G) { return G == 1 || G == 2 || G == 4 || G == 8 || G == 16; }

constexpr int kDecodeRowQuantum = 16;    // split lengths are multiples of this
constexpr int kDecodeTargetWaves = 2048;  // wavefronts per decode launch the heuristic aims for
constexpr int kDecodeMinRowsPerWave = 64; // shortest automatic share of a wavefront
constexpr int kDecodeShortSplit = 512;    // splits this short or shorter run as "short"

int round_up(int64_t x, int64_t q) { return (int)(((x + q - 1) / q) * q); }

int decode_rows_per_split(int T, int S) { return round_up((T + (int64_t)S - 1) / S, kDecodeRowQuantum); }

yoco_status check_decode(const void* q, const yoco_tensor4& k, const yoco_tensor4& v, int B, int T, int Hq, int Hkv,
                         int D, yoco_dtype dt) {
  if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0)
    return fail(YOCO_ERR_INVALID_ARG, "sizes must be positive (B=%d T=%d Hq=%d Hkv=%d D=%d)", B, T, Hq, Hkv, D);
  if (Hq % Hkv) return fail(YOCO_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (!valid_dtype(dt)) return fail(YOCO_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (D != 64 && D != 128) return fail(YOCO_ERR_UNSUPPORTED, "decode supports D in {64, 128}, got %d", D);
  if (!supported_group(Hq / Hkv))
    return fail(YOCO_ERR_UNSUPPORTED, "decode supports Hq/Hkv in {1,2,4,8,16}, got %d", Hq / Hkv);
  if (!q) return fail(YOCO_ERR_INVALID_ARG, "q: null pointer");
  if (!aligned16(q)) return fail(YOCO_ERR_ALIGNMENT, "q: not 16-byte aligned");
  size_t es = esize(dt);
  yoco_status st;
  if ((st = check_tensor("k_cache", k, T, es)) != YOCO_OK) return st;
  if ((st = check_tensor("v_cache", v, T, es)) != YOCO_OK) return st;
  if ((st = check_row_stride("k_cache", k, D)) != YOCO_OK) return st;
  if ((st = check_row_stride("v_cache", v, D)) != YOCO_OK) return st;
  if ((st = check_head_span("k_cache", k, T, es)) != YOCO_OK) return st;
  if ((st = check_head_span("v_cache", v, T, es)) != YOCO_OK) return st;
  return YOCO_OK;
}

// Layout of the allocation-free decode's scratch array (decode_noalloc.hip):
// the merge counters in a fixed leading section, so that they never share
// bytes with the partials of a call with a different shape, then the partials.
constexpr size_t kScratchBytes = YOCO_NOALLOC_SCRATCH_BYTES;
constexpr size_t kScratchCounterBytes = YOCO_NOALLOC_COUNTER_BYTES;

}  // namespace

extern "C" {

const char* yoco_status_string(yoco_status s) {
  switch (s) {
    case YOCO_OK: return "ok";
    case YOCO_ERR_INVALID_ARG: return "invalid argument";
    case YOCO_ERR_UNSUPPORTED: return "unsupported";
    case YOCO_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case YOCO_ERR_WORKSPACE: return "workspace missing or too small";
    case YOCO_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* yoco_last_error(void) { return g_err; }

int yoco_version(void) { return YOCO_VERSION; }

yoco_status yoco_compose_kv(yoco_tensor4 k1, yoco_tensor4 ki, yoco_tensor4 v1, yoco_tensor4 vi, yoco_tensor4 k_cache,
                            yoco_tensor4 v_cache, int t0, int B, int n, int Hkv, int D, float lambda, float aK1,
                            float aK2, float aV1, float aV2, yoco_dtype dtype, hipStream_t stream) {
  if (B <= 0 || n <= 0 || Hkv <= 0 || D <= 0 || t0 < 0)
    return fail(YOCO_ERR_INVALID_ARG, "sizes must be positive and t0 >= 0 (B=%d n=%d Hkv=%d D=%d t0=%d)", B, n, Hkv,
                D, t0);
  if (!valid_dtype(dtype)) return fail(YOCO_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  const size_t es = esize(dtype);
  if ((D * es) % 16 || D > 1024)
    return fail(YOCO_ERR_UNSUPPORTED, "compose needs D*elemsize a multiple of 16 bytes and D <= 1024 (D=%d)", D);
  if (!isfinite(lambda) || !isfinite(aK1) || !isfinite(aK2) || !isfinite(aV1) || !isfinite(aV2))
    return fail(YOCO_ERR_INVALID_ARG, "lambda and the weights must be finite");
  if ((uint64_t)B * n * Hkv * (D * es / 16) >= (1ull << 31))
    return fail(YOCO_ERR_UNSUPPORTED, "compose call too large (more than 2^31 16-byte vectors)");
  yoco_status st;
  const char* names[6] = {"k1", "ki", "v1", "vi", "k_cache", "v_cache"};
  const yoco_tensor4* ts[6] = {&k1, &ki, &v1, &vi, &k_cache, &v_cache};
  for (int i = 0; i < 6; ++i) {
    int64_t need = i < 4 ? (int64_t)n : (int64_t)t0 + n;
    if ((st = check_tensor(names[i], *ts[i], need, es)) != YOCO_OK) return st;
  }
  if ((st = check_distinct("k_cache", k_cache, B, Hkv, n, D)) != YOCO_OK) return st;
  if ((st = check_distinct("v_cache", v_cache, B, Hkv, n, D)) != YOCO_OK) return st;
  // Overlap rules: a source may alias a destination exactly (in-place, t0 = 0);
  // any other overlap of a source with a destination is rejected, and so is
  // k_cache overlapping v_cache with the same layout.
  Span dst[2] = {span_of(k_cache, B, Hkv, t0, (int64_t)t0 + n, D, es),
                 span_of(v_cache, B, Hkv, t0, (int64_t)t0 + n, D, es)};
  for (int i = 0; i < 4; ++i) {
    Span src = span_of(*ts[i], B, Hkv, 0, n, D, es);
    for (int d = 0; d < 2; ++d) {
      if (!overlap(src, dst[d])) continue;
      const yoco_tensor4& a = *ts[i];
      const yoco_tensor4& c = d == 0 ? k_cache : v_cache;
      bool exact = a.ptr == c.ptr && a.stride_b == c.stride_b && a.stride_h == c.stride_h &&
                   a.stride_t == c.stride_t && t0 == 0;
      if (!exact)
        return fail(YOCO_ERR_INVALID_ARG, "%s overlaps %s without aliasing it exactly", names[i], names[4 + d]);
    }
  }
  if (k_cache.ptr == v_cache.ptr && k_cache.stride_b == v_cache.stride_b && k_cache.stride_h == v_cache.stride_h &&
      k_cache.stride_t == v_cache.stride_t)
    return fail(YOCO_ERR_INVALID_ARG, "k_cache and v_cache are the same buffer");

  yoco::ComposeParams p;
  p.k1 = view(k1);
  p.ki = view(ki);
  p.v1 = view(v1);
  p.vi = view(vi);
  p.kc = view(k_cache);
  p.vc = view(v_cache);
  p.t0 = t0;
  p.B = B;
  p.n = n;
  p.Hkv = Hkv;
  p.D = D;
  p.cK1 = fold(lambda, aK1);
  p.cK2 = fold(lambda, aK2);
  p.cV1 = fold(lambda, aV1);
  p.cV2 = fold(lambda, aV2);
  return launched(yoco::launch_compose(p, dtype == YOCO_BF16, stream), "compose");
}

// Launch shape of the split pass. Measured on MI355X (bf16, D = 128, G = 4):
// a launch wants about kDecodeTargetWaves wavefronts; long splits run best with
// 8 wavefronts per workgroup and one register set, short splits with 8
// wavefronts per workgroup (4 for the shortest) and double-buffered row loads,
// which hide the load latency that few rows per wavefront expose.
struct DecodeShape {
  int splits, waves;
  bool prefetch;
};

static DecodeShape decode_shape(int B, int T, int Hkv, int S_req) {
  DecodeShape sh;
  const int64_t pairs = (int64_t)B * Hkv;
  int S = S_req;
  if (S <= 0) {
    int64_t want = (kDecodeTargetWaves / 4 + pairs - 1) / pairs;
    int64_t most = std::max<int64_t>(1, T / (4 * kDecodeMinRowsPerWave));
    S = (int)std::max<int64_t>(1, std::min(want, most));
    const int rps0 = decode_rows_per_split(T, S);
    // short splits: fewer, fuller ones; long splits: 8 wavefronts per workgroup
    // and half as many workgroups (the same wavefront count, measured faster)
    if ((rps0 <= kDecodeShortSplit || rps0 > 2 * kDecodeShortSplit) && S >= 2) S /= 2;
  }
  const int rps = decode_rows_per_split(T, S);
  sh.splits = (int)((T + (int64_t)rps - 1) / rps);   // drop splits the rounding leaves empty
  sh.prefetch = rps <= 2 * kDecodeShortSplit;
  sh.waves = !sh.prefetch || rps >= 8 * kDecodeMinRowsPerWave ? 8 : 4;
  return sh;
}

size_t yoco_compose_backward_workspace_size(int B, int n, int Hkv, int D, yoco_dtype dtype) {
  if (B <= 0 || n <= 0 || Hkv <= 0 || D <= 0 || !valid_dtype(dtype)) return 0;
  yoco::ComposeBackwardParams p{};
  p.B = B;
  p.n = n;
  p.Hkv = Hkv;
  p.D = D;
  return (size_t)yoco::compose_backward_blocks(p) * 4 * sizeof(float);
}

yoco_status yoco_compose_kv_backward(yoco_tensor4 gk, yoco_tensor4 gv, int t0, yoco_tensor4 k1, yoco_tensor4 ki,
                                     yoco_tensor4 v1, yoco_tensor4 vi, yoco_tensor4 dk1, yoco_tensor4 dki,
                                     yoco_tensor4 dv1, yoco_tensor4 dvi, int B, int n, int Hkv, int D, float lambda,
                                     float aK1, float aK2, float aV1, float aV2, float* dalpha, void* workspace,
                                     size_t workspace_bytes, yoco_dtype dtype, hipStream_t stream) {
  if (B <= 0 || n <= 0 || Hkv <= 0 || D <= 0 || t0 < 0)
    return fail(YOCO_ERR_INVALID_ARG, "sizes must be positive and t0 >= 0 (B=%d n=%d Hkv=%d D=%d t0=%d)", B, n, Hkv,
                D, t0);
  if (!valid_dtype(dtype)) return fail(YOCO_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  const size_t es = esize(dtype);
  if ((D * es) % 16 || D > 1024)
    return fail(YOCO_ERR_UNSUPPORTED, "compose backward needs D*elemsize a multiple of 16 bytes and D <= 1024");
  if (!isfinite(lambda) || !isfinite(aK1) || !isfinite(aK2) || !isfinite(aV1) || !isfinite(aV2))
    return fail(YOCO_ERR_INVALID_ARG, "lambda and the weights must be finite");
  if ((uint64_t)B * n * Hkv * (D / 4) >= (1ull << 31))
    return fail(YOCO_ERR_UNSUPPORTED, "compose backward call too large (more than 2^31 four-element vectors)");
  yoco_status st;
  const char* in_names[6] = {"gk", "gv", "k1", "ki", "v1", "vi"};
  const yoco_tensor4* ins[6] = {&gk, &gv, &k1, &ki, &v1, &vi};
  for (int i = 0; i < 6; ++i) {
    int64_t need = i < 2 ? (int64_t)t0 + n : (int64_t)n;
    if ((st = check_tensor(in_names[i], *ins[i], need, es)) != YOCO_OK) return st;
  }
  const char* out_names[4] = {"dk1", "dki", "dv1", "dvi"};
  const yoco_tensor4* outs[4] = {&dk1, &dki, &dv1, &dvi};
  for (int i = 0; i < 4; ++i)
    if ((st = check_tensor(out_names[i], *outs[i], n, 4)) != YOCO_OK ||
        (st = check_distinct(out_names[i], *outs[i], B, Hkv, n, D)) != YOCO_OK)
      return st;
  // the four gradient outputs must not overlap one another or any input
  for (int i = 0; i < 4; ++i) {
    Span so = span_of(*outs[i], B, Hkv, 0, n, D, 4);
    for (int j = i + 1; j < 4; ++j)
      if (overlap(so, span_of(*outs[j], B, Hkv, 0, n, D, 4)))
        return fail(YOCO_ERR_INVALID_ARG, "%s overlaps %s", out_names[i], out_names[j]);
    for (int j = 0; j < 6; ++j) {
      int64_t r0 = j < 2 ? t0 : 0;
      if (overlap(so, span_of(*ins[j], B, Hkv, r0, r0 + n, D, es)))
        return fail(YOCO_ERR_INVALID_ARG, "%s overlaps %s", out_names[i], in_names[j]);
    }
  }
  if (!dalpha) return fail(YOCO_ERR_INVALID_ARG, "dalpha: null pointer");
  if (reinterpret_cast<uintptr_t>(dalpha) & 3u) return fail(YOCO_ERR_ALIGNMENT, "dalpha: not 4-byte aligned");
  const size_t need = yoco_compose_backward_workspace_size(B, n, Hkv, D, dtype);
  if (!workspace) return fail(YOCO_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
  if (workspace_bytes < need) return fail(YOCO_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(YOCO_ERR_ALIGNMENT, "workspace not 16-byte aligned");
  yoco::ComposeBackwardParams p;
  p.gk = view(gk);
  p.gv = view(gv);
  p.k1 = view(k1);
  p.ki = view(ki);
  p.v1 = view(v1);
  p.vi = view(vi);
  p.dk1 = view(dk1);
  p.dki = view(dki);
  p.dv1 = view(dv1);
  p.dvi = view(dvi);
  p.t0 = t0;
  p.B = B;
  p.n = n;
  p.Hkv = Hkv;
  p.D = D;
  p.cK1 = fold(lambda, aK1);
  p.cK2 = fold(lambda, aK2);
  p.cV1 = fold(lambda, aV1);
  p.cV2 = fold(lambda, aV2);
  p.lambda = lambda;
  p.dalpha = dalpha;
  return launched(yoco::launch_compose_backward(p, dtype == YOCO_BF16, static_cast<float*>(workspace), stream),
                  "compose backward");
}

int yoco_decode_num_splits(int B, int T, int Hq, int Hkv, int D) {
  (void)Hq;
  (void)D;
  if (B <= 0 || T <= 0 || Hkv <= 0) return 0;
  return decode_shape(B, T, Hkv, 0).splits;
}

// Workspace layout: tickets [B, Hkv] u32 | part_o [B, Hq, S, D] f32 | part_lse [B, Hq, S] f32,
// each section starting on a 16-byte boundary. The counters come first so that
// their place does not move when the split count (or T) changes between calls.
struct WsLayout {
  size_t o_off, lse_off, total;
};

static WsLayout ws_layout(int B, int Hq, int Hkv, int D, int S) {
  WsLayout w;
  size_t rows = (size_t)B * Hq * S;
  w.o_off = (size_t)round_up((int64_t)B * Hkv * 4, 16);
  w.lse_off = w.o_off + rows * D * sizeof(float);
  w.total = w.lse_off + (size_t)round_up((int64_t)(rows * sizeof(float)), 16);
  return w;
}

size_t yoco_decode_workspace_size(int B, int T, int Hq, int Hkv, int D, int num_splits) {
  if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || num_splits < 0) return 0;
  int S = num_splits ? num_splits : yoco_decode_num_splits(B, T, Hq, Hkv, D);
  if (S <= 1) return 0;
  return ws_layout(B, Hq, Hkv, D, S).total;
}

// Checks and launch parameters of a decode call. With attach_workspace the
// partials are placed in the caller's workspace (when the split count is above
// one); otherwise the caller places them.
static yoco_status decode_setup(const void* q, yoco_tensor4 k, yoco_tensor4 v, const int32_t* seq_lens, int B, int T,
                                int Hq, int Hkv, int D, float scale, void* workspace, size_t ws_bytes, int S,
                                yoco_dtype dt, yoco::DecodeParams* p, bool attach_workspace = true) {
  yoco_status st = check_decode(q, k, v, B, T, Hq, Hkv, D, dt);
  if (st != YOCO_OK) return st;
  if (S < 1) return fail(YOCO_ERR_INVALID_ARG, "num_splits must be >= 1 (got %d)", S);
  if (S > T) return fail(YOCO_ERR_INVALID_ARG, "num_splits=%d exceeds T=%d", S, T);
  if (seq_lens && (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return fail(YOCO_ERR_ALIGNMENT, "seq_lens: not 4-byte aligned");
  if (!(scale > 0.f)) scale = 1.0f / sqrtf((float)D);
  if (!isfinite(scale)) return fail(YOCO_ERR_INVALID_ARG, "scale must be finite");
  p->q = q;
  p->k = view(k);
  p->v = view(v);
  p->seq_lens = seq_lens;
  p->B = B;
  p->T = T;
  p->Hq = Hq;
  p->Hkv = Hkv;
  p->D = D;
  p->scale_log2 = (float)((double)scale * 1.4426950408889634);
  const DecodeShape sh = decode_shape(B, T, Hkv, S);
  p->num_splits = S;
  p->rows_per_split = decode_rows_per_split(T, S);
  p->waves = sh.waves;
  p->prefetch = sh.prefetch;
  p->out = nullptr;
  p->lse = nullptr;
  p->part_o = nullptr;
  p->part_lse = nullptr;
  p->tickets = nullptr;
  p->compose_on_read = false;
  p->k1 = p->v1 = yoco::View4{nullptr, 0, 0, 0};
  p->append = false;
  p->nk1 = p->nki = p->nv1 = p->nvi = yoco::View4{nullptr, 0, 0, 0};
  p->cK1 = p->cK2 = p->cV1 = p->cV2 = 0.f;
  p->termsK = p->termsV = 0;
  if (S > 1 && attach_workspace) {
    WsLayout w = ws_layout(B, Hq, Hkv, D, S);
    if (!workspace) return fail(YOCO_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", w.total);
    if (ws_bytes < w.total) return fail(YOCO_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, w.total);
    if (!aligned16(workspace)) return fail(YOCO_ERR_ALIGNMENT, "workspace not 16-byte aligned");
    char* base = static_cast<char*>(workspace);
    p->part_o = reinterpret_cast<float*>(base + w.o_off);
    p->part_lse = reinterpret_cast<float*>(base + w.lse_off);
  }
  return YOCO_OK;
}

yoco_status yoco_cross_attn_decode(const void* q, yoco_tensor4 k_cache, yoco_tensor4 v_cache,
                                   const int32_t* seq_lens, int B, int T, int Hq, int Hkv, int D, float scale,
                                   float* out, float* lse, void* workspace, size_t workspace_bytes, int num_splits,
                                   yoco_dtype kv_dtype, hipStream_t stream) {
  if (num_splits < 0) return fail(YOCO_ERR_INVALID_ARG, "num_splits must be >= 0");
  int S = num_splits ? num_splits : yoco_decode_num_splits(B, T, Hq, Hkv, D);
  if (S == 0) return fail(YOCO_ERR_INVALID_ARG, "sizes must be positive");
  yoco::DecodeParams p;
  yoco_status st =
      decode_setup(q, k_cache, v_cache, seq_lens, B, T, Hq, Hkv, D, scale, workspace, workspace_bytes, S, kv_dtype, &p);
  if (st != YOCO_OK) return st;
  if (!out) return fail(YOCO_ERR_INVALID_ARG, "out: null pointer");
  if (!aligned16(out)) return fail(YOCO_ERR_ALIGNMENT, "out: not 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(YOCO_ERR_ALIGNMENT, "lse: not 4-byte aligned");
  p.out = out;
  p.lse = lse;
  if (S > 1) {
    // fused merge: the tickets live after the partials
    p.tickets = static_cast<unsigned*>(workspace);
  }
  return launched(yoco::launch_decode_partial(p, kv_dtype == YOCO_BF16, stream), "decode");
}

yoco_status yoco_cross_attn_decode_noalloc(const void* q, yoco_tensor4 k_cache, yoco_tensor4 v_cache,
                                           const int32_t* seq_lens, int B, int T, int Hq, int Hkv, int D, float scale,
                                           float* out, float* lse, int num_splits, yoco_dtype kv_dtype,
                                           hipStream_t stream) {
  if (num_splits < 0) return fail(YOCO_ERR_INVALID_ARG, "num_splits must be >= 0");
  int S = num_splits ? num_splits : yoco_decode_num_splits(B, T, Hq, Hkv, D);
  if (S == 0) return fail(YOCO_ERR_INVALID_ARG, "sizes must be positive");
  yoco::DecodeParams p;
  yoco_status st = decode_setup(q, k_cache, v_cache, seq_lens, B, T, Hq, Hkv, D, scale, nullptr, 0, S, kv_dtype, &p,
                                /*attach_workspace=*/false);
  if (st != YOCO_OK) return st;
  if (!out) return fail(YOCO_ERR_INVALID_ARG, "out: null pointer");
  if (!aligned16(out)) return fail(YOCO_ERR_ALIGNMENT, "out: not 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(YOCO_ERR_ALIGNMENT, "lse: not 4-byte aligned");
  p.out = out;
  p.lse = lse;
  if (S > 1) {
    // counters in the fixed leading section, then part_o and part_lse (16-byte aligned)
    const size_t rows = (size_t)B * Hq * S;
    const size_t o_bytes = rows * D * sizeof(float);
    const size_t need = kScratchCounterBytes + o_bytes + (size_t)round_up((int64_t)(rows * sizeof(float)), 16);
    if ((size_t)B * Hkv * 4 > kScratchCounterBytes)
      return fail(YOCO_ERR_WORKSPACE, "B*Hkv = %lld exceeds the %zu merge counters of the scratch array",
                  (long long)B * Hkv, kScratchCounterBytes / 4);
    if (need > kScratchBytes)
      return fail(YOCO_ERR_WORKSPACE, "this call needs %zu bytes of scratch; the scratch array holds %zu", need,
                  kScratchBytes);
    char* base = nullptr;
    const hipError_t e = yoco::noalloc_scratch(stream, &base);
    if (e != hipSuccess) return fail(YOCO_ERR_LAUNCH, "scratch array: %s", hipGetErrorString(e));
    p.tickets = reinterpret_cast<unsigned*>(base);
    p.part_o = reinterpret_cast<float*>(base + kScratchCounterBytes);
    p.part_lse = reinterpret_cast<float*>(base + kScratchCounterBytes + o_bytes);
  }
  return launched(yoco::launch_decode_partial(p, kv_dtype == YOCO_BF16, stream), "decode (no allocation)");
}

yoco_status yoco_cross_attn_decode_compose_on_read(const void* q, yoco_tensor4 k1_cache, yoco_tensor4 ki_cache,
                                                   yoco_tensor4 v1_cache, yoco_tensor4 vi_cache,
                                                   const int32_t* seq_lens, int B, int T, int Hq, int Hkv, int D,
                                                   float lambda, float aK1, float aK2, float aV1, float aV2,
                                                   float scale, float* out, float* lse, void* workspace,
                                                   size_t workspace_bytes, int num_splits, yoco_dtype kv_dtype,
                                                   hipStream_t stream) {
  if (num_splits < 0) return fail(YOCO_ERR_INVALID_ARG, "num_splits must be >= 0");
  int S = num_splits ? num_splits : yoco_decode_num_splits(B, T, Hq, Hkv, D);
  if (S == 0) return fail(YOCO_ERR_INVALID_ARG, "sizes must be positive");
  yoco::DecodeParams p;
  yoco_status st = decode_setup(q, ki_cache, vi_cache, seq_lens, B, T, Hq, Hkv, D, scale, workspace,
                                workspace_bytes, S, kv_dtype, &p);
  if (st != YOCO_OK) return st;
  const size_t es = esize(kv_dtype);
  if ((st = check_tensor("k1_cache", k1_cache, T, es)) != YOCO_OK) return st;
  if ((st = check_tensor("v1_cache", v1_cache, T, es)) != YOCO_OK) return st;
  if ((st = check_row_stride("k1_cache", k1_cache, D)) != YOCO_OK) return st;
  if ((st = check_row_stride("v1_cache", v1_cache, D)) != YOCO_OK) return st;
  if ((st = check_head_span("k1_cache", k1_cache, T, es)) != YOCO_OK) return st;
  if ((st = check_head_span("v1_cache", v1_cache, T, es)) != YOCO_OK) return st;
  if (!isfinite(lambda) || !isfinite(aK1) || !isfinite(aK2) || !isfinite(aV1) || !isfinite(aV2))
    return fail(YOCO_ERR_INVALID_ARG, "lambda and the weights must be finite");
  if (!out) return fail(YOCO_ERR_INVALID_ARG, "out: null pointer");
  if (!aligned16(out)) return fail(YOCO_ERR_ALIGNMENT, "out: not 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(YOCO_ERR_ALIGNMENT, "lse: not 4-byte aligned");
  p.out = out;
  p.lse = lse;
  if (S > 1) p.tickets = static_cast<unsigned*>(workspace);
  p.compose_on_read = true;
  p.k1 = view(k1_cache);
  p.v1 = view(v1_cache);
  p.cK1 = fold(lambda, aK1);
  p.cK2 = fold(lambda, aK2);
  p.cV1 = fold(lambda, aV1);
  p.cV2 = fold(lambda, aV2);
  p.termsK = yoco::compose_terms(p.cK1, p.cK2);
  p.termsV = yoco::compose_terms(p.cV1, p.cV2);
  return launched(yoco::launch_decode_partial(p, kv_dtype == YOCO_BF16, stream), "decode (compose on read)");
}

yoco_status yoco_self_attn_decode(const void* q, yoco_tensor4 k1_new, yoco_tensor4 ki_new, yoco_tensor4 v1_new,
                                  yoco_tensor4 vi_new, yoco_tensor4 k_cache, yoco_tensor4 v_cache,
                                  const int32_t* seq_lens, int B, int T, int Hq, int Hkv, int D, float lambda,
                                  float aK1, float aK2, float aV1, float aV2, float scale, float* out, float* lse,
                                  void* workspace, size_t workspace_bytes, int num_splits, yoco_dtype kv_dtype,
                                  hipStream_t stream) {
  if (num_splits < 0) return fail(YOCO_ERR_INVALID_ARG, "num_splits must be >= 0");
  int S = num_splits ? num_splits : yoco_decode_num_splits(B, T, Hq, Hkv, D);
  if (S == 0) return fail(YOCO_ERR_INVALID_ARG, "sizes must be positive");
  yoco::DecodeParams p;
  yoco_status st =
      decode_setup(q, k_cache, v_cache, seq_lens, B, T, Hq, Hkv, D, scale, workspace, workspace_bytes, S, kv_dtype, &p);
  if (st != YOCO_OK) return st;
  if (!isfinite(lambda) || !isfinite(aK1) || !isfinite(aK2) || !isfinite(aV1) || !isfinite(aV2))
    return fail(YOCO_ERR_INVALID_ARG, "lambda and the weights must be finite");
  const size_t es = esize(kv_dtype);
  const char* names[4] = {"k1_new", "ki_new", "v1_new", "vi_new"};
  const yoco_tensor4* src[4] = {&k1_new, &ki_new, &v1_new, &vi_new};
  for (int i = 0; i < 4; ++i) {
    // a source is read at row seq_len - 1 <= T - 1; a one-token buffer has stride_t = 0
    const int64_t need = src[i]->stride_t == 0 ? 1 : T;
    if ((st = check_tensor(names[i], *src[i], need, es)) != YOCO_OK) return st;
    // The cache is read at rows below seq_len - 1 and written at that row, so a
    // source may share its memory only as the very same view (in-place compose).
    const yoco_tensor4& c = i < 2 ? k_cache : v_cache;
    const yoco_tensor4& c_other = i < 2 ? v_cache : k_cache;
    const bool same = src[i]->ptr == c.ptr && src[i]->stride_b == c.stride_b && src[i]->stride_h == c.stride_h &&
                      src[i]->stride_t == c.stride_t;
    const Span ss = span_of(*src[i], B, Hkv, 0, src[i]->stride_t == 0 ? 1 : T, D, es);
    if (!same && overlap(ss, span_of(c, B, Hkv, 0, T, D, es)))
      return fail(YOCO_ERR_INVALID_ARG, "%s overlaps %s without being the same view", names[i],
                  i < 2 ? "k_cache" : "v_cache");
    if (overlap(ss, span_of(c_other, B, Hkv, 0, T, D, es)))
      return fail(YOCO_ERR_INVALID_ARG, "%s overlaps %s", names[i], i < 2 ? "v_cache" : "k_cache");
  }
  if (overlap(span_of(k_cache, B, Hkv, 0, T, D, es), span_of(v_cache, B, Hkv, 0, T, D, es)))
    return fail(YOCO_ERR_INVALID_ARG, "k_cache and v_cache overlap");
  // each (sequence, kv head) writes its own row n - 1
  if ((st = check_distinct("k_cache", k_cache, B, Hkv, T, D)) != YOCO_OK) return st;
  if ((st = check_distinct("v_cache", v_cache, B, Hkv, T, D)) != YOCO_OK) return st;
  if (!out) return fail(YOCO_ERR_INVALID_ARG, "out: null pointer");
  if (!aligned16(out)) return fail(YOCO_ERR_ALIGNMENT, "out: not 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(YOCO_ERR_ALIGNMENT, "lse: not 4-byte aligned");
  p.out = out;
  p.lse = lse;
  if (S > 1) p.tickets = static_cast<unsigned*>(workspace);
  p.append = true;
  p.nk1 = view(k1_new);
  p.nki = view(ki_new);
  p.nv1 = view(v1_new);
  p.nvi = view(vi_new);
  p.cK1 = fold(lambda, aK1);
  p.cK2 = fold(lambda, aK2);
  p.cV1 = fold(lambda, aV1);
  p.cV2 = fold(lambda, aV2);
  p.termsK = yoco::compose_terms(p.cK1, p.cK2);
  p.termsV = yoco::compose_terms(p.cV1, p.cV2);
  return launched(yoco::launch_decode_partial(p, kv_dtype == YOCO_BF16, stream), "self-decoder decode step");
}

yoco_status yoco_cross_attn_decode_partial(const void* q, yoco_tensor4 k_cache, yoco_tensor4 v_cache,
                                           const int32_t* seq_lens, int B, int T, int Hq, int Hkv, int D, float scale,
                                           void* workspace, size_t workspace_bytes, int num_splits,
                                           yoco_dtype kv_dtype, hipStream_t stream) {
  if (num_splits < 2)
    return fail(YOCO_ERR_INVALID_ARG, "the split pass alone needs num_splits >= 2 (got %d)", num_splits);
  yoco::DecodeParams p;
  yoco_status st = decode_setup(q, k_cache, v_cache, seq_lens, B, T, Hq, Hkv, D, scale, workspace, workspace_bytes,
                                num_splits, kv_dtype, &p);
  if (st != YOCO_OK) return st;
  return launched(yoco::launch_decode_partial(p, kv_dtype == YOCO_BF16, stream), "decode split pass");
}

yoco_status yoco_decode_merge(const void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int D,
                              int num_splits, float* out, float* lse, hipStream_t stream) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || num_splits < 2)
    return fail(YOCO_ERR_INVALID_ARG, "B, Hq, Hkv must be positive and num_splits >= 2");
  if (Hq % Hkv) return fail(YOCO_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (D != 64 && D != 128) return fail(YOCO_ERR_UNSUPPORTED, "merge supports D in {64, 128}, got %d", D);
  WsLayout w = ws_layout(B, Hq, Hkv, D, num_splits);
  if (!workspace) return fail(YOCO_ERR_WORKSPACE, "workspace is NULL");
  if (workspace_bytes < w.total)
    return fail(YOCO_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, w.total);
  if (!aligned16(workspace)) return fail(YOCO_ERR_ALIGNMENT, "workspace not 16-byte aligned");
  if (!out) return fail(YOCO_ERR_INVALID_ARG, "out: null pointer");
  if (!aligned16(out)) return fail(YOCO_ERR_ALIGNMENT, "out: not 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(YOCO_ERR_ALIGNMENT, "lse: not 4-byte aligned");
  const char* base = static_cast<const char*>(workspace);
  const float* po = reinterpret_cast<const float*>(base + w.o_off);
  const float* pl = reinterpret_cast<const float*>(base + w.lse_off);
  return launched(yoco::launch_decode_merge(po, pl, B, Hq, D, num_splits, out, lse, stream), "decode merge");
}

yoco_status yoco_cross_attn_prefill(const void* q, yoco_tensor4 k_cache, yoco_tensor4 v_cache, int B, int C, int p0,
                                    int Hq, int Hkv, int D, float scale, void* out, yoco_dtype out_dtype, float* lse,
                                    yoco_dtype dtype, hipStream_t stream) {
  if (B <= 0 || C <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || p0 < 0)
    return fail(YOCO_ERR_INVALID_ARG, "sizes must be positive and p0 >= 0 (B=%d C=%d Hq=%d Hkv=%d D=%d p0=%d)", B, C,
                Hq, Hkv, D, p0);
  if (Hq % Hkv) return fail(YOCO_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return fail(YOCO_ERR_INVALID_ARG, "unknown dtype");
  if (dtype != YOCO_BF16) return fail(YOCO_ERR_UNSUPPORTED, "prefill runs on bf16 inputs only");
  if (D != 64 && D != 128) return fail(YOCO_ERR_UNSUPPORTED, "prefill supports D in {64, 128}, got %d", D);
  if (!supported_group(Hq / Hkv))
    return fail(YOCO_ERR_UNSUPPORTED, "prefill supports Hq/Hkv in {1,2,4,8,16}, got %d", Hq / Hkv);
  if (!q) return fail(YOCO_ERR_INVALID_ARG, "q: null pointer");
  if (!aligned16(q)) return fail(YOCO_ERR_ALIGNMENT, "q: not 16-byte aligned");
  if (!out) return fail(YOCO_ERR_INVALID_ARG, "out: null pointer");
  if (!aligned16(out)) return fail(YOCO_ERR_ALIGNMENT, "out: not 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(YOCO_ERR_ALIGNMENT, "lse: not 4-byte aligned");
  yoco_status st;
  int64_t need = (int64_t)p0 + C;
  if ((st = check_tensor("k_cache", k_cache, need, 2)) != YOCO_OK) return st;
  if ((st = check_tensor("v_cache", v_cache, need, 2)) != YOCO_OK) return st;
  if ((st = check_row_stride("k_cache", k_cache, D)) != YOCO_OK) return st;
  if ((st = check_row_stride("v_cache", v_cache, D)) != YOCO_OK) return st;
  // the kernel addresses the rows of a 64-key step with 32-bit byte offsets
  if (k_cache.stride_t >= (int64_t(1) << 24) || v_cache.stride_t >= (int64_t(1) << 24))
    return fail(YOCO_ERR_UNSUPPORTED, "prefill: cache stride_t must be below 2^24 elements");
  if (need > INT32_MAX / 2) return fail(YOCO_ERR_UNSUPPORTED, "cache too long");
  if (!(scale > 0.f)) scale = 1.0f / sqrtf((float)D);
  if (!isfinite(scale)) return fail(YOCO_ERR_INVALID_ARG, "scale must be finite");
  yoco::PrefillParams p;
  p.q = q;
  p.k = view(k_cache);
  p.v = view(v_cache);
  p.B = B;
  p.C = C;
  p.p0 = p0;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.out = out;
  p.out_bf16 = out_dtype == YOCO_BF16;
  p.lse = lse;
  return launched(yoco::launch_prefill(p, stream), "prefill");
}

}  // extern "C"
