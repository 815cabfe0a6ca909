// Host-only driver of the C ABI layer (yoco_api.cpp), built with the test-only
// launchers of launch_stubs.cpp under AddressSanitizer and
// UndefinedBehaviorSanitizer. Device pointers are fake addresses that the ABI
// layer only does arithmetic on. It checks that valid calls reach the
// launchers with the parameters the header promises (folded weights, split
// counts, workspace and scratch layouts), that a launcher's failure becomes
// YOCO_ERR_LAUNCH with a message, that rejected calls launch nothing, and that
// the largest decode the 32-bit row offsets allow is accepted while the next
// is refused. Prints "ok" and exits 0 on success.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "../../include/yoco.h"
#include "stubs.h"

#define CHECK(cond)                                                               \
  do {                                                                            \
    if (!(cond)) {                                                                \
      fprintf(stderr, "FAIL %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond,          \
              yoco_last_error());                                                 \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

namespace {

constexpr uintptr_t kBase = 0x7F0000000000ull;
void* fake(uint64_t off) { return reinterpret_cast<void*>(kBase + off); }

// head-major [B, H, T, D] view
yoco_tensor4 hm(uint64_t off, int B, int H, int64_t T, int D) {
  (void)B;
  return {fake(off), (int64_t)H * T * D, T * D, D, T};
}
// token-major [B, n, H, D] view
yoco_tensor4 tm(uint64_t off, int B, int64_t n, int H, int D) {
  (void)B;
  return {fake(off), n * H * D, D, (int64_t)H * D, n};
}

float folded(float lambda, float a) { return (float)((double)lambda * (double)a); }

int test_compose() {
  const int B = 2, n = 300, H = 8, D = 128;
  const float a[4] = {0.0125f, -0.03f, 0.02f, 0.04f};
  yoco_tensor4 s[4];
  for (int i = 0; i < 4; ++i) s[i] = tm((uint64_t)(i + 1) << 28, B, n, H, D);
  yoco_tensor4 kc = hm(5ull << 28, B, H, 512, D), vc = hm(6ull << 28, B, H, 512, D);
  stubs::result = hipSuccess;
  int before = stubs::launches;
  CHECK(yoco_compose_kv(s[0], s[1], s[2], s[3], kc, vc, 100, B, n, H, D, 35.f, a[0], a[1], a[2], a[3], YOCO_BF16,
                        nullptr) == YOCO_OK);
  CHECK(stubs::launches == before + 1);
  CHECK(stubs::compose.cK1 == folded(35.f, a[0]) && stubs::compose.cK2 == folded(35.f, a[1]));
  CHECK(stubs::compose.cV1 == folded(35.f, a[2]) && stubs::compose.cV2 == folded(35.f, a[3]));
  CHECK(stubs::compose.t0 == 100 && stubs::compose.n == n && stubs::compose.B == B && stubs::compose.Hkv == H);
  CHECK(stubs::compose.kc.st == D && stubs::compose.k1.st == H * D);
  // the initialisation a1 = 0, a2 = fl32(1/35) folds to exactly (0, 1)
  const float inv = 1.0f / 35.0f;
  CHECK(yoco_compose_kv(s[0], s[1], s[2], s[3], kc, vc, 0, B, n, H, D, 35.f, 0.f, inv, 0.f, inv, YOCO_BF16,
                        nullptr) == YOCO_OK);
  CHECK(stubs::compose.cK1 == 0.f && stubs::compose.cK2 == 1.0f && stubs::compose.cV2 == 1.0f);
  // a launcher failure maps to YOCO_ERR_LAUNCH with the runtime's message
  stubs::result = hipErrorInvalidValue;
  CHECK(yoco_compose_kv(s[0], s[1], s[2], s[3], kc, vc, 0, B, n, H, D, 35.f, a[0], a[1], a[2], a[3], YOCO_BF16,
                        nullptr) == YOCO_ERR_LAUNCH);
  CHECK(strstr(yoco_last_error(), "stub launch error") != nullptr);
  stubs::result = hipSuccess;
  // rejected calls launch nothing
  before = stubs::launches;
  CHECK(yoco_compose_kv(s[0], s[1], s[2], s[3], kc, vc, 300, B, n, H, D, 35.f, a[0], a[1], a[2], a[3], YOCO_BF16,
                        nullptr) == YOCO_ERR_INVALID_ARG);   // t0 + n beyond the cache
  CHECK(yoco_compose_kv(s[0], s[1], s[2], s[3], kc, kc, 0, B, n, H, D, 35.f, a[0], a[1], a[2], a[3], YOCO_BF16,
                        nullptr) == YOCO_ERR_INVALID_ARG);   // one buffer for both caches
  CHECK(stubs::launches == before);
  CHECK(yoco_compose_kv(s[0], s[1], s[2], s[3], kc, vc, 0, B, n, H, D, 35.f, a[0], a[1], a[2], a[3], YOCO_BF16,
                        nullptr) == YOCO_OK);
  CHECK(yoco_last_error()[0] == '\0');   // a successful call clears the message
  return 0;
}

int test_backward() {
  const int B = 1, n = 1000, H = 8, D = 128;
  yoco_tensor4 g[2] = {hm(1ull << 28, B, H, n, D), hm(2ull << 28, B, H, n, D)};
  yoco_tensor4 s[4], d[4];
  for (int i = 0; i < 4; ++i) s[i] = tm((uint64_t)(3 + i) << 28, B, n, H, D);
  for (int i = 0; i < 4; ++i) d[i] = tm((uint64_t)(7 + i) << 28, B, n, H, D);
  const size_t need = yoco_compose_backward_workspace_size(B, n, H, D, YOCO_BF16);
  CHECK(need == (size_t)((B * n * H * (D / 4) + 1023) / 1024) * 16);
  float* dalpha = static_cast<float*>(fake(12ull << 28));
  void* ws = fake(13ull << 28);
  stubs::result = hipSuccess;
  CHECK(yoco_compose_kv_backward(g[0], g[1], 0, s[0], s[1], s[2], s[3], d[0], d[1], d[2], d[3], B, n, H, D, 35.f,
                                 0.f, 0.02f, 0.01f, 0.03f, dalpha, ws, need, YOCO_BF16, nullptr) == YOCO_OK);
  CHECK(stubs::backward_partial == ws && stubs::backward.dalpha == dalpha && stubs::backward.lambda == 35.f);
  CHECK(stubs::backward.cK2 == folded(35.f, 0.02f));
  CHECK(yoco_compose_kv_backward(g[0], g[1], 0, s[0], s[1], s[2], s[3], d[0], d[1], d[2], d[3], B, n, H, D, 35.f,
                                 0.f, 0.02f, 0.01f, 0.03f, dalpha, ws, need - 16, YOCO_BF16, nullptr) ==
        YOCO_ERR_WORKSPACE);
  stubs::result = hipErrorLaunchFailure;
  CHECK(yoco_compose_kv_backward(g[0], g[1], 0, s[0], s[1], s[2], s[3], d[0], d[1], d[2], d[3], B, n, H, D, 35.f,
                                 0.f, 0.02f, 0.01f, 0.03f, dalpha, ws, need, YOCO_BF16, nullptr) == YOCO_ERR_LAUNCH);
  stubs::result = hipSuccess;
  return 0;
}

int test_decode() {
  const int B = 8, T = 4096, Hq = 32, Hkv = 8, D = 128;
  yoco_tensor4 k = hm(1ull << 30, B, Hkv, T, D), v = hm(2ull << 30, B, Hkv, T, D);
  void* q = fake(0);
  float* out = static_cast<float*>(fake(3ull << 30));
  float* lse = static_cast<float*>(fake(4ull << 30));
  char* ws = static_cast<char*>(fake(5ull << 30));
  const int S = yoco_decode_num_splits(B, T, Hq, Hkv, D);
  const size_t need = yoco_decode_workspace_size(B, T, Hq, Hkv, D, 0);
  CHECK(S >= 2 && need == 256 + (size_t)B * Hq * S * D * 4 + (size_t)B * Hq * S * 4);
  stubs::result = hipSuccess;
  CHECK(yoco_cross_attn_decode(q, k, v, nullptr, B, T, Hq, Hkv, D, 0.f, out, lse, ws, need, 0, YOCO_BF16, nullptr) ==
        YOCO_OK);
  const yoco::DecodeParams& p = stubs::decode;
  CHECK(stubs::decode_bf16 && p.num_splits == S && p.rows_per_split * S >= T && p.rows_per_split % 16 == 0);
  CHECK((void*)p.tickets == ws && (char*)p.part_o == ws + 256 && (char*)p.part_lse == ws + 256 + (size_t)B * Hq * S * D * 4);
  CHECK(p.out == out && p.lse == lse && !p.append && !p.compose_on_read);
  CHECK(fabsf(p.scale_log2 - (float)(1.4426950408889634 / sqrt(128.0))) <= 1e-7f);
  // one split: no workspace needed, none read
  CHECK(yoco_cross_attn_decode(q, k, v, nullptr, B, T, Hq, Hkv, D, 0.f, out, lse, nullptr, 0, 1, YOCO_BF16, nullptr) ==
        YOCO_OK);
  CHECK(stubs::decode.num_splits == 1 && stubs::decode.tickets == nullptr && stubs::decode.part_o == nullptr);
  // the split pass alone and the standalone merge
  CHECK(yoco_cross_attn_decode_partial(q, k, v, nullptr, B, T, Hq, Hkv, D, 0.f, ws, need, S, YOCO_BF16, nullptr) ==
        YOCO_OK);
  CHECK(stubs::decode.tickets == nullptr && stubs::decode.out == nullptr);
  CHECK(yoco_decode_merge(ws, need, B, Hq, Hkv, D, S, out, lse, nullptr) == YOCO_OK);
  CHECK((const char*)stubs::merge.part_o == ws + 256 && stubs::merge.S == S && stubs::merge.out == out);
  // the allocation-free decode: counters at the scratch array's start, partials after its counter section
  CHECK(yoco_cross_attn_decode_noalloc(q, k, v, nullptr, B, T, Hq, Hkv, D, 0.f, out, lse, 0, YOCO_BF16, nullptr) ==
        YOCO_OK);
  CHECK((char*)stubs::decode.tickets == stubs::scratch_bytes);
  CHECK((char*)stubs::decode.part_o == stubs::scratch_bytes + YOCO_NOALLOC_COUNTER_BYTES);
  // compose on read and the self-decoder step carry their sources and folded weights
  CHECK(yoco_cross_attn_decode_compose_on_read(q, hm(6ull << 30, B, Hkv, T, D), k, hm(7ull << 30, B, Hkv, T, D), v,
                                               nullptr, B, T, Hq, Hkv, D, 35.f, 0.f, 0.02f, 0.01f, 0.03f, 0.f, out,
                                               lse, ws, need, 0, YOCO_BF16, nullptr) == YOCO_OK);
  CHECK(stubs::decode.compose_on_read && stubs::decode.termsK == 2 && stubs::decode.termsV == 3);
  yoco_tensor4 one = {fake(8ull << 30), (int64_t)Hkv * D, D, 0, 1};
  CHECK(yoco_self_attn_decode(q, one, one, one, one, k, v, nullptr, B, T, Hq, Hkv, D, 35.f, 0.f, 0.02f, 0.01f, 0.03f,
                              0.f, out, lse, ws, need, 0, YOCO_BF16, nullptr) == YOCO_OK);
  CHECK(stubs::decode.append && stubs::decode.nk1.st == 0);
  // launcher failures
  stubs::result = hipErrorInvalidValue;
  CHECK(yoco_cross_attn_decode(q, k, v, nullptr, B, T, Hq, Hkv, D, 0.f, out, lse, ws, need, 0, YOCO_BF16, nullptr) ==
        YOCO_ERR_LAUNCH);
  CHECK(yoco_cross_attn_decode_noalloc(q, k, v, nullptr, B, T, Hq, Hkv, D, 0.f, out, lse, 0, YOCO_BF16, nullptr) ==
        YOCO_ERR_LAUNCH);
  CHECK(yoco_decode_merge(ws, need, B, Hq, Hkv, D, S, out, lse, nullptr) == YOCO_ERR_LAUNCH);
  stubs::result = hipSuccess;
  return 0;
}

// The decode addresses a (sequence, kv head)'s rows through a buffer resource
// with 32-bit byte offsets. A wavefront's loads touch rows below te + R, R <= 64
// rows past the split's end (those read as zeros), each at most D * elemsize
// bytes into its row, so the largest offset is (T + 63) * stride_t * es +
// D * es - 1. The host accepts T while (T + 64) * stride_t * es < 2^31.
int test_decode_offset_limit() {
  const int D = 128;
  const int64_t es = 2;
  for (int64_t st : {(int64_t)D, (int64_t)8 * D, (int64_t)32 * D}) {
    const int64_t T_ok = ((((int64_t)1 << 31) - 1) / (st * es)) - 64;   // the largest T the host accepts
    yoco_tensor4 k = {fake(1ull << 34), 0, 0, st, T_ok + 1};
    yoco_tensor4 v = {fake(1ull << 36), 0, 0, st, T_ok + 1};
    float* out = static_cast<float*>(fake(1ull << 38));
    CHECK(yoco_cross_attn_decode(fake(0), k, v, nullptr, 1, (int)T_ok, 4, 1, D, 0.f, out, nullptr, nullptr, 0, 1,
                                 YOCO_BF16, nullptr) == YOCO_OK);
    const uint64_t max_offset = (uint64_t)(T_ok + 63) * st * es + D * es - 1;
    CHECK(max_offset < ((uint64_t)1 << 31));
    CHECK(yoco_cross_attn_decode(fake(0), k, v, nullptr, 1, (int)T_ok + 1, 4, 1, D, 0.f, out, nullptr, nullptr, 0, 1,
                                 YOCO_BF16, nullptr) == YOCO_ERR_UNSUPPORTED);
  }
  return 0;
}

int test_prefill() {
  const int B = 1, C = 4096, p0 = 4096, Hq = 32, Hkv = 8, D = 128;
  yoco_tensor4 k = hm(1ull << 30, B, Hkv, 8192, D), v = hm(2ull << 30, B, Hkv, 8192, D);
  stubs::result = hipSuccess;
  CHECK(yoco_cross_attn_prefill(fake(0), k, v, B, C, p0, Hq, Hkv, D, 0.f, fake(3ull << 30), YOCO_F32, nullptr,
                                YOCO_BF16, nullptr) == YOCO_OK);
  CHECK(stubs::prefill.p0 == p0 && stubs::prefill.C == C && !stubs::prefill.out_bf16);
  CHECK(yoco_cross_attn_prefill(fake(0), k, v, B, C, p0 + 1, Hq, Hkv, D, 0.f, fake(3ull << 30), YOCO_F32, nullptr,
                                YOCO_BF16, nullptr) == YOCO_ERR_INVALID_ARG);   // p0 + C beyond the cache rows
  stubs::result = hipErrorInvalidConfiguration;
  CHECK(yoco_cross_attn_prefill(fake(0), k, v, B, C, p0, Hq, Hkv, D, 0.f, fake(3ull << 30), YOCO_BF16, nullptr,
                                YOCO_BF16, nullptr) == YOCO_ERR_LAUNCH);
  CHECK(strstr(yoco_last_error(), "prefill") != nullptr);
  stubs::result = hipSuccess;
  return 0;
}

}  // namespace

int main() {
  if (test_compose() || test_backward() || test_decode() || test_decode_offset_limit() || test_prefill()) return 1;
  CHECK(strcmp(yoco_status_string(YOCO_ERR_LAUNCH), "kernel launch failed") == 0);
  CHECK(yoco_version() == YOCO_VERSION);
  printf("ok\n");
  return 0;
}
