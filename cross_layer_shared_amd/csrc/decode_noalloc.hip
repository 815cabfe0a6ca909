// Scratch memory of the allocation-free decode (yoco_cross_attn_decode_noalloc):
// one array per GPU, held until the process ends. The merge counters sit in a
// fixed leading section (so they never share bytes with the partials of a call
// with a different shape), the split partials after it. In host code `scratch`
// only names the symbol: its device address on the current GPU is looked up
// once per device with hipGetSymbolAddress, and only that address is handed to
// kernels.

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/yoco.h"
#include "common.h"

namespace yoco {
namespace {

constexpr size_t kScratchBytes = YOCO_NOALLOC_SCRATCH_BYTES;
constexpr size_t kCounterBytes = YOCO_NOALLOC_COUNTER_BYTES;
static_assert(kCounterBytes % 256 == 0 && kCounterBytes < kScratchBytes, "scratch layout");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void zero_words(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
char* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    // the counters must start at zero; every completed decode leaves them so
    const int words = (int)(kCounterBytes / 4);
    zero_words<<<(words + 255) / 256, 256, 0, stream>>>(static_cast<uint32_t*>(ptr), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace yoco
