// Decode attention without a caller workspace: the split partials and arrival
// counters live in a fixed device array of this library (one copy per GPU),
// for callers that cannot allocate device memory (code under graph capture,
// serving loops that forbid allocation).
//
// The array is a file-scope __device__ variable. Its name in host code is a
// host-side stand-in, not a device address, so the address is looked up once
// per device with hipGetSymbolAddress (that device current) and only that
// pointer is ever passed to a kernel. Every call on a device shares its array:
// the counters at its start are zero when the code object is loaded, are
// cleared once more by a small kernel before the device's first call, and
// every decode leaves them at zero again; the partials after them are
// overwritten by each call. Calls that overlap on one device race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvq_internal.h"

namespace kvq {
namespace {

__device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device, once looked up

__global__ void zero_words(uint32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// Device address of this device's scratch array; the first call on a device
// looks it up and enqueues the clearing of the counter region on `st`.
int32_t device_scratch(int64_t counter_bytes, hipStream_t st, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return KVQ_ERR_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return KVQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_ERR_DEVICE;
    // counters: every (sequence, KV head) of any configuration that fits
    const int64_t words = (counter_bytes + 3) / 4;
    hipLaunchKernelGGL(zero_words, dim3(64), dim3(256), 0, st, static_cast<uint32_t*>(p), words);
    if (hipGetLastError() != hipSuccess) return KVQ_ERR_DEVICE;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return KVQ_OK;
}

}  // namespace
}  // namespace kvq

extern "C" int32_t kvq_decode_attention_noalloc(const kvq_config* cfg, const void* cache,
                                                int32_t layer, int64_t tokens, const void* q,
                                                const float* k_scale, const float* v_scale,
                                                float* out, void* stream) {
  // validate everything first, against a placeholder workspace of the array's size
  void* const placeholder = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
  kvq::DecodeArgs a;
  const int32_t st = kvq::decode_prepare(cfg, cache, layer, tokens, nullptr, 1, q, k_scale,
                                         v_scale, out, placeholder, KVQ_NOALLOC_SCRATCH_BYTES, &a);
  if (st != KVQ_OK) return st;
  void* ws = nullptr;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  // the whole array may hold counters of some later configuration: clear all of it once
  const int32_t sst = kvq::device_scratch(KVQ_NOALLOC_SCRATCH_BYTES, hs, &ws);
  if (sst != KVQ_OK) return sst;
  a.workspace = static_cast<uint8_t*>(ws);
  const hipError_t e = kvq::launch_decode(a, hs);
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_DEVICE;
}
