// attn_decode_noalloc: attn_decode for callers that cannot allocate (code
// under HIP graph capture, serving loops and harnesses that forbid
// hipMalloc). The per-split partial results that attn_decode keeps in the
// caller's workspace go to a static device array of this library instead.
// Each GPU the library runs on holds its own copy of the array until the
// process ends. Calls on one GPU share it, so calls that overlap on one GPU
// (different streams, or several threads) race; the partials need no
// clearing, because every split a call merges is written by that call.
#include <mutex>

#include "../../include/hgqa.h"
#include "hgqa_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB per GPU

// In host code this name is a stand-in, not a device address: the kernels
// get the address that hipGetSymbolAddress returns for the GPU they run on.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of the stream's GPU copy of `scratch`, looked up once per
// GPU with that GPU current.
hipError_t scratch_address(hipStream_t stream, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int attn_decode_noalloc(const hgqa_layer* layer, int32_t batch, const void* q,
                                   const void* gate, const void* k_cache, const void* v_cache,
                                   int32_t cache_capacity, const int32_t* seq_lens,
                                   int32_t max_seq_len, void* out, void* stream) {
  return hgqa::decode_call(layer, batch, q, gate, k_cache, v_cache, cache_capacity, seq_lens,
                           max_seq_len, nullptr, 0, out, stream, &scratch_address, kScratchBytes);
}
