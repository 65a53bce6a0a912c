// decode_step_self_static: decode_step_self with the split-merge workspace
// in a file-scope device array instead of a caller's buffer, for callers that
// cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid allocation). It runs the same validation,
// plans and kernels as decode_step_self, so its results are the same bit for
// bit; nothing here allocates.
//
// The array holds kScratchBytes: the arrival-counter block (which must be
// zero at rest; the kernels reset every counter they use) and the per-split
// partials. Each GPU the library runs on holds its own copy until the
// process ends. Host code never passes the array's name to a kernel (in host
// code that name is a host-side stand-in, not a device address): the
// device address is taken once per device with hipGetSymbolAddress, with that
// device current, and only that address is used. The first call on a device
// clears the counter block with a fill kernel on the caller's stream.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvd_internal.hpp"
#include "kvdecode.h"

namespace {

constexpr size_t kScratchBytes = (size_t)4 << 20;  // counters (512 KiB), then partials
constexpr size_t kCounterWords = (size_t)kvd::kMaxCounters * kvd::kCounterStride;
static_assert(kCounterWords * sizeof(uint32_t) < kScratchBytes, "counters fit the scratch");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct DeviceScratch {
  void *ptr = nullptr;                // device address of `scratch` on this device
  bool cleared = false;               // counter block cleared by an eager call's fill
  unsigned long long capture = 0;     // the stream capture that last recorded a fill
};
std::mutex g_lock;
DeviceScratch g_dev[kMaxDevices];

__global__ __launch_bounds__(256) void clear_counters(uint32_t *p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// The calling thread's current device's scratch address (looked up once).
int device_scratch(DeviceScratch *&slot) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVD_ERR_LAUNCH;
  std::lock_guard<std::mutex> hold(g_lock);
  DeviceScratch &d = g_dev[dev];
  if (!d.ptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVD_ERR_LAUNCH;
    d.ptr = p;
  }
  slot = &d;
  return KVD_OK;
}

}  // namespace

extern "C" {

int decode_step_self_static(const void *q, const void *k_new, const void *v_new, int32_t Hq,
                            int32_t N, const kvd_cache *cache, int32_t len, float scale,
                            float rope_base, float *out, void *stream) {
  DeviceScratch *d = nullptr;
  int st = device_scratch(d);
  if (st) return st;
  // every check first (nothing is enqueued when one fails)
  st = kvd::step_self(q, k_new, v_new, Hq, N, cache, len, scale, rope_base, out, d->ptr,
                      kScratchBytes, stream, true);
  if (st == KVD_ERR_WORKSPACE) return KVD_ERR_SCRATCH;
  if (st) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  {
    // the counter block is cleared once: by the first eager call, or, in a
    // stream capture before that, once in each captured graph (a fill kernel,
    // not a memset, so that replays clear it too)
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    unsigned long long cap = 0;
    if (hipStreamGetCaptureInfo(s, &cs, &cap) != hipSuccess) return KVD_ERR_LAUNCH;
    const bool capturing = cs == hipStreamCaptureStatusActive;
    std::lock_guard<std::mutex> hold(g_lock);
    if (!d->cleared && !(capturing && d->capture == cap)) {
      clear_counters<<<dim3(512), dim3(256), 0, s>>>(static_cast<uint32_t *>(d->ptr),
                                                      kCounterWords);
      if (hipGetLastError() != hipSuccess) return KVD_ERR_LAUNCH;
      if (capturing) d->capture = cap;
      else d->cleared = true;
    }
  }
  return kvd::step_self(q, k_new, v_new, Hq, N, cache, len, scale, rope_base, out, d->ptr,
                        kScratchBytes, stream, false);
}

size_t kvd_static_scratch_bytes(void) { return kScratchBytes; }

}  // extern "C"
