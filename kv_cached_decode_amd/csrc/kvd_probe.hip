// Streaming-read probe: the attainable rate of a plain read of a given number
// of bytes in one launch on this GPU, to price the attention kernels against
// (they read their K/V once, in one launch per layer).
//
// Every thread keeps four 16-byte loads in flight per round (grid-stride over
// the buffer) and folds what it read into one word; the fold is stored only
// if it equals a value no input makes likely, so the loads stay live and the
// kernel writes (almost) nothing.
#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kMaxBlocks = 4096;

__global__ __launch_bounds__(kThreads) void read_kernel(ProbeArgs a) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  for (int part = 0; part < 2; ++part) {
    const u32x4 *src = static_cast<const u32x4 *>(part == 0 ? a.a : a.b);
    if (!src) continue;
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < a.vecs; i += kUnroll * stride) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < a.vecs; i += stride) {
      const u32x4 v = src[i];
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  if (acc == 0x9e3779b9u) *a.sink = acc;
}

}  // namespace

hipError_t launch_probe(const ProbeArgs &a, hipStream_t s) {
  const size_t per_block = (size_t)kThreads * kUnroll;
  size_t blocks = (a.vecs + per_block - 1) / per_block;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  if (blocks < 1) blocks = 1;
  launch_kernel(read_kernel, dim3((unsigned)blocks), dim3(kThreads), s, a);
  return hipGetLastError();
}

}  // namespace kvd
