// Streaming-read probe: the attainable rate of a plain read of a given number
// of bytes in one launch on this GPU, to price the attention kernels against
// (they read their K/V once, in one launch per layer).
//
// The two buffers are read as one sequence of 16-byte vectors (a's, then
// b's). Every thread keeps U loads in flight per round (grid-stride over the
// sequence) and folds what it read into one word; the fold is stored only if
// it equals a value no input makes likely, so the loads stay live and the
// kernel writes (almost) nothing. U and the grid are parameters, so the
// yardstick can be the best of several shapes.
#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 65535;

template <int U>
__global__ __launch_bounds__(kThreads) void read_kernel(ProbeArgs a) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  const size_t total = a.b ? 2 * a.vecs : a.vecs;
  const u32x4 *pa = static_cast<const u32x4 *>(a.a);
  // b's vectors are indexed from vecs on
  const u32x4 *pb = a.b ? static_cast<const u32x4 *>(a.b) - a.vecs : pa;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (U - 1) * stride < total; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + u * stride;
      v[u] = (j < a.vecs ? pa : pb)[j];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < total; i += stride) {
    const u32x4 v = (i < a.vecs ? pa : pb)[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) *a.sink = acc;
}

}  // namespace

int probe_unroll_ok(int u) { return u == 1 || u == 2 || u == 4 || u == 8 || u == 16; }

hipError_t launch_probe(const ProbeArgs &a, hipStream_t s) {
  const size_t total = a.b ? 2 * a.vecs : a.vecs;
  size_t blocks = a.blocks;
  if (blocks == 0) {  // one round: every thread issues its U loads once
    const size_t per_block = (size_t)kThreads * a.unroll;
    blocks = (total + per_block - 1) / per_block;
  }
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks), block(kThreads);
  switch (a.unroll) {
    case 1: launch_kernel(read_kernel<1>, grid, block, s, a); break;
    case 2: launch_kernel(read_kernel<2>, grid, block, s, a); break;
    case 8: launch_kernel(read_kernel<8>, grid, block, s, a); break;
    case 16: launch_kernel(read_kernel<16>, grid, block, s, a); break;
    default: launch_kernel(read_kernel<4>, grid, block, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace kvd
