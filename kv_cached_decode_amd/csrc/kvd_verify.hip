// Speculative verification epilogue on gfx950: row argmax over the
// vocabulary (lowest index among equal maxima) and the accepted length /
// corrected token of each batch row.
//
// Workgroup (chunk, r, b) reduces 4096 logits of row r to a (value, index)
// pair: every thread issues all 16 of its loads before comparing, then the
// pairs are reduced across the wavefront and the workgroup. The last
// workgroup of batch row b to arrive stages every pair of that row in LDS
// (all loads in flight at once), reduces each logits row in chunk order, and
// scans the drafts for the first mismatch.
#include <limits.h>

#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {

namespace {

constexpr int kThreads = 256;
constexpr int kItems = 16;                 // logits per thread
constexpr int kChunk = kThreads * kItems;  // logits per workgroup
constexpr int kStageIters = kMaxVerifyPartials / kThreads;

template <int DT>
__device__ __forceinline__ float load_logit(const char *row, int e) {
  if constexpr (DT == F32) return reinterpret_cast<const float *>(row)[e];
  else if constexpr (DT == F16) return (float)reinterpret_cast<const _Float16 *>(row)[e];
  else return __builtin_bit_cast(float, (uint32_t)reinterpret_cast<const uint16_t *>(row)[e] << 16);
}

// (v, i) beats (bv, bi): larger value, or equal value and lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void verify_kernel(VerifyArgs a) {
  const int ch = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int e0 = ch * kChunk;
  const char *row = static_cast<const char *>(a.logits) +
                    (size_t)(b * a.R + r) * a.V * Storage<DT>::bytes;
  float x[kItems];
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int e = e0 + j * kThreads + tid;
    x[j] = (e < a.V) ? load_logit<DT>(row, e) : 0.f;
  }
  float best = -INFINITY;
  int bi = INT_MAX;
#pragma unroll
  for (int j = 0; j < kItems; ++j) {  // ascending index within the thread
    const int e = e0 + j * kThreads + tid;
    if (e < a.V && better(x[j], e, best, bi)) {
      best = x[j];
      bi = e;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(best, off);
    const int oi = __shfl_xor(bi, off);
    if (better(ov, oi, best, bi)) {
      best = ov;
      bi = oi;
    }
  }
  __shared__ float sv[kMaxVerifyPartials];
  __shared__ int si[kMaxVerifyPartials];
  __shared__ int s_am[64];
  __shared__ int s_draft[64];
  __shared__ int s_last;
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kThreads / 64; ++w)
      if (better(sv[w], si[w], best, bi)) {
        best = sv[w];
        bi = si[w];
      }
    const size_t slot = (size_t)(b * a.R + r) * a.chunks + ch;
    publish(a.ws_val + slot, best);
    publish(a.ws_idx + slot, bi);
    wait_stores();
    s_last = (arrive(&a.ws_count[b]) == (uint32_t)(a.R * a.chunks - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;

  // stage this batch row's pairs (and its drafts) in LDS, every load at once
  const int n = a.R * a.chunks;
  const size_t base = (size_t)b * a.R * a.chunks;
  float pv[kStageIters];
  int pi[kStageIters];
#pragma unroll
  for (int j = 0; j < kStageIters; ++j) {
    const int i = tid + j * kThreads;
    if (i < n) {
      pv[j] = __builtin_bit_cast(float, fetch_u32(a.ws_val + base + i));
      pi[j] = (int)fetch_u32(a.ws_idx + base + i);
    }
  }
  const int dr = (tid < a.N) ? a.draft[b * a.N + tid] : 0;
#pragma unroll
  for (int j = 0; j < kStageIters; ++j) {
    const int i = tid + j * kThreads;
    if (i < n) {
      sv[i] = pv[j];
      si[i] = pi[j];
    }
  }
  if (tid < a.N) s_draft[tid] = dr;
  __syncthreads();
  if (tid < a.R) {
    float bv = -INFINITY;
    int bix = INT_MAX;
    for (int c = 0; c < a.chunks; ++c) {
      const float v = sv[tid * a.chunks + c];
      const int ix = si[tid * a.chunks + c];
      if (better(v, ix, bv, bix)) {
        bv = v;
        bix = ix;
      }
    }
    if (bix == INT_MAX) bix = 0;  // only reachable with NaN rows
    s_am[tid] = bix;
    if (a.argmax_out) a.argmax_out[b * a.R + tid] = bix;
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    while (acc < a.N && s_draft[acc] == s_am[acc]) ++acc;
    a.accept_len[b] = acc;
    a.next_token[b] = (acc < a.R) ? s_am[acc] : -1;
    reset_counter(&a.ws_count[b]);
  }
}

}  // namespace

void plan_verify(int B, int R, int V, int &chunk, int &chunks) {
  (void)B;
  (void)R;
  chunk = kChunk;
  chunks = (V + kChunk - 1) / kChunk;
}

hipError_t launch_verify(const VerifyArgs &a, hipStream_t s) {
  const dim3 grid(a.chunks, a.R, a.B);
  switch (a.dtype) {
    case F32: launch_kernel(verify_kernel<F32>, grid, dim3(kThreads), s, a); break;
    case F16: launch_kernel(verify_kernel<F16>, grid, dim3(kThreads), s, a); break;
    default: launch_kernel(verify_kernel<BF16>, grid, dim3(kThreads), s, a); break;
  }
  return hipGetLastError();
}

}  // namespace kvd
