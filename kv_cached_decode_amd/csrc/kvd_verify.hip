// Speculative verification epilogue on gfx950: row argmax over the
// vocabulary (lowest index among equal maxima), optionally after the logit
// filters, and the accepted length / corrected token of each batch row.
//
// Every (logit, token) pair is one 64-bit order key (larger logit first,
// equal logits lower token first), so an argmax is a max over keys.
// Workgroup (chunk, r, b) reads 2048 logits of row r, 4 per thread with every
// load issued first, and with the filters it reads the suppression bits of
// its tokens too (a suppressed logit counts as -inf). Each wavefront reduces
// its keys in lane exchanges; wavefront 0 takes the best of the eight,
// publishes it and counts the arrival. The last workgroup of batch row b
// gives each logits row to a wavefront (the row's chunk keys, up to 8 per
// lane, one more wavefront max) and scans the drafts with one ballot.
#include <limits.h>

#include "kvd_device.hpp"
#include "kvd_internal.hpp"
#include "kvd_select.hpp"

namespace kvd {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kItems = 4;                      // logits per thread
constexpr int kChunk = kThreads * kItems;      // logits per workgroup
constexpr int kChunkLane = kMaxVerifyChunks / 64;  // chunk keys per lane in the row merge

template <int DT, bool MASKED>
__global__ __launch_bounds__(kThreads) void verify_kernel(VerifyArgs a) {
  const int ch = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e0 = ch * kChunk;
  const char *row = static_cast<const char *>(a.logits) +
                    (size_t)(b * a.R + r) * a.V * Storage<DT>::bytes;
  float x[kItems];
  uint32_t sup[kItems];
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int e = e0 + q * kThreads + tid;
    x[q] = (e < a.V) ? load_logit<DT>(row, e) : 0.f;
    sup[q] = 0;
    if constexpr (MASKED) {
      if (e < a.V) {
        if (a.suppress) sup[q] = a.suppress[e >> 5];
        if (r == 0 && a.suppress_first) sup[q] |= a.suppress_first[e >> 5];
      }
    }
  }
  uint64_t best = 0;  // padding past V stays 0, below every real key
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int e = e0 + q * kThreads + tid;
    float v = x[q];
    if constexpr (MASKED) v = ((sup[q] >> (e & 31)) & 1u) ? -INFINITY : v;
    if (e < a.V) {
      const uint64_t k = value_key(v, e);
      best = k > best ? k : best;
    }
  }
  int owner;
  best = wave_max_key(best, owner);

  __shared__ uint64_t s_key[kWaves];
  __shared__ int s_am[64];
  __shared__ int s_last;
  if (lane == 0) s_key[wave] = best;
  __syncthreads();
  if (wave == 0) {
    uint64_t k = (lane < kWaves) ? s_key[lane] : 0;
    k = wave_max_key(k, owner);
    if (lane == 0) publish(a.ws_key + (size_t)(b * a.R + r) * a.chunks + ch, k);
    wait_stores();  // the key is in place before it counts
    if (lane == 0) s_last = (arrive(&a.ws_count[b * kCounterStride]) == (uint32_t)(a.R * a.chunks - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;

  // ---- last workgroup of batch row b: row rr on wavefront rr mod 8
  const int dr = (wave == 0 && lane < a.N) ? a.draft[b * a.N + lane] : 0;
  for (int rr = wave; rr < a.R; rr += kWaves) {
    const uint64_t *src = a.ws_key + (size_t)(b * a.R + rr) * a.chunks;
    uint64_t k[kChunkLane];
#pragma unroll
    for (int q = 0; q < kChunkLane; ++q) {
      const int c = lane + 64 * q;
      k[q] = (c < a.chunks) ? fetch_u64(src + c) : 0;
    }
    uint64_t m = k[0];
#pragma unroll
    for (int q = 1; q < kChunkLane; ++q) m = k[q] > m ? k[q] : m;
    m = wave_max_key(m, owner);
    const int am = (int)~(uint32_t)m;  // V >= 1: some chunk key is real
    if (lane == 0) {
      s_am[rr] = am;
      if (a.argmax_out) a.argmax_out[b * a.R + rr] = am;
    }
  }
  __syncthreads();
  if (wave == 0) {
    // accepted length: the first draft that differs from its row's argmax
    const uint64_t miss = __builtin_amdgcn_ballot_w64(lane < a.N && dr != s_am[lane]);
    const int acc = miss ? __builtin_ctzll(miss) : a.N;
    if (lane == 0) {
      a.accept_len[b] = acc;
      a.next_token[b] = (acc < a.R) ? s_am[acc] : -1;
      reset_counter(&a.ws_count[b * kCounterStride]);
    }
  }
}

template <int DT>
void launch_dt(const VerifyArgs &a, dim3 grid, hipStream_t s) {
  if (a.suppress || a.suppress_first)
    launch_kernel(verify_kernel<DT, true>, grid, dim3(kThreads), s, a);
  else
    launch_kernel(verify_kernel<DT, false>, grid, dim3(kThreads), s, a);
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
    case F32: launch_dt<F32>(a, grid, s); break;
    case F16: launch_dt<F16>(a, grid, s); break;
    default: launch_dt<BF16>(a, grid, s); break;
  }
  return hipGetLastError();
}

}  // namespace kvd
