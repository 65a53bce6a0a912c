// Beam-search candidate scoring on gfx950: for each audio row, the K beams'
// logits rows give log-probabilities, each beam's K + 1 best tokens, the
// K (K + 1) candidate scores, and the next K beams (parent, token, score) with
// the end-of-text candidates met on the way recorded as finished. Follows the
// update steps of the beam-search decoder on "Whisper のデコーダー内部：Beam
// Search、Logit フィルター、KV キャッシュ" (the step after them, reordering the
// cache, is kv_reorder).
//
// Workgroup (chunk, beam, row) reads 4096 logits (16 per thread, all loads
// issued first) and publishes a record: the chunk's max, its sum of
// exp(x - max), and its K + 1 best (value, index) pairs, found in K + 1
// rounds of a (value, index) argmax in which the owner of each round's winner
// drops it. The last workgroup of the audio row to arrive stages every record
// in LDS, combines the chunks of each beam (log-sum-exp and the K + 1 best),
// ranks the candidates in parallel and walks them in order.
#include <limits.h>
#include <math.h>

#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {

namespace {

constexpr int kThreads = 256;
constexpr int kItems = 16;
constexpr int kChunk = kThreads * kItems;
constexpr int kStageIters = kMaxBeamWords / kThreads;
constexpr int kMaxCand = kMaxBeamWidth * (kMaxBeamWidth + 1);

template <int DT>
__device__ __forceinline__ float load_logit(const char *row, int e) {
  if constexpr (DT == F32) return reinterpret_cast<const float *>(row)[e];
  else if constexpr (DT == F16) return (float)reinterpret_cast<const _Float16 *>(row)[e];
  else return __builtin_bit_cast(float, (uint32_t)reinterpret_cast<const uint16_t *>(row)[e] << 16);
}

// (v, i) ranks before (bv, bi): larger value, or equal value and lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void beam_kernel(BeamArgs a) {
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, KP = a.K + 1;
  const int e0 = c * kChunk;
  const char *row = static_cast<const char *>(a.logits) +
                    (size_t)(b * K + j) * a.V * Storage<DT>::bytes;
  float x[kItems];
  uint32_t avail = 0;  // bit jj: element e0 + jj * kThreads + tid exists and is not taken
#pragma unroll
  for (int jj = 0; jj < kItems; ++jj) {
    const int e = e0 + jj * kThreads + tid;
    x[jj] = -INFINITY;
    if (e < a.V) {
      x[jj] = load_logit<DT>(row, e);
      avail |= 1u << jj;
    }
  }

  __shared__ float s_f[4];
  __shared__ int s_i[4];
  __shared__ float s_tv[kMaxBeamWidth + 1];
  __shared__ int s_ti[kMaxBeamWidth + 1];
  __shared__ int s_last;

  // ---- chunk max and sum of exp(x - max)
  float mx = -INFINITY;
#pragma unroll
  for (int jj = 0; jj < kItems; ++jj) mx = fmaxf(mx, x[jj]);
  mx = groups_max<1>(mx);
  if (lane == 0) s_f[wave] = mx;
  __syncthreads();
  const float cmax = fmaxf(fmaxf(s_f[0], s_f[1]), fmaxf(s_f[2], s_f[3]));
  __syncthreads();
  float se = 0.f;
#pragma unroll
  for (int jj = 0; jj < kItems; ++jj)
    if (avail & (1u << jj)) se += expf(x[jj] - cmax);
  se = groups_sum<1>(se);
  if (lane == 0) s_f[wave] = se;
  __syncthreads();
  const float csum = (s_f[0] + s_f[1]) + (s_f[2] + s_f[3]);

  // ---- the chunk's K + 1 best (value, index), one argmax round each
  for (int r = 0; r < KP; ++r) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int jj = 0; jj < kItems; ++jj) {  // ascending index within the thread
      const int e = e0 + jj * kThreads + tid;
      if ((avail & (1u << jj)) && better(x[jj], e, bv, bi)) {
        bv = x[jj];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    __syncthreads();  // the previous round's readers are done with s_f / s_i
    if (lane == 0) {
      s_f[wave] = bv;
      s_i[wave] = bi;
    }
    __syncthreads();
    bv = s_f[0];
    bi = s_i[0];
    for (int w = 1; w < 4; ++w)
      if (better(s_f[w], s_i[w], bv, bi)) {
        bv = s_f[w];
        bi = s_i[w];
      }
    if (tid == 0) {
      s_tv[r] = bv;
      s_ti[r] = bi;
    }
    if (bi != INT_MAX && ((bi - e0) & (kThreads - 1)) == tid)  // its owner drops it
      avail &= ~(1u << ((bi - e0) / kThreads));
  }
  __syncthreads();

  // ---- publish the record, count the arrival
  uint32_t *rec = a.ws_rec + ((size_t)(b * K + j) * a.chunks + c) * kBeamRec;
  if (tid == 0) publish(reinterpret_cast<float *>(rec), cmax);
  if (tid == 1) publish(reinterpret_cast<float *>(rec) + 1, csum);
  if (tid < KP) {
    publish(reinterpret_cast<float *>(rec) + 2 + 2 * tid, s_tv[tid]);
    publish(reinterpret_cast<int32_t *>(rec) + 3 + 2 * tid, s_ti[tid]);
  }
  wait_stores();
  __syncthreads();
  if (tid == 0) s_last = (arrive(&a.ws_count[b]) == (uint32_t)(K * a.chunks - 1)) ? 1 : 0;
  __syncthreads();
  if (!s_last) return;

  // ---- last workgroup of audio row b: stage every record (all loads in
  // flight), then merge
  __shared__ uint32_t s_rec[kMaxBeamWords];
  __shared__ float s_cs[kMaxCand];
  __shared__ int s_ct[kMaxCand];
  __shared__ int s_order[kMaxCand];
  const int n = K * a.chunks * kBeamRec;
  const uint32_t *src = a.ws_rec + (size_t)b * K * a.chunks * kBeamRec;
  uint32_t st[kStageIters];
#pragma unroll
  for (int it = 0; it < kStageIters; ++it) {
    const int i = tid + it * kThreads;
    if (i < n) st[it] = fetch_u32(src + i);
  }
#pragma unroll
  for (int it = 0; it < kStageIters; ++it) {
    const int i = tid + it * kThreads;
    if (i < n) s_rec[i] = st[it];
  }
  __syncthreads();

  if (tid < K) {  // beam tid: log-sum-exp over chunks, then its K + 1 best tokens
    const uint32_t *br = s_rec + (size_t)tid * a.chunks * kBeamRec;
    float M = -INFINITY;
    for (int cc = 0; cc < a.chunks; ++cc) M = fmaxf(M, __builtin_bit_cast(float, br[cc * kBeamRec]));
    float S = 0.f;
    for (int cc = 0; cc < a.chunks; ++cc) {
      const float cm = __builtin_bit_cast(float, br[cc * kBeamRec]);
      S += __builtin_bit_cast(float, br[cc * kBeamRec + 1]) * expf(cm - M);
    }
    const float lse = M + logf(S);
    const float base = a.sum_logprobs[b * K + tid];
    // round r takes the best entry ranked after round r - 1's (entries are
    // distinct tokens, so the order is strict)
    float pv = INFINITY;
    int pi = -1;
    for (int r = 0; r < KP; ++r) {
      float bv = -INFINITY;
      int bi = INT_MAX;
      for (int cc = 0; cc < a.chunks; ++cc) {
        for (int q = 0; q < KP; ++q) {
          const float v = __builtin_bit_cast(float, br[cc * kBeamRec + 2 + 2 * q]);
          const int i = (int)br[cc * kBeamRec + 3 + 2 * q];
          if (i == INT_MAX) continue;  // chunk had fewer than K + 1 elements
          if (better(pv, pi, v, i) && better(v, i, bv, bi)) {
            bv = v;
            bi = i;
          }
        }
      }
      s_cs[tid * KP + r] = base + (bv - lse);
      s_ct[tid * KP + r] = bi;
      pv = bv;
      pi = bi;
    }
  }
  __syncthreads();

  // ---- rank the K (K + 1) candidates: larger score first, equal scores in
  // the order beam, then rank (the candidate's number)
  const int nc = K * KP;
  for (int t = tid; t < nc; t += kThreads) {
    const float sc = s_cs[t];
    int rank = 0;
    for (int u = 0; u < nc; ++u) {
      const float su = s_cs[u];
      rank += (su > sc || (su == sc && u < t)) ? 1 : 0;
    }
    s_order[rank] = t;
  }
  __syncthreads();

  if (tid == 0) {
    int kept = 0, nf = 0;
    for (int i = 0; i < nc && kept < K; ++i) {
      const int t = s_order[i];
      const int beam = t / KP, tok = s_ct[t];
      if (tok == a.eot) {
        a.fin_parent[b * K + nf] = beam;
        a.fin_score[b * K + nf] = s_cs[t];
        ++nf;
      } else {
        a.parent[b * K + kept] = beam;
        a.token[b * K + kept] = tok;
        a.score[b * K + kept] = s_cs[t];
        ++kept;
      }
    }
    for (int i = nf; i < K; ++i) {
      a.fin_parent[b * K + i] = -1;
      a.fin_score[b * K + i] = __builtin_nanf("");
    }
    a.fin_count[b] = nf;
    reset_counter(&a.ws_count[b]);
  }
}

}  // namespace

int beam_chunks(int V) { return (V + kChunk - 1) / kChunk; }

hipError_t launch_beam(const BeamArgs &a, hipStream_t s) {
  const dim3 grid(a.chunks, a.K, a.B);
  switch (a.dtype) {
    case F32: launch_kernel(beam_kernel<F32>, grid, dim3(kThreads), s, a); break;
    case F16: launch_kernel(beam_kernel<F16>, grid, dim3(kThreads), s, a); break;
    default: launch_kernel(beam_kernel<BF16>, grid, dim3(kThreads), s, a); break;
  }
  return hipGetLastError();
}

}  // namespace kvd
