// Beam-search candidate scoring on gfx950: for each audio row, the K beams'
// logits rows give log-probabilities, each beam's K + 1 best tokens, the
// K (K + 1) candidate scores, and the next K beams (parent, token, score) with
// the end-of-text candidates met on the way recorded as finished. Follows the
// update steps of the beam-search decoder on "Whisper のデコーダー内部：Beam
// Search、Logit フィルター、KV キャッシュ" (the step after them, reordering the
// cache, is kv_reorder).
//
// Orders are taken on 64-bit keys whose unsigned order is the order wanted:
// (logit, token) pairs and candidates become one integer each, so a selection
// step is a max over the wavefront in lane exchanges (DPP and permlane swaps)
// with no LDS round trip and no barrier.
//
// Workgroup (chunk, beam, row) reads 2048 logits (4 per thread) and publishes
// a record: the chunk's max, its sum of exp(x - max), and its K + 1 best keys.
// Each wavefront finds its own K + 1 best in K + 1 rounds (each lane sorts its
// keys once; the lane holding a round's winner shifts its list); wavefront 0
// merges the eight lists the same way. The last workgroup of the audio row to arrive gives each
// beam to a wavefront: log-sum-exp over the chunk records, then the beam's
// K + 1 best out of every chunk's entries, again in rounds. The K (K + 1)
// candidates are then placed in parallel: a candidate's position in the walk
// is the number of candidates ranked before it, and the end-of-text ones among
// them fix whether the walk reaches it and which output slot it takes.
#include <limits.h>
#include <math.h>

#include "kvd_device.hpp"
#include "kvd_internal.hpp"
#include "kvd_select.hpp"

namespace kvd {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kItems = 4;
constexpr int kChunk = kThreads * kItems;
constexpr int kMaxKP = kMaxBeamWidth + 1;
constexpr int kTopLane = (kWaves * kMaxKP + 63) / 64;       // wave lists merged per lane
constexpr int kEntLane = kMaxBeamEntries / 64;              // chunk entries per lane
constexpr int kChunkLane = (kMaxBeamEntries / 2 + 63) / 64;  // chunk records per lane (K >= 1)
constexpr int kMaxCand = kMaxBeamWidth * kMaxKP;
constexpr uint32_t kTokBits = 23;                            // tokens < 2^23 (V <= 2048 * 256)
static_assert(kMaxCand <= kThreads, "one thread per candidate");
static_assert((kMaxCand - 1) < (1 << (32 - kTokBits)), "candidate number fits its field");

// Candidate t = beam * (K + 1) + rank with token tok: larger score first,
// equal scores smaller t first; the token rides in the low bits.
__device__ __forceinline__ uint64_t cand_key(float score, int t, int tok) {
  return ((uint64_t)order_bits(score) << 32) |
         ((uint32_t)(kMaxCand - 1 - t) << kTokBits) | (uint32_t)tok;
}
__device__ __forceinline__ int cand_token(uint64_t k) { return (int)(k & ((1u << kTokBits) - 1)); }

template <int DT>
__global__ __launch_bounds__(kThreads) void beam_kernel(BeamArgs a) {
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, KP = a.K + 1;
  const int e0 = c * kChunk;
  const char *row = static_cast<const char *>(a.logits) +
                    (size_t)(b * K + j) * a.V * Storage<DT>::bytes;
  float x[kItems];
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int e = e0 + q * kThreads + tid;
    x[q] = (e < a.V) ? load_logit<DT>(row, e) : -INFINITY;
  }

  __shared__ float s_max[kWaves], s_sum[kWaves];
  __shared__ uint64_t s_top[kWaves * kMaxKP];
  __shared__ int s_last;

  // ---- chunk max, then the sum of exp(x - max) (a chunk of -inf sums to 0)
  float mx = x[0];
#pragma unroll
  for (int q = 1; q < kItems; ++q) mx = fmaxf(mx, x[q]);
  mx = groups_max<1>(mx);
  if (lane == 0) s_max[wave] = mx;
  uint64_t k[kItems];
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int e = e0 + q * kThreads + tid;
    k[q] = (e < a.V) ? value_key(x[q], e) : 0;
  }
  __syncthreads();
  float cmax = s_max[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) cmax = fmaxf(cmax, s_max[w]);
  const float ref = (cmax == -INFINITY) ? 0.f : cmax;
  float se = 0.f;
#pragma unroll
  for (int q = 0; q < kItems; ++q) se += expf(x[q] - ref);  // padding is -inf: adds 0
  se = groups_sum<1>(se);
  if (lane == 0) s_sum[wave] = se;

  // ---- each wavefront's K + 1 best, then wavefront 0 merges the lists
  const uint64_t top = wave_top(k, KP, lane);
  if (lane < KP) s_top[wave * KP + lane] = top;
  __syncthreads();
  if (wave == 0) {
    uint64_t m[kTopLane];
#pragma unroll
    for (int q = 0; q < kTopLane; ++q) {
      const int t = lane + 64 * q;
      m[q] = (t < kWaves * KP) ? s_top[t] : 0;
    }
    float csum = s_sum[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) csum += s_sum[w];
    const uint64_t best = wave_top(m, KP, lane);
    uint32_t *rec = a.ws_rec + ((size_t)(b * K + j) * a.chunks + c) * kBeamRec;
    if (lane == 0) publish(reinterpret_cast<float *>(rec), cmax);
    if (lane == 1) publish(reinterpret_cast<float *>(rec) + 1, csum);
    if (lane < KP) publish(reinterpret_cast<uint64_t *>(rec + 2) + lane, best);
    wait_stores();  // the wavefront's record is in place before it counts
    if (lane == 0)
      s_last = (arrive(&a.ws_count[b * kCounterStride]) == (uint32_t)(K * a.chunks - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;

  // ---- last workgroup of audio row b: beam bj on wavefront bj mod 8
  __shared__ __align__(16) uint64_t s_cand[kMaxCand + 7];
  __shared__ __align__(16) uint64_t s_eot[kMaxBeamWidth];
  __shared__ int s_nf;
  if (tid == 0) s_nf = 0;
  const int E = a.chunks * KP;
  for (int bj = wave; bj < K; bj += kWaves) {
    const uint32_t *br = a.ws_rec + (size_t)(b * K + bj) * a.chunks * kBeamRec;
    uint64_t ent[kEntLane];
#pragma unroll
    for (int q = 0; q < kEntLane; ++q) {
      const int e = lane + 64 * q;
      ent[q] = (e < E) ? fetch_u64(br + (e / KP) * kBeamRec + 2 + 2 * (e % KP)) : 0;
    }
    float cm[kChunkLane], cs[kChunkLane];
#pragma unroll
    for (int q = 0; q < kChunkLane; ++q) {
      const int cc = lane + 64 * q;
      const bool in = cc < a.chunks;
      cm[q] = in ? __builtin_bit_cast(float, fetch_u32(br + cc * kBeamRec)) : -INFINITY;
      cs[q] = in ? __builtin_bit_cast(float, fetch_u32(br + cc * kBeamRec + 1)) : 0.f;
    }
    const float sl = a.sum_logprobs[b * K + bj];
    float M = cm[0];
#pragma unroll
    for (int q = 1; q < kChunkLane; ++q) M = fmaxf(M, cm[q]);
    M = groups_max<1>(M);  // finite: the row has a finite maximum
    float S = 0.f;
#pragma unroll
    for (int q = 0; q < kChunkLane; ++q) S += cs[q] * expf(cm[q] - M);
    S = groups_sum<1>(S);
    const float lse = M + logf(S);
    const uint64_t best = wave_top(ent, KP, lane);
    const int tok = (int)~(uint32_t)best;
    uint64_t ck = 0;
    if (lane < KP) {
      const float v = order_value((uint32_t)(best >> 32));
      const int t = bj * KP + lane;
      ck = cand_key(sl + (v - lse), t, tok);
      s_cand[t] = ck;
    }
    // a beam's tokens are distinct: at most one of its candidates is end-of-text
    const uint64_t is_eot = __builtin_amdgcn_ballot_w64(lane < KP && tok == a.eot);
    if (lane == (is_eot ? __builtin_ctzll(is_eot) : 0)) s_eot[bj] = is_eot ? ck : 0;
  }
  if (tid < 7) s_cand[K * KP + tid] = 0;                   // pad to whole blocks of 8
  if (tid >= K && tid < kMaxBeamWidth) s_eot[tid] = 0;
  __syncthreads();

  // ---- the walk, in parallel: candidate t ranks after `rank` others, `eots`
  // of them end-of-text. The walk reaches it while fewer than K others were
  // kept; end-of-text then goes to finished slot `eots`, any other token to
  // next-beam slot rank - eots.
  const int nc = K * KP;
  if (tid < nc) {
    const uint64_t me = s_cand[tid];
    int rank = 0, eots = 0;
    for (int u = 0; u < nc; u += 8) {  // 0 (the pad) ranks after every candidate
#pragma unroll
      for (int v = 0; v < 8; ++v) rank += (s_cand[u + v] > me) ? 1 : 0;
    }
#pragma unroll
    for (int bj = 0; bj < kMaxBeamWidth; ++bj) eots += (s_eot[bj] > me) ? 1 : 0;
    const int kept = rank - eots;
    if (kept < K) {
      const int beam = tid / KP, tok = cand_token(me);
      const float sc = order_value((uint32_t)(me >> 32));
      if (tok == a.eot) {
        a.fin_parent[b * K + eots] = beam;
        a.fin_score[b * K + eots] = sc;
        atomicAdd(&s_nf, 1);
      } else {
        a.parent[b * K + kept] = beam;
        a.token[b * K + kept] = tok;
        a.score[b * K + kept] = sc;
      }
    }
  }
  __syncthreads();
  const int nf = s_nf;
  if (tid >= nf && tid < K) {
    a.fin_parent[b * K + tid] = -1;
    a.fin_score[b * K + tid] = __builtin_nanf("");
  }
  if (tid == 0) {
    a.fin_count[b] = nf;
    reset_counter(&a.ws_count[b * kCounterStride]);
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
