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

template <int DT>
__device__ __forceinline__ float load_logit(const char *row, int e) {
  if constexpr (DT == F32) return reinterpret_cast<const float *>(row)[e];
  else if constexpr (DT == F16) return (float)reinterpret_cast<const _Float16 *>(row)[e];
  else return __builtin_bit_cast(float, (uint32_t)reinterpret_cast<const uint16_t *>(row)[e] << 16);
}

// Unsigned integers that compare as the floats do (-0 taken as +0; NaN is
// outside the contract), and back.
__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_value(uint32_t k) {
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// (logit, token): larger logit first, equal logits lower token first. Every
// such key is nonzero; 0 stands for "none" and ranks last.
__device__ __forceinline__ uint64_t entry_key(float v, int tok) {
  return ((uint64_t)order_bits(v) << 32) | (uint32_t)~tok;
}
// Candidate t = beam * (K + 1) + rank with token tok: larger score first,
// equal scores smaller t first; the token rides in the low bits.
__device__ __forceinline__ uint64_t cand_key(float score, int t, int tok) {
  return ((uint64_t)order_bits(score) << 32) |
         ((uint32_t)(kMaxCand - 1 - t) << kTokBits) | (uint32_t)tok;
}
__device__ __forceinline__ int cand_token(uint64_t k) { return (int)(k & ((1u << kTokBits) - 1)); }

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
// Unsigned max over the wavefront; every lane ends with it. (permlane swaps
// with both operands x leave {x[lane], x[lane ^ 16]} (resp. ^ 32) in the two
// results, and max is symmetric.)
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
  x = umax(x, dpp_u32<kDppQuadXor1>(x));
  x = umax(x, dpp_u32<kDppQuadXor2>(x));
  x = umax(x, dpp_u32<kDppHalfMirror>(x));
  x = umax(x, dpp_u32<kDppRowRor8>(x));
  const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = umax((uint32_t)r16[0], (uint32_t)r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return umax((uint32_t)r32[0], (uint32_t)r32[1]);
}

// Sorting networks (larger first) for the few keys one lane holds.
__device__ __forceinline__ void order2(uint64_t &x, uint64_t &y) {
  const uint64_t hi = x > y ? x : y, lo = x > y ? y : x;
  x = hi;
  y = lo;
}
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&k)[N]) {
  static_assert(N == 3 || N == 4 || N == 8, "sorting network sizes");
  if constexpr (N == 3) {
    order2(k[0], k[1]); order2(k[0], k[2]); order2(k[1], k[2]);
  } else if constexpr (N == 4) {
    order2(k[0], k[1]); order2(k[2], k[3]); order2(k[0], k[2]); order2(k[1], k[3]);
    order2(k[1], k[2]);
  } else {  // Batcher's odd-even merge sort, 19 comparators
    order2(k[0], k[1]); order2(k[2], k[3]); order2(k[4], k[5]); order2(k[6], k[7]);
    order2(k[0], k[2]); order2(k[1], k[3]); order2(k[4], k[6]); order2(k[5], k[7]);
    order2(k[1], k[2]); order2(k[5], k[6]);
    order2(k[0], k[4]); order2(k[1], k[5]); order2(k[2], k[6]); order2(k[3], k[7]);
    order2(k[2], k[4]); order2(k[3], k[5]);
    order2(k[1], k[2]); order2(k[3], k[4]); order2(k[5], k[6]);
  }
}

// The wavefront's n best keys among the N keys each lane holds (0 = none;
// real keys are distinct): lane r (r < n) returns the r-th. With each lane's
// keys sorted, a round reduces the high words (the value) over the wavefront;
// when one lane holds that value its low word is read from it, otherwise a
// second reduction over the tied lanes' low words decides. The lane holding
// the winner then shifts its list.
template <int N>
__device__ __forceinline__ uint64_t wave_top(uint64_t (&k)[N], int n, int lane) {
  sort_desc(k);
  uint64_t mine = 0;
  for (int r = 0; r < n; ++r) {
    const uint32_t hi = (uint32_t)(k[0] >> 32), lo = (uint32_t)k[0];
    const uint32_t whi = wave_umax(hi);
    const uint64_t tied = __builtin_amdgcn_ballot_w64(hi == whi);
    uint32_t wlo;
    int owner;
    if (__builtin_popcountll(tied) == 1) {
      owner = __builtin_ctzll(tied);
      wlo = (uint32_t)__builtin_amdgcn_readlane((int)lo, owner);
    } else {
      wlo = wave_umax(hi == whi ? lo : 0u);
      owner = __builtin_ctzll(__builtin_amdgcn_ballot_w64(hi == whi && lo == wlo));
    }
    if (lane == r) mine = ((uint64_t)whi << 32) | wlo;
    if (lane == owner) {
#pragma unroll
      for (int q = 0; q + 1 < N; ++q) k[q] = k[q + 1];
      k[N - 1] = 0;
    }
  }
  return mine;
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
    k[q] = (e < a.V) ? entry_key(x[q], e) : 0;
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
      s_last = (arrive(&a.ws_count[b]) == (uint32_t)(K * a.chunks - 1)) ? 1 : 0;
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
