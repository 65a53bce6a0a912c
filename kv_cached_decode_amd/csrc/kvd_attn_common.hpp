// Pieces shared by the two decode-attention kernels (the streaming kernel for
// one query per head and the MFMA tile for blocks of queries): query-row
// numbering, the layout of split partials, and the merge of the splits by the
// last workgroup of a tile to arrive.
#pragma once

#include <stddef.h>

#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {

constexpr int kPStride = kHeadDim + 4;  // partial row: o[D], m, l, 2 pad floats (16-byte rows)
constexpr int kMaxWaves = 8;            // the widest workgroup (512 threads; 16 measured slower)

struct RowId {
  int b, h, i;
};

__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

// Query row gg of unit (bkv, hk): numbered (bl * group + j) * N + i.
__device__ __forceinline__ RowId row_id(const AttnArgs &a, int bkv, int hk, int gg) {
  RowId r;
  const int q = (int)fast_div((uint32_t)gg, a.div_N);  // gg / N
  r.i = gg - q * a.N;
  const int bl = (int)fast_div((uint32_t)q, a.div_group);  // gg / (N * group)
  const int j = q - bl * a.group;
  r.b = (a.Bkv == 1) ? bl : bkv;
  r.h = hk * a.group + j;
  return r;
}

__device__ __forceinline__ size_t out_row(const AttnArgs &a, const RowId &r) {
  return ((size_t)(r.b * a.Hq + r.h) * a.N + r.i) * kHeadDim;
}

// The key range of unit row bkv: the call's L, causal base and new-row base,
// or, with per-row lengths (RAGGED: a ragged batch), that row's len clamped
// into [N, L] (L is the planned maximum; a clamped len is flagged in
// dev_status, so no access ever leaves the planned range). RAGGED is a
// template flag so that kernels without per-row lengths carry no trace of
// them.
struct RowSpan {
  int L, causal_base, new_base;
};
template <bool RAGGED>
__device__ __forceinline__ RowSpan row_span(const AttnArgs &a, int bkv, int L, int causal_base,
                                            int new_base) {
  RowSpan s{L, causal_base, new_base};
  if constexpr (RAGGED) {
    const int len = a.lens[bkv];
    const int c = min(max(len, a.N), a.L);
    if (c != len && a.dev_status && threadIdx.x == 0) *a.dev_status = kStatusCapacity;
    s.L = c;
    s.causal_base = c - a.N;
    if (a.new_base != INT_MAX) s.new_base = c - a.T_new;
  }
  return s;
}
template <bool RAGGED>
__device__ __forceinline__ RowSpan row_span(const AttnArgs &a, int bkv) {
  return row_span<RAGGED>(a, bkv, a.L, a.causal_base, a.new_base);
}

// The values a kernel's first key loads need, passed ahead of the argument
// struct as plain scalar kernel arguments, which the code object has the
// hardware preload into SGPRs at wave start (about 0.25 us before a load of
// the struct would return): the K and V bases, the unit split (Hkv and its
// divider), the cache row stride, the keys per split and the key range.
struct Lead {
  char *k, *v;
  FastDiv div_Hkv;
  int Hkv, S_max, chunk, L, causal_base, new_base, nw;  // nw: waves per workgroup
};
// A kernel's leading parameters that carry a Lead (in preload order), and the
// Lead they make.
#define KVD_LEAD_PARAMS                                                                      \
  char *lead_k, char *lead_v, uint32_t lead_hkv_m, uint32_t lead_hkv_s, int lead_hkv,       \
      int lead_smax, int lead_chunk, int lead_L, int lead_cb, int lead_nb, int lead_nw
#define KVD_LEAD                                                                             \
  Lead {                                                                                     \
    lead_k, lead_v, FastDiv{lead_hkv_m, lead_hkv_s}, lead_hkv, lead_smax, lead_chunk, lead_L, \
        lead_cb, lead_nb, lead_nw                                                            \
  }
typedef void (*LeadKernel)(char *, char *, uint32_t, uint32_t, int, int, int, int, int, int,
                           int, AttnArgs);
// The kernarg segment of such a kernel: its parameters laid out in order with
// their natural alignment, then the hidden arguments.
struct LeadLayout {
  char *k, *v;
  uint32_t hkv_m, hkv_s;
  int hkv, smax, chunk, L, cb, nb, nw;
  AttnArgs args;
};
constexpr size_t kLeadArgsOffset = offsetof(LeadLayout, args);
static_assert(kLeadArgsOffset == 56, "13 dwords of lead parameters, then the struct 8-aligned");
// The argument struct of a kernel with Lead parameters, read from the kernarg
// segment where this is called and not earlier: the segment pointer passes
// through an empty asm the compiler cannot move, so the struct's scalar loads
// are issued after the code before the call (the first key loads). Scalar
// loads complete out of order, so a wait for one of them (the compiler puts
// one wherever it reuses a register a pending load targets) is a wait for
// all; issued at the top, they held back the first key loads.
__device__ __forceinline__ AttnArgs lead_struct() {
#if __HIP_DEVICE_COMPILE__
  typedef const __attribute__((address_space(4))) char cchar4;
  typedef const __attribute__((address_space(4))) uint32_t cword4;
  cchar4 *p = (cchar4 *)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  // word by word: constant-memory words (scalar loads) into the local struct
  cword4 *w = reinterpret_cast<cword4 *>(p + kLeadArgsOffset);
  AttnArgs r;
  uint32_t *d = reinterpret_cast<uint32_t *>(&r);
  static_assert(sizeof(AttnArgs) % 4 == 0, "whole words");
#pragma unroll
  for (size_t i = 0; i < sizeof(AttnArgs) / 4; ++i) d[i] = w[i];
  return r;
#else
  return AttnArgs{};  // host pass: never called
#endif
}
// Launch of a kernel with Lead parameters: the Lead from the call's arguments.
inline void launch_lead(LeadKernel kernel, dim3 grid, dim3 block, hipStream_t s,
                        const AttnArgs &a) {
  const FastDiv fd = make_fast_div((uint32_t)a.Hkv);
  launch_kernel(kernel, grid, block, s, static_cast<char *>(a.k), static_cast<char *>(a.v), fd.m,
                fd.s, a.Hkv, a.S_max, a.chunk, a.L, a.causal_base, a.new_base,
                (int)(block.x / 64), AttnArgs(a));
}

// Online softmax (log2 domain), one row, one step of keys: mt is the step's
// largest score and each(fn) calls fn(score, v) for every key of the step.
// The row's reference m moves only when a score passes it by more than
// kLazySoftmax, so p = 2^(score - m) stays below 2^kLazySoftmax and o and l
// are rescaled only when some lane of the wavefront moved (exact: o and l
// always share the reference m; the merges weigh partials by their m).
constexpr float kLazySoftmax = 8.f;
template <int VE, typename Each>
__device__ __forceinline__ void online_update(float &m, float &l, float (&o)[VE], float mt,
                                              Each each) {
  const bool move = mt > m + kLazySoftmax;
  if (__builtin_amdgcn_ballot_w64(move)) {
    const float mn = move ? mt : m;
    const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
    for (int e = 0; e < VE; ++e) o[e] *= alpha;
    l *= alpha;
    m = mn;
  }
  if (m != -INFINITY) {
    each([&](float sc, const float (&v)[VE]) {
      const float p = __builtin_amdgcn_exp2f(sc - m);
      l += p;
#pragma unroll
      for (int e = 0; e < VE; ++e) o[e] = fmaf(p, v[e], o[e]);
    });
  }
}

// Every kernel argument the first loads depend on, fetched in one go: the
// empty asm keeps the compiler from sinking a fetch into a later branch,
// which would add a serial round trip before the first key load.
__device__ __forceinline__ void hoist_args(const AttnArgs &a) {
  const int f0 = a.Hkv, f1 = a.S_max, f2 = a.G, f3 = a.L, f4 = a.N, f5 = a.group, f6 = a.Bkv,
            f7 = a.causal_base, f8 = a.new_base, f9 = a.chunk, f10 = a.Hq, f11 = a.T_new;
  asm volatile("" ::"s"(f0), "s"(f1), "s"(f2), "s"(f3), "s"(f4), "s"(f5), "s"(f6), "s"(f7),
               "s"(f8), "s"(f9), "s"(f10), "s"(f11), "s"(a.k), "s"(a.v), "s"(a.q));
  asm volatile("" ::"s"(a.div_N.m), "s"(a.div_N.s), "s"(a.div_group.m), "s"(a.div_group.s));
}

// Merge of S published partials (o, m, l) of tile `tile_id`, numbered
// 0..S-1 in a fixed order, by one wavefront: it takes rows g_first,
// g_first + g_step, ... (< gcount), one dim per lane (D equals the wavefront
// width). Lane j reads m and l of partial j, so the max, the weights and
// their sum are wavefront reductions; every lane reads o[dim] of all S
// partials with every load in flight (one memory round trip whatever S is:
// NB >= S is the load count a lane keeps ready), and the outputs are summed
// in partial order so that the result does not depend on the arrival order.
template <int GM, int NB, int MR>
__device__ __forceinline__ void merge_rows_nb(const AttnArgs &a, size_t tile_id, int S, int g0, int gcount,
                              int bkv, int hk, int g_first, int g_step) {
  constexpr int D = kHeadDim;
  constexpr int SS = GM * kPStride;  // floats between two partials of one row
  static_assert(D == 64, "one lane per dim");
  const int lane = threadIdx.x & 63;
  const float *src = a.ws_part + tile_id * S * SS;
  for (int g1 = g_first; g1 < gcount; g1 += MR * g_step) {
    // the loads of up to MR rows go out before any of them is reduced, with
    // no branch around a load: rows past gcount read row g1 again and
    // partials past S partial 0, and those values go unused
    float mj[MR], lj[MR], ob[MR][NB];
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const int g = (g1 + r * g_step < gcount) ? g1 + r * g_step : g1;
      const float *row = src + g * kPStride;
      const int jl = (lane < S) ? lane : 0;
      mj[r] = __builtin_bit_cast(float, fetch_u32(row + jl * SS + D));
      lj[r] = __builtin_bit_cast(float, fetch_u32(row + jl * SS + D + 1));
#pragma unroll
      for (int j = 0; j < NB; ++j)
        ob[r][j] = __builtin_bit_cast(float, fetch_u32(row + ((j < S) ? j : 0) * SS + lane));
    }
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const int g = g1 + r * g_step;
      if (g < gcount) {
        const float m = (lane < S) ? mj[r] : -INFINITY;
        const float l = (lane < S) ? lj[r] : 0.f;
        // over the first NB lanes only (every partial sits in one; the rest
        // add -inf and zeros, so the full wavefront reduction gives the same
        // bits): the max where the weights are taken, the sum broadcast
        const float M = lanes_max<NB>(m);
        const float wj = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - M);
        const float inv = __builtin_amdgcn_rcpf(lanes_sum_all<NB>(l * wj));
        float O = 0.f;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if (j < S) {
            const float w = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wj), j));
            O = fmaf(ob[r][j], w, O);
          }
        }
        store_f32(a.out + out_row(a, row_id(a, bkv, hk, g0 + g)) + lane, O * inv);
      }
    }
  }
}

// The merge with a load count sized to S (at most kMaxSplits): up to 8
// partials, up to 4 rows of a wave load together; more partials, fewer rows.
template <int GM>
__device__ __forceinline__ void merge_rows(const AttnArgs &a, size_t tile_id, int S, int g0, int gcount, int bkv,
                           int hk, int g_first, int g_step) {
  constexpr int MR = GM < 4 ? GM : 4;
  static_assert(kMaxSplits == 64, "the largest load count below covers kMaxSplits");
  if (S <= 8)
    merge_rows_nb<GM, 8, MR>(a, tile_id, S, g0, gcount, bkv, hk, g_first, g_step);
  else if (S <= 16)
    merge_rows_nb<GM, 16, (MR < 2 ? MR : 2)>(a, tile_id, S, g0, gcount, bkv, hk, g_first, g_step);
  else if (S <= 32)
    merge_rows_nb<GM, 32, 1>(a, tile_id, S, g0, gcount, bkv, hk, g_first, g_step);
  else
    merge_rows_nb<GM, 64, 1>(a, tile_id, S, g0, gcount, bkv, hk, g_first, g_step);
}

// After every thread has published its part of this workgroup's partial
// (rows g < gcount of tile `tile_id`, partial blockIdx.x of a.splits), count
// the arrival; the last workgroup of the tile to arrive merges the partials,
// each of its waves taking every nw-th row. No LDS and no barrier in the
// merge.
template <int GM>
__device__ __forceinline__ void merge_splits(const AttnArgs &a, size_t tile_id, int g0, int gcount, int bkv,
                             int hk, int nw) {
  __shared__ int s_last;
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t *counter = a.ws_count + tile_id * kCounterStride;
    const bool last = arrive(counter) == (uint32_t)(a.splits - 1);
    if (last) reset_counter(counter);  // every split has arrived
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  merge_rows<GM>(a, tile_id, a.splits, g0, gcount, bkv, hk, threadIdx.x >> 6, nw);
}

}  // namespace kvd
