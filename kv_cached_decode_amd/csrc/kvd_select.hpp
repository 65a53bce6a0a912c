// Selection on gfx950 wavefronts with order keys: a (value, index) pair, or
// any ranked item, is one 64-bit integer whose unsigned order is the order
// wanted, so a max or a top-n over the wavefront runs in lane exchanges (DPP
// and permlane swaps) with no LDS round trip and no barrier.
#pragma once

#include <stdint.h>

#include "kvd_device.hpp"

namespace kvd {

// Element e of a logits row of storage type DT, widened to fp32 (exact).
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

// (value, index): larger value first, equal values lower index first. Every
// such key is nonzero; 0 stands for "none" and ranks last.
__device__ __forceinline__ uint64_t value_key(float v, int tok) {
  return ((uint64_t)order_bits(v) << 32) | (uint32_t)~tok;
}
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

// Max of a 64-bit key over the wavefront (every lane ends with it) and the
// lowest lane holding it. The high words (the value) are reduced first; when
// one lane holds that value its low word is read from it, otherwise a second
// reduction over the tied lanes' low words decides.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k, int &owner) {
  const uint32_t hi = (uint32_t)(k >> 32), lo = (uint32_t)k;
  const uint32_t whi = wave_umax(hi);
  const uint64_t tied = __builtin_amdgcn_ballot_w64(hi == whi);
  uint32_t wlo;
  if (__builtin_popcountll(tied) == 1) {
    owner = __builtin_ctzll(tied);
    wlo = (uint32_t)__builtin_amdgcn_readlane((int)lo, owner);
  } else {
    wlo = wave_umax(hi == whi ? lo : 0u);
    owner = __builtin_ctzll(__builtin_amdgcn_ballot_w64(hi == whi && lo == wlo));
  }
  return ((uint64_t)whi << 32) | wlo;
}

// The wavefront's n best keys among the N keys each lane holds (0 = none;
// real keys are distinct): lane r (r < n) returns the r-th. Each lane sorts
// its keys once; a round takes the wavefront max and the lane holding it
// shifts its list.
template <int N>
__device__ __forceinline__ uint64_t wave_top(uint64_t (&k)[N], int n, int lane) {
  sort_desc(k);
  uint64_t mine = 0;
  for (int r = 0; r < n; ++r) {
    int owner;
    const uint64_t win = wave_max_key(k[0], owner);
    if (lane == r) mine = win;
    if (lane == owner) {
#pragma unroll
      for (int q = 0; q + 1 < N; ++q) k[q] = k[q + 1];
      k[N - 1] = 0;
    }
  }
  return mine;
}

}  // namespace kvd
