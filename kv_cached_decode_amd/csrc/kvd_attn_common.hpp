// Pieces shared by the two decode-attention kernels (the streaming kernel for
// one query per head and the MFMA tile for blocks of queries): query-row
// numbering, the layout of split partials, and the merge of the splits by the
// last workgroup of a tile to arrive.
#pragma once

#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {

constexpr int kPStride = kHeadDim + 4;  // partial row: o[D], m, l, 2 pad floats (16-byte rows)
constexpr int kMergeRows = 128;         // splits * rows per tile the merge can stage
constexpr int kMaxWaves = 16;           // the widest workgroup (1024 threads)

// Floats each thread stages in the final merge, for workgroups of 64 * NWMAX.
template <int NWMAX>
constexpr int stage_iters() { return (kMergeRows * kPStride + 64 * NWMAX - 1) / (64 * NWMAX); }

struct RowId {
  int b, h, i;
};

// Query row gg of unit (bkv, hk): numbered (bl * group + j) * N + i.
__device__ __forceinline__ RowId row_id(const AttnArgs &a, int bkv, int hk, int gg) {
  RowId r;
  r.i = gg % a.N;
  const int j = (gg / a.N) % a.group;
  const int bl = gg / (a.N * a.group);
  r.b = (a.Bkv == 1) ? bl : bkv;
  r.h = hk * a.group + j;
  return r;
}

__device__ __forceinline__ size_t out_row(const AttnArgs &a, const RowId &r) {
  return ((size_t)(r.b * a.Hq + r.h) * a.N + r.i) * kHeadDim;
}

// Every kernel argument the first loads depend on, fetched in one go: the
// empty asm keeps the compiler from sinking a fetch into a later branch,
// which would add a serial round trip before the first key load.
__device__ __forceinline__ void hoist_args(const AttnArgs &a) {
  const int f0 = a.Hkv, f1 = a.S_max, f2 = a.G, f3 = a.L, f4 = a.N, f5 = a.group, f6 = a.Bkv,
            f7 = a.causal_base, f8 = a.new_base, f9 = a.chunk, f10 = a.Hq, f11 = a.T_new;
  asm volatile("" ::"s"(f0), "s"(f1), "s"(f2), "s"(f3), "s"(f4), "s"(f5), "s"(f6), "s"(f7),
               "s"(f8), "s"(f9), "s"(f10), "s"(f11), "s"(a.k), "s"(a.v), "s"(a.q));
}

// After every thread has published its part of this workgroup's partial
// (rows g < gcount of tile `tile_id`, split blockIdx.x), count the arrival;
// the last workgroup of the tile stages every split's partial in LDS (all
// loads in flight at once), weighs the splits (one lane per split in wave 0)
// and writes the rows' outputs, combining splits in split order so that the
// result does not depend on arrival order. smem holds kMergeRows * kPStride
// floats.
template <int GM, int NWMAX>
__device__ void merge_splits(const AttnArgs &a, size_t tile_id, int g0, int gcount, int bkv, int hk,
                             float *smem) {
  constexpr int D = kHeadDim;
  __shared__ int s_last;
  __shared__ float s_w[kMergeRows], s_inv[GM];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (arrive(&a.ws_count[tile_id]) == (uint32_t)(a.splits - 1)) ? 1 : 0;
  __syncthreads();
  if (!s_last) return;

  const int n = a.splits * GM * kPStride;
  const float *src = a.ws_part + tile_id * a.splits * GM * kPStride;
  constexpr int kStageIters = stage_iters<NWMAX>();
  uint32_t stage[kStageIters];
#pragma unroll
  for (int j = 0; j < kStageIters; ++j) {
    const int i = threadIdx.x + j * blockDim.x;
    if (i < n) stage[j] = fetch_u32(src + i);
  }
#pragma unroll
  for (int j = 0; j < kStageIters; ++j) {
    const int i = threadIdx.x + j * blockDim.x;
    if (i < n) smem[i] = __builtin_bit_cast(float, stage[j]);
  }
  __syncthreads();
  if (wave == 0) {
    for (int g = 0; g < gcount; ++g) {
      const bool on = lane < a.splits;
      const float ms = on ? smem[(lane * GM + g) * kPStride + D] : -INFINITY;
      const float ls = on ? smem[(lane * GM + g) * kPStride + D + 1] : 0.f;
      const float M = groups_max<1>(ms);
      const float w = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
      const float L = groups_sum<1>(ls * w);
      if (on) s_w[lane * GM + g] = w;
      if (lane == 0) s_inv[g] = 1.f / L;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < GM * D; idx += blockDim.x) {
    const int g = idx / D, d = idx % D;
    if (g >= gcount) continue;
    float O = 0.f;
#pragma unroll 8
    for (int sp = 0; sp < a.splits; ++sp)
      O = fmaf(smem[(sp * GM + g) * kPStride + d], s_w[sp * GM + g], O);
    a.out[out_row(a, row_id(a, bkv, hk, g0 + g)) + d] = O * s_inv[g];
  }
  if (threadIdx.x == 0) reset_counter(&a.ws_count[tile_id]);
}

}  // namespace kvd
