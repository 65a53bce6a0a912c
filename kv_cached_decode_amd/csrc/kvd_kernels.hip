// gfx950 kernels of the decoder step: cache append (optional rotary keys),
// in-place beam reorder, split-K decode attention with an in-kernel merge,
// and the speculative verify epilogue (row argmax + accepted length).
//
// Every kernel checks its own indices against the sizes it is given; the
// host entry points have already validated those sizes.
#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdlib.h>

#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {

namespace {

constexpr int kThreads = 256;
constexpr int kStatusBadShape = -2;  // KVD_ERR_SHAPE

// ---------------------------------------------------------------------------
// kv_append: thread (row, j) moves the 16-byte chunk j of the first half of a
// row and its partner chunk in the second half, so a rotary pair (i, i+D/2)
// is rotated by one thread.
// ---------------------------------------------------------------------------
template <int DT, bool ROPE>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
  constexpr int VE = vec_elems<DT>();
  constexpr int EB = Storage<DT>::bytes;
  constexpr int HALF_VECS = kHeadDim / 2 / VE;
  const long tid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long total = (long)a.B * a.H * a.T * HALF_VECS;
  if (tid >= total) return;
  const int j = (int)(tid % HALF_VECS);
  const long row = tid / HALF_VECS;  // (b * H + h) * T + t
  const int t = (int)(row % a.T);
  const long bh = row / a.T;
  const size_t src = (size_t)row * kHeadDim;
  const size_t dst = ((size_t)bh * a.S_max + a.pos + t) * kHeadDim;
  const int lo_e = j * VE, hi_e = kHeadDim / 2 + j * VE;

  const char *kn = static_cast<const char *>(a.k_new);
  const char *vn = static_cast<const char *>(a.v_new);
  char *kc = static_cast<char *>(a.k_cache);
  char *vc = static_cast<char *>(a.v_cache);

  u32x4 klo = load16(kn + (src + lo_e) * EB), khi = load16(kn + (src + hi_e) * EB);
  const u32x4 vlo = load16(vn + (src + lo_e) * EB), vhi = load16(vn + (src + hi_e) * EB);
  if constexpr (ROPE) {
    float lo[VE], hi[VE];
    unpack16<DT>(klo, lo);
    unpack16<DT>(khi, hi);
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      float c, s;
      rope_cos_sin(a.pos + t, lo_e + e, a.rope_base, c, s);
      rope_rotate(lo[e], hi[e], c, s);
    }
    klo = pack16<DT>(lo);
    khi = pack16<DT>(hi);
  }
  store16(kc + (dst + lo_e) * EB, klo);
  store16(kc + (dst + hi_e) * EB, khi);
  store16(vc + (dst + lo_e) * EB, vlo);
  store16(vc + (dst + hi_e) * EB, vhi);
}

// ---------------------------------------------------------------------------
// kv_reorder: thread (h, s, c) owns the 16-byte column c of position s of head
// h in every beam. It reads every source it needs, waits for all of them, and
// only then writes, so an in-place gather with repeated parents is safe: no
// other thread touches that column.
// ---------------------------------------------------------------------------
constexpr int kMaxBeams = 16;

template <int DT>
__global__ __launch_bounds__(kThreads) void reorder_kernel(ReorderArgs a) {
  constexpr int VPR = kHeadDim * Storage<DT>::bytes / 16;  // vectors per row
  const long tid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long total = (long)a.H * a.len * VPR;
  if (tid >= total) return;
  const int c = (int)(tid % VPR);
  const long hs = tid / VPR;
  const int s = (int)(hs % a.len);
  const int h = (int)(hs / a.len);

  int par[kMaxBeams];
  bool bad = false;
#pragma unroll
  for (int b = 0; b < kMaxBeams; ++b) {
    par[b] = b;
    if (b < a.B) {
      const int p = a.parent[b];
      if (p < 0 || p >= a.B) bad = true;
      else par[b] = p;
    }
  }
  const size_t beam_stride = (size_t)a.H * a.S_max * VPR;  // in 16-byte vectors
  const size_t off = ((size_t)h * a.S_max + s) * VPR + c;
  u32x4 *K = static_cast<u32x4 *>(a.k_cache);
  u32x4 *V = static_cast<u32x4 *>(a.v_cache);
  u32x4 kr[kMaxBeams], vr[kMaxBeams];
#pragma unroll
  for (int b = 0; b < kMaxBeams; ++b) {
    if (b < a.B && par[b] != b) {
      kr[b] = K[par[b] * beam_stride + off];
      vr[b] = V[par[b] * beam_stride + off];
    }
  }
  // every load has returned before the first store is issued
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int b = 0; b < kMaxBeams; ++b) {
    if (b < a.B && par[b] != b) {
      K[b * beam_stride + off] = kr[b];
      V[b * beam_stride + off] = vr[b];
    }
  }
  if (bad && tid == 0 && a.dev_status) *a.dev_status = kStatusBadShape;
}

// ---------------------------------------------------------------------------
// Decode attention, split over keys.
//
// Workgroup (split, row tile, unit) takes keys [split*chunk, +chunk) of one
// (cache row, kv head) for up to GM query rows. A wave loads TILE keys per
// iteration: LPR lanes share a key row (16 bytes each, one 128/256-byte row
// per LPR lanes, fully coalesced), so one wave load covers RPL rows. Scores
// are reduced across the LPR lanes; the softmax runs online in the log2
// domain (running max m, sum l, unnormalised o per row). Waves are merged in
// LDS; splits are merged by the last workgroup of the unit to arrive, in
// split order, so the result does not depend on arrival order.
// ---------------------------------------------------------------------------
constexpr int kMaxWaves = 4;
constexpr int kSteps = 4;

template <int DT>
struct AttnGeom {
  static constexpr int VE = vec_elems<DT>();      // elements per lane load
  static constexpr int LPR = kHeadDim / VE;       // lanes per key row
  static constexpr int RPL = 64 / LPR;            // key rows per wave load
  static constexpr int TILE = RPL * kSteps;       // keys per wave iteration
  static constexpr int ROWB = kHeadDim * Storage<DT>::bytes;
};

template <int DT, int GM>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
  using Geo = AttnGeom<DT>;
  constexpr int D = kHeadDim;
  constexpr int EB = Storage<DT>::bytes;
  constexpr int VE = Geo::VE, LPR = Geo::LPR, RPL = Geo::RPL, TILE = Geo::TILE;
  constexpr int ROWB = Geo::ROWB;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int kr = lane / LPR;   // key row within a wave load
  const int ds = lane % LPR;   // dims [ds*VE, ds*VE + VE)

  const int split = blockIdx.x, rt = blockIdx.y, unit = blockIdx.z;
  const int bkv = unit / a.Hkv, hk = unit % a.Hkv;
  const int g0 = rt * GM;
  const int gcount = min(GM, a.G - g0);

  // ---- query rows: load, rotate, fold in scale*log2(e)
  float qf[GM][VE];
  int lim[GM];
  int kvis = 0;
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    lim[g] = 0;
#pragma unroll
    for (int e = 0; e < VE; ++e) qf[g][e] = 0.f;
    if (g < gcount) {
      const int gg = g0 + g;
      const int i = gg % a.N;
      const int j = (gg / a.N) % a.group;
      const int bl = gg / (a.N * a.group);
      const int b = (a.Bkv == 1) ? bl : bkv;
      const int h = hk * a.group + j;
      const size_t qrow = ((size_t)(b * a.Hq + h) * a.N + i) * D;
      const char *qp = static_cast<const char *>(a.q);
      unpack16<DT>(load16(qp + (qrow + ds * VE) * EB), qf[g]);
      if (a.rope_base > 0.f) {
        float pf[VE];
        unpack16<DT>(load16(qp + (qrow + (ds ^ (LPR / 2)) * VE) * EB), pf);
        const int pos = a.causal_base + i;
        const bool is_lo = ds < LPR / 2;
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          float c, s;
          rope_cos_sin(pos, (ds % (LPR / 2)) * VE + e, a.rope_base, c, s);
          float lo = is_lo ? qf[g][e] : pf[e];
          float hi = is_lo ? pf[e] : qf[g][e];
          rope_rotate(lo, hi, c, s);
          qf[g][e] = is_lo ? lo : hi;
        }
      }
#pragma unroll
      for (int e = 0; e < VE; ++e) qf[g][e] *= a.scale_log2;
      lim[g] = (a.causal_base < 0) ? a.L : a.causal_base + i + 1;
      kvis = max(kvis, lim[g]);
    }
  }

  const int k0 = split * a.chunk;
  const int kend = min(min(k0 + a.chunk, a.L), kvis);
  const size_t head_off = (size_t)(bkv * a.Hkv + hk) * a.S_max * ROWB;
  const char *kb = static_cast<const char *>(a.k) + head_off + ds * 16;
  const char *vb = static_cast<const char *>(a.v) + head_off + ds * 16;

  float m[GM], l[GM], o[GM][VE];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) o[g][e] = 0.f;
  }

  for (int t0 = k0 + wave * TILE; t0 < kend; t0 += nw * TILE) {
    u32x4 kv[kSteps], vv[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int key = t0 + s * RPL + kr;
      if (key < kend) {
        kv[s] = load16(kb + (size_t)key * ROWB);
        vv[s] = load16(vb + (size_t)key * ROWB);
      } else {
        kv[s] = u32x4{0, 0, 0, 0};
        vv[s] = u32x4{0, 0, 0, 0};
      }
    }
    float sc[kSteps][GM];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      float kf[VE];
      unpack16<DT>(kv[s], kf);
      const int key = t0 + s * RPL + kr;
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) d = fmaf(qf[g][e], kf[e], d);
#pragma unroll
        for (int off = 1; off < LPR; off <<= 1) d += __shfl_xor(d, off);
        sc[s][g] = (key < lim[g] && key < kend) ? d : -INFINITY;
      }
    }
    float vf[kSteps][VE];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) unpack16<DT>(vv[s], vf[s]);
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      if (g < gcount) {
        float mt = sc[0][g];
#pragma unroll
        for (int s = 1; s < kSteps; ++s) mt = fmaxf(mt, sc[s][g]);
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off));
        const float mn = fmaxf(m[g], mt);
        if (mn != -INFINITY) {  // wave-uniform
          const float alpha = exp2f(m[g] - mn);
          l[g] *= alpha;
#pragma unroll
          for (int e = 0; e < VE; ++e) o[g][e] *= alpha;
#pragma unroll
          for (int s = 0; s < kSteps; ++s) {
            const float p = exp2f(sc[s][g] - mn);
            l[g] += p;
#pragma unroll
            for (int e = 0; e < VE; ++e) o[g][e] = fmaf(p, vf[s][e], o[g][e]);
          }
          m[g] = mn;
        }
      }
    }
  }

  // ---- reduce l and o over the key rows of the wave
#pragma unroll
  for (int g = 0; g < GM; ++g) {
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
      l[g] += __shfl_xor(l[g], off);
#pragma unroll
      for (int e = 0; e < VE; ++e) o[g][e] += __shfl_xor(o[g][e], off);
    }
  }

  // ---- merge the waves of the workgroup in LDS
  __shared__ float sm_m[kMaxWaves][GM], sm_l[kMaxWaves][GM];
  __shared__ float sm_o[kMaxWaves][GM][D];
  if (kr == 0) {
#pragma unroll
    for (int g = 0; g < GM; ++g) {
#pragma unroll
      for (int e = 0; e < VE; ++e) sm_o[wave][g][ds * VE + e] = o[g][e];
      if (ds == 0) {
        sm_m[wave][g] = m[g];
        sm_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();

  constexpr int PART = D + 2;  // o[D], m, l per row in the workspace
  const size_t tile_id = (size_t)unit * a.row_tiles + rt;
  float *part = a.ws_part + (tile_id * a.splits + split) * GM * PART;
  for (int idx = threadIdx.x; idx < GM * D; idx += blockDim.x) {
    const int g = idx / D, d = idx % D;
    if (g >= gcount) continue;
    float M = -INFINITY;
    for (int w = 0; w < nw; ++w) M = fmaxf(M, sm_m[w][g]);
    float Ls = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int w = 0; w < nw; ++w) {
        const float f = exp2f(sm_m[w][g] - M);
        Ls = fmaf(sm_l[w][g], f, Ls);
        O = fmaf(sm_o[w][g][d], f, O);
      }
    }
    if (a.splits == 1) {
      const int gg = g0 + g;
      const int i = gg % a.N, j = (gg / a.N) % a.group, bl = gg / (a.N * a.group);
      const int b = (a.Bkv == 1) ? bl : bkv;
      const int h = hk * a.group + j;
      a.out[((size_t)(b * a.Hq + h) * a.N + i) * D + d] = O / Ls;
    } else {
      part[g * PART + d] = O;
      if (d == 0) {
        part[g * PART + D] = M;
        part[g * PART + D + 1] = Ls;
      }
    }
  }
  if (a.splits == 1) return;

  // ---- arrival: the last workgroup of this (unit, row tile) merges the splits
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(&a.ws_count[tile_id], 1u);
    s_last = (prev == (uint32_t)(a.splits - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const float *tparts = a.ws_part + tile_id * a.splits * GM * PART;
  for (int idx = threadIdx.x; idx < GM * D; idx += blockDim.x) {
    const int g = idx / D, d = idx % D;
    if (g >= gcount) continue;
    float M = -INFINITY;
    for (int sp = 0; sp < a.splits; ++sp) M = fmaxf(M, tparts[(sp * GM + g) * PART + D]);
    float Ls = 0.f, O = 0.f;
    for (int sp = 0; sp < a.splits; ++sp) {
      const float *p = tparts + (sp * GM + g) * PART;
      const float ms = p[D];
      if (ms != -INFINITY) {
        const float f = exp2f(ms - M);
        Ls = fmaf(p[D + 1], f, Ls);
        O = fmaf(p[d], f, O);
      }
    }
    const int gg = g0 + g;
    const int i = gg % a.N, j = (gg / a.N) % a.group, bl = gg / (a.N * a.group);
    const int b = (a.Bkv == 1) ? bl : bkv;
    const int h = hk * a.group + j;
    a.out[((size_t)(b * a.Hq + h) * a.N + i) * D + d] = O / Ls;
  }
  if (threadIdx.x == 0) a.ws_count[tile_id] = 0u;
}

// ---------------------------------------------------------------------------
// verify_accept: workgroup (chunk, r, b) finds (max, lowest index) over its
// slice of row r; the last workgroup of batch row b to arrive reduces the
// slices of every row in order, then scans the drafts for the first mismatch.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float load_logit(const void *row, int e) {
  if constexpr (DT == F32) return static_cast<const float *>(row)[e];
  else if constexpr (DT == F16) return (float)static_cast<const _Float16 *>(row)[e];
  else return __builtin_bit_cast(float, (uint32_t)static_cast<const uint16_t *>(row)[e] << 16);
}

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void verify_kernel(VerifyArgs a) {
  const int ch = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int e0 = ch * a.chunk;
  const int e1 = min(e0 + a.chunk, a.V);
  const char *row = static_cast<const char *>(a.logits) +
                    (size_t)(b * a.R + r) * a.V * Storage<DT>::bytes;
  float best = -INFINITY;
  int bi = INT_MAX;
  for (int e = e0 + (int)threadIdx.x; e < e1; e += kThreads) {
    const float x = load_logit<DT>(row, e);
    if (better(x, e, best, bi)) {
      best = x;
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
  __shared__ float sv[kThreads / 64];
  __shared__ int si[kThreads / 64];
  __shared__ int s_last;
  __shared__ int s_am[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / 64; ++w)
      if (better(sv[w], si[w], best, bi)) {
        best = sv[w];
        bi = si[w];
      }
    const size_t slot = (size_t)(b * a.R + r) * a.chunks + ch;
    a.ws_val[slot] = best;
    a.ws_idx[slot] = bi;
    __threadfence();
    const uint32_t prev = atomicAdd(&a.ws_count[b], 1u);
    s_last = (prev == (uint32_t)(a.R * a.chunks - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if ((int)threadIdx.x < a.R) {
    const int rr = threadIdx.x;
    float bv = -INFINITY;
    int bix = INT_MAX;
    for (int c = 0; c < a.chunks; ++c) {
      const size_t slot = (size_t)(b * a.R + rr) * a.chunks + c;
      const float v = a.ws_val[slot];
      const int ix = a.ws_idx[slot];
      if (better(v, ix, bv, bix)) {
        bv = v;
        bix = ix;
      }
    }
    if (bix == INT_MAX) bix = 0;  // only reachable with NaN rows
    s_am[rr] = bix;
    if (a.argmax_out) a.argmax_out[b * a.R + rr] = bix;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    while (n < a.N && a.draft[b * a.N + n] == s_am[n]) ++n;
    a.accept_len[b] = n;
    a.next_token[b] = (n < a.R) ? s_am[n] : -1;
    a.ws_count[b] = 0u;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

hipError_t launch_append(int dtype, const AppendArgs &a, hipStream_t s) {
  const int ve = (dtype == F32) ? 4 : 8;
  const long total = (long)a.B * a.H * a.T * (kHeadDim / 2 / ve);
  const dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
  const bool rope = a.rope_base > 0.f;
  switch (dtype) {
    case F32:
      if (rope) hipLaunchKernelGGL((append_kernel<F32, true>), grid, dim3(kThreads), 0, s, a);
      else hipLaunchKernelGGL((append_kernel<F32, false>), grid, dim3(kThreads), 0, s, a);
      break;
    case F16:
      if (rope) hipLaunchKernelGGL((append_kernel<F16, true>), grid, dim3(kThreads), 0, s, a);
      else hipLaunchKernelGGL((append_kernel<F16, false>), grid, dim3(kThreads), 0, s, a);
      break;
    default:
      if (rope) hipLaunchKernelGGL((append_kernel<BF16, true>), grid, dim3(kThreads), 0, s, a);
      else hipLaunchKernelGGL((append_kernel<BF16, false>), grid, dim3(kThreads), 0, s, a);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_reorder(int dtype, const ReorderArgs &a, hipStream_t s) {
  if (a.len == 0) return hipSuccess;
  const int vpr = kHeadDim * ((dtype == F32) ? 4 : 2) / 16;
  const long total = (long)a.H * a.len * vpr;
  const dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
  switch (dtype) {
    case F32: hipLaunchKernelGGL((reorder_kernel<F32>), grid, dim3(kThreads), 0, s, a); break;
    case F16: hipLaunchKernelGGL((reorder_kernel<F16>), grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((reorder_kernel<BF16>), grid, dim3(kThreads), 0, s, a); break;
  }
  return hipGetLastError();
}

template <int DT>
static void launch_attn_dt(const AttnArgs &a, dim3 grid, dim3 block, hipStream_t s) {
  switch (a.gm) {
    case 1: hipLaunchKernelGGL((attn_kernel<DT, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((attn_kernel<DT, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_kernel<DT, 4>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((attn_kernel<DT, 8>), grid, block, 0, s, a); break;
  }
}

hipError_t launch_attn(int dtype, const AttnArgs &a, hipStream_t s) {
  const dim3 grid(a.splits, a.row_tiles, a.Bkv * a.Hkv);
  const dim3 block(64 * a.waves);
  switch (dtype) {
    case F32: launch_attn_dt<F32>(a, grid, block, s); break;
    case F16: launch_attn_dt<F16>(a, grid, block, s); break;
    default: launch_attn_dt<BF16>(a, grid, block, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_verify(const VerifyArgs &a, hipStream_t s) {
  const dim3 grid(a.chunks, a.R, a.B);
  switch (a.dtype) {
    case F32: hipLaunchKernelGGL((verify_kernel<F32>), grid, dim3(kThreads), 0, s, a); break;
    case F16: hipLaunchKernelGGL((verify_kernel<F16>), grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((verify_kernel<BF16>), grid, dim3(kThreads), 0, s, a); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Plans
// ---------------------------------------------------------------------------

static int env_int(const char *name, int dflt) {
  const char *v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

AttnPlan plan_attn(int dtype, int units, int G, int L) {
  AttnPlan p{};
  p.gm = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8;
  p.row_tiles = (G + p.gm - 1) / p.gm;
  p.waves = env_int("KVD_ATTN_WAVES", 4);
  if (p.waves != 1 && p.waves != 2 && p.waves != 4) p.waves = 4;
  const int tile = (dtype == F32) ? AttnGeom<F32>::TILE : AttnGeom<F16>::TILE;
  const int min_chunk = tile * p.waves;
  const int per_split = units * p.row_tiles;
  int target_wgs = env_int("KVD_ATTN_TARGET_WGS", 512);
  if (target_wgs < 1 || target_wgs > kMaxCounters) target_wgs = 512;
  int want = (target_wgs + per_split - 1) / per_split;
  want = want < 1 ? 1 : (want > 64 ? 64 : want);
  int chunk = (L + want - 1) / want;
  chunk = ((chunk + min_chunk - 1) / min_chunk) * min_chunk;
  const int forced = env_int("KVD_ATTN_CHUNK", 0);
  if (forced > 0) chunk = ((forced + min_chunk - 1) / min_chunk) * min_chunk;
  if (chunk < min_chunk) chunk = min_chunk;
  p.chunk = chunk;
  p.splits = (L + chunk - 1) / chunk;
  if (p.splits > 64) {  // keep the merge and the workspace bounded
    p.splits = 64;
    p.chunk = (((L + 63) / 64 + min_chunk - 1) / min_chunk) * min_chunk;
    p.splits = (L + p.chunk - 1) / p.chunk;
  }
  const size_t tiles = (size_t)units * p.row_tiles;
  if (p.splits > 1 && tiles > (size_t)kMaxCounters) {  // one counter per tile
    p.chunk = ((L + min_chunk - 1) / min_chunk) * min_chunk;
    p.splits = 1;
  }
  p.part_floats = (p.splits > 1) ? tiles * p.splits * p.gm * (kHeadDim + 2) : 0;
  p.counters = tiles;
  return p;
}

void plan_verify(int B, int R, int V, int &chunk, int &chunks) {
  (void)B;
  (void)R;
  chunk = 4096;
  chunks = (V + chunk - 1) / chunk;
}

}  // namespace kvd
