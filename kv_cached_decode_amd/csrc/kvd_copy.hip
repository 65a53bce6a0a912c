// Cache writes on gfx950: kv_append (optionally rotating keys) and the
// in-place beam reorder. Both are pure data movement with 16-byte accesses.
#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxBeams = 16;

// Thread (row, j) moves rotary pair j of one new row; rows are ordered
// (b, h, t) like the input.
template <int DT>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
  constexpr int HALF_VECS = kHeadDim / 2 / vec_elems<DT>();
  constexpr int ROWB = kHeadDim * Storage<DT>::bytes;
  const long tid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long total = (long)a.B * a.H * a.T * HALF_VECS;
  if (tid >= total) return;
  const int j = (int)(tid % HALF_VECS);
  const long row = tid / HALF_VECS;
  const int t = (int)(row % a.T);
  const long bh = row / a.T;
  int pos = a.pos;
  if (a.pos_rows) {  // ragged batch: row b writes at its own position
    pos = a.pos_rows[bh / a.H];
    if (pos < 0 || pos > a.S_max - a.T) {  // outside the cache: skipped, never written
      if (a.dev_status && t == 0 && j == 0) *a.dev_status = kStatusCapacity;
      return;
    }
  }
  const size_t src = (size_t)row * ROWB;
  const size_t dst = ((size_t)bh * a.S_max + pos + t) * ROWB;
  constexpr int VE = vec_elems<DT>();
  double th[VE];  // angles of the thread's VE rotary pairs (zeros without rotation)
#pragma unroll
  for (int e = 0; e < VE; ++e) th[e] = rope_theta_at(a.rope_theta, j * VE + e);
  const PairChunks c = load_pair<DT>(static_cast<const char *>(a.k_new) + src,
                                     static_cast<const char *>(a.v_new) + src, j, pos + t,
                                     a.rope_base > 0.f ? th : nullptr);
  store_pair<DT>(static_cast<char *>(a.k_cache) + dst, static_cast<char *>(a.v_cache) + dst, j, c);
}

// Thread (h, s, c) owns the 16-byte column c of position s of head h in
// every beam. It reads every source it needs, waits for all of them, and only
// then writes, so an in-place gather with repeated parents is safe: no other
// thread touches that column.
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

}  // namespace

hipError_t launch_append(int dtype, const AppendArgs &a, hipStream_t s) {
  const int ve = (dtype == F32) ? 4 : 8;
  const long total = (long)a.B * a.H * a.T * (kHeadDim / 2 / ve);
  const dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
  switch (dtype) {
    case F32: launch_kernel(append_kernel<F32>, grid, dim3(kThreads), s, a); break;
    case F16: launch_kernel(append_kernel<F16>, grid, dim3(kThreads), s, a); break;
    default: launch_kernel(append_kernel<BF16>, grid, dim3(kThreads), s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_reorder(int dtype, const ReorderArgs &a, hipStream_t s) {
  if (a.len == 0) return hipSuccess;
  const int vpr = kHeadDim * ((dtype == F32) ? 4 : 2) / 16;
  const long total = (long)a.H * a.len * vpr;
  const dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
  switch (dtype) {
    case F32: launch_kernel(reorder_kernel<F32>, grid, dim3(kThreads), s, a); break;
    case F16: launch_kernel(reorder_kernel<F16>, grid, dim3(kThreads), s, a); break;
    default: launch_kernel(reorder_kernel<BF16>, grid, dim3(kThreads), s, a); break;
  }
  return hipGetLastError();
}

}  // namespace kvd
