// Device helpers shared by the gfx950 kernels: 16-byte vector loads of the
// storage types, conversion to fp32, round-to-nearest-even stores, and the
// rotary rotation of one (i, i + D/2) pair.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvd_internal.hpp"

namespace kvd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int DT> struct Storage;
template <> struct Storage<F32> { static constexpr int bytes = 4; };
template <> struct Storage<F16> { static constexpr int bytes = 2; };
template <> struct Storage<BF16> { static constexpr int bytes = 2; };

// Elements per 16-byte vector.
template <int DT> constexpr int vec_elems() { return 16 / Storage<DT>::bytes; }

// Global memory, named as such: pointers that arrive through the argument
// struct would otherwise be accessed with flat instructions (an address
// space check per access, and counted in lgkmcnt as well as vmcnt).
template <typename T>
using global_ptr = __attribute__((address_space(1))) T *;
__device__ __forceinline__ u32x4 load16(const void *p) {
  return *(const global_ptr<u32x4>)p;
}
__device__ __forceinline__ void store16(void *p, u32x4 v) {
  *(global_ptr<u32x4>)p = v;
}
__device__ __forceinline__ void store_f32(float *p, float v) { *(global_ptr<float>)p = v; }

// Two storage elements packed in one dword -> two floats (element 2i is the
// low half of dword i, little endian).
template <int DT> __device__ __forceinline__ void unpack2(uint32_t w, float &lo, float &hi);
template <> __device__ __forceinline__ void unpack2<F16>(uint32_t w, float &lo, float &hi) {
  f16x2 h = __builtin_bit_cast(f16x2, w);
  lo = (float)h[0];
  hi = (float)h[1];
}
template <> __device__ __forceinline__ void unpack2<BF16>(uint32_t w, float &lo, float &hi) {
  lo = __builtin_bit_cast(float, w << 16);
  hi = __builtin_bit_cast(float, w & 0xffff0000u);
}

// One 16-bit storage element -> float.
template <int DT> __device__ __forceinline__ float widen16(uint16_t b);
template <> __device__ __forceinline__ float widen16<F16>(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
template <> __device__ __forceinline__ float widen16<BF16>(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// A 16-byte vector -> vec_elems<DT>() floats.
template <int DT> __device__ __forceinline__ void unpack16(u32x4 v, float *out) {
  if constexpr (DT == F32) {
    // copy each element out first: bit-casting a vector element lvalue
    // directly reads element 0 with this compiler
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = v[i];
      out[i] = __builtin_bit_cast(float, w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = v[i];
      unpack2<DT>(w, out[2 * i], out[2 * i + 1]);
    }
  }
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).

// Two floats -> one dword of two storage elements, round to nearest even.
template <int DT> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<F16>(float lo, float hi) {
  f16x2 h;
  h[0] = (_Float16)lo;
  h[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, h);
}
template <> __device__ __forceinline__ uint32_t pack2<BF16>(float lo, float hi) {
  // v_cvt_pk_bf16_f32: round to nearest even (checked against the rounding
  // (u + 0x7fff + ((u >> 16) & 1)) >> 16 over every non-NaN float)
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

template <int DT> __device__ __forceinline__ u32x4 pack16(const float *in) {
  u32x4 v;
  if constexpr (DT == F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_bit_cast(uint32_t, in[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack2<DT>(in[2 * i], in[2 * i + 1]);
  }
  return v;
}

// Rotary angles. Pair (i, i + D/2) at absolute position pos turns by
// pos * theta_i, theta_i = base^(-2i/D). The angle is one fp64 product,
// reduced modulo pi/2 in fp64 (Cody-Waite: k = nearest integer to
// angle * 2/pi, then angle - k * pi/2 with pi/2 split into three doubles, the
// first step exact), which leaves |y| <= pi/4 + a rounding.
//  - Stored keys (rope_theta_at, rope_angle_cs64, rotate_elem64): theta_i
//    exactly as the host's C library pow gives it (RopeTheta), cos y and
//    sin y as fp64 Taylor polynomials (sin through y^17, cos through y^18:
//    truncation below 2^-60 on |y| <= pi/4; cos as w + ((1 - w) - z/2 +
//    z^2 r(z)) with w = 1 - z/2, z = y^2, so the rounding of w is carried),
//    the rotation in fp64 and one rounding to the storage type. The result
//    is the correctly rounded rotation unless the exact value lies within
//    about 2^-50 (relative) of a rounding boundary of the storage type.
//  - Queries (RopeStep, rope_angle_cs): theta_i = ratio^i in fp64 with the
//    host's ratio = 2^(-step), step = 2 log2(base) / D (squarings and a few
//    multiplies; a few ulps from the exact theta_i), the reduction with the
//    first double of pi/2 only (the rest moves y by k * 2^-53.9, below 2^-30
//    for every position under 2^24, far below fp32's resolution), fp32
//    Taylor polynomials of y (degree 10 and 9, truncation below 2^-28) and
//    the rotation in fp32: queries are not stored, so they only need to be
//    accurate, and one definition serves every kernel and plan, so a query
//    is rotated with the same bits everywhere. No memory access.
// The quadrant k mod 4 maps cos y / sin y onto cos / sin of the full angle.
// A double in the constant address space (read with scalar loads).
typedef const __attribute__((address_space(4))) double const_double;

__device__ __forceinline__ double rope_reduce(int pos, double theta, int &quadrant) {
  const double ang = (double)pos * theta;                   // >= 0, < 2^31
  const double k = rint(ang * 0x1.45f306dc9c883p-1);      // 2 / pi
  double y = fma(-k, 0x1.921fb54442d18p+0, ang);          // pi/2, first 53 bits (exact step)
  y = fma(-k, 0x1.1a62633145c07p-54, y);                  // next 53 bits
  y = fma(-k, -0x1.f1976b7ed8fbcp-110, y);                // next 53 bits
  quadrant = (int)k & 3;
  return y;
}

__device__ __forceinline__ void rope_angle_cs(int pos, double theta, float &c, float &s) {
  const double ang = (double)pos * theta;
  const double k = rint(ang * 0x1.45f306dc9c883p-1);  // 2 / pi
  const int q = (int)k & 3;
  const float y = (float)fma(-k, 0x1.921fb54442d18p+0, ang), y2 = y * y;  // pi/2, first 53 bits
  float ps = fmaf(y2, 2.7557319e-06f, -1.9841270e-04f);  // 1/9!, -1/7!
  ps = fmaf(ps, y2, 8.3333333e-03f);                     // 1/5!
  ps = fmaf(ps, y2, -1.6666667e-01f);                    // -1/3!
  const float sy = fmaf(ps * y2, y, y);
  float pc = fmaf(y2, -2.7557319e-07f, 2.4801587e-05f);  // -1/10!, 1/8!
  pc = fmaf(pc, y2, -1.3888889e-03f);                    // -1/6!
  pc = fmaf(pc, y2, 4.1666668e-02f);                     // 1/4!
  pc = fmaf(pc, y2, -0.5f);
  const float cy = fmaf(pc, y2, 1.0f);
  const float sv = (q & 1) ? cy : sy, cv = (q & 1) ? sy : cy;
  s = (q & 2) ? -sv : sv;                           // sin: s, c, -s, -c
  c = (q == 1 || q == 2) ? -cv : cv;                // cos: c, -s, -c, s
}

// Taylor coefficients 1/n! (rounded to nearest) of the fp64 cos / sin:
// sin y = y + y z p(z) with p from 1/17! down to -1/3!, cos y = 1 - z/2 +
// z^2 r(z) with r from -1/18! down to 1/4!.
#define KVD_SIN64_COEFS                                                                      \
  0x1.952c77030ad4ap-49, -0x1.ae7f3e733b81fp-41, 0x1.6124613a86d09p-33, -0x1.ae64567f544e4p-26, \
      0x1.71de3a556c734p-19, -0x1.a01a01a01a01ap-13, 0x1.1111111111111p-7, -0x1.5555555555555p-3
#define KVD_COS64_COEFS                                                                        \
  -0x1.6827863b97d97p-53, 0x1.ae7f3e733b81fp-45, -0x1.93974a8c07c9dp-37, 0x1.1eed8eff8d898p-29, \
      -0x1.27e4fb7789f5cp-22, 0x1.a01a01a01a01ap-16, -0x1.6c16c16c16c17p-10, 0x1.5555555555555p-5
__constant__ const double kSinCos64[16] = {KVD_SIN64_COEFS, KVD_COS64_COEFS};

// fp64 cos / sin at pos * theta. OPAQUE: read the coefficients from constant
// memory at the call (scalar loads the optimiser cannot hoist), for callers in
// a loop where 32 hoisted scalar registers of constants make a kernel spill;
// otherwise they are immediates.
template <bool OPAQUE = false>
__device__ __forceinline__ void rope_angle_cs64(int pos, double theta, double &c, double &s) {
  int q;
  const double y = rope_reduce(pos, theta, q), z = y * y;
  constexpr double kImm[16] = {KVD_SIN64_COEFS, KVD_COS64_COEFS};
  const_double *tab = (const_double *)kSinCos64;
  if constexpr (OPAQUE) asm volatile("" : "+s"(tab));  // constant address space kept: scalar loads
  auto k = [&](int i) -> double {
    if constexpr (OPAQUE) return tab[i];
    else return kImm[i];
  };
  double p = fma(z, k(0), k(1));
#pragma unroll
  for (int i = 2; i < 8; ++i) p = fma(p, z, k(i));
  const double sy = fma(y * z, p, y);
  double r = fma(z, k(8), k(9));
#pragma unroll
  for (int i = 10; i < 16; ++i) r = fma(r, z, k(i));
  const double hz = 0.5 * z, w = 1.0 - hz;
  const double cy = w + (((1.0 - w) - hz) + (z * z) * r);
  const double sv = (q & 1) ? cy : sy, cv = (q & 1) ? sy : cy;
  s = (q & 2) ? -sv : sv;
  c = (q == 1 || q == 2) ? -cv : cv;
}

// theta_i (i in [0, 32), may differ per lane) rebuilt from the kernel
// arguments' RopeTheta: the product of pw[k] over the set bits of i in
// ascending k (a factor 1.0 for a clear bit leaves the product exact), then
// the byte correction added to the bit pattern. The words are read at
// constant indices (scalar loads) and picked per lane by selects: no vector
// memory access, so nothing waits behind the key loads.
__device__ __forceinline__ double rope_theta_at(const RopeTheta &r, int i) {
  double t = 1.0;
#pragma unroll
  for (int k = 0; k < 5; ++k) t = t * (((i >> k) & 1) ? r.pw[k] : 1.0);
  // (each word taken as a wave-uniform value first: a select between the
  // words themselves, which the optimiser would otherwise turn into one load
  // at a selected offset, a per-lane memory access)
  uint32_t w = __builtin_amdgcn_readfirstlane(r.delta[0]);
#pragma unroll
  for (int q = 1; q < kHeadDim / 8; ++q)
    w = ((i >> 2) == q) ? __builtin_amdgcn_readfirstlane(r.delta[q]) : w;
  const int d = (int)(int8_t)(w >> (8 * (i & 3)));
  return __builtin_bit_cast(double, __builtin_bit_cast(int64_t, t) + (int64_t)d);
}

// Query angles: pair i's theta from RopeStep. For a run of n consecutive
// pairs i0 .. i0 + n - 1 (n a power of two, i0 a multiple of n), theta_i0 =
// (ratio^n)^(i0 / n), ratio^n by squarings and its power by the bits of
// i0 / n, and each next theta one fp64 multiply by ratio; rope_cos_sin_pair
// gives pair i alone bit for bit what the run that holds it gives.
struct RopeStep {
  double ratio;  // 2^(-step), step = 2 log2(base) / D
};
template <int n>
__device__ __forceinline__ double rope_theta_q(int i0, double ratio) {
  static_assert(n >= 1 && (n & (n - 1)) == 0 && n <= kHeadDim / 2, "runs of a power of two");
  double p = ratio;
#pragma unroll
  for (int b = 1; b < n; b *= 2) p *= p;  // ratio^n
  const int j = i0 / n;
  double t = (j & 1) ? p : 1.0;
#pragma unroll
  for (int b = 1; (1 << b) < kHeadDim / 2 / n; ++b) {
    p *= p;
    t = ((j >> b) & 1) ? t * p : t;
  }
  return t;
}
template <int n>
__device__ __forceinline__ void rope_cos_sin_run(int pos, int i0, RopeStep r, float *c, float *s) {
  double theta = rope_theta_q<n>(i0, r.ratio);
#pragma unroll
  for (int e = 0; e < n; ++e) {
    rope_angle_cs(pos, theta, c[e], s[e]);
    theta *= r.ratio;
  }
}
template <int n>
__device__ __forceinline__ void rope_cos_sin_pair(int pos, int i, RopeStep r, float &c, float &s) {
  const int e = i & (n - 1);
  double theta = rope_theta_q<n>(i - e, r.ratio);
#pragma unroll
  for (int t = 0; t < n - 1; ++t) theta = (t < e) ? theta * r.ratio : theta;
  rope_angle_cs(pos, theta, c, s);
}
// Key angles: n pairs whose exact angles th[0 .. n) are given.
template <int n>
__device__ __forceinline__ void rope_cos_sin_run64(int pos, const double *th, double *c, double *s) {
#pragma unroll
  for (int e = 0; e < n; ++e) rope_angle_cs64(pos, th[e], c[e], s[e]);
}
// Query rotation (fp32).
__device__ __forceinline__ void rope_rotate(float &lo, float &hi, float c, float s) {
  const float l = lo, h = hi;
  lo = fmaf(l, c, -(h * s));
  hi = fmaf(h, c, l * s);
}

// fp64 -> fp32 rounded to odd: truncated, with the last bit set when the
// conversion is inexact. Rounding that to nearest in a format with at least
// two fewer significant bits (fp16, bf16) gives the nearest value of the
// original fp64, which a direct fp32 rounding first would not always give.
__device__ __forceinline__ float f64_to_f32_odd(double x) {
  const float f = (float)x;  // nearest
  const double back = (double)f;
  if (back == x || x != x) return f;
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (fabs(back) > fabs(x)) u -= 1;  // rounded away from zero: one step back
  return __builtin_bit_cast(float, u | 1u);
}


// ---------------------------------------------------------------------------
// Cross-lane sums with DPP (no LDS round trip). Every lane of an aligned group
// ends with the same bits: each step adds a value and its partner's value,
// and IEEE addition is commutative.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;   // lane i <- lane 15-i within 16 lanes
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i within 8 lanes

constexpr int kDppRowRor8 = 0x128;     // lane i <- lane (i + 8) mod 16 within 16 lanes

// Value of lane (this lane ^ 8) in a 64-lane wavefront.
__device__ __forceinline__ float lane_xor8(float x) { return dpp_mov<kDppRowRor8>(x); }

// v_permlane16_swap / v_permlane32_swap with both operands x leave, in every
// lane, the pair {x[lane], x[lane ^ 16]} (resp. ^ 32) in the two results, in
// an order that depends on the lane; sum and max are symmetric, so they need
// no select. (Lane layout checked on gfx950.)
__device__ __forceinline__ float pair_sum16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float pair_max16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float pair_max32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

// The value x holds in the lane 16 (resp. 32) apart: v_permlane16_swap with
// both operands x leaves the lower row of each pair of 16-lane rows its own
// value in the first result and the partner's in the second, the upper row
// the other way round (resp. the lower and upper 32 lanes); `upper` is this
// lane's bit 4 (resp. 5).
__device__ __forceinline__ float partner16(float x, bool upper) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)(upper ? r[0] : r[1]));
}
__device__ __forceinline__ float partner32(float x, bool upper) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)(upper ? r[0] : r[1]));
}

// Reduce over the 64 / FROM aligned groups of FROM lanes (lanes that differ
// only in the bits >= FROM): max or sum, every lane ends with the result.
// (FROM = 1: the whole wavefront.)
template <int FROM>
__device__ __forceinline__ float groups_max(float x) {
  if constexpr (FROM <= 1) x = fmaxf(x, dpp_mov<kDppQuadXor1>(x));
  if constexpr (FROM <= 2) x = fmaxf(x, dpp_mov<kDppQuadXor2>(x));
  if constexpr (FROM <= 4) x = fmaxf(x, dpp_mov<kDppHalfMirror>(x));
  if constexpr (FROM <= 8) x = fmaxf(x, lane_xor8(x));
  if constexpr (FROM <= 16) x = pair_max16(x);
  return pair_max32(x);
}
template <int FROM>
__device__ __forceinline__ float groups_sum(float x) {
  if constexpr (FROM <= 1) x += dpp_mov<kDppQuadXor1>(x);
  if constexpr (FROM <= 2) x += dpp_mov<kDppQuadXor2>(x);
  if constexpr (FROM <= 4) x += dpp_mov<kDppHalfMirror>(x);
  if constexpr (FROM <= 8) x += lane_xor8(x);
  if constexpr (FROM <= 16) x = pair_sum16(x);
  return pair_sum32(x);
}

// Max over lanes 0 .. N - 1 (N a power of two, 8 to 64), left in those
// lanes; sum over them, given to every lane. The same steps, in the same
// order, as the first ones of the wavefront reductions above.
template <int N>
__device__ __forceinline__ float lanes_max(float x) {
  static_assert(N >= 8 && N <= 64 && (N & (N - 1)) == 0, "8, 16, 32 or 64 lanes");
  if constexpr (N == 64) return groups_max<1>(x);
  x = fmaxf(x, dpp_mov<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_mov<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_mov<kDppHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, lane_xor8(x));
  if constexpr (N >= 32) x = pair_max16(x);
  return x;
}
template <int N>
__device__ __forceinline__ float lanes_sum_all(float x) {
  static_assert(N >= 8 && N <= 64 && (N & (N - 1)) == 0, "8, 16, 32 or 64 lanes");
  if constexpr (N == 64) return groups_sum<1>(x);
  x += dpp_mov<kDppQuadXor1>(x);
  x += dpp_mov<kDppQuadXor2>(x);
  x += dpp_mov<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += lane_xor8(x);
  if constexpr (N >= 32) x = pair_sum16(x);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
}

template <int LANES> __device__ __forceinline__ float group_sum(float x);
template <> __device__ __forceinline__ float group_sum<8>(float x) {
  x += dpp_mov<kDppQuadXor1>(x);
  x += dpp_mov<kDppQuadXor2>(x);
  x += dpp_mov<kDppHalfMirror>(x);
  return x;
}
template <> __device__ __forceinline__ float group_sum<16>(float x) {
  x = group_sum<8>(x);
  x += dpp_mov<kDppRowMirror>(x);
  return x;
}

// Query cos / sin of the VE rotary pairs held by lane slice `ds` of a row at
// position pos (slice ds and ds ^ (LPR/2) hold the two halves of the pairs
// (ds % (LPR/2)) * VE + e).
template <int DT>
__device__ __forceinline__ void rope_slice_cs(int ds, int pos, RopeStep r, float *c, float *s) {
  constexpr int VE = vec_elems<DT>();
  constexpr int LPR = kHeadDim / VE;
  rope_cos_sin_run<VE>(pos, (ds % (LPR / 2)) * VE, r, c, s);
}

// The 16-byte slice `ds` of a query row rotated with those cos / sin, in fp32
// (queries are not stored, so they are not rounded): `partner` is slice
// ds ^ (LPR/2) of the same row.
template <int DT>
__device__ __forceinline__ void rope_slice_f32(u32x4 mine, u32x4 partner, int ds, const float *c,
                                               const float *s, float *x) {
  constexpr int VE = vec_elems<DT>();
  constexpr int LPR = kHeadDim / VE;
  float p[VE];
  unpack16<DT>(mine, x);
  unpack16<DT>(partner, p);
  const bool is_lo = ds < LPR / 2;
#pragma unroll
  for (int e = 0; e < VE; ++e) {
    float lo = is_lo ? x[e] : p[e];
    float hi = is_lo ? p[e] : x[e];
    rope_rotate(lo, hi, c[e], s[e]);
    x[e] = is_lo ? lo : hi;
  }
}

// ---------------------------------------------------------------------------
// Handing small partial results from many workgroups to the last one to
// arrive. The partials are written with agent-scope atomic stores, which go
// through the caches that other XCDs cannot see; each thread waits for its
// stores to complete before the workgroup barrier, and one thread then counts
// the arrival with an agent-scope atomic. The last arriver reads the partials
// back with agent-scope atomic loads, which bypass those caches too, and only
// after its own count has returned. No L2 write-back or invalidate is needed
// because the handed-over data never sits in a non-coherent cache.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void publish(float *p, float v) {
  __hip_atomic_store((global_ptr<uint32_t>)p, __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish(int32_t *p, int32_t v) {
  __hip_atomic_store((global_ptr<int32_t>)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish(uint64_t *p, uint64_t v) {
  __hip_atomic_store((global_ptr<uint64_t>)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t fetch_u64(const void *p) {
  return __hip_atomic_load((global_ptr<const uint64_t>)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t fetch_u32(const void *p) {
  return __hip_atomic_load((global_ptr<const uint32_t>)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// (the asm orders the compiler's memory accesses around the wait; the
// builtin, the same wait again and free, tells the compiler's wait counting
// that nothing is outstanding, so it guards no later load with waits for
// loads issued before this point; gfx9 encoding: vmcnt 0, expcnt and lgkmcnt
// at their maxima)
__device__ __forceinline__ void wait_stores() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
}
// Returns the arrival count before this one (call from one thread).
__device__ __forceinline__ uint32_t arrive(uint32_t *counter) {
  return __hip_atomic_fetch_add((global_ptr<uint32_t>)counter, 1u, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_counter(uint32_t *counter) {
  __hip_atomic_store((global_ptr<uint32_t>)counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One rotary pair of 16-byte chunks of a new K/V row (chunk j in the first
// half of the row, j + D/2 in the second), the key rotated at position pos
// when there is a rotation, rounded to the storage type.
struct PairChunks {
  u32x4 klo, khi, vlo, vhi;
};
// One rotary pair of a new key, (lo, hi) -> (lo c - hi s, hi c + lo s) with
// the fp64 cos / sin c, s: each product and the sum rounded in fp64 (no fused
// multiply-add), then one rounding to the storage type (fp32 storage: to
// nearest; 16-bit storage: to odd here, to nearest when packed). The one
// definition of a stored rotated key.
template <int DT>
__device__ __forceinline__ void rotate_elem64(float &lo, float &hi, double c, double s) {
  const double l = lo, h = hi;
  const double lc = l * c, hs = h * s, hc = h * c, ls = l * s;
  if constexpr (DT == F32) {
    lo = (float)(lc - hs);
    hi = (float)(hc + ls);
  } else {
    lo = f64_to_f32_odd(lc - hs);
    hi = f64_to_f32_odd(hc + ls);
  }
}
// Chunk j of each half of a new key row (dims [j*VE, +VE) and their rotary
// partners [D/2 + j*VE, +VE)) rotated with the fp64 cos / sin cs, sn of those
// VE pairs.
template <int DT>
__device__ __forceinline__ void rotate_key_pair_cs(u32x4 &klo, u32x4 &khi, const double *cs,
                                                   const double *sn) {
  constexpr int VE = vec_elems<DT>();
  float lo[VE], hi[VE];
  unpack16<DT>(klo, lo);
  unpack16<DT>(khi, hi);
#pragma unroll
  for (int e = 0; e < VE; ++e) rotate_elem64<DT>(lo[e], hi[e], cs[e], sn[e]);
  klo = pack16<DT>(lo);
  khi = pack16<DT>(hi);
}
// The same at position pos, each pair's cos / sin computed just before its
// rotation (two doubles live at a time); th: the VE pairs' angles, or null
// for no rotation.
template <int DT, bool OPAQUE = false>
__device__ __forceinline__ void rotate_key_pair(u32x4 &klo, u32x4 &khi, int pos, const double *th) {
  constexpr int VE = vec_elems<DT>();
  if (th) {
    float lo[VE], hi[VE];
    unpack16<DT>(klo, lo);
    unpack16<DT>(khi, hi);
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      double c, s;
      rope_angle_cs64<OPAQUE>(pos, th[e], c, s);
      rotate_elem64<DT>(lo[e], hi[e], c, s);
    }
    klo = pack16<DT>(lo);
    khi = pack16<DT>(hi);
  }
}
// th: the angles of pairs j*VE .. j*VE + VE - 1, or null.
template <int DT, bool OPAQUE = false>
__device__ __forceinline__ void load_key_pair(const char *k_src, int j, int pos, const double *th,
                                              u32x4 &klo, u32x4 &khi) {
  constexpr int VE = vec_elems<DT>();
  constexpr int EB = Storage<DT>::bytes;
  klo = load16(k_src + j * VE * EB);
  khi = load16(k_src + (kHeadDim / 2 + j * VE) * EB);
  rotate_key_pair<DT, OPAQUE>(klo, khi, pos, th);
}

template <int DT, bool OPAQUE = false>
__device__ __forceinline__ PairChunks load_pair(const char *k_src, const char *v_src, int j,
                                                int pos, const double *th) {
  constexpr int VE = vec_elems<DT>();
  constexpr int EB = Storage<DT>::bytes;
  const int lo_off = j * VE * EB, hi_off = (kHeadDim / 2 + j * VE) * EB;
  PairChunks c;
  c.vlo = load16(v_src + lo_off);
  c.vhi = load16(v_src + hi_off);
  load_key_pair<DT, OPAQUE>(k_src, j, pos, th, c.klo, c.khi);
  return c;
}
template <int DT>
__device__ __forceinline__ void store_pair(char *k_dst, char *v_dst, int j, const PairChunks &c) {
  constexpr int VE = vec_elems<DT>();
  constexpr int EB = Storage<DT>::bytes;
  const int lo_off = j * VE * EB, hi_off = (kHeadDim / 2 + j * VE) * EB;
  store16(k_dst + lo_off, c.klo);
  store16(k_dst + hi_off, c.khi);
  store16(v_dst + lo_off, c.vlo);
  store16(v_dst + hi_off, c.vhi);
}

}  // namespace kvd
