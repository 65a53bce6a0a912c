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

__device__ __forceinline__ u32x4 load16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void store16(void *p, u32x4 v) {
  *reinterpret_cast<u32x4 *>(p) = v;
}

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
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> one dword of two storage elements, round to nearest even.
template <int DT> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<F16>(float lo, float hi) {
  f16x2 h;
  h[0] = (_Float16)lo;
  h[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, h);
}
template <> __device__ __forceinline__ uint32_t pack2<BF16>(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
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

// Rotary embedding of pair (i, i + D/2) at absolute position pos: angle
// pos * base^(-2i/D). The angle and its cosine/sine are evaluated in fp64 and
// rounded to fp32 once; the rotation itself is fp32.
__device__ __forceinline__ void rope_cos_sin(int pos, int i, float base, float &c, float &s) {
  const double theta = pow((double)base, -2.0 * (double)i / (double)kHeadDim);
  const double ang = (double)pos * theta;
  double sd, cd;
  sincos(ang, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}
__device__ __forceinline__ void rope_rotate(float &lo, float &hi, float c, float s) {
  const float l = lo, h = hi;
  lo = fmaf(l, c, -(h * s));
  hi = fmaf(h, c, l * s);
}

}  // namespace kvd
