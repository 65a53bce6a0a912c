// Matrix-core pieces shared by the attention tiles on gfx950: the
// 16x16x32 fp16/bf16 MFMA, rounding eight floats into the storage type, the
// high/low split that feeds an fp32 operand to a 16-bit MFMA, and the byte
// permutation that builds a transposed V operand from 8-byte row chunks.
#pragma once

#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {

constexpr int kMfmaRows = 16;  // query rows per MFMA tile
constexpr int kMfmaStep = 32;  // keys per MFMA step

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Eight floats rounded to nearest-even into the storage type (bf16 through
// the hardware conversion, v_cvt_pk_bf16_f32).
template <int DT>
__device__ __forceinline__ u32x4 round8(const float *x) {
  if constexpr (DT == BF16) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[2 * i], x[2 * i + 1]}, bf16x2));
    return v;
  } else {
    return pack16<DT>(x);
  }
}

// x as a high and a low part in the storage type: hi = round(x), lo = round(x - hi).
template <int DT>
__device__ __forceinline__ void split_hi_lo(const float *x, u32x4 &hi, u32x4 &lo) {
  float h[8], r[8];
  hi = round8<DT>(x);
  unpack16<DT>(hi, h);
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = x[e] - h[e];
  lo = round8<DT>(r);
}

__device__ __forceinline__ void store_f32x4(float *p, f32x4 v) { *(global_ptr<f32x4>)p = v; }

// Element t (0..3) of two 8-byte chunks as one dword: (c0's, c1's << 16).
template <int t>
__device__ __forceinline__ uint32_t pair16(u32x2 c0, u32x2 c1) {
  constexpr uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
  return __builtin_amdgcn_perm(c1[t >> 1], c0[t >> 1], sel);
}

}  // namespace kvd
