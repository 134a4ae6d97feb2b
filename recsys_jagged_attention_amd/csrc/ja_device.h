// Device helpers for the gfx950 (CDNA4) jagged attention kernels.
#pragma once

#include <hip/hip_ext.h>

#include "ja_gelu_poly.h"
#include "ja_internal.h"

namespace ja {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// D(32x32) += A(32x16) * B(16x32), bf16 operands, fp32 accumulate.
// Lane l supplies A[l%32][8*(l/32) .. +8) and B[8*(l/32) .. +8)[l%32]; the
// result register i of lane l holds C[8*(i/4) + 4*(l/32) + i%4][l%32].
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum and max of lane l's value and lane l^32's (the two 32-lane halves that
// hold one MFMA column), on the VALU: v_permlane32_swap with both operands x
// leaves the pair {x[l], x[l^32]} in lane l (its order depends on the half,
// which a symmetric operation does not see, so every lane gets the same bits).
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Decode 8 e4m3 ("fn") codes (little-endian in a u32x2) scaled by 2^(e8m0-127)
// into bf16.  Exact: an e4m3 value has at most 4 significant bits and the
// product with a power of two fits bf16 unless it leaves bf16's exponent range.
__device__ __forceinline__ bf16x8 decode_mx8(u32x2 codes, unsigned scale_byte) {
  // 2^(E-127) as a float; E == 0 gives the subnormal 2^-127, E == 255 is NaN.
  const unsigned sb = scale_byte & 0xFFu;
  const float s = sb == 0 ? __uint_as_float(0x00400000u)
                          : (sb == 255u ? __builtin_nanf("") : __uint_as_float(sb << 23));
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const unsigned c = (codes[j >> 2] >> (8 * (j & 3))) & 0xFFu;
    const unsigned e = (c >> 3) & 0xFu, m = c & 7u;
    // |value| = (e ? 8+m : m) * 2^(max(e,1) - 10)
    const float mag = float(e ? (8u + m) : m) * __uint_as_float((max(e, 1u) + 117u) << 23);
    float v = (c & 0x80u) ? -mag : mag;
    if (e == 15u && m == 7u) v = __builtin_nanf("");
    r[j] = (__bf16)(v * s);
  }
  return r;
}

// Launch a kernel of one by-value argument on `st`; with events in `tm` the
// dispatch itself records its start and end time into them (no separate
// event packets around the launch).
template <typename A>
inline hipError_t launch1(void (*kernel)(A), dim3 grid, dim3 block, hipStream_t st, const A& arg,
                          const KTiming& tm) {
  void* args[] = {const_cast<A*>(&arg)};
  if (tm.start || tm.stop)
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, st, tm.start, tm.stop, 0);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, st);
}

// gelu_tanh(x) = x * sigmoid(2u), u = sqrt(2/pi) (x + 0.044715 x^3):
// the identity 1 + tanh(u) = 2 sigmoid(2u) needs one exp2 and one reciprocal.
// The exponent -2 log2(e) u is taken as x (kB + kA x^2): two multiplies per
// score fewer than forming u first.
__device__ __forceinline__ float gelu_tanh(float x) {
  constexpr float kB = static_cast<float>(-2.0 * 1.4426950408889634 * 0.7978845608028654);  // -2 log2(e) sqrt(2/pi)
  constexpr float kA = static_cast<float>(-2.0 * 1.4426950408889634 * 0.7978845608028654 * 0.044715);
  const float e = fast_exp2(x * fmaf(kA, x * x, kB));
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// gelu(x) = x t and gelu'(x) = t + 2 x t (1 - t) u'(x), where t = sigmoid(2u),
// u = sqrt(2/pi) (x + 0.044715 x^3) (from 1 + tanh(u) = 2 sigmoid(2u)); the
// backward's form, with IEEE division and exp2f.
__device__ __forceinline__ void gelu_and_grad(float x, float& g, float& gp) {
  constexpr float kC = 0.7978845608028654f;  // sqrt(2/pi)
  constexpr float kA = 0.044715f;
  const float u = kC * fmaf(kA * x, x * x, x);
  const float t = 1.0f / (1.0f + exp2f(-2.0f * 1.4426950408889634f * u));
  g = x * t;
  gp = fmaf(2.0f * x * t * (1.0f - t), kC * fmaf(3.0f * kA, x * x, 1.0f), t);
}

// The GELU of a score for the GELU-family activations.
template <int ACT>
__device__ __forceinline__ float gelu_act(float x) {
  if constexpr (ACT == ACT_GELU_POLY) return gelu_poly(x);
  else return gelu_tanh(x);
}

}  // namespace ja
