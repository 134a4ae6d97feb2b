// MX (microscaling FP8) quantisation on the device: float32 or bfloat16 values
// -> e4m3 ("fn") codes and one E8M0 scale per 32 contiguous elements, the
// input format of the MXFP8 attention path (techfeed.io summary of "GEM
// Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation
// Model", section "MXFP8による超低精度トレーニング").  The page gives no encoding
// rule; this one takes the scale exponent floor(log2 max|x|) - 8 (8 is the
// exponent of e4m3's largest power of two), clamped to [-127, 127] and -127
// for an all-zero block, and rounds x / 2^E to the nearest e4m3 value (ties to
// even) after saturating to +-448.
//
// Streaming and HBM-bound: four lanes per 32-element block, eight elements
// each (one 16-byte bf16 load or two for f32), the block max over the four
// lanes, one 8-byte store of codes per lane and one scale byte per block; a
// lane handles four such chunks, all loaded before the first is encoded.
#include "ja_internal.h"
#include "jagged_attn.h"

namespace ja {

namespace {

constexpr int kQuantThreads = 256;

__device__ __forceinline__ unsigned e4m3_code(float y) {
  const unsigned sign = (__float_as_uint(y) >> 31) << 7;
  const float a = fminf(fabsf(y), 448.0f);
  unsigned code;
  if (a < 0.015625f) {
    // subnormal e4m3: multiples of 2^-9 (8 of them rounds up to 2^-6, code 8)
    code = unsigned(__builtin_rintf(a * 512.0f));
  } else {
    // round the float's mantissa to 3 bits, ties to even (a carry moves the
    // exponent up); the exponent is in [-6, 8] here
    unsigned b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    const unsigned e = (b >> 23) - 127u + 7u;
    code = (e << 3) | ((b >> 20) & 7u);
  }
  return code | sign;
}

constexpr int kQuantPer = 4;  // 8-element chunks per lane, loaded before any is used

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v) {
  if constexpr (sizeof(T) == 2) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const unsigned u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Lane t of the grid handles chunks t + c * n_threads, c < kQuantPer: chunk
// u is elements [8u, 8u + 8) of block u / 4, and the four lanes of a block are
// neighbours in every round.
template <typename T>
__global__ __launch_bounds__(kQuantThreads) void mx_quant_kernel(const T* __restrict__ x, int64_t n_blocks,
                                                                 uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales) {
  const int64_t n_threads = int64_t(gridDim.x) * kQuantThreads;
  const int64_t t = int64_t(blockIdx.x) * kQuantThreads + threadIdx.x;
  float v[kQuantPer][8];
#pragma unroll
  for (int c = 0; c < kQuantPer; ++c) {
    const int64_t u = t + c * n_threads;
    // (n_threads is a multiple of 4, so the four lanes of a block are all in
    // range or all out of it; those out of range take part in the shuffles
    // with zeros and store nothing)
    if (u < 4 * n_blocks) {
      load8(x + u * 8, v[c]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[c][i] = 0.f;
    }
  }
#pragma unroll
  for (int c = 0; c < kQuantPer; ++c) {
    const int64_t u = t + c * n_threads;
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
    // max over the block's four lanes (a quad): DPP quad permutations
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(amax), 0xB1, 0xF, 0xF, true)));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(amax), 0x4E, 0xF, 0xF, true)));
    // E = floor(log2 amax) - 8 from the exponent field; a zero or subnormal
    // block max gives -127 (the clamp)
    const int ex = int((__float_as_uint(amax) >> 23) & 0xFFu);
    const int E = ex == 0 ? -127 : max(-127, min(127, ex - 127 - 8));
    // 2^-E as a float: normal for -E >= -126, the subnormal 2^-127 otherwise
    const float mul = -E >= -126 ? __uint_as_float(unsigned(127 - E) << 23) : __uint_as_float(0x00400000u);
    if (u < 4 * n_blocks) {
      unsigned lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= e4m3_code(v[c][i] * mul) << (8 * i);
        hi |= e4m3_code(v[c][4 + i] * mul) << (8 * i);
      }
      *reinterpret_cast<uint2*>(codes + u * 8) = make_uint2(lo, hi);
      if ((u & 3) == 0) scales[u >> 2] = uint8_t(E + 127);
    }
  }
}

}  // namespace

hipError_t launch_mx_quant(bool bf16, const void* x, int64_t n_blocks, uint8_t* codes, uint8_t* scales,
                           hipStream_t st) {
  if (n_blocks <= 0) return hipSuccess;
  const int64_t chunks = n_blocks * 4;  // eight elements each
  const int64_t per_group = int64_t(kQuantThreads) * kQuantPer;
  const dim3 gd(unsigned((chunks + per_group - 1) / per_group)), bd(kQuantThreads);
  if (bf16)
    hipLaunchKernelGGL(mx_quant_kernel<uint16_t>, gd, bd, 0, st, reinterpret_cast<const uint16_t*>(x), n_blocks,
                       codes, scales);
  else
    hipLaunchKernelGGL(mx_quant_kernel<float>, gd, bd, 0, st, reinterpret_cast<const float*>(x), n_blocks, codes,
                       scales);
  return hipGetLastError();
}

}  // namespace ja
