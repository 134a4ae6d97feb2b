// Jagged attention forward in fp32 (fp32 in, fp32 accumulate, fp32 out).
//
// The fp32 path exists for exactness checks at 1e-5 relative error, where
// bf16 operands would be far too coarse; its workloads are small (a few
// hundred tokens), so it is latency-bound and uses plain VALU arithmetic:
// one lane per query row, keys streamed through the cache (every lane of a
// wave reads the same key row, a broadcast).  Same semantics as the MFMA
// path: softmax over the sample's keys (optionally the 64-token block window
// of the "BlockAttention" section of the techfeed.io summary of "GEM
// Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation
// Model", or the token sliding window it grew out of), or RMS-normalised
// GELU-tanh scores divided by the key count (same page, "Generalized
// Dot-Product Attention（GDPA）").
#include "ja_device.h"
#include "jagged_attn.h"

namespace ja {

namespace {

constexpr int kF32Rows = 64;  // query rows per work item (one wave)

// WMODE: 0 all keys, 1 block window, 2 token sliding window.
template <int D, int ACT, int WMODE>
__global__ __launch_bounds__(kF32Rows) void attn_f32_kernel(AttnArgs a) {
  const int n_items = a.hdr->n_items;
  const float* qv = reinterpret_cast<const float*>(a.q);
  const float* kv = reinterpret_cast<const float*>(a.k);
  const float* vv = reinterpret_cast<const float*>(a.v);
  float* out = reinterpret_cast<float*>(a.out);
  for (int idx = blockIdx.x; idx < n_items; idx += gridDim.x) {
    const WorkItem it = a.items[idx];
    const int h = it.h, q0 = it.q0;
    const int qbeg = it.qbeg, lq = it.lq;
    const int kbeg = it.kbeg, lk = it.lk;
    const int qrow = q0 + int(threadIdx.x);
    if (qrow >= lq) continue;
    float q[D], o[D];
    const float* qp = qv + (size_t(qbeg + qrow) * a.H + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      q[d] = qp[d];
      o[d] = 0.f;
    }
    float rq = 1.f;
    if constexpr (ACT != ACT_SOFTMAX) {
      float ss = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) ss = fmaf(q[d], q[d], ss);
      rq = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
    }
    int lo = 0, hi = lk;
    if constexpr (WMODE == 1) {
      const int blk = qrow / kBlock;
      lo = max(0, blk - a.window_blocks + 1) * kBlock;
      hi = min(lk, (blk + 1) * kBlock);
    } else if constexpr (WMODE == 2) {
      lo = max(0, qrow - a.window_tokens + 1);
      hi = min(lk, qrow + 1);
    }
    float m = -__builtin_huge_valf(), l = 0.f;
    for (int j = lo; j < hi; ++j) {
      const float* kp = kv + (size_t(kbeg + j) * a.H + h) * D;
      const float* vp = vv + (size_t(kbeg + j) * a.H + h) * D;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(q[d], kp[d], s);
      float p;
      if constexpr (ACT == ACT_SOFTMAX) {
        const float x = s * a.score_scale;  // log2 units
        if (x > m) {
          const float alpha = exp2f(m - x);
          l *= alpha;
#pragma unroll
          for (int d = 0; d < D; ++d) o[d] *= alpha;
          m = x;
        }
        p = exp2f(x - m);
        l += p;
      } else {
        float ss = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) ss = fmaf(kp[d], kp[d], ss);
        const float rk = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
        const float x = s * rq * rk * a.score_scale;
        if constexpr (ACT == ACT_GELU_POLY) {
          p = gelu_poly(x);
        } else {
          constexpr float kC = 0.7978845608028654f;
          p = 0.5f * x * (1.0f + tanhf(kC * fmaf(0.044715f * x, x * x, x)));
        }
      }
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, vp[d], o[d]);
    }
    float scale;
    if constexpr (ACT == ACT_SOFTMAX) scale = l > 0.f ? 1.0f / l : 0.f;
    else scale = lk > 0 ? 1.0f / float(lk) : 0.f;
    float* op = out + (size_t(qbeg + qrow) * a.H + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = o[d] * scale;
  }
}

template <int D>
hipError_t launch_d(int act, int window_mode, const AttnArgs& a, int grid, const KTiming& tm, hipStream_t st) {
  const dim3 gd(grid), bd(kF32Rows);
  if (act == ACT_GELU) return launch1(attn_f32_kernel<D, ACT_GELU, 0>, gd, bd, st, a, tm);
  if (act == ACT_GELU_POLY) return launch1(attn_f32_kernel<D, ACT_GELU_POLY, 0>, gd, bd, st, a, tm);
  if (window_mode == 1) return launch1(attn_f32_kernel<D, ACT_SOFTMAX, 1>, gd, bd, st, a, tm);
  if (window_mode == 2) return launch1(attn_f32_kernel<D, ACT_SOFTMAX, 2>, gd, bd, st, a, tm);
  return launch1(attn_f32_kernel<D, ACT_SOFTMAX, 0>, gd, bd, st, a, tm);
}

}  // namespace

// grid: workgroups of the grid-stride loop over the work items.
hipError_t launch_attn_f32(int D, int act, int window_mode, const AttnArgs& a, int grid, const KTiming& tm,
                           hipStream_t st) {
  if (D == 32) return launch_d<32>(act, window_mode, a, grid, tm, st);
  if (D == 64) return launch_d<64>(act, window_mode, a, grid, tm, st);
  return launch_d<128>(act, window_mode, a, grid, tm, st);
}

}  // namespace ja
