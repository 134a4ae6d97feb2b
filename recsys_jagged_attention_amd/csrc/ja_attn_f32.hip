// Jagged attention forward in fp32 (fp32 in, fp32 accumulate, fp32 out).
//
// The fp32 path exists for exactness checks at 1e-5 relative error, where
// bf16 operands would be far too coarse; its workloads are small (a few
// hundred tokens), so it is latency-bound and uses plain VALU arithmetic.
// Same semantics as the MFMA path: softmax over the sample's keys
// (optionally the 64-token block window of the "BlockAttention" section of
// the techfeed.io summary of "GEM Training: How Meta Doubled the Efficiency
// of Its LLM-Scale Ads Foundation Model", or the token sliding window it grew
// out of), or RMS-normalised GELU-tanh scores divided by the key count (same
// page, "Generalized Dot-Product Attention（GDPA）").
//
// One workgroup per work item (64 query rows of one sample and head, one row
// per lane).  The item's keys are split into NW contiguous chunks, one per
// wave, so that the per-key chain (dot product, softmax update, P V) runs NW
// times shorter; every wave keeps its own (m, l, O) for its 64 rows, and the
// partials are merged through LDS in wave order (softmax: rescaled to the
// largest m; GELU: summed), so the result does not depend on the grid.
// Each wave stages its keys' K and V rows, 32 keys at a time, in its own
// part of that LDS area (free until the partials are written), with all
// lanes loading at once: one round trip to memory per 32 keys instead of one
// per key, and the key loop then reads broadcast LDS.
#include "ja_device.h"
#include "jagged_attn.h"

namespace ja {

namespace {

constexpr int kF32Rows = 64;  // query rows per work item (one lane each)

template <int D>
struct F32Shape {
  static constexpr int kWaves = D == 128 ? 4 : 8;  // key chunks per item (LDS: kWaves x 64 x (D+1) floats)
  static constexpr int kStride = D + 1;            // floats per partial row in LDS (odd: no bank conflicts)
  static constexpr int kStage = 32;                // keys staged per round (2 x 32 x D floats fit 64 x (D+1))
  // waves per SIMD the registers must leave room for: at D = 32 two
  // workgroups per CU (LDS: 2 x 71.5 KB), else one
  static constexpr int kMinWavesPerSimd = D == 32 ? 4 : 1;
};

// WMODE: 0 all keys, 1 block window, 2 token sliding window.
template <int D, int ACT, int WMODE>
__global__ __launch_bounds__(64 * F32Shape<D>::kWaves, F32Shape<D>::kMinWavesPerSimd) void attn_f32_kernel(
    AttnArgs a) {
  constexpr int NW = F32Shape<D>::kWaves, kS = F32Shape<D>::kStride;
  __shared__ __attribute__((aligned(16))) float s_o[NW * kF32Rows * kS];
  __shared__ float s_m[NW * kF32Rows], s_l[NW * kF32Rows];
  const int n_items = a.hdr->n_items;
  const float* qv = reinterpret_cast<const float*>(a.q);
  const float* kv = reinterpret_cast<const float*>(a.k);
  const float* vv = reinterpret_cast<const float*>(a.v);
  float* out = reinterpret_cast<float*>(a.out);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int idx = blockIdx.x; idx < n_items; idx += gridDim.x) {
    const WorkItem it = a.items[idx];
    const int h = it.h, q0 = it.q0;
    const int qbeg = it.qbeg, lq = it.lq;
    const int kbeg = it.kbeg, lk = it.lk;
    // (rows past the sample compute on its last row and are not stored)
    const int qrow = min(q0 + lane, lq - 1);
    // keys of this lane's row, and their union over the item's rows (items
    // start at multiples of 64 rows, so a block window is the same for all)
    int lo = 0, hi = lk, ulo = 0, uhi = lk;
    if constexpr (WMODE == 1) {
      const int blk = q0 / kBlock;
      lo = ulo = max(0, blk - a.window_blocks + 1) * kBlock;
      hi = uhi = min(lk, (blk + 1) * kBlock);
    } else if constexpr (WMODE == 2) {
      lo = max(0, qrow - a.window_tokens + 1);
      hi = min(lk, qrow + 1);
      ulo = max(0, q0 - a.window_tokens + 1);
      uhi = min(lk, min(q0 + kF32Rows, lq));
    }
    // this wave's chunk of the union (the same for all lanes: the stage is shared)
    const int chunk = (max(uhi - ulo, 0) + NW - 1) / NW;
    const int jlo = ulo + wave * chunk, jhi = min(ulo + (wave + 1) * chunk, uhi);
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
    float m = -__builtin_huge_valf(), l = 0.f;
    constexpr int SK = F32Shape<D>::kStage, kPieces = 2 * SK * D / (4 * 64);  // 16-byte loads per lane
    static_assert(2 * SK * D <= kF32Rows * kS, "a stage fits the wave's partial area");
    float* stage = s_o + wave * kF32Rows * kS;  // K rows [SK][D], then V rows [SK][D]
    for (int j = jlo; j < jhi; ++j) {
      const int js = (j - jlo) % SK;
      if (js == 0) {
        // stage keys j .. j+SK-1 (those below jhi): piece p, lane: 16 bytes at
        // float offset 4 (64 p + lane) of the stage
        const int nk = min(SK, jhi - j);
#pragma unroll 8
        for (int pc = 0; pc < kPieces; ++pc) {
          const int f = 4 * (64 * pc + lane);
          const bool is_v = f >= SK * D;
          const int fk = is_v ? f - SK * D : f;
          const int key = fk / D, col = fk % D;
          if (key < nk) {
            const float* src = (is_v ? vv : kv) + (size_t(kbeg + j + key) * a.H + h) * D + col;
            *reinterpret_cast<float4*>(stage + f) = *reinterpret_cast<const float4*>(src);
          }
        }
      }
      if (j < lo || j >= hi) continue;  // (sliding window: keys outside this row's)
      const float* kp = stage + js * D;
      const float* vp = stage + SK * D + js * D;
      // q . k as four independent partial sums (a dependent chain of D fmas
      // would set the pace)
      float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int d = 0; d < D; ++d) s4[d & 3] = fmaf(q[d], kp[d], s4[d & 3]);
      const float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
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
        float k4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < D; ++d) k4[d & 3] = fmaf(kp[d], kp[d], k4[d & 3]);
        const float ss = (k4[0] + k4[1]) + (k4[2] + k4[3]);
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
    // partials of this wave's chunk
    float* po = s_o + (wave * kF32Rows + lane) * kS;
#pragma unroll
    for (int d = 0; d < D; ++d) po[d] = o[d];
    s_m[wave * kF32Rows + lane] = m;
    s_l[wave * kF32Rows + lane] = l;
    __syncthreads();
    // merge, in wave order: thread t takes row t % 64 and dims t / 64 + NW i
    {
      const int r = threadIdx.x & 63, dg = threadIdx.x >> 6;
      const int orow = q0 + r;
      float c[NW];
      float scale;
      if constexpr (ACT == ACT_SOFTMAX) {
        float mx = -__builtin_huge_valf();
#pragma unroll
        for (int w = 0; w < NW; ++w) mx = fmaxf(mx, s_m[w * kF32Rows + r]);
        float lt = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float mw = s_m[w * kF32Rows + r];
          c[w] = mw == -__builtin_huge_valf() ? 0.f : exp2f(mw - mx);
          lt = fmaf(c[w], s_l[w * kF32Rows + r], lt);
        }
        scale = lt > 0.f ? 1.0f / lt : 0.f;
        // log-sum-exp output: m is in log2 units of the scaled scores, so
        // ln(sum_j exp(s_j / sqrt(D))) = (mx + log2 lt) ln 2 (-inf without keys)
        if (a.lse != nullptr && dg == 0 && orow < lq)
          a.lse[size_t(qbeg + orow) * a.H + h] =
              lt > 0.f ? (mx + log2f(lt)) * 0.69314718055994531f : -__builtin_huge_valf();
      } else {
#pragma unroll
        for (int w = 0; w < NW; ++w) c[w] = 1.f;
        scale = lk > 0 ? 1.0f / float(lk) : 0.f;
      }
      if (orow < lq) {
        float* op = out + (size_t(qbeg + orow) * a.H + h) * D;
        for (int d = dg; d < D; d += NW) {
          float acc = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) acc = fmaf(c[w], s_o[(w * kF32Rows + r) * kS + d], acc);
          op[d] = acc * scale;
        }
      }
    }
    __syncthreads();  // (the LDS partials are rewritten by the next item)
  }
}

template <int D>
hipError_t launch_d(int act, int window_mode, const AttnArgs& a, int grid, const KTiming& tm, hipStream_t st) {
  const dim3 gd(grid), bd(64 * F32Shape<D>::kWaves);
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
