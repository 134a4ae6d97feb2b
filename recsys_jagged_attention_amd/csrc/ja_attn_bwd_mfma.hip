// Backward of jagged softmax attention on bf16 MFMA (training; the chain rule
// of the forward as defined -- the pages, e.g. the techfeed.io summary of
// "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads
// Foundation Model", describe the training system but not its backward):
//   P = softmax(Q K^T / sqrt(D)),  dV = P^T dO,  dS = P * (dO V^T - D_i),
//   D_i = rowsum(P * (dO V^T)),    dQ = dS K / sqrt(D),  dK = dS^T Q / sqrt(D).
//
// Two kernels of two waves each, 32 rows per wave, all products on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation (P and dS enter their
// products in bf16, as P does in the forward):
//  * bwd_dq_mfma_kernel, 64 query rows per item.  Lane column = query.  Over
//    the item's key tiles it forms S^T = K Q^T and dP^T = V dO^T; a first pass
//    keeps the online max, sum and sum of p * dP (giving the log-sum-exp and
//    D_i, stored for the second kernel), a second pass accumulates
//    dQ^T += K^T dS^T.
//  * bwd_dkv_mfma_kernel, 64 key rows per item (kept in LDS).  Lane column =
//    key.  Over the 32-query tiles that see the item it forms S = Q K^T and
//    dP = dO V^T, P from the stored statistics, then dV^T += dO^T P and
//    dK^T += Q^T dS.
// The score products read their A rows in key_perm order so that the result
// registers of lane half h hold, for each 16-row step, the 8 contiguous rows
// 8h..8h+7: exactly the B operand of the next product (no shuffle).  The
// transposed A operands (K^T, dO^T, Q^T) come from ds_read_b64_tr_b16 on
// row-major LDS tiles.  Plain synchronous tile loads; several workgroups per
// CU hide their latency.
#include "ja_mfma_util.h"
#include "jagged_attn.h"

namespace ja {
namespace {

constexpr int kMT = 128;  // two waves

template <int D>
struct BT {
  static constexpr int kRS = D + 8;  // LDS row stride in bf16 (16-byte pad: rows 4 banks apart)
  static constexpr int kS = D / 16;  // k-steps over D
  static constexpr int kT = D / 32;  // 32-row output tiles over D
};

// Rows [0, nrows) of a global [*, H, D] slice (row stride `gstride` elements)
// into an LDS tile with row stride kRS; rows >= valid are zero-filled.
template <int D, int NROWS>
__device__ __forceinline__ void load_tile(__bf16* lds, const __bf16* g, size_t gstride, int valid) {
  constexpr int kChunks = D / 8;
#pragma unroll 4
  for (int c = threadIdx.x; c < NROWS * kChunks; c += kMT) {
    const int r = c / kChunks, cc = c % kChunks;
    bf16x8 x = zero8();
    if (r < valid) x = *reinterpret_cast<const bf16x8*>(g + size_t(r) * gstride + 8 * cc);
    *reinterpret_cast<bf16x8*>(lds + r * BT<D>::kRS + 8 * cc) = x;
  }
}

// A operand (row `row` of a row-major tile, k-step cc): lane half g supplies
// dims (D/2) g + 8 cc .. +8.  B operands held in registers use the same split.
template <int D>
__device__ __forceinline__ bf16x8 read_a(const __bf16* lds, int row, int g, int cc) {
  return *reinterpret_cast<const bf16x8*>(lds + row * BT<D>::kRS + (D / 2) * g + 8 * cc);
}

// Transposed A operand X^T (row d = 32 t + lane%32, k = tile rows
// row0 + 8 (lane/32) + 0..7) of a row-major tile, by two transpose reads.
// In each 16-lane group, lane 4j + q addresses row row0 + 8 (lane/32) + j
// (+4 for the second read) at dims 32 t + 16 ((lane/16)%2) + 4q; lane i of the
// group then receives element i%4 of the chunks addressed by lanes 4j + i/4.
template <int D>
__device__ __forceinline__ bf16x8 read_at(const __bf16* lds, int row0, int t, int lane) {
  const int grp = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
  const __bf16* p = lds + (row0 + 8 * (grp >> 1) + j) * BT<D>::kRS + 32 * t + 16 * (grp & 1) + 4 * q;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * BT<D>::kRS));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
  u32x4 w;
  w[0] = lo2[0];
  w[1] = lo2[1];
  w[2] = hi2[0];
  w[3] = hi2[1];
  return __builtin_bit_cast(bf16x8, w);
}

// Registers 8 (kc%2) .. +8 of a score block as the bf16 B operand of k-step kc.
__device__ __forceinline__ bf16x8 to_b(const f32x16& c, int half) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)c[8 * half + e];
  return r;
}

// Tile-local row (key or query) of result register i in lane half g, for A
// rows read in key_perm order.
__device__ __forceinline__ int c_row(int i, int g) { return key_perm(8 * (i >> 2) + 4 * g + (i & 3)); }

// Keys [lo, hi) seen by the 32 queries r0 .. r0+31 of one wave (sample-local;
// empty when r0 >= lq).  Block items start on a 64-row boundary, so the 32
// rows share one block.
template <int WMODE>
__device__ __forceinline__ void wave_keys(const BwdArgs& a, int r0, int lq, int lk, int& lo, int& hi) {
  lo = 0;
  hi = r0 < lq ? lk : 0;
  if constexpr (WMODE == 1) {
    const int blk = r0 / kBlock;
    lo = max(0, blk - a.window_blocks + 1) * kBlock;
    hi = r0 < lq ? min(lk, (blk + 1) * kBlock) : 0;
  } else if constexpr (WMODE == 2) {
    lo = max(0, r0 - a.window_tokens + 1);
    hi = r0 < lq ? min(lk, min(r0 + 31, lq - 1) + 1) : 0;
  }
}

// Queries [lo, hi) that see the 32 keys k0 .. k0+31 of one wave.
template <int WMODE>
__device__ __forceinline__ void wave_queries(const BwdArgs& a, int k0, int lq, int lk, int& lo, int& hi) {
  lo = 0;
  hi = k0 < lk ? lq : 0;
  if constexpr (WMODE == 1) {
    const int blk = k0 / kBlock;
    lo = min(lq, blk * kBlock);
    hi = k0 < lk ? min(lq, (blk + a.window_blocks) * kBlock) : 0;
  } else if constexpr (WMODE == 2) {
    lo = min(lq, k0);
    hi = k0 < lk ? min(lq, min(k0 + 31, lk - 1) + a.window_tokens) : 0;
  }
}

// Does query i see key j (both sample-local, both in range)?
template <int WMODE>
__device__ __forceinline__ bool allowed(const BwdArgs& a, int i, int j) {
  if constexpr (WMODE == 1) {
    const int bi = i / kBlock, bj = j / kBlock;
    return bj <= bi && bi - bj < a.window_blocks;
  } else if constexpr (WMODE == 2) {
    return j <= i && i - j < a.window_tokens;
  } else {
    return true;
  }
}

template <int D, int WMODE>
__global__ __launch_bounds__(kMT) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_mfma_kernel(BwdArgs a) {
  using L = BT<D>;
  __shared__ __attribute__((aligned(16))) __bf16 ks[64 * L::kRS];
  __shared__ __attribute__((aligned(16))) __bf16 vs[64 * L::kRS];
  const __bf16* qg = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* kg = reinterpret_cast<const __bf16*>(a.k);
  const __bf16* vg = reinterpret_cast<const __bf16*>(a.v);
  const __bf16* gg = reinterpret_cast<const __bf16*>(a.dout);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int kp = key_perm(l32);
  const size_t gstride = size_t(a.H) * D;
  const int n_items = a.hdr_q->n_items;
  for (int idx = blockIdx.x; idx < n_items; idx += gridDim.x) {
    const WorkItem it = a.items_q[idx];
    const int r0 = it.q0 + 32 * wave;
    const int qrow = r0 + l32;
    const int qr = min(qrow, it.lq - 1);
    bf16x8 qf[L::kS], gf[L::kS];
    {
      const size_t off = (size_t(it.qbeg + qr) * a.H + it.h) * D + (D / 2) * g;
#pragma unroll
      for (int cc = 0; cc < L::kS; ++cc) {
        qf[cc] = *reinterpret_cast<const bf16x8*>(qg + off + 8 * cc);
        gf[cc] = *reinterpret_cast<const bf16x8*>(gg + off + 8 * cc);
      }
    }
    int klo, khi, olo, ohi;
    wave_keys<WMODE>(a, r0, it.lq, it.lk, klo, khi);
    wave_keys<WMODE>(a, it.q0 + 32 * (1 - wave), it.lq, it.lk, olo, ohi);
    const int wt_lo = klo / 64, wt_hi = khi > klo ? (khi + 63) / 64 : wt_lo;
    const int ot_lo = olo / 64, ot_hi = ohi > olo ? (ohi + 63) / 64 : ot_lo;
    int t_lo = min(wt_hi > wt_lo ? wt_lo : 1 << 30, ot_hi > ot_lo ? ot_lo : 1 << 30);
    const int t_hi = max(wt_hi > wt_lo ? wt_hi : 0, ot_hi > ot_lo ? ot_hi : 0);
    if (t_lo > t_hi) t_lo = t_hi;
    const __bf16* kbase = kg + size_t(it.kbeg) * gstride + size_t(it.h) * D;
    const __bf16* vbase = vg + size_t(it.kbeg) * gstride + size_t(it.h) * D;

    // Scores and dP^T of keys 64 t + 32 kb .. +32 for this wave's queries
    // (one 32-key block at a time keeps the live registers down).
    auto scores = [&](int t, int kb, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
      f32x16 x = {}, y = {};
#pragma unroll
      for (int cc = 0; cc < L::kS; ++cc) {
        x = mfma_32x32x16(read_a<D>(ks, 32 * kb + kp, g, cc), qf[cc], x);
        y = mfma_32x32x16(read_a<D>(vs, 32 * kb + kp, g, cc), gf[cc], y);
      }
      // scale to log2 units; disallowed and ragged keys -> -inf
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = 64 * t + 32 * kb + c_row(i, g);
        const bool ok = j < it.lk && allowed<WMODE>(a, qrow, j);
        x[i] = ok ? x[i] * a.c2 : -__builtin_huge_valf();
      }
      s = x;
      dp = y;
    };
    auto load_kv = [&](int t) __attribute__((always_inline)) {
      __syncthreads();  // the previous tile's readers are done
      const int valid = min(64, it.lk - 64 * t);
      load_tile<D, 64>(ks, kbase + size_t(64 * t) * gstride, gstride, valid);
      load_tile<D, 64>(vs, vbase + size_t(64 * t) * gstride, gstride, valid);
      __syncthreads();
    };

    // Pass 1: log-sum-exp (base 2) and D_i = sum_j p_ij dP_ij.
    float m = -__builtin_huge_valf(), l = 0.f, acc = 0.f;
    for (int t = t_lo; t < t_hi; ++t) {
      load_kv(t);
      if (t < wt_lo || t >= wt_hi) continue;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 s, dp;
        scores(t, kb, s, dp);
        float mx = -__builtin_huge_valf();
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
        const float mn = fmaxf(m, max_halves(mx));
        // (no branch: the MFMAs of the next block run with the whole wave)
        const float mref = mn == -__builtin_huge_valf() ? 0.f : mn;  // nothing allowed yet
        const float sc = exp2f(m - mref);                             // m = -inf -> 0
        l *= sc;
        acc *= sc;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = exp2f(s[i] - mref);
          l += p;
          acc = fmaf(p, dp[i], acc);
        }
        m = mn;
      }
    }
    l = sum_halves(l);
    acc = sum_halves(acc);
    const float lse = l > 0.f ? m + log2f(l) : 0.f;
    const float di = l > 0.f ? acc / l : 0.f;
    if (g == 0 && qrow < it.lq) a.stats[size_t(it.qbeg + qrow) * a.H + it.h] = make_float2(lse, di);

    // Pass 2: dQ^T += K^T dS^T.
    f32x16 dq[L::kT];
#pragma unroll
    for (int t2 = 0; t2 < L::kT; ++t2) dq[t2] = f32x16{};
    for (int t = t_lo; t < t_hi; ++t) {
      load_kv(t);
      if (t < wt_lo || t >= wt_hi) continue;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 s, dp;
        scores(t, kb, s, dp);
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = exp2f(s[i] - lse) * (dp[i] - di);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const bf16x8 db = to_b(s, half);
#pragma unroll
          for (int t2 = 0; t2 < L::kT; ++t2)
            dq[t2] = mfma_32x32x16(read_at<D>(ks, 32 * kb + 16 * half, t2, lane), db, dq[t2]);
          __builtin_amdgcn_sched_barrier(0);  // (bounds the operand reads in flight: registers)
        }
      }
    }
    if (qrow < it.lq) {
      float* out = a.dq + (size_t(it.qbeg + qrow) * a.H + it.h) * D;
#pragma unroll
      for (int t2 = 0; t2 < L::kT; ++t2)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          float4 w;
          w.x = dq[t2][4 * gi + 0] * a.inv_sqrt_d;
          w.y = dq[t2][4 * gi + 1] * a.inv_sqrt_d;
          w.z = dq[t2][4 * gi + 2] * a.inv_sqrt_d;
          w.w = dq[t2][4 * gi + 3] * a.inv_sqrt_d;
          *reinterpret_cast<float4*>(out + 32 * t2 + 8 * gi + 4 * g) = w;
        }
    }
  }
}

template <int D, int WMODE>
__global__ __launch_bounds__(kMT) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dkv_mfma_kernel(BwdArgs a) {
  using L = BT<D>;
  __shared__ __attribute__((aligned(16))) __bf16 kst[64 * L::kRS];  // the item's keys and values
  __shared__ __attribute__((aligned(16))) __bf16 vst[64 * L::kRS];
  __shared__ __attribute__((aligned(16))) __bf16 qs[32 * L::kRS];   // one 32-query tile and its dO
  __shared__ __attribute__((aligned(16))) __bf16 gs[32 * L::kRS];
  __shared__ float2 st[32];
  const __bf16* qg = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* kg = reinterpret_cast<const __bf16*>(a.k);
  const __bf16* vg = reinterpret_cast<const __bf16*>(a.v);
  const __bf16* gg = reinterpret_cast<const __bf16*>(a.dout);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int kp = key_perm(l32);
  const size_t gstride = size_t(a.H) * D;
  const int n_items = a.hdr_k->n_items;
  for (int idx = blockIdx.x; idx < n_items; idx += gridDim.x) {
    // (items over key tiles: the plan ran on the swapped offsets, so the
    // record's "query" fields describe keys and its "key" fields queries)
    const WorkItem it = a.items_k[idx];
    const int lk = it.lq, lq = it.lk, kbeg = it.qbeg, qbeg = it.kbeg;
    const int k0 = it.q0 + 32 * wave;
    const int krow = k0 + l32;
    // K and V rows of the item stay in LDS (B operands read per use: the
    // dK^T and dV^T accumulators take the registers).
    __syncthreads();  // the previous item's readers are done
    {
      const int valid = min(64, lk - it.q0);
      const size_t off = size_t(kbeg + it.q0) * gstride + size_t(it.h) * D;
      load_tile<D, 64>(kst, kg + off, gstride, valid);
      load_tile<D, 64>(vst, vg + off, gstride, valid);
    }
    int qlo, qhi, olo, ohi;
    wave_queries<WMODE>(a, k0, lq, lk, qlo, qhi);
    wave_queries<WMODE>(a, it.q0 + 32 * (1 - wave), lq, lk, olo, ohi);
    const int wt_lo = qlo / 32, wt_hi = qhi > qlo ? (qhi + 31) / 32 : wt_lo;
    const int ot_lo = olo / 32, ot_hi = ohi > olo ? (ohi + 31) / 32 : ot_lo;
    int t_lo = min(wt_hi > wt_lo ? wt_lo : 1 << 30, ot_hi > ot_lo ? ot_lo : 1 << 30);
    const int t_hi = max(wt_hi > wt_lo ? wt_hi : 0, ot_hi > ot_lo ? ot_hi : 0);
    if (t_lo > t_hi) t_lo = t_hi;
    const __bf16* qbase = qg + size_t(qbeg) * gstride + size_t(it.h) * D;
    const __bf16* gbase = gg + size_t(qbeg) * gstride + size_t(it.h) * D;

    f32x16 dk[L::kT], dv[L::kT];
#pragma unroll
    for (int t2 = 0; t2 < L::kT; ++t2) {
      dk[t2] = f32x16{};
      dv[t2] = f32x16{};
    }
    for (int t = t_lo; t < t_hi; ++t) {
      __syncthreads();  // the previous tile's readers are done
      const int valid = min(32, lq - 32 * t);
      load_tile<D, 32>(qs, qbase + size_t(32 * t) * gstride, gstride, valid);
      load_tile<D, 32>(gs, gbase + size_t(32 * t) * gstride, gstride, valid);
      if (threadIdx.x < 32)
        st[threadIdx.x] = int(threadIdx.x) < valid
                              ? a.stats[size_t(qbeg + 32 * t + int(threadIdx.x)) * a.H + it.h]
                              : make_float2(0.f, 0.f);
      __syncthreads();
      if (t < wt_lo || t >= wt_hi) continue;
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int cc = 0; cc < L::kS; ++cc) {
        s = mfma_32x32x16(read_a<D>(qs, kp, g, cc), read_a<D>(kst, 32 * wave + l32, g, cc), s);
        dp = mfma_32x32x16(read_a<D>(gs, kp, g, cc), read_a<D>(vst, 32 * wave + l32, g, cc), dp);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = c_row(i, g);
        const int q = 32 * t + qi;
        const float2 sv = st[qi];
        const bool ok = q < lq && krow < lk && allowed<WMODE>(a, q, krow);
        const float p = ok ? exp2f(s[i] * a.c2 - sv.x) : 0.f;
        s[i] = p;
        dp[i] = p * (dp[i] - sv.y);
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const bf16x8 pb = to_b(s, kc), db = to_b(dp, kc);
#pragma unroll
        for (int t2 = 0; t2 < L::kT; ++t2) {
          dv[t2] = mfma_32x32x16(read_at<D>(gs, 16 * kc, t2, lane), pb, dv[t2]);
          dk[t2] = mfma_32x32x16(read_at<D>(qs, 16 * kc, t2, lane), db, dk[t2]);
        }
        __builtin_amdgcn_sched_barrier(0);  // (bounds the operand reads in flight: registers)
      }
    }
    if (krow < lk) {
      float* odk = a.dk + (size_t(kbeg + krow) * a.H + it.h) * D;
      float* odv = a.dv + (size_t(kbeg + krow) * a.H + it.h) * D;
#pragma unroll
      for (int t2 = 0; t2 < L::kT; ++t2)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          float4 wk, wv;
          wk.x = dk[t2][4 * gi + 0] * a.inv_sqrt_d;
          wk.y = dk[t2][4 * gi + 1] * a.inv_sqrt_d;
          wk.z = dk[t2][4 * gi + 2] * a.inv_sqrt_d;
          wk.w = dk[t2][4 * gi + 3] * a.inv_sqrt_d;
          wv.x = dv[t2][4 * gi + 0];
          wv.y = dv[t2][4 * gi + 1];
          wv.z = dv[t2][4 * gi + 2];
          wv.w = dv[t2][4 * gi + 3];
          *reinterpret_cast<float4*>(odk + 32 * t2 + 8 * gi + 4 * g) = wk;
          *reinterpret_cast<float4*>(odv + 32 * t2 + 8 * gi + 4 * g) = wv;
        }
    }
  }
}

template <int D, int WMODE>
hipError_t launch_w(const BwdArgs& a, int grid_q, int grid_k, hipStream_t st) {
  hipLaunchKernelGGL((bwd_dq_mfma_kernel<D, WMODE>), dim3(grid_q), dim3(kMT), 0, st, a);
  hipLaunchKernelGGL((bwd_dkv_mfma_kernel<D, WMODE>), dim3(grid_k), dim3(kMT), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dm(int wmode, const BwdArgs& a, int grid_q, int grid_k, hipStream_t st) {
  if (wmode == 1) return launch_w<D, 1>(a, grid_q, grid_k, st);
  if (wmode == 2) return launch_w<D, 2>(a, grid_q, grid_k, st);
  return launch_w<D, 0>(a, grid_q, grid_k, st);
}

}  // namespace

hipError_t launch_attn_bwd_mfma(int D, int wmode, const BwdArgs& a, int grid_q, int grid_k, hipStream_t st) {
  if (D == 32) return launch_dm<32>(wmode, a, grid_q, grid_k, st);
  if (D == 64) return launch_dm<64>(wmode, a, grid_q, grid_k, st);
  return launch_dm<128>(wmode, a, grid_q, grid_k, st);
}

}  // namespace ja
