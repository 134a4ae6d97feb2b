// Backward of jagged softmax attention (training): dQ, dK, dV of the forward
// as defined, by the chain rule (the pages describe the training system --
// techfeed.io summary of "GEM Training: How Meta Doubled the Efficiency of
// Its LLM-Scale Ads Foundation Model" -- but not its backward pass).  For one
// (sample, head):
//   P = softmax(Q K^T / sqrt(D)) on the allowed keys,
//   dV = P^T dO,  dS = P * (dO V^T - rowsum(P * (dO V^T))),
//   dQ = dS K / sqrt(D),  dK = dS^T Q / sqrt(D).
// Nothing is kept from the forward: the row statistics are recomputed.
//
// fp32 VALU kernels for fp32 inputs (bf16 inputs take the MFMA kernels of
// ja_attn_bwd_mfma.hip), four lanes per row (D/4 dimensions each, dot
// products finished by two lane shuffles):
//  * bwd_q_kernel, one row per query: the row's max and sum (log-sum-exp,
//    base 2), then D_i = sum_j p_ij (dO_i . v_j), then dQ_i; it leaves
//    (lse_i, D_i) for the second kernel;
//  * bwd_kv_kernel, one row per key: over the queries that see the key,
//    dV_j += p_ij dO_i and dK_j += p_ij (dO_i . v_j - D_i) q_i.
// Work items are the forward's 64-row query tiles (plan over q) and 64-row key
// tiles (the same plan over the swapped offsets); no atomics.
//
// GELU scores (tanh form, QK-RMSNorm, no window): with Qn = rms(Q), Kn = rms(K),
// S = Qn Kn^T / sqrt(D) and O = gelu(S) V / Lk,
//   dV = gelu(S)^T dO / Lk,  dS = gelu'(S) * (dO V^T) / Lk,
//   dQn = dS Kn / sqrt(D),   dKn = dS^T Qn / sqrt(D),
// and through the RMSNorm, per row, dx = r dxn - x r^3 (dxn . x) / D with
// r = (mean(x^2) + eps)^(-1/2).  No statistics pass is needed; bwd_rms_kernel
// writes r for every query and key row first.
#include "ja_device.h"
#include "ja_internal.h"
#include "jagged_attn.h"

namespace ja {

namespace {

constexpr int kBwdThreads = 256;  // 64 rows x 4 lanes
constexpr int kLpr = 4;           // lanes per row

template <typename T>
__device__ __forceinline__ float ld(const T* p, int i) {
  if constexpr (sizeof(T) == 2) return __uint_as_float(unsigned(reinterpret_cast<const uint16_t*>(p)[i]) << 16);
  else return p[i];
}

// Sum over the four lanes of a row (a quad), by DPP quad permutations on the
// VALU: lanes 1,0,3,2 then 2,3,0,1 of the quad.
template <int CTRL>
__device__ __forceinline__ float quad_perm(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_sum(float x) {
  x += quad_perm<0xB1>(x);  // lanes [1, 0, 3, 2] of the quad
  x += quad_perm<0x4E>(x);  // lanes [2, 3, 0, 1]
  return x;
}

// RMS factor (mean(x^2) + eps)^(-1/2) of every row of a [rows, D] tensor,
// four lanes per row.
template <int D, typename T>
__global__ __launch_bounds__(kBwdThreads) void bwd_rms_kernel(const T* x, int64_t rows, float eps, float* out) {
  constexpr int DL = D / kLpr;
  const int64_t r = int64_t(blockIdx.x) * (kBwdThreads / kLpr) + threadIdx.x / kLpr;
  if (r >= rows) return;  // (all four lanes of a row together)
  const T* p = x + r * D + (threadIdx.x % kLpr) * DL;
  float ss = 0.f;
#pragma unroll
  for (int d = 0; d < DL; ++d) {
    const float e = ld(p, d);
    ss = fmaf(e, e, ss);
  }
  ss = row_sum(ss);
  if (threadIdx.x % kLpr == 0) out[r] = 1.0f / sqrtf(ss * (1.0f / D) + eps);
}

// Keys of a query row (sample-local), [lo, hi).
template <int WMODE>
__device__ __forceinline__ void key_range(const BwdArgs& a, int qrow, int lk, int& lo, int& hi) {
  lo = 0;
  hi = lk;
  if constexpr (WMODE == 1) {
    const int blk = qrow / kBlock;
    lo = max(0, blk - a.window_blocks + 1) * kBlock;
    hi = min(lk, (blk + 1) * kBlock);
  } else if constexpr (WMODE == 2) {
    lo = max(0, qrow - a.window_tokens + 1);
    hi = min(lk, qrow + 1);
  }
}

// Queries of a key row (sample-local), [lo, hi): the inverse of key_range.
template <int WMODE>
__device__ __forceinline__ void query_range(const BwdArgs& a, int krow, int lq, int& lo, int& hi) {
  lo = 0;
  hi = lq;
  if constexpr (WMODE == 1) {
    const int blk = krow / kBlock;
    lo = min(lq, blk * kBlock);
    hi = min(lq, (blk + a.window_blocks) * kBlock);
  } else if constexpr (WMODE == 2) {
    lo = min(lq, krow);
    hi = min(lq, krow + a.window_tokens);
  }
}

template <int D, typename T, int WMODE, int ACT>
__global__ __launch_bounds__(kBwdThreads) void bwd_q_kernel(BwdArgs a) {
  constexpr int DL = D / kLpr;
  const T* qv = reinterpret_cast<const T*>(a.q);
  const T* kv = reinterpret_cast<const T*>(a.k);
  const T* vv = reinterpret_cast<const T*>(a.v);
  const T* gv = reinterpret_cast<const T*>(a.dout);
  const int part = threadIdx.x % kLpr;
  const int n_items = a.hdr_q->n_items;
  for (int idx = blockIdx.x; idx < n_items; idx += gridDim.x) {
    const WorkItem it = a.items_q[idx];
    const int qrow = it.q0 + int(threadIdx.x) / kLpr;
    if (qrow >= it.lq) continue;  // (all four lanes of a row together)
    const size_t qoff = (size_t(it.qbeg + qrow) * a.H + it.h) * D + part * DL;
    float q[DL], g[DL], dq[DL];
#pragma unroll
    for (int d = 0; d < DL; ++d) {
      q[d] = ld(qv + qoff, d);
      g[d] = ld(gv + qoff, d);
      dq[d] = 0.f;
    }
    int lo, hi;
    key_range<WMODE>(a, qrow, it.lk, lo, hi);
    auto krow = [&](const T* base, int j) { return base + (size_t(it.kbeg + j) * a.H + it.h) * D + part * DL; };
    if constexpr (ACT == ACT_GELU) {
      // dQn_i = sum_j gelu'(s_ij) (dO_i . v_j) / Lk * Kn_j / sqrt(D), then the RMSNorm
      const float ri = a.rq[size_t(it.qbeg + qrow) * a.H + it.h];
      const float sc = ri * a.inv_sqrt_d;
      const float inv_lk = 1.0f / float(it.lk);
      for (int j = lo; j < hi; ++j) {
        const T* kp = krow(kv, j);
        const T* vp = krow(vv, j);
        const float ck = a.rk[size_t(it.kbeg + j) * a.H + it.h];
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int d = 0; d < DL; ++d) {
          s = fmaf(q[d], ld(kp, d), s);
          dp = fmaf(g[d], ld(vp, d), dp);
        }
        float gl, gp;
        gelu_and_grad(row_sum(s) * sc * ck, gl, gp);
        const float ds = gp * row_sum(dp) * inv_lk * ck;
#pragma unroll
        for (int d = 0; d < DL; ++d) dq[d] = fmaf(ds, ld(kp, d), dq[d]);
      }
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < DL; ++d) {
        dq[d] *= a.inv_sqrt_d;
        dot = fmaf(dq[d], q[d], dot);
      }
      const float c3 = ri * ri * ri * row_sum(dot) * (1.0f / D);
      float* out = a.dq + qoff;
#pragma unroll
      for (int d = 0; d < DL; ++d) out[d] = fmaf(ri, dq[d], -q[d] * c3);
      continue;
    }
    float lse, di = 0.f;
    if (a.lse_in != nullptr) {
      // the forward's log-sum-exp (natural log -> base 2 of the scaled
      // scores; a row without keys takes 0) and D_i = dO_i . O_i
      const float ln = a.lse_in[size_t(it.qbeg + qrow) * a.H + it.h];
      lse = ln > -__builtin_huge_valf() ? ln * 1.4426950408889634f : 0.f;
      const T* op = reinterpret_cast<const T*>(a.o_in) + qoff;
#pragma unroll
      for (int d = 0; d < DL; ++d) di = fmaf(g[d], ld(op, d), di);
      di = row_sum(di);
    } else {
      // row max and sum, base 2
      float m = -__builtin_huge_valf(), l = 0.f;
      for (int j = lo; j < hi; ++j) {
        const T* kp = krow(kv, j);
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < DL; ++d) s = fmaf(q[d], ld(kp, d), s);
        s = row_sum(s) * a.c2;
        if (s > m) {
          l *= exp2f(m - s);
          m = s;
        }
        l += exp2f(s - m);
      }
      lse = hi > lo ? m + log2f(l) : 0.f;
      // D_i = sum_j p_ij (dO_i . v_j)
      for (int j = lo; j < hi; ++j) {
        const T* kp = krow(kv, j);
        const T* vp = krow(vv, j);
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int d = 0; d < DL; ++d) {
          s = fmaf(q[d], ld(kp, d), s);
          dp = fmaf(g[d], ld(vp, d), dp);
        }
        const float p = exp2f(row_sum(s) * a.c2 - lse);
        di = fmaf(p, row_sum(dp), di);
      }
    }
    // dQ_i = sum_j p_ij (dO_i . v_j - D_i) k_j / sqrt(D)
    for (int j = lo; j < hi; ++j) {
      const T* kp = krow(kv, j);
      const T* vp = krow(vv, j);
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < DL; ++d) {
        s = fmaf(q[d], ld(kp, d), s);
        dp = fmaf(g[d], ld(vp, d), dp);
      }
      const float ds = exp2f(row_sum(s) * a.c2 - lse) * (row_sum(dp) - di);
#pragma unroll
      for (int d = 0; d < DL; ++d) dq[d] = fmaf(ds, ld(kp, d), dq[d]);
    }
    float* out = a.dq + qoff;
#pragma unroll
    for (int d = 0; d < DL; ++d) out[d] = dq[d] * a.inv_sqrt_d;
    if (part == 0) a.stats[size_t(it.qbeg + qrow) * a.H + it.h] = make_float2(lse, di);
  }
}

template <int D, typename T, int WMODE, int ACT>
__global__ __launch_bounds__(kBwdThreads) void bwd_kv_kernel(BwdArgs a) {
  constexpr int DL = D / kLpr;
  const T* qv = reinterpret_cast<const T*>(a.q);
  const T* kv = reinterpret_cast<const T*>(a.k);
  const T* vv = reinterpret_cast<const T*>(a.v);
  const T* gv = reinterpret_cast<const T*>(a.dout);
  const int part = threadIdx.x % kLpr;
  const int n_items = a.hdr_k->n_items;
  for (int idx = blockIdx.x; idx < n_items; idx += gridDim.x) {
    // (items over key tiles: the plan ran on the swapped offsets, so the
    // record's "query" fields describe keys and its "key" fields queries)
    const WorkItem it = a.items_k[idx];
    const int krow = it.q0 + int(threadIdx.x) / kLpr;
    const int lk = it.lq, lq = it.lk, kbeg = it.qbeg, qbeg = it.kbeg;
    if (krow >= lk) continue;
    const size_t koff = (size_t(kbeg + krow) * a.H + it.h) * D + part * DL;
    float k[DL], v[DL], dk[DL], dv[DL];
#pragma unroll
    for (int d = 0; d < DL; ++d) {
      k[d] = ld(kv + koff, d);
      v[d] = ld(vv + koff, d);
      dk[d] = 0.f;
      dv[d] = 0.f;
    }
    int lo, hi;
    query_range<WMODE>(a, krow, lq, lo, hi);
    if constexpr (ACT == ACT_GELU) {
      // dV_j = sum_i gelu(s_ij) dO_i / Lk; dKn_j = sum_i gelu'(s_ij) (dO_i . v_j) / Lk * Qn_i / sqrt(D)
      const float ck = a.rk[size_t(kbeg + krow) * a.H + it.h];
      const float sc = ck * a.inv_sqrt_d;
      const float inv_lk = 1.0f / float(lk);
      for (int i = lo; i < hi; ++i) {
        const size_t qoff = (size_t(qbeg + i) * a.H + it.h) * D + part * DL;
        const float ri = a.rq[size_t(qbeg + i) * a.H + it.h];
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int d = 0; d < DL; ++d) {
          s = fmaf(ld(qv + qoff, d), k[d], s);
          dp = fmaf(ld(gv + qoff, d), v[d], dp);
        }
        float gl, gp;
        gelu_and_grad(row_sum(s) * sc * ri, gl, gp);
        gl *= inv_lk;
        const float ds = gp * row_sum(dp) * inv_lk * ri;
#pragma unroll
        for (int d = 0; d < DL; ++d) {
          dv[d] = fmaf(gl, ld(gv + qoff, d), dv[d]);
          dk[d] = fmaf(ds, ld(qv + qoff, d), dk[d]);
        }
      }
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < DL; ++d) {
        dk[d] *= a.inv_sqrt_d;
        dot = fmaf(dk[d], k[d], dot);
      }
      const float c3 = ck * ck * ck * row_sum(dot) * (1.0f / D);
      float* odk = a.dk + koff;
      float* odv = a.dv + koff;
#pragma unroll
      for (int d = 0; d < DL; ++d) {
        odk[d] = fmaf(ck, dk[d], -k[d] * c3);
        odv[d] = dv[d];
      }
      continue;
    }
    for (int i = lo; i < hi; ++i) {
      const size_t qoff = (size_t(qbeg + i) * a.H + it.h) * D + part * DL;
      const float2 st = a.stats[size_t(qbeg + i) * a.H + it.h];
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < DL; ++d) {
        s = fmaf(ld(qv + qoff, d), k[d], s);
        dp = fmaf(ld(gv + qoff, d), v[d], dp);
      }
      const float p = exp2f(row_sum(s) * a.c2 - st.x);
      const float ds = p * (row_sum(dp) - st.y);
#pragma unroll
      for (int d = 0; d < DL; ++d) {
        dv[d] = fmaf(p, ld(gv + qoff, d), dv[d]);
        dk[d] = fmaf(ds, ld(qv + qoff, d), dk[d]);
      }
    }
    float* odk = a.dk + koff;
    float* odv = a.dv + koff;
#pragma unroll
    for (int d = 0; d < DL; ++d) {
      odk[d] = dk[d] * a.inv_sqrt_d;
      odv[d] = dv[d];
    }
  }
}

template <int D, typename T, int ACT>
hipError_t launch_d(int wmode, const BwdArgs& a, int grid_q, int grid_k, hipStream_t st) {
  const dim3 bd(kBwdThreads);
  if constexpr (ACT == ACT_GELU) {  // (no window with GELU scores)
    hipLaunchKernelGGL((bwd_q_kernel<D, T, 0, ACT>), dim3(grid_q), bd, 0, st, a);
    hipLaunchKernelGGL((bwd_kv_kernel<D, T, 0, ACT>), dim3(grid_k), bd, 0, st, a);
  } else if (wmode == 1) {
    hipLaunchKernelGGL((bwd_q_kernel<D, T, 1, ACT>), dim3(grid_q), bd, 0, st, a);
    hipLaunchKernelGGL((bwd_kv_kernel<D, T, 1, ACT>), dim3(grid_k), bd, 0, st, a);
  } else if (wmode == 2) {
    hipLaunchKernelGGL((bwd_q_kernel<D, T, 2, ACT>), dim3(grid_q), bd, 0, st, a);
    hipLaunchKernelGGL((bwd_kv_kernel<D, T, 2, ACT>), dim3(grid_k), bd, 0, st, a);
  } else {
    hipLaunchKernelGGL((bwd_q_kernel<D, T, 0, ACT>), dim3(grid_q), bd, 0, st, a);
    hipLaunchKernelGGL((bwd_kv_kernel<D, T, 0, ACT>), dim3(grid_k), bd, 0, st, a);
  }
  return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_rms(const void* x, int64_t rows, float eps, float* out, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  constexpr int kRowsPerBlock = kBwdThreads / kLpr;
  hipLaunchKernelGGL((bwd_rms_kernel<D, T>), dim3(unsigned((rows + kRowsPerBlock - 1) / kRowsPerBlock)),
                     dim3(kBwdThreads), 0, st, reinterpret_cast<const T*>(x), rows, eps, out);
  return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_all(int act, int wmode, const BwdArgs& a, int64_t rows_q, int64_t rows_k, int grid_q,
                      int grid_k, hipStream_t st) {
  if (act != ACT_GELU) return launch_d<D, T, ACT_SOFTMAX>(wmode, a, grid_q, grid_k, st);
  hipError_t e = launch_rms<D, T>(a.q, rows_q, a.eps, a.rq, st);
  if (e != hipSuccess) return e;
  e = launch_rms<D, T>(a.k, rows_k, a.eps, a.rk, st);
  if (e != hipSuccess) return e;
  return launch_d<D, T, ACT_GELU>(0, a, grid_q, grid_k, st);
}

}  // namespace

// RMS factors of every query and key row (the GELU backward's prepass).
hipError_t launch_bwd_rms(int D, bool bf16, const BwdArgs& a, int64_t rows_q, int64_t rows_k, hipStream_t st) {
  hipError_t e;
  if (bf16) {
    e = D == 32 ? launch_rms<32, __bf16>(a.q, rows_q, a.eps, a.rq, st)
        : D == 64 ? launch_rms<64, __bf16>(a.q, rows_q, a.eps, a.rq, st)
                  : launch_rms<128, __bf16>(a.q, rows_q, a.eps, a.rq, st);
    if (e != hipSuccess) return e;
    return D == 32 ? launch_rms<32, __bf16>(a.k, rows_k, a.eps, a.rk, st)
           : D == 64 ? launch_rms<64, __bf16>(a.k, rows_k, a.eps, a.rk, st)
                     : launch_rms<128, __bf16>(a.k, rows_k, a.eps, a.rk, st);
  }
  e = D == 32 ? launch_rms<32, float>(a.q, rows_q, a.eps, a.rq, st)
      : D == 64 ? launch_rms<64, float>(a.q, rows_q, a.eps, a.rq, st)
                : launch_rms<128, float>(a.q, rows_q, a.eps, a.rq, st);
  if (e != hipSuccess) return e;
  return D == 32 ? launch_rms<32, float>(a.k, rows_k, a.eps, a.rk, st)
         : D == 64 ? launch_rms<64, float>(a.k, rows_k, a.eps, a.rk, st)
                   : launch_rms<128, float>(a.k, rows_k, a.eps, a.rk, st);
}

// fp32 inputs (bf16 inputs take the MFMA kernels of ja_attn_bwd_mfma.hip).
hipError_t launch_attn_bwd(int D, bool bf16, int act, int wmode, const BwdArgs& a, int64_t rows_q, int64_t rows_k,
                           int grid_q, int grid_k, hipStream_t st) {
  if (bf16) return hipErrorInvalidValue;
  if (D == 32) return launch_all<32, float>(act, wmode, a, rows_q, rows_k, grid_q, grid_k, st);
  if (D == 64) return launch_all<64, float>(act, wmode, a, rows_q, rows_k, grid_q, grid_k, st);
  return launch_all<128, float>(act, wmode, a, rows_q, rows_k, grid_q, grid_k, st);
}

}  // namespace ja
