// Backward of jagged attention on bf16 MFMA (training; the chain rule
// of the forward as defined -- the pages, e.g. the techfeed.io summary of
// "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads
// Foundation Model", describe the training system but not its backward):
//   P = softmax(Q K^T / sqrt(D)),  dV = P^T dO,  dS = P * (dO V^T - D_i),
//   D_i = rowsum(P * (dO V^T)),    dQ = dS K / sqrt(D),  dK = dS^T Q / sqrt(D).
// GELU scores (QK-RMSNorm, no window; RMS factors r from a prepass):
//   S = Qn Kn^T / sqrt(D), dV = gelu(S)^T dO / Lk, dS = gelu'(S) * (dO V^T) / Lk,
//   dQn = dS Kn / sqrt(D), dKn = dS^T Qn / sqrt(D), dx = r dxn - x r^3 (dxn . x) / D;
// the RMS factors are folded into the scores and into dS, so the products
// take the raw bf16 rows, and the dQ kernel needs no first pass.
//
// Two kernels, 32 rows per wave, all products on v_mfma_f32_32x32x16_bf16
// with fp32 accumulation (P and dS enter their products in bf16, as P does in
// the forward):
//  * bwd_dq_mfma_kernel, 4 waves, 128 query rows per item.  Lane column = query.  Over
//    the item's key tiles it forms S^T = K Q^T and dP^T = V dO^T; a first pass
//    keeps the online max, sum and sum of p * dP (giving the log-sum-exp and
//    D_i, stored for the second kernel), a second pass accumulates
//    dQ^T += K^T dS^T.
//  * bwd_dkv_pair_kernel, 4 waves, 64 key rows per item (kept in LDS).  Lane
//    column = key.  Each 32-key group is split over a wave pair: over the
//    32-query tiles that see the item, one wave forms S = Q K^T, the weights
//    and dV^T += dO^T W, the other dP = dO V^T and, with a factor handed over
//    through LDS, dK^T += Q^T dS.
// The score products read their A rows in key_perm order so that the result
// registers of lane half h hold, for each 16-row step, the 8 contiguous rows
// 8h..8h+7: exactly the B operand of the next product (no shuffle).  The
// transposed A operands (K^T, dO^T, Q^T) come from ds_read_b64_tr_b16 on
// row-major LDS tiles (rows padded by 16 bytes).  Tiles arrive by
// direct-to-LDS loads into two stages: tile s + 1 loads while tile s is used.
#include "ja_mfma_util.h"
#include "jagged_attn.h"

namespace ja {
namespace {

template <int D>
struct BT {
  static constexpr int kRS = D + 8;  // LDS row stride in bf16 (16-byte pad: rows 4 banks apart)
  static constexpr int kS = D / 16;  // k-steps over D
  static constexpr int kT = D / 32;  // 32-row output tiles over D
};

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

// Direct-to-LDS tile loads into the padded layout: slot L (16 bytes) of an
// LDS tile is row L / kCpr, chunk L % kCpr; the last chunk of every row is
// padding (it loads a duplicate) and the tile is rounded up to whole wave
// instructions (1 KB each).  Rows at or past `valid` load row valid-1: finite
// values whose weights are zero.
template <int D, int NROWS>
struct Dma {
  static constexpr int kCpr = D / 8 + 1;                   // slots per padded row
  static constexpr int kInstr = (NROWS * kCpr + 63) / 64;  // wave instructions per tile
  static constexpr int kBytes = kInstr * 1024;
  // instructions issued by wave w of nw (i = w, w + nw, ...)
  static constexpr int count(int w, int nw) { return (kInstr - w + nw - 1) / nw; }
};

template <int D, int NROWS, int NW>
__device__ __forceinline__ void dma_tile(unsigned lds, const void* g, unsigned grow_bytes, int valid, int wave,
                                         int lane) {
  using T = Dma<D, NROWS>;
  for (int i = wave; i < T::kInstr; i += NW) {
    const int slot = 64 * i + lane;
    int row = slot / T::kCpr;
    int c = slot - row * T::kCpr;
    if (c == T::kCpr - 1) c = 0;
    row = min(row, valid - 1);
    lds_dma16(g, unsigned(row) * grow_bytes + 16u * unsigned(c), lds + 1024u * unsigned(i));
  }
}

// Wait until at most N of this wave's VMEM instructions are outstanding (N < 64).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

constexpr int kQWaves = 4;  // dq kernel: 4 waves x 32 query rows (128-row items)

template <int D, int WMODE, int ACT>
__global__ __launch_bounds__(64 * kQWaves) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_mfma_kernel(BwdArgs a) {
  using L = BT<D>;
  using T = Dma<D, 64>;
  constexpr bool kGelu = ACT == ACT_GELU;
  // per-wave DMA count of one K + V tile (every wave past the first issues the
  // same number; with GELU wave 0 also loads the tile's key RMS factors)
  constexpr int kN0 = 2 * T::count(0, kQWaves) + (kGelu ? 1 : 0), kN1 = 2 * T::count(1, kQWaves);
  static_assert(T::count(1, kQWaves) == T::count(kQWaves - 1, kQWaves), "waves 1.. issue equally");
  __shared__ __attribute__((aligned(1024))) unsigned char buf[2][2][T::kBytes];  // [stage][K, V]
  __shared__ __attribute__((aligned(256))) float rkb[2][64];                    // GELU: [stage] key RMS factors
  const __bf16* qg = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* kg = reinterpret_cast<const __bf16*>(a.k);
  const __bf16* vg = reinterpret_cast<const __bf16*>(a.v);
  const __bf16* gg = reinterpret_cast<const __bf16*>(a.dout);
  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // (scalar: uniform loops)
  const int kp = key_perm(l32);
  const size_t gstride = size_t(a.H) * D;
  const unsigned grow = unsigned(gstride) * 2u;
  const unsigned lds0 = lds_addr_of(&buf[0][0][0]);
  const unsigned lds_rk = lds_addr_of(&rkb[0][0]);
  const int n_items = a.hdr_q->n_items;
  for (int idx = blockIdx.x; idx < n_items; idx += gridDim.x) {
    const WorkItem it = a.items_q[idx];
    const int r0 = it.q0 + 32 * wave;
    const int qrow = r0 + l32;
    const int qr = min(qrow, it.lq - 1);
    bf16x8 qf[L::kS], gf[L::kS];
    // With the forward's log-sum-exp and output: D_i = dO_i . O_i (this lane's
    // half of the row; the halves are added below) instead of the first pass.
    const bool saved = !kGelu && a.lse_in != nullptr;
    float dot_o = 0.f, lse_ln = 0.f;
    {
      const size_t off = (size_t(it.qbeg + qr) * a.H + it.h) * D + (D / 2) * g;
#pragma unroll
      for (int cc = 0; cc < L::kS; ++cc) {
        qf[cc] = *reinterpret_cast<const bf16x8*>(qg + off + 8 * cc);
        gf[cc] = *reinterpret_cast<const bf16x8*>(gg + off + 8 * cc);
      }
      if (saved) {
        lse_ln = a.lse_in[size_t(it.qbeg + qr) * a.H + it.h];
        const __bf16* og = reinterpret_cast<const __bf16*>(a.o_in) + off;
#pragma unroll
        for (int cc = 0; cc < L::kS; ++cc) {
          const bf16x8 o8 = *reinterpret_cast<const bf16x8*>(og + 8 * cc);
#pragma unroll
          for (int j = 0; j < 8; ++j) dot_o = fmaf(float(gf[cc][j]), float(o8[j]), dot_o);
        }
      }
      // Wait here, before any tile load: the compiler then knows these are
      // complete and puts no wait for them (which would also drain the
      // untracked tile loads) inside the loops.
      wait_vm<0>();
    }
    // this wave's key tiles [wt_lo, wt_hi) and the workgroup's [t_lo, t_hi)
    int klo, khi;
    wave_keys<WMODE>(a, r0, it.lq, it.lk, klo, khi);
    const int wt_lo = klo / 64, wt_hi = khi > klo ? (khi + 63) / 64 : wt_lo;
    int t_lo = 1 << 30, t_hi = 0;
    for (int w = 0; w < kQWaves; ++w) {
      int lo, hi;
      wave_keys<WMODE>(a, it.q0 + 32 * w, it.lq, it.lk, lo, hi);
      if (hi > lo) {
        t_lo = min(t_lo, lo / 64);
        t_hi = max(t_hi, (hi + 63) / 64);
      }
    }
    if (t_lo > t_hi) t_lo = t_hi;
    const int nt = t_hi - t_lo;
    const __bf16* kbase = kg + size_t(it.kbeg) * gstride + size_t(it.h) * D;
    const __bf16* vbase = vg + size_t(it.kbeg) * gstride + size_t(it.h) * D;

    // Each pass walks tiles t_lo .. t_hi - 1; tile s + 1 loads into the other
    // stage while tile s is used.
    auto issue = [&](int s) __attribute__((always_inline)) {
      const int t = t_lo + s;
      const int valid = min(64, it.lk - 64 * t);
      const unsigned st = lds0 + unsigned(s & 1) * 2u * T::kBytes;
      dma_tile<D, 64, kQWaves>(st, kbase + size_t(64 * t) * gstride, grow, valid, wave, lane);
      dma_tile<D, 64, kQWaves>(st + T::kBytes, vbase + size_t(64 * t) * gstride, grow, valid, wave, lane);
      if (kGelu && wave == 0)
        lds_dma4(a.rk + (size_t(it.kbeg) + 64 * t) * a.H + it.h, unsigned(min(lane, valid - 1) * a.H) * 4u,
                 lds_rk + unsigned(s & 1) * 256u);
    };
    // Start of step s: issue tile s + 1, wait for tile s, barrier.
    auto step_begin = [&](int s) __attribute__((always_inline)) {
      if (s + 1 < nt) {
        issue(s + 1);
        if (wave == 0) wait_vm<kN0>();
        else wait_vm<kN1>();
      } else {
        wait_vm<0>();
      }
      lds_barrier();  // tile s is in LDS for every wave
    };

    // Scores and dP^T of keys 64 t + 32 kb .. +32 for this wave's queries
    // (one 32-key block at a time keeps the live registers down).
    auto scores = [&](const __bf16* ks, const __bf16* vs, int t, int kb, f32x16& s, f32x16& dp)
                      __attribute__((always_inline)) {
      f32x16 x = {}, y = {};
#pragma unroll
      for (int cc = 0; cc < L::kS; ++cc) {
        x = mfma_32x32x16(read_a<D>(ks, 32 * kb + kp, g, cc), qf[cc], x);
        y = mfma_32x32x16(read_a<D>(vs, 32 * kb + kp, g, cc), gf[cc], y);
      }
      if constexpr (!kGelu) {
        // scale to log2 units; disallowed and ragged keys -> -inf.  (Branch
        // free: bitwise tests, no short circuit.  A block window is uniform
        // here: the wave's 32 queries share a block, and so do the tile's keys.)
        bool uok = true;
        if constexpr (WMODE == 1) {
          const int bi = r0 / kBlock, bj = t;
          uok = bj <= bi && bi - bj < a.window_blocks;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = 64 * t + 32 * kb + c_row(i, g);
          bool ok = uok & (j < it.lk);
          if constexpr (WMODE == 2) ok = ok & (j <= qrow) & (qrow - j < a.window_tokens);
          x[i] = ok ? x[i] * a.c2 : -__builtin_huge_valf();
        }
      }
      s = x;
      dp = y;
    };

    // Pass 1: online max, sum and sum of p * dP -> log-sum-exp (base 2) and
    // D_i = sum_j p_ij dP_ij of the row, for pass 2 and the dK/dV kernel.
    float m = -__builtin_huge_valf(), l = 0.f, acc = 0.f;
    if (!kGelu && !saved && nt > 0) issue(0);
    for (int s = 0; s < (kGelu || saved ? 0 : nt); ++s) {
      step_begin(s);
      const int t = t_lo + s;
      if (t >= wt_lo && t < wt_hi) {
        const __bf16* ks = reinterpret_cast<const __bf16*>(&buf[s & 1][0][0]);
        const __bf16* vs = reinterpret_cast<const __bf16*>(&buf[s & 1][1][0]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          f32x16 sc, dp;
          scores(ks, vs, t, kb, sc, dp);
          float mx = -__builtin_huge_valf();
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[i]);
          const float mn = fmaxf(m, max_halves(mx));
          // (no branch: the MFMAs of the next block run with the whole wave)
          const float mref = mn == -__builtin_huge_valf() ? 0.f : mn;  // nothing allowed yet
          const float r = fast_exp2(m - mref);                          // m = -inf -> 0
          l *= r;
          acc *= r;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(sc[i] - mref);
            l += p;
            acc = fmaf(p, dp[i], acc);
          }
          m = mn;
        }
      }
      lds_barrier();  // every wave is done with stage s & 1 before tile s + 2 loads into it
    }
    float lse, di;
    if (saved) {
      // natural log -> log2 units of the scaled scores; a row without keys
      // (-inf) takes 0, as below, so that its masked weights stay 0
      lse = lse_ln > -__builtin_huge_valf() ? lse_ln * 1.4426950408889634f : 0.f;
      di = sum_halves(dot_o);
    } else {
      l = sum_halves(l);
      acc = sum_halves(acc);
      lse = l > 0.f ? m + log2f(l) : 0.f;
      di = l > 0.f ? acc / l : 0.f;
    }
    if (!kGelu && g == 0 && qrow < it.lq) a.stats[size_t(it.qbeg + qrow) * a.H + it.h] = make_float2(lse, di);
    // GELU: RMS factor of the query row, times 1/sqrt(D); 1/Lk
    const float rsc = kGelu ? a.rq[size_t(it.qbeg + qr) * a.H + it.h] * a.inv_sqrt_d : 0.f;
    const float inv_lk = kGelu ? 1.0f / float(max(it.lk, 1)) : 0.f;
    if constexpr (kGelu) wait_vm<0>();  // (complete before the tile loads, as the Q fragments)

    // Pass 2: dQ^T += K^T dS^T.
    f32x16 dq[L::kT];
#pragma unroll
    for (int t2 = 0; t2 < L::kT; ++t2) dq[t2] = f32x16{};
    if (nt > 0) issue(0);
    for (int s = 0; s < nt; ++s) {
      step_begin(s);
      const int t = t_lo + s;
      if (t >= wt_lo && t < wt_hi) {
        const __bf16* ks = reinterpret_cast<const __bf16*>(&buf[s & 1][0][0]);
        const __bf16* vs = reinterpret_cast<const __bf16*>(&buf[s & 1][1][0]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          f32x16 sc, dp;
          scores(ks, vs, t, kb, sc, dp);
          if constexpr (kGelu) {
            // dSn = gelu'(s) dP / Lk, times the key's RMS factor (dQn = dSn Kn / sqrt(D))
            const float* rk = &rkb[s & 1][0];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int jl = 32 * kb + c_row(i, g);
              const float ck = rk[jl];
              float gl, gp;
              gelu_and_grad(sc[i] * rsc * ck, gl, gp);
              sc[i] = 64 * t + jl < it.lk ? gp * dp[i] * inv_lk * ck : 0.f;
            }
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[i] = fast_exp2(sc[i] - lse) * (dp[i] - di);
          }
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const bf16x8 db = to_b(sc, half);
#pragma unroll
            for (int t2 = 0; t2 < L::kT; ++t2)
              dq[t2] = mfma_32x32x16(read_at<D>(ks, 32 * kb + 16 * half, t2, lane), db, dq[t2]);
            __builtin_amdgcn_sched_barrier(0);  // (bounds the operand reads in flight: registers)
          }
        }
      }
      lds_barrier();  // every wave is done with stage s & 1 before tile s + 2 loads into it
    }
#pragma unroll
    for (int t2 = 0; t2 < L::kT; ++t2) dq[t2] *= a.inv_sqrt_d;
    if constexpr (kGelu) {
      // through the RMSNorm: dq = r dqn - q r^3 (dqn . q) / D; the lane holds
      // dims 32 t2 + 8 gi + 4 g + 0..3, the other lane half the rest
      const float r = a.rq[size_t(it.qbeg + qr) * a.H + it.h];
      const __bf16* qrow_p = qg + (size_t(it.qbeg + qr) * a.H + it.h) * D;
      float dot = 0.f;
#pragma unroll
      for (int t2 = 0; t2 < L::kT; ++t2)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
          for (int e = 0; e < 4; ++e) dot = fmaf(dq[t2][4 * gi + e], float(qrow_p[32 * t2 + 8 * gi + 4 * g + e]), dot);
      const float c3 = r * r * r * sum_halves(dot) * (1.0f / D);
#pragma unroll
      for (int t2 = 0; t2 < L::kT; ++t2)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            dq[t2][4 * gi + e] = fmaf(r, dq[t2][4 * gi + e], -float(qrow_p[32 * t2 + 8 * gi + 4 * g + e]) * c3);
    }
    if (qrow < it.lq) {
      float* out = a.dq + (size_t(it.qbeg + qrow) * a.H + it.h) * D;
#pragma unroll
      for (int t2 = 0; t2 < L::kT; ++t2)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          float4 w;
          w.x = dq[t2][4 * gi + 0];
          w.y = dq[t2][4 * gi + 1];
          w.z = dq[t2][4 * gi + 2];
          w.w = dq[t2][4 * gi + 3];
          *reinterpret_cast<float4*>(out + 32 * t2 + 8 * gi + 4 * g) = w;
        }
    }
  }
}

// dK/dV with the work of a 32-key group split over a wave pair: the "V wave"
// forms S = Q K^T and the weights W (softmax: P from the stored statistics;
// GELU: gelu(s) / Lk on the RMS-normalised scores) and accumulates
// dV^T += dO^T W; the "K wave" forms dP = dO V^T, takes a factor F through
// LDS (softmax: P; GELU: gelu'(s) r_q / Lk) and accumulates dK^T += Q^T dS
// with dS = P (dP - D_i) (softmax) or F dP (GELU; dK then goes through the
// key RMSNorm's backward).  Each wave holds 64 accumulators and issues 16
// MFMAs per query step, so two workgroups of 4 waves (64-key items, 78.5 KB
// of LDS at D = 128) share a CU: two waves per SIMD, one's VALU work under the
// other's MFMAs (one wave forming all four products of its keys holds 128
// accumulators and runs alone on its SIMD).  Query tiles in two stages; the
// next tile's loads are issued after the step's first barrier, into the stage
// every wave has finished with.
constexpr int kPairWaves = 4;  // 2 pairs x (V wave, K wave), 32 keys per pair

template <int D, int WMODE, int ACT>
__global__ __launch_bounds__(64 * kPairWaves) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dkv_pair_kernel(
    BwdArgs a) {
  using L = BT<D>;
  constexpr bool kGelu = ACT == ACT_GELU;
  static_assert(!kGelu || WMODE == 0, "GELU takes no window");
  using TK = Dma<D, 64>;
  using TQ = Dma<D, 32>;
  __shared__ __attribute__((aligned(1024))) unsigned char kvb[2][TK::kBytes];    // the item's K, V (64 rows)
  __shared__ __attribute__((aligned(1024))) unsigned char qb[2][2][TQ::kBytes];  // [stage][Q, dO]
  __shared__ __attribute__((aligned(256))) float2 stb[2][32];  // [stage] (lse, D_i); GELU: 64 floats, RMS factors
  __shared__ __attribute__((aligned(256))) float pxb[2][16][64];  // [pair] P or the GELU factor, lane-major
  const __bf16* qg = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* kg = reinterpret_cast<const __bf16*>(a.k);
  const __bf16* vg = reinterpret_cast<const __bf16*>(a.v);
  const __bf16* gg = reinterpret_cast<const __bf16*>(a.dout);
  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // (scalar: uniform branches)
  const int pair = wave >> 1;
  const bool vwave = (wave & 1) == 0;
  const int kp = key_perm(l32);
  const size_t gstride = size_t(a.H) * D;
  const unsigned grow = unsigned(gstride) * 2u;
  const unsigned lds_kv = lds_addr_of(&kvb[0][0]), lds_q = lds_addr_of(&qb[0][0][0]);
  const unsigned lds_st = lds_addr_of(&stb[0][0]);
  const __bf16* kst = reinterpret_cast<const __bf16*>(&kvb[0][0]);
  const __bf16* vst = reinterpret_cast<const __bf16*>(&kvb[1][0]);
  float* px = &pxb[pair][0][0];
  const int n_items = a.hdr_k->n_items;
  for (int idx = blockIdx.x; idx < n_items; idx += gridDim.x) {
    // (items over key tiles: the plan ran on the swapped offsets)
    const WorkItem it = a.items_k[idx];
    const int lk = it.lq, lq = it.lk, kbeg = it.qbeg, qbeg = it.kbeg;
    const int k0 = it.q0 + 32 * pair;
    const int krow = k0 + l32;
    int qlo, qhi;
    wave_queries<WMODE>(a, k0, lq, lk, qlo, qhi);
    const int wt_lo = qlo / 32, wt_hi = qhi > qlo ? (qhi + 31) / 32 : wt_lo;
    int t_lo = 1 << 30, t_hi = 0;
    for (int pp = 0; pp < 2; ++pp) {
      int lo, hi;
      wave_queries<WMODE>(a, it.q0 + 32 * pp, lq, lk, lo, hi);
      if (hi > lo) {
        t_lo = min(t_lo, lo / 32);
        t_hi = max(t_hi, (hi + 31) / 32);
      }
    }
    if (t_lo > t_hi) t_lo = t_hi;
    const int nt = t_hi - t_lo;
    const __bf16* qbase = qg + size_t(qbeg) * gstride + size_t(it.h) * D;
    const __bf16* gbase = gg + size_t(qbeg) * gstride + size_t(it.h) * D;
    const float2* sbase = a.stats + size_t(qbeg) * a.H + it.h;

    // Query tile t_lo + s into stage s & 1: Q, dO and the statistics.
    auto issue_q = [&](int s) __attribute__((always_inline)) {
      const int t = t_lo + s;
      const int valid = min(32, lq - 32 * t);
      const unsigned stage = unsigned(s & 1);
      const unsigned st = lds_q + stage * 2u * TQ::kBytes;
      dma_tile<D, 32, kPairWaves>(st, qbase + size_t(32 * t) * gstride, grow, valid, wave, lane);
      dma_tile<D, 32, kPairWaves>(st + TQ::kBytes, gbase + size_t(32 * t) * gstride, grow, valid, wave, lane);
      if (wave == 0) {
        if constexpr (kGelu) {
          const unsigned row = unsigned(min(lane, valid - 1));
          lds_dma4(a.rq + (size_t(qbeg) + 32 * t) * a.H + it.h, row * unsigned(a.H) * 4u, lds_st + stage * 256u);
        } else {
          const unsigned row = unsigned(min(lane >> 1, valid - 1));
          lds_dma4(sbase + size_t(32 * t) * a.H, (row * unsigned(a.H)) * 8u + 4u * unsigned(lane & 1),
                   lds_st + stage * 256u);
        }
      }
    };

    // GELU: RMS factor of this lane's key row times 1/sqrt(D); 1/Lk (loaded
    // and waited for before the tile loads, see the dQ kernel)
    const int kr = min(krow, lk - 1);
    const float csc = kGelu ? a.rk[size_t(kbeg + kr) * a.H + it.h] * a.inv_sqrt_d : 0.f;
    const float inv_lk = kGelu ? 1.0f / float(lk) : 0.f;
    if constexpr (kGelu) wait_vm<0>();

    f32x16 acc[L::kT];  // dV^T (V wave) or dK^T (K wave) of the pair's 32 keys
#pragma unroll
    for (int t2 = 0; t2 < L::kT; ++t2) acc[t2] = f32x16{};
    if (nt > 0) {
      const int valid = min(64, lk - it.q0);
      const size_t off = size_t(kbeg + it.q0) * gstride + size_t(it.h) * D;
      dma_tile<D, 64, kPairWaves>(lds_kv, kg + off, grow, valid, wave, lane);
      dma_tile<D, 64, kPairWaves>(lds_kv + TK::kBytes, vg + off, grow, valid, wave, lane);
      issue_q(0);
    }
    // the pair's key range is uniform over its window per step: a block
    // window tests it once (the step's 32 queries lie in block t / 2)
    for (int s = 0; s < nt; ++s) {
      wait_vm<0>();   // tile s (and the item's K, V): nothing else is in flight
      lds_barrier();  // ... in LDS for every wave; every wave is done with step s - 1
      if (s + 1 < nt) issue_q(s + 1);
      const int t = t_lo + s;
      const int stage = s & 1;
      const bool active = t >= wt_lo && t < wt_hi;
      const __bf16* qs = reinterpret_cast<const __bf16*>(&qb[stage][0][0]);
      const __bf16* gs = reinterpret_cast<const __bf16*>(&qb[stage][1][0]);
      const float2* st = &stb[stage][0];
      f32x16 x = {};
      if (active) {
        // V wave: S = Q K^T; K wave: dP = dO V^T (key as lane column)
        const __bf16* as = vwave ? qs : gs;
        const __bf16* bs = vwave ? kst : vst;
#pragma unroll
        for (int cc = 0; cc < L::kS; ++cc)
          x = mfma_32x32x16(read_a<D>(as, kp, g, cc), read_a<D>(bs, 32 * pair + l32, g, cc), x);
        if (vwave && kGelu) {
          // W = gelu(s) / Lk for dV; F = gelu'(s) r_q / Lk for the K wave
          const float* rq = reinterpret_cast<const float*>(st);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int qi = c_row(i, g);
            const float ri = rq[qi];
            const bool ok = 32 * t + qi < lq && krow < lk;
            float gl, gp;
            gelu_and_grad(x[i] * csc * ri, gl, gp);
            x[i] = ok ? gl * inv_lk : 0.f;
            px[64 * i + lane] = ok ? gp * inv_lk * ri : 0.f;
          }
        } else if (vwave) {
          // P from the stored log-sum-exp, masked without branches (the
          // mask enters as an added 0 or -inf under the raw exp2)
          bool kok = krow < lk;
          if constexpr (WMODE == 1) {
            const int bq = t >> 1, bk = krow / kBlock;
            kok = kok && bk <= bq && bq - bk < a.window_blocks;
          }
          const int qn = lq - 32 * t;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int qi = c_row(i, g);
            const float2 sv = st[qi];
            bool ok = kok & (qi < qn);
            if constexpr (WMODE == 2) {
              const int q = 32 * t + qi;
              ok = ok & (krow <= q) & (q - krow < a.window_tokens);
            }
            x[i] = fast_exp2(fmaf(x[i], a.c2, -sv.x) + (ok ? 0.f : -__builtin_huge_valf()));
            px[64 * i + lane] = x[i];
          }
        }
      }
      lds_barrier();  // P of the step in LDS for the pair's K wave
      if (active) {
        if (!vwave) {
          // dS = P (dP - D_i); GELU: F dP
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if constexpr (kGelu) x[i] = px[64 * i + lane] * x[i];
            else x[i] = px[64 * i + lane] * (x[i] - st[c_row(i, g)].y);
          }
        }
        // V wave: dV^T += dO^T P; K wave: dK^T += Q^T dS
        const __bf16* ts = vwave ? gs : qs;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const bf16x8 xb = to_b(x, kc);
#pragma unroll
          for (int t2 = 0; t2 < L::kT; ++t2) acc[t2] = mfma_32x32x16(read_at<D>(ts, 16 * kc, t2, lane), xb, acc[t2]);
        }
      }
    }
    lds_barrier();  // every wave is done with the item's LDS before the next item's loads
    // dV^T is acc; dK^T is acc / sqrt(D) (GELU: then through the RMSNorm)
    float osc = vwave ? 1.f : a.inv_sqrt_d;
    if (kGelu && !vwave) {
      // dk = c dKn - k c^3 (dKn . k) / D, dKn = acc / sqrt(D), c the key's RMS
      // factor (the lane holds dims 32 t2 + 8 gi + 4 g + 0..3)
      const float c = a.rk[size_t(kbeg + kr) * a.H + it.h];
      const __bf16* krow_p = kg + (size_t(kbeg + kr) * a.H + it.h) * D;
      float dot = 0.f;
#pragma unroll
      for (int t2 = 0; t2 < L::kT; ++t2) {
        acc[t2] *= osc;
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
          for (int e = 0; e < 4; ++e) dot = fmaf(acc[t2][4 * gi + e], float(krow_p[32 * t2 + 8 * gi + 4 * g + e]), dot);
      }
      const float c3 = c * c * c * sum_halves(dot) * (1.0f / D);
#pragma unroll
      for (int t2 = 0; t2 < L::kT; ++t2)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[t2][4 * gi + e] = fmaf(c, acc[t2][4 * gi + e], -float(krow_p[32 * t2 + 8 * gi + 4 * g + e]) * c3);
      osc = 1.f;
    }
    if (krow < lk) {
      float* o = (vwave ? a.dv : a.dk) + (size_t(kbeg + krow) * a.H + it.h) * D;
#pragma unroll
      for (int t2 = 0; t2 < L::kT; ++t2)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          float4 w;
          w.x = acc[t2][4 * gi + 0] * osc;
          w.y = acc[t2][4 * gi + 1] * osc;
          w.z = acc[t2][4 * gi + 2] * osc;
          w.w = acc[t2][4 * gi + 3] * osc;
          *reinterpret_cast<float4*>(o + 32 * t2 + 8 * gi + 4 * g) = w;
        }
    }
  }
}

template <int D, int WMODE, int ACT>
hipError_t launch_w(const BwdArgs& a, int grid_q, int grid_k, hipStream_t st) {
  hipLaunchKernelGGL((bwd_dq_mfma_kernel<D, WMODE, ACT>), dim3(grid_q), dim3(64 * kQWaves), 0, st, a);
  hipLaunchKernelGGL((bwd_dkv_pair_kernel<D, WMODE, ACT>), dim3(grid_k), dim3(64 * kPairWaves), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dm(int act, int wmode, const BwdArgs& a, int grid_q, int grid_k, hipStream_t st) {
  if (act == ACT_GELU) return launch_w<D, 0, ACT_GELU>(a, grid_q, grid_k, st);  // (no window with GELU)
  if (wmode == 1) return launch_w<D, 1, ACT_SOFTMAX>(a, grid_q, grid_k, st);
  if (wmode == 2) return launch_w<D, 2, ACT_SOFTMAX>(a, grid_q, grid_k, st);
  return launch_w<D, 0, ACT_SOFTMAX>(a, grid_q, grid_k, st);
}

}  // namespace

hipError_t launch_attn_bwd_mfma(int D, int act, int wmode, const BwdArgs& a, int grid_q, int grid_k,
                                hipStream_t st) {
  if (D == 32) return launch_dm<32>(act, wmode, a, grid_q, grid_k, st);
  if (D == 64) return launch_dm<64>(act, wmode, a, grid_q, grid_k, st);
  return launch_dm<128>(act, wmode, a, grid_q, grid_k, st);
}

}  // namespace ja
