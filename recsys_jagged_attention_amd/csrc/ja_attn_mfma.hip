// Jagged generalized dot-product attention forward on gfx950 MFMA (bf16 and
// MX-fp8 inputs, bf16 output).
//
// One kernel family covers the three shapes of GDPA (techfeed.io summary of
// "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads
// Foundation Model", sections "なぜLLM向けのインフラをそのまま使えないのか" and
// "Generalized Dot-Product Attention（GDPA）"): the four waves of a workgroup
// are split NWQ x NWK between query rows (32 per wave) and key tiles (64 keys
// per tile), so long-query shapes use NWQ=4, the 64-token block window uses
// NWQ=2 x NWK=2 (one query block, its window split over two wave pairs) and
// PMA (32 queries, long keys) uses NWK=4 plus a key split across workgroups.
//
// Score tiles are computed transposed, S^T = K Q^T, with K from LDS as the A
// operand and Q resident in registers as the B operand: the 32x32 result then
// leaves every lane holding one query's scores, so softmax row statistics need
// only one exchange between the two half-waves, and P^T is already the B
// operand of O^T = V^T P^T.  V is stored transposed in LDS for that product.
// Two free index permutations are used:
//  * the A rows of S^T (keys) are fed with bits 2 and 3 of the row swapped, so
//    lane-half g ends up holding keys 16*(i/8) + 8g + i%8 in register i -- eight
//    consecutive keys per MFMA k-chunk, read from V^T with one 16-byte load;
//  * the A rows of O^T (head dims) of output tile t are chosen so that lane-half
//    g holds dims (D/2)g + 16t + i: each lane owns a contiguous half row of O,
//    and Q is loaded the same way (contraction order is free for a dot product).
// Softmax (online, base 2) is kept per lane; GELU needs no statistics
// (techfeed.io GDPA section: the QK-norm bounds the activation input, and no
// correction stage is needed); the block window needs no element mask because
// 64-key tiles coincide with the 64-token blocks ("BlockAttention" section).
#include "ja_device.h"
#include "jagged_attn.h"

namespace ja {

namespace {

constexpr int kVtStride = 80;  // bf16 per V^T row: 64 keys + 16 pad (bank spread)

template <int D>
struct Lds {
  static constexpr int kKStride = D + 8;                 // bf16 per K row
  static constexpr int kKSize = 64 * kKStride;           // bf16 elements
  static constexpr int kVtSize = D * kVtStride + 8;      // rows >= D/2 shifted by 8
  static constexpr int kGroup = kKSize + kVtSize;        // one key tile (K + V^T)
};

// V^T row offset (bf16 units): rows of the upper half start 16 bytes later so
// that a 16-lane LDS phase reading dims {d, d + D/2} hits distinct banks.
template <int D>
__device__ __forceinline__ int vt_row(int d) {
  return d * kVtStride + (d >= D / 2 ? 8 : 0);
}

// Key row feeding A row r of S^T: bits 2 and 3 of r swapped.
__device__ __forceinline__ int key_perm(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Head dim feeding A row r of output tile t of O^T.
template <int D>
__device__ __forceinline__ int dim_perm(int t, int r) {
  return (D / 2) * ((r >> 2) & 1) + 16 * t + ((r >> 3) << 2) + (r & 3);
}

template <int IN>
__device__ __forceinline__ bf16x8 load_row8(const void* base, size_t elem, const uint8_t* scales,
                                            size_t scale_idx) {
  if constexpr (IN == IN_BF16) {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(base) + elem);
  } else {
    const u32x2 c = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(base) + elem);
    return decode_mx8(c, scales[scale_idx]);
  }
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = (__bf16)0.0f;
  return z;
}

template <int D, int NWQ, int NWK, int ACT, int IN, bool WINDOW, bool SPLIT>
struct Attn {
  using L = Lds<D>;
  static constexpr int kQChunks = D / 16;   // MFMA k-chunks over D
  static constexpr int kOTiles = D / 32;    // 32-dim output tiles

  // Cooperative load of 64 key rows [key0, key0+64) of (sample, head) into
  // K (row-major) and V^T; rows at or beyond kv_end are zero.  GELU also
  // stores each key's RMSNorm factor.
  static __device__ __forceinline__ void load_tile(const AttnArgs& a, __bf16* grp, float* kscale,
                                                   size_t kv_row0, int h, int key0, int kv_end) {
    const int tid = threadIdx.x;
    __bf16* ks = grp;
    __bf16* vt = grp + L::kKSize;
    constexpr int kChunks = D / 8;             // 8-element chunks per row
    constexpr int kKUnits = 64 * kChunks;
#pragma unroll
    for (int u0 = 0; u0 < kKUnits; u0 += kThreads) {
      const int u = u0 + tid;
      const int key = u / kChunks, ch = u % kChunks;
      bf16x8 x = zero8();
      if (key0 + key < kv_end) {
        const size_t row = (kv_row0 + key0 + key) * a.H + h;
        x = load_row8<IN>(a.k, row * D + 8 * ch, a.ks, row * (D / kMxBlock) + (8 * ch) / kMxBlock);
      }
      *reinterpret_cast<bf16x8*>(ks + key * L::kKStride + 8 * ch) = x;
      if constexpr (ACT == ACT_GELU) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fmaf(float(x[j]), float(x[j]), ss);
#pragma unroll
        for (int o = 1; o < kChunks; o <<= 1) ss += __shfl_xor(ss, o, 64);
        if (ch == 0) kscale[key] = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.eps);
      }
    }
    constexpr int kVUnits = 32 * kChunks;      // (key pair, chunk)
#pragma unroll
    for (int u0 = 0; u0 < kVUnits; u0 += kThreads) {
      const int u = u0 + tid;
      if (kVUnits % kThreads == 0 || u < kVUnits) {
        const int p = u % 32, ch = u / 32;
        bf16x8 x0 = zero8(), x1 = zero8();
        const int k0 = key0 + 2 * p;
        if (k0 < kv_end) {
          const size_t row = (kv_row0 + k0) * a.H + h;
          x0 = load_row8<IN>(a.v, row * D + 8 * ch, a.vs, row * (D / kMxBlock) + (8 * ch) / kMxBlock);
        }
        if (k0 + 1 < kv_end) {
          const size_t row = (kv_row0 + k0 + 1) * a.H + h;
          x1 = load_row8<IN>(a.v, row * D + 8 * ch, a.vs, row * (D / kMxBlock) + (8 * ch) / kMxBlock);
        }
        // Pair element j of key 2p (low half) with element j of key 2p+1 (high
        // half).  Whole-vector casts only: hipcc folds a bit_cast of a single
        // bf16 vector element to element 0.
        const u32x4 w0 = __builtin_bit_cast(u32x4, x0), w1 = __builtin_bit_cast(u32x4, x1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          *reinterpret_cast<unsigned*>(vt + vt_row<D>(8 * ch + 2 * i) + 2 * p) =
              (w0[i] & 0xFFFFu) | (w1[i] << 16);
          *reinterpret_cast<unsigned*>(vt + vt_row<D>(8 * ch + 2 * i + 1) + 2 * p) =
              (w0[i] >> 16) | (w1[i] & 0xFFFF0000u);
        }
      }
    }
  }

  static __device__ void run_item(const AttnArgs& a, const int4 item, __bf16* lds, float* kscale_all,
                                  float* cbuf) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wq = wave % NWQ, wk = wave / NWQ;
    const int l32 = lane & 31, g = lane >> 5;
    const int b = item.x, h = item.y, q0 = item.z, split = item.w;
    const int qbeg = a.qo[b], lq = a.qo[b + 1] - qbeg;
    const int kbeg = a.ko[b], lk = a.ko[b + 1] - kbeg;

    int kv_lo = 0, kv_hi = lk;
    if constexpr (SPLIT) {
      if (a.nsplit[b] > 1) {
        kv_lo = split * a.kvc;
        kv_hi = min(lk, kv_lo + a.kvc);
      }
    }
    if constexpr (WINDOW) {
      const int qlast = min(q0 + 32 * NWQ, lq) - 1;
      kv_lo = max(0, q0 / kBlock - a.window_blocks + 1) * kBlock;
      kv_hi = min(lk, (qlast / kBlock + 1) * kBlock);
    }
    const int ntiles = kv_hi > kv_lo ? (kv_hi - kv_lo + 63) / 64 : 0;

    const int qrow_w = q0 + 32 * wq;          // first row of this wave (sample-local)
    const bool wave_has_rows = qrow_w < lq;
    const int qrow = qrow_w + l32;
    const bool qvalid = qrow < lq;
    const int wblk = qrow_w / kBlock;

    // Q fragment: lane holds dims [(D/2)g, (D/2)g + D/2) of its query row.
    bf16x8 qf[kQChunks];
    if (qvalid) {
      const size_t row = size_t(qbeg + qrow) * a.H + h;
#pragma unroll
      for (int c = 0; c < kQChunks; ++c) {
        const int d0 = (D / 2) * g + 8 * c;
        qf[c] = load_row8<IN>(a.q, row * D + d0, a.qs, row * (D / kMxBlock) + d0 / kMxBlock);
      }
    } else {
#pragma unroll
      for (int c = 0; c < kQChunks; ++c) qf[c] = zero8();
    }
    float rq = 1.0f;
    if constexpr (ACT == ACT_GELU) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < kQChunks; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fmaf(float(qf[c][j]), float(qf[c][j]), ss);
      ss += other_half(ss);
      rq = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.eps) * a.score_scale;
    }

    f32x16 o[kOTiles];
#pragma unroll
    for (int t = 0; t < kOTiles; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
    float m = -__builtin_huge_valf(), l = 0.f;

    const size_t kv_row0 = size_t(kbeg);
    for (int t0 = 0; t0 < ntiles; t0 += NWK) {
      __syncthreads();  // the previous tiles are no longer read
#pragma unroll
      for (int kg = 0; kg < NWK; ++kg)
        if (t0 + kg < ntiles)
          load_tile(a, lds + kg * L::kGroup, kscale_all + kg * 64, kv_row0, h,
                    kv_lo + 64 * (t0 + kg), kv_hi);
      __syncthreads();
      const int tile = t0 + wk;
      if (tile >= ntiles || !wave_has_rows) continue;
      const int key0 = kv_lo + 64 * tile;
      if constexpr (WINDOW) {
        const int kb = key0 / kBlock;
        if (kb > wblk || kb < wblk - a.window_blocks + 1) continue;
      }
      const __bf16* ks = lds + wk * L::kGroup;
      const __bf16* vt = ks + L::kKSize;
      const float* kscale = kscale_all + wk * 64;

      // S^T for two 32-key halves of the tile.
      f32x16 s[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[st][i] = 0.f;
        const __bf16* krow = ks + (32 * st + key_perm(l32)) * L::kKStride + (D / 2) * g;
#pragma unroll
        for (int c = 0; c < kQChunks; ++c)
          s[st] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(krow + 8 * c), qf[c], s[st]);
      }
      // Register i of half st holds key 32*st + 16*(i/8) + 8g + i%8 of the tile.
      const int nvalid = kv_hi - key0;  // keys at or beyond this index are outside
      if constexpr (ACT == ACT_SOFTMAX) {
        float mt = -__builtin_huge_valf();
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kk = 32 * st + 16 * (i >> 3) + 8 * g + (i & 7);
            const float x = kk < nvalid ? s[st][i] * a.score_scale : -__builtin_huge_valf();
            s[st][i] = x;
            mt = fmaxf(mt, x);
          }
        mt = fmaxf(mt, other_half(mt));
        const float m_new = fmaxf(m, mt);
        const float m_use = m_new == -__builtin_huge_valf() ? 0.f : m_new;
        const float alpha = fast_exp2(m - m_use);
        l *= alpha;
#pragma unroll
        for (int t = 0; t < kOTiles; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(s[st][i] - m_use);
            s[st][i] = p;
            l += p;
          }
        m = m_new;
      } else {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kk = 32 * st + 16 * (i >> 3) + 8 * g + (i & 7);
            s[st][i] = kk < nvalid ? gelu_tanh(s[st][i] * rq * kscale[kk]) : 0.f;
          }
      }
      // O^T += V^T P^T over four 16-key chunks.
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        bf16x8 pf;
#pragma unroll
        for (int j = 0; j < 8; ++j) pf[j] = (__bf16)s[kc >> 1][8 * (kc & 1) + j];
#pragma unroll
        for (int t = 0; t < kOTiles; ++t) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
              vt + vt_row<D>(dim_perm<D>(t, l32)) + 16 * kc + 8 * g);
          o[t] = mfma_32x32x16(vf, pf, o[t]);
        }
      }
    }

    // Merge the key groups of a query group (NWK > 1) through LDS.
    if constexpr (NWK > 1) {
      constexpr int kRec = D / 2 + 2;  // floats per lane record: O half row, m, l
      __syncthreads();
      if (wk > 0) {
        float* rec = cbuf + (((wk - 1) * NWQ + wq) * 64 + lane) * kRec;
#pragma unroll
        for (int t = 0; t < kOTiles; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) rec[16 * t + i] = o[t][i];
        rec[D / 2] = m;
        rec[D / 2 + 1] = l;
      }
      __syncthreads();
      if (wk == 0) {
#pragma unroll
        for (int w = 1; w < NWK; ++w) {
          const float* rec = cbuf + (((w - 1) * NWQ + wq) * 64 + lane) * kRec;
          if constexpr (ACT == ACT_SOFTMAX) {
            const float m2 = rec[D / 2], l2 = rec[D / 2 + 1];
            const float mn = fmaxf(m, m2);
            const float mu = mn == -__builtin_huge_valf() ? 0.f : mn;
            const float a1 = fast_exp2(m - mu), a2 = fast_exp2(m2 - mu);
#pragma unroll
            for (int t = 0; t < kOTiles; ++t)
#pragma unroll
              for (int i = 0; i < 16; ++i) o[t][i] = o[t][i] * a1 + rec[16 * t + i] * a2;
            l = l * a1 + l2 * a2;
            m = mn;
          } else {
#pragma unroll
            for (int t = 0; t < kOTiles; ++t)
#pragma unroll
              for (int i = 0; i < 16; ++i) o[t][i] += rec[16 * t + i];
          }
        }
      }
    }
    if (wk != 0 || !qvalid) return;

    const float l_tot = l + other_half(l);
    if constexpr (SPLIT) {
      const int ns = a.nsplit[b];
      if (ns > 1) {
        const size_t slot = size_t(a.pbase[b]) + size_t(h) * ns + split;
        float* po = a.part_o + (slot * kPmaRows + qrow) * D + (D / 2) * g;
#pragma unroll
        for (int t = 0; t < kOTiles; ++t)
#pragma unroll
          for (int i = 0; i < 16; i += 4)
            *reinterpret_cast<float4*>(po + 16 * t + i) =
                make_float4(o[t][i], o[t][i + 1], o[t][i + 2], o[t][i + 3]);
        if (g == 0) a.part_ml[slot * kPmaRows + qrow] = make_float2(m, l_tot);
        return;
      }
    }
    float scale;
    if constexpr (ACT == ACT_SOFTMAX) {
      scale = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    } else {
      scale = lk > 0 ? 1.0f / float(lk) : 0.f;
    }
    __bf16* orow = reinterpret_cast<__bf16*>(a.out) + (size_t(qbeg + qrow) * a.H + h) * D + (D / 2) * g;
#pragma unroll
    for (int t = 0; t < kOTiles; ++t)
#pragma unroll
      for (int i = 0; i < 16; i += 8) {
        bf16x8 ov;
#pragma unroll
        for (int j = 0; j < 8; ++j) ov[j] = (__bf16)(o[t][i + j] * scale);
        *reinterpret_cast<bf16x8*>(orow + 16 * t + i) = ov;
      }
  }
};

template <int D, int NWQ, int NWK, int ACT, int IN, bool WINDOW, bool SPLIT>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(AttnArgs a) {
  using K = Attn<D, NWQ, NWK, ACT, IN, WINDOW, SPLIT>;
  using L = Lds<D>;
  constexpr int kTileBytes = NWK * L::kGroup * 2;
  constexpr int kCombBytes = NWK > 1 ? (NWK - 1) * NWQ * 64 * (D / 2 + 2) * 4 : 0;
  constexpr int kBytes = kTileBytes > kCombBytes ? kTileBytes : kCombBytes;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kBytes];
  __shared__ float kscale[ACT == ACT_GELU ? NWK * 64 : 1];
  const int n_items = a.hdr->n_items;
  for (int idx = blockIdx.x; idx < n_items; idx += gridDim.x) {
    K::run_item(a, a.items[idx], reinterpret_cast<__bf16*>(smem), kscale,
                reinterpret_cast<float*>(smem));
    __syncthreads();
  }
}

// Merge of the key splits of one (sample, head): softmax partials hold an
// unnormalised O with the running max m (base 2) and sum l; GELU partials hold
// plain sums.  Fixed split order, so the result is deterministic.
template <int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh % a.H;
  const int ns = a.nsplit[b];
  if (ns <= 1 || a.hdr->status != JA_OK) return;
  const int qbeg = a.qo[b], lq = a.qo[b + 1] - qbeg;
  const int lk = a.ko[b + 1] - a.ko[b];
  constexpr int kPer = D / 8;               // threads per row, 8 dims each
  const int c = threadIdx.x % kPer;
  const int nrows = min(lq, kPmaRows);
  const size_t slot0 = size_t(a.pbase[b]) + size_t(h) * ns;
  for (int r = threadIdx.x / kPer; r < nrows; r += kThreads / kPer) {
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
    float scale;
    if (a.act == ACT_SOFTMAX) {
      float mx = -__builtin_huge_valf();
      for (int s = 0; s < ns; ++s) mx = fmaxf(mx, a.part_ml[(slot0 + s) * kPmaRows + r].x);
      const float mu = mx == -__builtin_huge_valf() ? 0.f : mx;
      float lsum = 0.f;
      for (int s = 0; s < ns; ++s) {
        const float2 ml = a.part_ml[(slot0 + s) * kPmaRows + r];
        const float w = fast_exp2(ml.x - mu);
        lsum += w * ml.y;
        const float* po = a.part_o + ((slot0 + s) * kPmaRows + r) * D + 8 * c;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(w, po[j], acc[j]);
      }
      scale = lsum > 0.f ? 1.0f / lsum : 0.f;
    } else {
      for (int s = 0; s < ns; ++s) {
        const float* po = a.part_o + ((slot0 + s) * kPmaRows + r) * D + 8 * c;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += po[j];
      }
      scale = lk > 0 ? 1.0f / float(lk) : 0.f;
    }
    bf16x8 ov;
#pragma unroll
    for (int j = 0; j < 8; ++j) ov[j] = (__bf16)(acc[j] * scale);
    *reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(a.out) + (size_t(qbeg + r) * a.H + h) * D + 8 * c) = ov;
  }
}

template <int D, int NWQ, int NWK, int ACT, int IN, bool WINDOW, bool SPLIT>
hipError_t launch(const AttnArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_kernel<D, NWQ, NWK, ACT, IN, WINDOW, SPLIT>), dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int D, int IN>
hipError_t launch_for_shape(int shape, int act, const AttnArgs& a, int grid, hipStream_t st) {
  switch (shape) {
    case 0:  // query-tiled (self full, cross)
      return act == ACT_SOFTMAX ? launch<D, 4, 1, ACT_SOFTMAX, IN, false, false>(a, grid, st)
                                : launch<D, 4, 1, ACT_GELU, IN, false, false>(a, grid, st);
    case 1:  // block window (softmax only)
      return launch<D, 2, 2, ACT_SOFTMAX, IN, true, false>(a, grid, st);
    default:  // key-split (PMA)
      return act == ACT_SOFTMAX ? launch<D, 1, 4, ACT_SOFTMAX, IN, false, true>(a, grid, st)
                                : launch<D, 1, 4, ACT_GELU, IN, false, true>(a, grid, st);
  }
}

}  // namespace

// shape: 0 = query-tiled, 1 = block window, 2 = key-split.
hipError_t launch_attn_mfma(int D, int in, int shape, int act, const AttnArgs& a, int grid,
                            hipStream_t st) {
  if (in == IN_BF16) {
    if (D == 32) return launch_for_shape<32, IN_BF16>(shape, act, a, grid, st);
    if (D == 64) return launch_for_shape<64, IN_BF16>(shape, act, a, grid, st);
    return launch_for_shape<128, IN_BF16>(shape, act, a, grid, st);
  }
  if (D == 32) return launch_for_shape<32, IN_MX>(shape, act, a, grid, st);
  if (D == 64) return launch_for_shape<64, IN_MX>(shape, act, a, grid, st);
  return launch_for_shape<128, IN_MX>(shape, act, a, grid, st);
}

hipError_t launch_combine(int D, const CombineArgs& a, hipStream_t st) {
  const int grid = a.B * a.H;
  if (D == 32) hipLaunchKernelGGL(combine_kernel<32>, dim3(grid), dim3(kThreads), 0, st, a);
  else if (D == 64) hipLaunchKernelGGL(combine_kernel<64>, dim3(grid), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL(combine_kernel<128>, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ja
