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
// Data path.  K and V tiles go from HBM straight into LDS (global_load_lds,
// 16 bytes per lane, no register staging), row-major with the 16-byte chunks
// of each row XOR-swizzled so that the MFMA operand reads below are free of
// bank conflicts.  Q stays in registers for the whole item.
//
// Score tiles are computed transposed, S^T = K Q^T, with K from LDS as the A
// operand and Q as the B operand: the 32x32 result leaves every lane holding
// one query's scores, so softmax row statistics need one exchange between the
// two half-waves, and P^T is already the B operand of O^T = V^T P^T.  The V^T
// operand is read from the row-major V tile with the LDS transpose read
// (ds_read_b64_tr_b16: within 16 lanes, lane i gets element i%4 of the 8-byte
// chunks addressed by lanes 4j + i/4).  Two free index permutations are used:
//  * the A rows of S^T (keys) are fed with bits 2 and 3 of the row swapped, so
//    lane-half g holds keys 16*(i/8) + 8g + i%8 in register i -- eight
//    consecutive keys per MFMA k-chunk;
//  * the A rows of O^T (head dims) of output tile t are chosen so lane-half g
//    holds dims (D/2)g + 16t + i: each lane owns a contiguous half row of O,
//    and Q is loaded the same way (the contraction order is free).
// Softmax is online in base 2 and rescales only when some row's max moved;
// GELU needs no statistics (techfeed.io GDPA section: the QK-norm bounds the
// activation input, no correction stage); the block window needs no element
// mask because 64-key tiles coincide with the 64-token blocks (same page,
// "BlockAttention"); only a sample's ragged last tile is masked.
#include "ja_device.h"
#include "jagged_attn.h"

namespace ja {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Key row feeding A row r of S^T: bits 2 and 3 of r swapped.
__device__ __forceinline__ int key_perm(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Head dim feeding A row r of output tile t of O^T.
template <int D>
__device__ __forceinline__ int dim_perm(int t, int r) {
  return (D / 2) * ((r >> 2) & 1) + 16 * t + ((r >> 3) << 2) + (r & 3);
}

// Chunk swizzles (16-byte chunk index XOR) of the K and V tiles, chosen so that
// a 16-lane phase of the K operand reads and a 32-lane phase of the V
// transpose reads touch 64 distinct banks.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (D == 128) return row & 15;
  else if constexpr (D == 64) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (D == 128) return 2 * (row & 3);
  else if constexpr (D == 64) return 2 * ((row >> 1) & 1);
  else return 0;
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = (__bf16)0.0f;
  return z;
}

__device__ __forceinline__ void wait_vmem() {
  // s_waitcnt vmcnt(0): direct-to-LDS loads complete before the barrier
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <int D, int NWQ, int NWK, int ACT, int IN, bool WINDOW, bool SPLIT>
struct Attn {
  static constexpr int kRowBytes = 2 * D;               // one bf16 row in LDS
  static constexpr int kTileBytes = 64 * kRowBytes;      // 64 keys
  static constexpr int kGroupBytes = 2 * kTileBytes;     // K tile + V tile
  static constexpr int kSegs = kTileBytes / 1024;        // 1 KB direct-load segments per tile
  static constexpr int kQChunks = D / 16;                // MFMA k-chunks over D
  static constexpr int kOTiles = D / 32;                 // 32-dim output tiles
  static constexpr int kChunks = D / 8;                  // 16-byte chunks per row

  // Issue the loads of one key tile (keys [key0, key0+64) of the item, rows
  // at or beyond kv_end replaced by row kv_end-1, which the mask removes).
  static __device__ __forceinline__ void issue_tile(unsigned char* grp, const __bf16* kb,
                                                    const __bf16* vb, const uint8_t* ksb,
                                                    const uint8_t* vsb, size_t rs, int key0,
                                                    int kv_end) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if constexpr (IN == IN_BF16) {
      // 2 * kSegs segments of 1 KB (K then V), 4 waves round-robin.
#pragma unroll
      for (int s = wave; s < 2 * kSegs; s += 4) {
        const bool is_v = s >= kSegs;
        const int seg = is_v ? s - kSegs : s;
        const int byte = seg * 1024 + 16 * lane;
        const int row = byte / kRowBytes;
        const int phys = (byte % kRowBytes) / 16;
        const int c = phys ^ (is_v ? swz_v<D>(row) : swz_k<D>(row));
        const int key = min(key0 + row, kv_end - 1);
        const __bf16* src = (is_v ? vb : kb) + size_t(key) * rs + 8 * c;
        unsigned char* dst = grp + (is_v ? kTileBytes : 0) + seg * 1024;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
      }
    } else {
      // MX: decode 8 e4m3 codes x 2^(E-127) to bf16 through registers.
#pragma unroll
      for (int u0 = 0; u0 < 2 * 64 * kChunks; u0 += kThreads) {
        const int u = u0 + tid;
        const bool is_v = u >= 64 * kChunks;
        const int uu = is_v ? u - 64 * kChunks : u;
        const int row = uu / kChunks, c = uu % kChunks;
        const int key = min(key0 + row, kv_end - 1);
        const size_t e = size_t(key) * rs + 8 * c;
        const uint8_t* codes = reinterpret_cast<const uint8_t*>(is_v ? (const void*)vb : (const void*)kb);
        const uint8_t* sc = is_v ? vsb : ksb;
        const bf16x8 x = decode_mx8(*reinterpret_cast<const u32x2*>(codes + e),
                                    sc[size_t(key) * (rs / kMxBlock) + (8 * c) / kMxBlock]);
        const int phys = c ^ (is_v ? swz_v<D>(row) : swz_k<D>(row));
        *reinterpret_cast<bf16x8*>(grp + (is_v ? kTileBytes : 0) + row * kRowBytes + 16 * phys) = x;
      }
    }
  }

  // RMSNorm factor of every key of a loaded K tile (GELU).
  static __device__ __forceinline__ void key_scales(float eps, const unsigned char* grp, float* kscale) {
    const int tid = threadIdx.x;
    const int row = tid >> 2, part = tid & 3;
    constexpr int kPer = kChunks / 4;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = part * kPer + i;
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(grp + row * kRowBytes + 16 * (c ^ swz_k<D>(row)));
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fmaf(float(x[j]), float(x[j]), ss);
    }
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    if (part == 0) kscale[row] = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
  }

  static __device__ void run_item(const AttnArgs& a, const int4 item, unsigned char* lds,
                                  float* kscale_all) {
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

    // Per-item base pointers: key row r of head h starts at base + r * rs.
    const size_t rs = size_t(a.H) * D;
    const size_t kv_off = size_t(kbeg) * rs + size_t(h) * D;
    const __bf16* kb;
    const __bf16* vb;
    const uint8_t* ksb = nullptr;
    const uint8_t* vsb = nullptr;
    if constexpr (IN == IN_BF16) {
      kb = reinterpret_cast<const __bf16*>(a.k) + kv_off;
      vb = reinterpret_cast<const __bf16*>(a.v) + kv_off;
    } else {
      // e4m3 codes are bytes: the element offset is the byte offset
      kb = reinterpret_cast<const __bf16*>(reinterpret_cast<const uint8_t*>(a.k) + kv_off);
      vb = reinterpret_cast<const __bf16*>(reinterpret_cast<const uint8_t*>(a.v) + kv_off);
      ksb = a.ks + (size_t(kbeg) * a.H + h) * (D / kMxBlock);
      vsb = a.vs + (size_t(kbeg) * a.H + h) * (D / kMxBlock);
    }

    // Q fragment: lane holds dims [(D/2)g, (D/2)g + D/2) of its query row.
    bf16x8 qf[kQChunks];
    if (qvalid) {
      const size_t row = size_t(qbeg + qrow) * a.H + h;
#pragma unroll
      for (int c = 0; c < kQChunks; ++c) {
        const int d0 = (D / 2) * g + 8 * c;
        if constexpr (IN == IN_BF16) {
          qf[c] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(a.q) + row * D + d0);
        } else {
          qf[c] = decode_mx8(*reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(a.q) + row * D + d0),
                             a.qs[row * (D / kMxBlock) + d0 / kMxBlock]);
        }
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

    // Lane-constant LDS byte offsets of the MFMA operand reads.
    const int kp = key_perm(l32);
    int k_off[kQChunks];
#pragma unroll
    for (int c = 0; c < kQChunks; ++c) k_off[c] = kp * kRowBytes + 16 * ((kQChunks * g + c) ^ swz_k<D>(kp));
    const int v_row = (8 * g + ((lane & 15) >> 2)) * kRowBytes;
    int v_col[kOTiles];
#pragma unroll
    for (int t = 0; t < kOTiles; ++t) {
      const int col = dim_perm<D>(t, 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
      v_col[t] = 16 * ((col >> 3) ^ swz_v<D>((lane & 15) >> 2)) + 8 * ((col & 7) >> 2);
    }

    f32x16 o[kOTiles];
#pragma unroll
    for (int t = 0; t < kOTiles; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
    float m = -__builtin_huge_valf(), l = 0.f;

    for (int t0 = 0; t0 < ntiles; t0 += NWK) {
      __syncthreads();  // the previous tiles are no longer read
#pragma unroll
      for (int kg = 0; kg < NWK; ++kg)
        if (t0 + kg < ntiles)
          issue_tile(lds + kg * kGroupBytes, kb, vb, ksb, vsb, rs, kv_lo + 64 * (t0 + kg), kv_hi);
      wait_vmem();
      __syncthreads();
      if constexpr (ACT == ACT_GELU) {
#pragma unroll
        for (int kg = 0; kg < NWK; ++kg)
          if (t0 + kg < ntiles) key_scales(a.eps, lds + kg * kGroupBytes, kscale_all + kg * 64);
        __syncthreads();
      }
      const int tile = t0 + wk;
      if (tile >= ntiles || !wave_has_rows) continue;
      const int key0 = kv_lo + 64 * tile;
      if constexpr (WINDOW) {
        const int kblk = key0 / kBlock;
        if (kblk > wblk || kblk < wblk - a.window_blocks + 1) continue;
      }
      const unsigned char* ks = lds + wk * kGroupBytes;
      const unsigned char* vs = ks + kTileBytes;
      const float* kscale = kscale_all + wk * 64;

      // S^T for two 32-key halves of the tile.
      f32x16 s[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[st][i] = 0.f;
#pragma unroll
        for (int c = 0; c < kQChunks; ++c)
          s[st] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(ks + st * 32 * kRowBytes + k_off[c]),
                                qf[c], s[st]);
      }
      // Register i of half st holds key 32*st + 16*(i/8) + 8g + i%8 of the tile.
      const int nvalid = kv_hi - key0;  // keys at or beyond this index are outside
      const bool ragged = nvalid < 64;
      if constexpr (ACT == ACT_SOFTMAX) {
        float mt = -__builtin_huge_valf();
        if (ragged) {
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int kk = 32 * st + 16 * (i >> 3) + 8 * g + (i & 7);
              s[st][i] = kk < nvalid ? s[st][i] * a.score_scale : -__builtin_huge_valf();
              mt = fmaxf(mt, s[st][i]);
            }
        } else {
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              s[st][i] *= a.score_scale;
              mt = fmaxf(mt, s[st][i]);
            }
        }
        mt = fmaxf(mt, other_half(mt));
        const float m_new = fmaxf(m, mt);
        const float m_use = m_new == -__builtin_huge_valf() ? 0.f : m_new;
        if (__any(m_new != m)) {
          const float alpha = fast_exp2(m - m_use);
          l *= alpha;
#pragma unroll
          for (int t = 0; t < kOTiles; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
          m = m_new;
        }
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(s[st][i] - m_use);
            s[st][i] = p;
            l += p;
          }
      } else {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kk = 32 * st + 16 * (i >> 3) + 8 * g + (i & 7);
            const float gl = gelu_tanh(s[st][i] * rq * kscale[kk]);
            s[st][i] = (!ragged || kk < nvalid) ? gl : 0.f;
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
          const unsigned char* p0 = vs + v_row + kc * 16 * kRowBytes + v_col[t];
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 4 * kRowBytes));
          const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
          u32x4 w;
          w[0] = lo2[0];
          w[1] = lo2[1];
          w[2] = hi2[0];
          w[3] = hi2[1];
          o[t] = mfma_32x32x16(__builtin_bit_cast(bf16x8, w), pf, o[t]);
        }
      }
    }

    // Merge the key groups of a query group (NWK > 1) through LDS.
    if constexpr (NWK > 1) {
      constexpr int kRec = D / 2 + 2;  // floats per lane record: O half row, m, l
      float* cbuf = reinterpret_cast<float*>(lds);
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
  constexpr int kTileBytes = NWK * K::kGroupBytes;
  constexpr int kCombBytes = NWK > 1 ? (NWK - 1) * NWQ * 64 * (D / 2 + 2) * 4 : 0;
  constexpr int kBytes = kTileBytes > kCombBytes ? kTileBytes : kCombBytes;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kBytes];
  __shared__ float kscale[ACT == ACT_GELU ? NWK * 64 : 1];
  // Items [xcd_begin[x], xcd_begin[x+1]) belong to XCD x = blockIdx.x % 8.
  const int n = a.hdr->n_items;
  const int x = blockIdx.x % kXcds;
  const int beg = min(a.hdr->xcd_begin[x], n);
  const int end = min(max(a.hdr->xcd_begin[x + 1], beg), n);
  const int stride = gridDim.x / kXcds;
  for (int idx = beg + int(blockIdx.x) / kXcds; idx < end; idx += stride) {
    K::run_item(a, a.items[idx], smem, kscale);
    __syncthreads();
  }
}

// Merge of the key splits of one (sample, head): softmax partials hold an
// unnormalised O with the running max m (base 2) and sum l; GELU partials hold
// plain sums.  Fixed split order, so the result is deterministic.
template <int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  if (a.hdr->status != JA_OK) return;
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh % a.H;
  const int ns = a.nsplit[b];
  if (ns <= 1) return;
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

// Workgroups resident per CU for one kernel instance (queried once).
template <int D, int NWQ, int NWK, int ACT, int IN, bool WINDOW, bool SPLIT>
int resident_per_cu() {
  static int cached = 0;
  if (cached == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, attn_kernel<D, NWQ, NWK, ACT, IN, WINDOW, SPLIT>, kThreads, 0) != hipSuccess || n < 1)
      n = 1;
    cached = n;
  }
  return cached;
}

template <int D, int NWQ, int NWK, int ACT, int IN, bool WINDOW, bool SPLIT>
hipError_t launch(const AttnArgs& a, int num_cu, int64_t max_items, hipStream_t st) {
  // Persistent grid: each resident slot once, a multiple of the XCD count.
  int64_t grid = int64_t(num_cu) * resident_per_cu<D, NWQ, NWK, ACT, IN, WINDOW, SPLIT>();
  const int64_t need = ((max_items + kXcds - 1) / kXcds) * kXcds;
  if (grid > need) grid = need;
  grid = (grid / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  hipLaunchKernelGGL((attn_kernel<D, NWQ, NWK, ACT, IN, WINDOW, SPLIT>), dim3(unsigned(grid)),
                     dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int D, int IN>
hipError_t launch_for_shape(int shape, int act, const AttnArgs& a, int num_cu, int64_t max_items,
                            hipStream_t st) {
  switch (shape) {
    case 0:  // query-tiled (self full, cross)
      return act == ACT_SOFTMAX ? launch<D, 4, 1, ACT_SOFTMAX, IN, false, false>(a, num_cu, max_items, st)
                                : launch<D, 4, 1, ACT_GELU, IN, false, false>(a, num_cu, max_items, st);
    case 1:  // block window (softmax only)
      return launch<D, 2, 2, ACT_SOFTMAX, IN, true, false>(a, num_cu, max_items, st);
    default:  // key-split (PMA)
      return act == ACT_SOFTMAX ? launch<D, 1, 4, ACT_SOFTMAX, IN, false, true>(a, num_cu, max_items, st)
                                : launch<D, 1, 4, ACT_GELU, IN, false, true>(a, num_cu, max_items, st);
  }
}

}  // namespace

// shape: 0 = query-tiled, 1 = block window, 2 = key-split.
hipError_t launch_attn_mfma(int D, int in, int shape, int act, const AttnArgs& a, int num_cu,
                            int64_t max_items, hipStream_t st) {
  if (in == IN_BF16) {
    if (D == 32) return launch_for_shape<32, IN_BF16>(shape, act, a, num_cu, max_items, st);
    if (D == 64) return launch_for_shape<64, IN_BF16>(shape, act, a, num_cu, max_items, st);
    return launch_for_shape<128, IN_BF16>(shape, act, a, num_cu, max_items, st);
  }
  if (D == 32) return launch_for_shape<32, IN_MX>(shape, act, a, num_cu, max_items, st);
  if (D == 64) return launch_for_shape<64, IN_MX>(shape, act, a, num_cu, max_items, st);
  return launch_for_shape<128, IN_MX>(shape, act, a, num_cu, max_items, st);
}

hipError_t launch_combine(int D, const CombineArgs& a, hipStream_t st) {
  const int grid = a.B * a.H;
  if (D == 32) hipLaunchKernelGGL(combine_kernel<32>, dim3(grid), dim3(kThreads), 0, st, a);
  else if (D == 64) hipLaunchKernelGGL(combine_kernel<64>, dim3(grid), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL(combine_kernel<128>, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ja
