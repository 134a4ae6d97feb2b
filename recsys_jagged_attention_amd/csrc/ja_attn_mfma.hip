// Jagged generalized dot-product attention forward on gfx950 MFMA (bf16 and
// MX-fp8 inputs, bf16 output).
//
// One kernel family covers the three shapes of GDPA (techfeed.io summary of
// "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads
// Foundation Model", sections "なぜLLM向けのインフラをそのまま使えないのか" and
// "Generalized Dot-Product Attention（GDPA）"): the waves of a workgroup are
// split NWQ x NWK between query rows and key tiles (64 keys per tile).  A wave
// owns 32*QSUB query rows (QSUB = 2 feeds every K and V^T operand read to two
// MFMAs but needs the whole register file at one wave per SIMD; measured
// slower, so the shapes below use QSUB = 1).  Long-query shapes use 4 waves x
// 32 rows (full self-attention 8 waves, so each key tile in LDS serves 256
// query rows); the 64-token block window uses 4 waves on two consecutive query
// blocks (their windows share all but one key block; each wave skips the tile
// outside its own window); PMA (32 queries, long keys) uses 4 key groups plus
// a key split across workgroups.
//
// Data path.  K and V tiles go from HBM straight into LDS (global_load_lds,
// 16 bytes per lane, no register staging), row-major with the 16-byte chunks
// of each row XOR-swizzled so that the MFMA operand reads below are free of
// bank conflicts.  Two LDS stages: while the waves compute on one, the next
// tile group -- or the next work item's first -- is already in flight into
// the other.  Q stays in registers for the whole item.
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
#include <atomic>
#include <type_traits>

#include "ja_device.h"
#include "ja_mfma_util.h"
#include "jagged_attn.h"

namespace ja {

namespace {


// D: head dim.  NWQ x NWK waves: NWQ query groups of 32*QSUB rows each, NWK
// key groups (each takes every NWK-th tile).  QSUB = 2 lets one wave reuse
// every K and V^T operand read from LDS for two 32-row query blocks.
template <int D, int NWQ, int NWK, int QSUB, int ACT, int IN, bool WINDOW, bool SPLIT>
struct Attn {
  static constexpr int kWaves = NWQ * NWK;
  static constexpr int kNT = 64 * kWaves;               // threads per workgroup
  static constexpr int kRowsPerWave = 32 * QSUB;
  static constexpr int kRowBytes = 2 * D;               // one bf16 row in LDS
  static constexpr int kTileBytes = 64 * kRowBytes;      // 64 keys
  // One key group in LDS.  bf16 / MX decoded: K tile, V tile (bf16).  MX8:
  // K codes, V codes (fp8), K and V scale rows (4 bytes each), V as bf16.
  static constexpr bool kMx8 = IN == IN_MX8;
  static constexpr int kKcOff = 0, kVcOff = 64 * D, kKsOff = 128 * D, kVsOff = 128 * D + 256;
  static constexpr int kVOff = kMx8 ? 128 * D + 512 : kTileBytes;   // bf16 V tile
  static constexpr int kGroupBytes = kMx8 ? 128 * D + 512 + kTileBytes : 2 * kTileBytes;
  static constexpr int kStageBytes = NWK * kGroupBytes;
  static constexpr int kStages = 2 * kStageBytes <= 128 * 1024 ? 2 : 1;
  static constexpr int kSegs = kTileBytes / 1024;        // 1 KB direct-load segments per tile
  static constexpr int kQChunks = D / 16;                // MFMA k-chunks over D
  static constexpr int kOTiles = D / 32;                 // 32-dim output tiles
  static constexpr int kChunks = D / 8;                  // 16-byte chunks per row
  static_assert((2 * kSegs) % kWaves == 0, "tile segments must split evenly over the waves");
  static_assert(!kMx8 || D == 128, "fp8 MFMA path needs D = 128");
  static constexpr int kCodeSegs = 64 * D / 1024;        // 1 KB segments of an fp8 code tile
  static_assert(NWK == 1 || QSUB == 1, "key groups are merged for single-block waves only");

  // ---- Direct-to-LDS loads (bf16 and MX8) --------------------------------
  // A key tile is loaded as 1 KB segments (K then V), shared round-robin by
  // the waves: job k of a wave moves segment wave + kWaves*k.  The lane part of
  // a job's source offset is the same for every full tile, so it is computed
  // once per kernel; only a sample's ragged last tile clamps rows.
  static constexpr int kRowLd = kMx8 ? D : kRowBytes;            // bytes per loaded row
  static constexpr int kSegsLd = 64 * kRowLd / 1024;             // segments per K (or V) tile
  static constexpr int kRowsPerSeg = 1024 / kRowLd;
  static constexpr int kChunksPerRow = kRowLd / 16;
  static constexpr int kDmaTile = (IN == IN_BF16 || kMx8) ? 2 * kSegsLd / kWaves : 0;  // jobs per wave per tile
  static constexpr int kDmaJobs = NWK * kDmaTile;                // jobs per wave per key group
  static constexpr int kVLoadOff = kMx8 ? kVcOff : kTileBytes;   // LDS offset of the V rows in a group

  // What the next direct loads fetch: tiles [t0, t0 + NWK) of an item (none
  // when t0 >= ntiles) into the stage at LDS byte address `lds`.  A tile that
  // does not exist is loaded from a valid stand-in row (dk/dv) instead, so that
  // every job is branch-free; its LDS copy is never read.
  struct Pf {
    const unsigned char* tk[NWK];  // first K row of tile t0 + kg (or the stand-in row)
    const unsigned char* tv[NWK];
    int lim[NWK];                  // last row of the tile that holds a key (0 for stand-ins)
    const uint8_t* ksb;            // MX8 scale rows of the item's head
    const uint8_t* vsb;
    int kv_lo, kv_hi, t0, ntiles;
    unsigned lds;
  };

  // Job j: segment wave + kWaves*(j % kDmaTile) of tile j / kDmaTile.  Rows of a
  // ragged tile are clamped to the last key (min(row, lim) * row_bytes, a
  // 24-bit product: row < 64, and H <= 4096, D <= 128 keep row_bytes <= 1 MiB).
  static __device__ __forceinline__ void pf_job(const Pf& p, int j, unsigned row_bytes) {
    const int kg = j / kDmaTile, k = j % kDmaTile;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int lane = int(threadIdx.x) & 63;
    const int sg = wave + kWaves * k;
    const bool is_v = sg >= kSegsLd;
    const int seg = is_v ? sg - kSegsLd : sg;
    const int lim = p.lim[kg];
    const unsigned char* tile = is_v ? p.tv[kg] : p.tk[kg];
    const int row = seg * kRowsPerSeg + lane / kChunksPerRow;
    const int phys = lane % kChunksPerRow;
    int c;
    if constexpr (kMx8) c = phys ^ swz_c<D>(row);
    else c = phys ^ (is_v ? swz_v<D>(row) : swz_k<D>(row));
    const unsigned off = __umul24(unsigned(min(row, lim)), row_bytes) + 16u * unsigned(c);
    lds_dma16(tile, off, p.lds + kg * kGroupBytes + (is_v ? kVLoadOff : 0) + seg * 1024);
  }

  // MX8: the 4 scale bytes of each of the tile's 64 key rows (wave 0 only).
  static __device__ __forceinline__ void pf_scales(const Pf& p, unsigned srow) {
    if constexpr (kMx8) {
      if (__builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6) != 0) return;
#pragma unroll
      for (int kg = 0; kg < NWK; ++kg) {
        if (p.t0 + kg >= p.ntiles) break;
        const int key0 = p.kv_lo + 64 * (p.t0 + kg);
        const unsigned r = unsigned(min(int(threadIdx.x) & 63, p.kv_hi - 1 - key0));
        lds_dma4(p.ksb + size_t(key0) * srow, r * srow, p.lds + kg * kGroupBytes + kKsOff);
        lds_dma4(p.vsb + size_t(key0) * srow, r * srow, p.lds + kg * kGroupBytes + kVsOff);
      }
    }
  }

  // MX (D < 128): decode 8 e4m3 codes x 2^(E-127) to bf16 through registers,
  // keys [key0, key0+64) of the item, rows at or beyond kv_end replaced by row
  // kv_end-1 (removed by the mask).
  static __device__ __forceinline__ void decode_tile(unsigned char* grp, const __bf16* kb, const __bf16* vb,
                                                     const uint8_t* ksb, const uint8_t* vsb, size_t rs, int key0,
                                                     int kv_end) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u0 = 0; u0 < 2 * 64 * kChunks; u0 += kNT) {
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

  // MX8: convert the V code tile to the bf16 V tile (exact: 4-bit e4m3
  // significands times a power of two), hardware scaled conversion.
  static __device__ __forceinline__ void convert_v(unsigned char* grp) {
    constexpr int kUnits = 64 * D / 8;  // 8 elements per unit
#pragma unroll
    for (int u0 = 0; u0 < kUnits; u0 += kNT) {
      const int u = u0 + int(threadIdx.x);
      const int row = u / (D / 8), j8 = u % (D / 8);
      const int phys16 = (j8 >> 1) ^ swz_c<D>(row);
      const u32x2 w = *reinterpret_cast<const u32x2*>(grp + kVcOff + row * D + 16 * phys16 + 8 * (j8 & 1));
      const unsigned sw = *reinterpret_cast<const unsigned*>(grp + kVsOff + 4 * row);
      const float sc = e8m0_to_float(sw >> (8 * ((8 * j8) / kMxBlock)));
      const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], sc, false);
      const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], sc, true);
      const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], sc, false);
      const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], sc, true);
      u32x4 o;
      o[0] = __builtin_bit_cast(unsigned, p0);
      o[1] = __builtin_bit_cast(unsigned, p1);
      o[2] = __builtin_bit_cast(unsigned, p2);
      o[3] = __builtin_bit_cast(unsigned, p3);
      *reinterpret_cast<u32x4*>(grp + kVOff + row * kRowBytes + 16 * (j8 ^ swz_v<D>(row))) = o;
    }
  }

  // RMSNorm factor of every key of a loaded K tile (GELU): 4 threads per row.
  static __device__ __forceinline__ void key_scales(float eps, const unsigned char* grp, float* kscale) {
#pragma unroll
    for (int t0 = 0; t0 < 256; t0 += kNT) {
      const int t = t0 + int(threadIdx.x);
      const int row = t >> 2, part = t & 3;
      constexpr int kPer = kChunks / 4;
      float ss = 0.f;
      if constexpr (kMx8) {
        // one thread per (row, 32-element block): decode its codes
        const unsigned sw = *reinterpret_cast<const unsigned*>(grp + kKsOff + 4 * row);
        const float sc = e8m0_to_float(sw >> (8 * part));
#pragma unroll
        for (int h16 = 0; h16 < 2; ++h16) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(
              grp + kKcOff + row * D + 16 * ((2 * part + h16) ^ swz_c<D>(row)));
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bf16x2 p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q], sc, false);
            const bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q], sc, true);
            ss = fmaf(float(p[0]), float(p[0]), ss);
            ss = fmaf(float(p[1]), float(p[1]), ss);
            ss = fmaf(float(r[0]), float(r[0]), ss);
            ss = fmaf(float(r[1]), float(r[1]), ss);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const int c = part * kPer + i;
          const bf16x8 x = *reinterpret_cast<const bf16x8*>(grp + row * kRowBytes + 16 * (c ^ swz_k<D>(row)));
#pragma unroll
          for (int j = 0; j < 8; ++j) ss = fmaf(float(x[j]), float(x[j]), ss);
        }
      }
      ss += __shfl_xor(ss, 1, 64);
      ss += __shfl_xor(ss, 2, 64);
      if (part == 0) kscale[row] = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
    }
  }

  // Per-item context (wave-uniform).
  struct Item {
    int b, h, q0, split, qbeg, lq, lk, kv_lo, kv_hi, ntiles;
    const __bf16* kb;   // key row r of this head starts at kb + r * rs (elements; bytes for MX)
    const __bf16* vb;
    const uint8_t* ksb;  // MX scales of key row r start at ksb + r * rs / 32
    const uint8_t* vsb;
  };

  static __device__ __forceinline__ Item make_item(const AttnArgs& a, const WorkItem& it, size_t rs) {
    Item c;
    c.b = it.b;
    c.h = it.h;
    c.q0 = it.q0;
    c.split = it.split;
    c.qbeg = it.qbeg;
    c.lq = it.lq;
    const int kbeg = it.kbeg;
    c.lk = it.lk;
    c.kv_lo = 0;
    c.kv_hi = c.lk;
    if constexpr (SPLIT) {
      if (a.nsplit[c.b] > 1) {
        c.kv_lo = c.split * a.kvc;
        c.kv_hi = min(c.lk, c.kv_lo + a.kvc);
      }
    }
    if constexpr (WINDOW) {
      const int qlast = min(c.q0 + kRowsPerWave * NWQ, c.lq) - 1;
      c.kv_lo = max(0, c.q0 / kBlock - a.window_blocks + 1) * kBlock;
      c.kv_hi = min(c.lk, (qlast / kBlock + 1) * kBlock);
    }
    c.ntiles = c.kv_hi > c.kv_lo ? (c.kv_hi - c.kv_lo + 63) / 64 : 0;
    const size_t kv_off = size_t(kbeg) * rs + size_t(c.h) * D;
    if constexpr (IN == IN_BF16) {
      c.kb = reinterpret_cast<const __bf16*>(a.k) + kv_off;
      c.vb = reinterpret_cast<const __bf16*>(a.v) + kv_off;
      c.ksb = nullptr;
      c.vsb = nullptr;
    } else {  // MX inputs: codes are bytes, scales one byte per 32 elements
      c.kb = reinterpret_cast<const __bf16*>(reinterpret_cast<const uint8_t*>(a.k) + kv_off);
      c.vb = reinterpret_cast<const __bf16*>(reinterpret_cast<const uint8_t*>(a.v) + kv_off);
      c.ksb = a.ks + (size_t(kbeg) * a.H + c.h) * (D / kMxBlock);
      c.vsb = a.vs + (size_t(kbeg) * a.H + c.h) * (D / kMxBlock);
    }
    return c;
  }

  // `stand` is an item with at least one tile (its first row stands in for
  // tiles that do not exist).
  static __device__ __forceinline__ Pf make_pf(const Item& c, int t0, unsigned lds, const Item& stand,
                                               unsigned row_bytes) {
    Pf p;
    const unsigned char* kb = reinterpret_cast<const unsigned char*>(c.kb);
    const unsigned char* vb = reinterpret_cast<const unsigned char*>(c.vb);
    const size_t stand_off = size_t(stand.kv_lo) * row_bytes;
#pragma unroll
    for (int kg = 0; kg < NWK; ++kg) {
      const bool exists = t0 + kg < c.ntiles;
      const int key0 = c.kv_lo + 64 * (t0 + kg);
      const size_t off = size_t(key0) * row_bytes;
      p.tk[kg] = uniform_ptr(exists ? kb + off : reinterpret_cast<const unsigned char*>(stand.kb) + stand_off);
      p.tv[kg] = uniform_ptr(exists ? vb + off : reinterpret_cast<const unsigned char*>(stand.vb) + stand_off);
      p.lim[kg] = exists ? min(63, c.kv_hi - 1 - key0) : 0;
    }
    p.ksb = c.ksb;
    p.vsb = c.vsb;
    p.kv_lo = c.kv_lo;
    p.kv_hi = c.kv_hi;
    p.t0 = t0;
    p.ntiles = c.ntiles;
    p.lds = lds;
    return p;
  }

  // Load the tiles [t0, t0 + NWK) of an item into one stage in one go.
  static __device__ __forceinline__ void issue_group(const Item& c, unsigned char* stage_base, int t0, size_t rs,
                                                     unsigned row_bytes, unsigned srow) {
    if constexpr (IN == IN_MX) {
#pragma unroll
      for (int kg = 0; kg < NWK; ++kg)
        if (t0 + kg < c.ntiles)
          decode_tile(stage_base + kg * kGroupBytes, c.kb, c.vb, c.ksb, c.vsb, rs, c.kv_lo + 64 * (t0 + kg), c.kv_hi);
    } else {
      const Pf p = make_pf(c, t0, lds_addr_of(stage_base), c, row_bytes);
#pragma unroll
      for (int j = 0; j < kDmaJobs; ++j)
        if (t0 + j / kDmaTile < c.ntiles) pf_job(p, j, row_bytes);
      pf_scales(p, srow);
    }
  }
};

template <int D, int NWQ, int NWK, int QSUB, int ACT, int IN, bool WINDOW, bool SPLIT>
__global__ __launch_bounds__(64 * NWQ * NWK, QSUB == 2 ? 1 : 2) void attn_kernel(AttnArgs a) {
  using K = Attn<D, NWQ, NWK, QSUB, ACT, IN, WINDOW, SPLIT>;
  using Item = typename K::Item;
  constexpr int kStageBytes = K::kStageBytes, kStages = K::kStages;
  constexpr int kQChunks = K::kQChunks, kOTiles = K::kOTiles, kRowBytes = K::kRowBytes;
  constexpr int kTileBytes = K::kTileBytes;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * kStageBytes];
  __shared__ float kscale_all[ACT != ACT_SOFTMAX ? kStages * NWK * 64 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wq = wave % NWQ, wk = wave / NWQ;
  const int l32 = lane & 31, g = lane >> 5;
  const size_t rs = size_t(a.H) * D;

  // Without dealing, items [xcd_begin[x], xcd_begin[x+1]) belong to XCD
  // x = blockIdx.x % 8.  Key splits (PMA) and windows come sorted by their key
  // tiles, most first, and are dealt in rounds of gridDim.x, forward on even
  // rounds and backward on odd ones: PMA costs differ by two orders of
  // magnitude, and contiguous ranges left the slowest workgroup at 1.5x the
  // mean.  Windows deal over positions that run XCD by XCD (the grid is a
  // multiple of 8): neighbouring query tiles share key tiles, and dealt over
  // plain workgroup ids they read 1.7x the bytes from HBM.
  const int n = a.hdr->n_items;
  const int x = blockIdx.x % kXcds;
  const int beg = min(a.hdr->xcd_begin[x], n);
  const int end = min(max(a.hdr->xcd_begin[x + 1], beg), n);
  const int stride = gridDim.x / kXcds;
  const bool deal = a.dealt != 0;
  const int G = int(gridDim.x);
  const int pos = SPLIT ? int(blockIdx.x) : x * stride + int(blockIdx.x) / kXcds;
  auto dealt = [&](int k) { return k * G + ((k & 1) ? G - 1 - pos : pos); };
  int n_mine = 0, k_mine = 0;  // (dealing) items of this workgroup, and which one is current
  if (deal) {
    const int full = n / G;
    n_mine = full + (dealt(full) < n ? 1 : 0);
  }
  int idx = deal ? dealt(0) : beg + int(blockIdx.x) / kXcds;
  if (deal ? n_mine == 0 : idx >= end) return;

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
  const float c2 = a.score_scale;  // softmax: log2(e)/sqrt(D); GELU: 1/sqrt(D)
  const float lazy_thr = kLazyLog2 / c2;  // raw-score growth that forces a rescale

  // Direct-load geometry: bytes between key rows.
  const unsigned row_bytes = K::kMx8 ? unsigned(rs) : 2u * unsigned(rs);  // bytes between key rows
  const unsigned srow = unsigned(rs / kMxBlock);                            // MX scale bytes between key rows

  Item cur = K::make_item(a, a.items[idx], rs);
  int stage = 0;
  K::issue_group(cur, smem, 0, rs, row_bytes, srow);

  while (true) {
    const int qrow_w = cur.q0 + K::kRowsPerWave * wq;   // first row of this wave (sample-local)
    const bool wave_has_rows = qrow_w < cur.lq;
    const int wblk = qrow_w / kBlock;

    // Q fragments: lane holds dims [(D/2)g, (D/2)g + D/2) of query row
    // qrow_w + 32*qs + l32.  Rows past the sample load its last row: their
    // results are finite and never stored, and nothing waits on the loads
    // before the first score MFMA.
    bf16x8 qf[QSUB][kQChunks];
    // MX8: operand c of lane-half g holds elements 64c+16g+[0,16) (bytes 0-15,
    // scaled by the lower lane-half's scale) and 64c+32+16g+[0,16) (bytes 16-31,
    // scaled by the upper lane-half's), so lane-half g carries the scale of
    // 32-element block 2c+g.
    i32x8 qc[QSUB][D / 64 > 0 ? D / 64 : 1];
    int qsc[QSUB][D / 64 > 0 ? D / 64 : 1];
    float rq[QSUB];
#pragma unroll
    for (int qs = 0; qs < QSUB; ++qs) {
      const int qrow = qrow_w + 32 * qs + l32;
      const size_t row = size_t(cur.qbeg + min(qrow, cur.lq - 1)) * a.H + cur.h;
      if constexpr (IN == IN_MX8) {
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < D / 64; ++c) {
          const uint8_t* src = reinterpret_cast<const uint8_t*>(a.q) + row * D + 64 * c + 16 * g;
          const u32x4 w0 = *reinterpret_cast<const u32x4*>(src);
          const u32x4 w1 = *reinterpret_cast<const u32x4*>(src + 32);
          const int sb0 = a.qs[row * (D / kMxBlock) + 2 * c];
          const int sb1 = a.qs[row * (D / kMxBlock) + 2 * c + 1];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            qc[qs][c][i] = int(w0[i]);
            qc[qs][c][4 + i] = int(w1[i]);
          }
          qsc[qs][c] = g ? sb1 : sb0;
          if constexpr (ACT != ACT_SOFTMAX) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float sc = e8m0_to_float(unsigned(i < 4 ? sb0 : sb1));
              const bf16x2 p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(unsigned(qc[qs][c][i]), sc, false);
              const bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(unsigned(qc[qs][c][i]), sc, true);
              ss = fmaf(float(p[0]), float(p[0]), ss);
              ss = fmaf(float(p[1]), float(p[1]), ss);
              ss = fmaf(float(r[0]), float(r[0]), ss);
              ss = fmaf(float(r[1]), float(r[1]), ss);
            }
          }
        }
        if constexpr (ACT != ACT_SOFTMAX) {
          ss = sum_halves(ss);
          rq[qs] = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.eps) * c2;
        } else {
          rq[qs] = 1.0f;
        }
        continue;
      }
#pragma unroll
      for (int c = 0; c < kQChunks; ++c) {
        const int d0 = (D / 2) * g + 8 * c;
        if constexpr (IN == IN_BF16) {
          qf[qs][c] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(a.q) + row * D + d0);
        } else {
          qf[qs][c] = decode_mx8(*reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(a.q) + row * D + d0),
                                 a.qs[row * (D / kMxBlock) + d0 / kMxBlock]);
        }
      }
      rq[qs] = 1.0f;
      if constexpr (ACT != ACT_SOFTMAX) {
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < kQChunks; ++c)
#pragma unroll
          for (int j = 0; j < 8; ++j) ss = fmaf(float(qf[qs][c][j]), float(qf[qs][c][j]), ss);
        ss = sum_halves(ss);
        rq[qs] = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.eps) * c2;
      }
    }

    const bool has_next = deal ? k_mine + 1 < n_mine : idx + stride < end;
    const int next_idx = deal ? (has_next ? dealt(k_mine + 1) : idx) : idx + stride;
    Item nxt = cur;
    if (has_next) nxt = K::make_item(a, a.items[next_idx], rs);

    f32x16 o[QSUB][kOTiles];
#pragma unroll
    for (int qs = 0; qs < QSUB; ++qs)
#pragma unroll
      for (int t = 0; t < kOTiles; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[qs][t][i] = 0.f;
    float m[QSUB], l[QSUB];  // m in raw score units
#pragma unroll
    for (int qs = 0; qs < QSUB; ++qs) {
      m[qs] = -__builtin_huge_valf();
      l[qs] = 0.f;
    }

    for (int t0 = 0; t0 < cur.ntiles; t0 += NWK) {
      // The next key group (or the next item's first) goes to the other stage.
      // Direct loads are issued between the score MFMAs below, after the first
      // half has consumed every Q fragment: the compiler waits for the Q loads
      // with counts that do not know about these loads.
      unsigned char* other = smem + (stage ^ 1) * kStageBytes;
      // (no next group: tiles past the end of the current item, i.e. stand-ins)
      const bool pf_cur = t0 + NWK < cur.ntiles || !has_next;
      const typename K::Pf pf =
          K::make_pf(pf_cur ? cur : nxt, pf_cur ? t0 + NWK : 0, lds_addr_of(other), cur, row_bytes);
      if constexpr (kStages == 2) {
        if constexpr (IN == IN_MX) {  // decoded through registers: done here, in one go
          if (t0 + NWK < cur.ntiles) K::issue_group(cur, other, t0 + NWK, rs, row_bytes, srow);
          else if (has_next) K::issue_group(nxt, other, 0, rs, row_bytes, srow);
        }
      } else {
        // group 0 was loaded before the item
        if (t0 > 0) K::issue_group(cur, smem, t0, rs, row_bytes, srow);
      }
      wait_vmcnt(0);
      lds_barrier();
      unsigned char* st_base = smem + stage * kStageBytes;
      float* kscale_st = kscale_all + (ACT != ACT_SOFTMAX ? stage * NWK * 64 : 0);
      if constexpr (ACT != ACT_SOFTMAX || IN == IN_MX8) {
#pragma unroll
        for (int kg = 0; kg < NWK; ++kg)
          if (t0 + kg < cur.ntiles) {
            if constexpr (ACT != ACT_SOFTMAX) K::key_scales(a.eps, st_base + kg * K::kGroupBytes, kscale_st + kg * 64);
            if constexpr (IN == IN_MX8) K::convert_v(st_base + kg * K::kGroupBytes);
          }
        lds_barrier();
      }
      const int tile = t0 + wk;
      bool active = tile < cur.ntiles && wave_has_rows;
      const int key0 = cur.kv_lo + 64 * tile;
      if constexpr (WINDOW) {
        const int kblk = key0 / kBlock;
        active = active && kblk <= wblk && kblk >= wblk - a.window_blocks + 1;
      }
      const unsigned char* ks = st_base + wk * K::kGroupBytes;
      const unsigned char* vs = ks + K::kVOff;
      const float* kscale = kscale_st + wk * 64;
      // S^T for two 32-key halves of the tile, each K operand read feeding QSUB MFMAs.
      f32x16 s[QSUB][2];
#pragma unroll
      for (int qs = 0; qs < QSUB; ++qs)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[qs][st][i] = 0.f;
      // Scores for the 32-key halves st = 0, 1 of the tile.  The next group's
      // direct loads go between the MFMAs of the second half: for a group of
      // full tiles (kFast) one branch-free job after each MFMA, else (ragged or
      // partial groups) all jobs between the two halves.  LDS reads are not
      // moved across volatile asm, so the K operand is read one MFMA ahead.
      // Direct loads run only with two stages (else the group was loaded above).
      constexpr bool kFast = kStages == 2 && (IN == IN_BF16 || IN == IN_MX8);
      auto scores = [&]() {
        if constexpr (IN == IN_MX8) {
          // block-scaled fp8 MFMA: key row operand laid out like the query's
          // (16-byte chunks 4c+g and 4c+2+g), lane-half g giving block 2c+g's scale
          constexpr int kNC = D / 64;
          auto kop = [&](int krow, int c) {
            const u32x4 w0 = *reinterpret_cast<const u32x4*>(ks + krow * D + 16 * ((4 * c + g) ^ swz_c<D>(krow)));
            const u32x4 w1 = *reinterpret_cast<const u32x4*>(ks + krow * D + 16 * ((4 * c + 2 + g) ^ swz_c<D>(krow)));
            i32x8 ka;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              ka[i] = int(w0[i]);
              ka[4 + i] = int(w1[i]);
            }
            return ka;
          };
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const int krow = 32 * st + kp;
            const unsigned ksw = *reinterpret_cast<const unsigned*>(ks + K::kKsOff + 4 * krow);
#pragma unroll
            for (int c = 0; c < kNC; ++c) {
              const i32x8 ka = kop(krow, c);  // two MFMAs per half: no read-ahead (registers)
              const int kscl = int((ksw >> (8 * (2 * c + g))) & 0xFFu);
#pragma unroll
              for (int qs = 0; qs < QSUB; ++qs)
                s[qs][st] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qc[qs][c], s[qs][st], 0, 0, 0, kscl,
                                                                             0, qsc[qs][c]);
              if constexpr (kFast) {
                if (st == 1) {
#pragma unroll
                  for (int j = c * K::kDmaJobs / kNC; j < (c + 1) * K::kDmaJobs / kNC; ++j)
                    K::pf_job(pf, j, row_bytes);
                }
              }
            }
          }
        } else {
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            bf16x8 knext = *reinterpret_cast<const bf16x8*>(ks + st * 32 * kRowBytes + k_off[0]);
#pragma unroll
            for (int c = 0; c < kQChunks; ++c) {
              const bf16x8 kf = knext;
              if (c + 1 < kQChunks) knext = *reinterpret_cast<const bf16x8*>(ks + st * 32 * kRowBytes + k_off[c + 1]);
#pragma unroll
              for (int qs = 0; qs < QSUB; ++qs) s[qs][st] = mfma_32x32x16(kf, qf[qs][c], s[qs][st]);
              if constexpr (kFast) {
                if (st == 1) {
#pragma unroll
                  for (int j = c * K::kDmaJobs / kQChunks; j < (c + 1) * K::kDmaJobs / kQChunks; ++j)
                    K::pf_job(pf, j, row_bytes);
                }
              }
            }
          }
        }
      };
      if (active) {
        scores();
      } else if constexpr (kFast) {
#pragma unroll
        for (int j = 0; j < K::kDmaJobs; ++j) K::pf_job(pf, j, row_bytes);
      }
      if constexpr (kFast) K::pf_scales(pf, srow);
      if (active) {
        // Register i of half st holds key 32*st + 16*(i/8) + 8g + i%8 of the tile.
        const int nvalid = cur.kv_hi - key0;  // keys at or beyond this index are outside
        const bool ragged = nvalid < 64;
#pragma unroll
        for (int qs = 0; qs < QSUB; ++qs) {
          if constexpr (ACT == ACT_SOFTMAX) {
            if (ragged) {
#pragma unroll
              for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                  const int kk = 32 * st + 16 * (i >> 3) + 8 * g + (i & 7);
                  if (kk >= nvalid) s[qs][st][i] = -__builtin_huge_valf();
                }
            }
            float mt = -__builtin_huge_valf();
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
              for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[qs][st][i]);
            mt = max_halves(mt);
            // Lazy rescale: the reference max moves only when a row's tile max
            // exceeds it by more than kLazyLog2 (base 2), so exponentials stay
            // below 2^kLazyLog2 and most tiles skip the O rescale.  Softmax is
            // unchanged by the choice of reference; the final 1/l uses the same one.
            if (__any(mt - m[qs] > lazy_thr)) {
              const float m_new = fmaxf(m[qs], mt);
              const float alpha = m[qs] == -__builtin_huge_valf() ? 0.f : fast_exp2((m[qs] - m_new) * c2);
              l[qs] *= alpha;
#pragma unroll
              for (int t = 0; t < kOTiles; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[qs][t][i] *= alpha;
              m[qs] = m_new;
            }
            const float mc = m[qs] == -__builtin_huge_valf() ? 0.f : m[qs] * c2;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const float p = fast_exp2(fmaf(s[qs][st][i], c2, -mc));
                s[qs][st][i] = p;
                l[qs] += p;
              }
          } else {
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int kk = 32 * st + 16 * (i >> 3) + 8 * g + (i & 7);
                const float gl = gelu_act<ACT>(s[qs][st][i] * rq[qs] * kscale[kk]);
                s[qs][st][i] = (!ragged || kk < nvalid) ? gl : 0.f;
              }
          }
        }
        // O^T += V^T P^T over four 16-key chunks, each V^T read feeding QSUB MFMAs.
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          bf16x8 pf8[QSUB];
#pragma unroll
          for (int qs = 0; qs < QSUB; ++qs)
#pragma unroll
            for (int j = 0; j < 8; ++j) pf8[qs][j] = (__bf16)s[qs][kc >> 1][8 * (kc & 1) + j];
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
            const bf16x8 vf = __builtin_bit_cast(bf16x8, w);
#pragma unroll
            for (int qs = 0; qs < QSUB; ++qs) o[qs][t] = mfma_32x32x16(vf, pf8[qs], o[qs][t]);
          }
        }
      }
      lds_barrier();  // this stage may be refilled from the next iteration on
      if constexpr (kStages == 2) stage ^= 1;
    }
    if constexpr (kStages == 2) {
      if (cur.ntiles == 0 && has_next) K::issue_group(nxt, smem + stage * kStageBytes, 0, rs, row_bytes, srow);
    }

    // Merge the key groups of a query group (NWK > 1, QSUB == 1) through the free stage.
    if constexpr (NWK > 1) {
      constexpr int kRec = D / 2 + 2;  // floats per lane record: O half row, m, l
      float* cbuf = reinterpret_cast<float*>(smem + (kStages == 2 ? (stage ^ 1) * kStageBytes : 0));
      if (wk > 0) {
        float* rec = cbuf + (((wk - 1) * NWQ + wq) * 64 + lane) * kRec;
#pragma unroll
        for (int t = 0; t < kOTiles; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) rec[16 * t + i] = o[0][t][i];
        rec[D / 2] = m[0];
        rec[D / 2 + 1] = l[0];
      }
      lds_barrier();
      if (wk == 0) {
#pragma unroll
        for (int w = 1; w < NWK; ++w) {
          const float* rec = cbuf + (((w - 1) * NWQ + wq) * 64 + lane) * kRec;
          if constexpr (ACT == ACT_SOFTMAX) {
            const float m2 = rec[D / 2], l2 = rec[D / 2 + 1];
            const float mn = fmaxf(m[0], m2);
            const float a1 = m[0] == -__builtin_huge_valf() ? 0.f : fast_exp2((m[0] - mn) * c2);
            const float a2 = m2 == -__builtin_huge_valf() ? 0.f : fast_exp2((m2 - mn) * c2);
#pragma unroll
            for (int t = 0; t < kOTiles; ++t)
#pragma unroll
              for (int i = 0; i < 16; ++i) o[0][t][i] = o[0][t][i] * a1 + rec[16 * t + i] * a2;
            l[0] = l[0] * a1 + l2 * a2;
            m[0] = mn;
          } else {
#pragma unroll
            for (int t = 0; t < kOTiles; ++t)
#pragma unroll
              for (int i = 0; i < 16; ++i) o[0][t][i] += rec[16 * t + i];
          }
        }
      }
      lds_barrier();  // the merge buffer may be refilled by the next prefetch
    }
    if constexpr (kStages == 1) {
      if (has_next) K::issue_group(nxt, smem, 0, rs, row_bytes, srow);  // LDS is free again
    }

    if (wk == 0) {
#pragma unroll
      for (int qs = 0; qs < QSUB; ++qs) {
        const int qrow = qrow_w + 32 * qs + l32;
        if (qrow >= cur.lq) continue;
        const float l_tot = sum_halves(l[qs]);
        bool done = false;
        if constexpr (SPLIT) {
          const int ns = a.nsplit[cur.b];
          if (ns > 1) {
            const size_t slot = size_t(a.pbase[cur.b]) + size_t(cur.h) * ns + cur.split;
            float* po = a.part_o + (slot * kPmaRows + qrow) * D + (D / 2) * g;
#pragma unroll
            for (int t = 0; t < kOTiles; ++t)
#pragma unroll
              for (int i = 0; i < 16; i += 4)
                *reinterpret_cast<float4*>(po + 16 * t + i) =
                    make_float4(o[qs][t][i], o[qs][t][i + 1], o[qs][t][i + 2], o[qs][t][i + 3]);
            // running max stored in base-2 units
            if (g == 0)
              a.part_ml[slot * kPmaRows + qrow] =
                  make_float2(m[qs] == -__builtin_huge_valf() ? m[qs] : m[qs] * c2, l_tot);
            done = true;
          }
        }
        if (!done) {
          float scale;
          if constexpr (ACT == ACT_SOFTMAX) {
            scale = l_tot > 0.f ? 1.0f / l_tot : 0.f;
          } else {
            scale = cur.lk > 0 ? 1.0f / float(cur.lk) : 0.f;
          }
          __bf16* orow = reinterpret_cast<__bf16*>(a.out) + (size_t(cur.qbeg + qrow) * a.H + cur.h) * D + (D / 2) * g;
#pragma unroll
          for (int t = 0; t < kOTiles; ++t)
#pragma unroll
            for (int i = 0; i < 16; i += 8) {
              bf16x8 ov;
#pragma unroll
              for (int j = 0; j < 8; ++j) ov[j] = (__bf16)(o[qs][t][i + j] * scale);
              *reinterpret_cast<bf16x8*>(orow + 16 * t + i) = ov;
            }
          if constexpr (ACT == ACT_SOFTMAX && SPLIT) {
            // log-sum-exp output of the key-split (PMA) shape, for a sample
            // taken whole: ln sum_j exp(s_j / sqrt(D)) = (m c2 + log2 l) ln 2,
            // m the row's reference max of the raw scores (-inf without keys).
            // (Not in the other instances: at D = 32 / 64 with MX inputs the
            // store cost them a third of their occupancy.)
            if (a.lse != nullptr && g == 0)
              a.lse[size_t(cur.qbeg + qrow) * a.H + cur.h] =
                  l_tot > 0.f ? (m[qs] * c2 + __log2f(l_tot)) * 0.69314718055994531f : -__builtin_huge_valf();
          }
        }
      }
    }
    if (!has_next) break;
    idx = next_idx;
    cur = nxt;
    ++k_mine;
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
      // log-sum-exp output (the partial maxima are in base-2 units)
      if (a.lse != nullptr && c == 0)
        a.lse[size_t(qbeg + r) * a.H + h] = lsum > 0.f ? (mu + __log2f(lsum)) * 0.69314718055994531f
                                                        : -__builtin_huge_valf();
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

// Workgroups resident per CU for one kernel instance (queried once; concurrent
// first calls may both query, and store the same value).
template <int D, int NWQ, int NWK, int QSUB, int ACT, int IN, bool WINDOW, bool SPLIT>
int resident_per_cu() {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, attn_kernel<D, NWQ, NWK, QSUB, ACT, IN, WINDOW, SPLIT>, 64 * NWQ * NWK, 0) != hipSuccess ||
        n < 1)
      n = 1;
    cached.store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D, int NWQ, int NWK, int QSUB, int ACT, int IN, bool WINDOW, bool SPLIT>
hipError_t launch(const AttnArgs& a, int num_cu, int64_t max_items, int64_t grid_cap, const KTiming& tm,
                  hipStream_t st) {
  // Persistent grid: each resident slot once, a multiple of the XCD count.
  const int64_t slots = int64_t(num_cu) * resident_per_cu<D, NWQ, NWK, QSUB, ACT, IN, WINDOW, SPLIT>();
  const int64_t grid = persistent_grid(slots, max_items, grid_cap);
  return launch1(attn_kernel<D, NWQ, NWK, QSUB, ACT, IN, WINDOW, SPLIT>, dim3(unsigned(grid)), dim3(64 * NWQ * NWK),
                 st, a, tm);
}

template <int D, int IN>
hipError_t launch_for_shape(int shape, int act, const AttnArgs& a, int num_cu, int64_t max_items, int64_t cap,
                            const KTiming& tm, hipStream_t st) {
  switch (shape) {
    case 0:  // query-tiled (self full, cross): 4 waves x 32 rows
      if (act == ACT_SOFTMAX) return launch<D, 4, 1, 1, ACT_SOFTMAX, IN, false, false>(a, num_cu, max_items, cap, tm, st);
      if (act == ACT_GELU_POLY) return launch<D, 4, 1, 1, ACT_GELU_POLY, IN, false, false>(a, num_cu, max_items, cap, tm, st);
      return launch<D, 4, 1, 1, ACT_GELU, IN, false, false>(a, num_cu, max_items, cap, tm, st);
    case 1:  // block window (softmax only): 4 waves x 32 rows on two 64-token query blocks
      return launch<D, 4, 1, 1, ACT_SOFTMAX, IN, true, false>(a, num_cu, max_items, cap, tm, st);
    case 3:  // full self-attention: 8 waves x 32 rows share every key tile
      return launch<D, 8, 1, 1, ACT_SOFTMAX, IN, false, false>(a, num_cu, max_items, cap, tm, st);
    default:  // key-split (PMA): 1 query group of 32 rows x 4 key groups
      if (act == ACT_SOFTMAX) return launch<D, 1, 4, 1, ACT_SOFTMAX, IN, false, true>(a, num_cu, max_items, cap, tm, st);
      if (act == ACT_GELU_POLY) return launch<D, 1, 4, 1, ACT_GELU_POLY, IN, false, true>(a, num_cu, max_items, cap, tm, st);
      return launch<D, 1, 4, 1, ACT_GELU, IN, false, true>(a, num_cu, max_items, cap, tm, st);
  }
}

}  // namespace

// shape: 0 = query-tiled, 1 = block window, 2 = key-split, 3 = full self-attention.
hipError_t launch_attn_mfma(int D, int in, int shape, int act, const AttnArgs& a, int num_cu,
                            int64_t max_items, int64_t grid_cap, const KTiming& tm, hipStream_t st) {
  if (in == IN_BF16) {
    if (D == 32) return launch_for_shape<32, IN_BF16>(shape, act, a, num_cu, max_items, grid_cap, tm, st);
    if (D == 64) return launch_for_shape<64, IN_BF16>(shape, act, a, num_cu, max_items, grid_cap, tm, st);
    return launch_for_shape<128, IN_BF16>(shape, act, a, num_cu, max_items, grid_cap, tm, st);
  }
  if (D == 32) return launch_for_shape<32, IN_MX>(shape, act, a, num_cu, max_items, grid_cap, tm, st);
  if (D == 64) return launch_for_shape<64, IN_MX>(shape, act, a, num_cu, max_items, grid_cap, tm, st);
  return launch_for_shape<128, IN_MX8>(shape, act, a, num_cu, max_items, grid_cap, tm, st);
}

hipError_t launch_combine(int D, const CombineArgs& a, hipStream_t st) {
  const int grid = a.B * a.H;
  if (D == 32) hipLaunchKernelGGL(combine_kernel<32>, dim3(grid), dim3(kThreads), 0, st, a);
  else if (D == 64) hipLaunchKernelGGL(combine_kernel<64>, dim3(grid), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL(combine_kernel<128>, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ja
