// Ping-pong MFMA attention for the query-tiled shapes of GDPA: self-attention
// without a window and cross-attention (long queries), bf16 inputs, softmax or
// GELU scores (techfeed.io summary of "GEM Training: How Meta Doubled the
// Efficiency of Its LLM-Scale Ads Foundation Model", section "Generalized
// Dot-Product Attention（GDPA）").
//
// A workgroup of 8 waves owns work items of 256 query rows (32 per wave) and
// walks the key tiles (64 keys) of all its items as one stream.  Step s of the
// stream has one MFMA phase per wave -- O += V_{s-1} P_{s-1} followed by the
// scores S_s = K_s Q^T -- and one VALU phase (softmax or GELU of a score tile).
// Waves 0-3 run "MFMA(s), VALU(s)", waves 4-7 run "VALU(s-1), MFMA(s)": every
// SIMD holds one wave of each kind, so while one wave keeps the matrix core
// busy the other does its exponentials, with one workgroup barrier per step.
// The stream does not stop at item boundaries: an item's Q is loaded at the
// start of its first step and the previous item's output is written between
// two MFMA phases.  The plan sorts the items by key tiles, most first, and
// they are dealt out in rounds that alternate direction (workgroup positions
// 0..G-1, then G-1..0, ...), so every workgroup gets about the same number of
// tile steps; consecutive positions lie on one XCD, so the query tiles of one
// (sample, head) mostly share its K/V through that XCD's L2.
//
// Block windows of at most four 64-token blocks run as a pipeline instead: an
// item is a run of up to kPipeBlocks query blocks of one (sample, head), and
// query block b belongs to the wave pair b mod 4 (32 rows per wave).  Every key
// tile of the run is loaded once and serves the (up to four) query blocks
// whose window holds it, so each step keeps every pair busy; when a pair's
// block ends, its next block starts on the following tile, with its Q already
// staged in LDS by direct loads issued two steps earlier (techfeed.io summary,
// section "BlockAttention": attention confined to whole blocks within a window).
//
// LDS holds a ring of 4 tiles (K and V, plus the key scales of the GELU path):
// in step s the waves read K_s and V_{s-1}, tile s+1 has landed and tile s+2
// is loaded by direct-to-LDS loads issued between the score MFMAs.  The next
// step's wait for tile s+1 lets an item's output stores, issued in this step,
// run on.  Operand
// layouts, swizzles and the transposed score tile are those of the main MFMA
// kernel (ja_attn_mfma.hip).
#include <type_traits>

#include "ja_device.h"
#include "ja_mfma_util.h"
#include "ja_sched.h"
#include "jagged_attn.h"

namespace ja {

namespace {

constexpr int kPPWaves = 8;
constexpr int kPPRows = 32 * kPPWaves;  // query rows per work item
constexpr int kPPItemCache = 256;       // work item records staged in LDS per workgroup
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSgMfma = 0x008, kSgDsRead = 0x100;
// Softmax: a lane's sum of one tile's exponentials (32 keys) against the lazy
// reference max may reach 2^12 before the reference moves up.
constexpr float kPartCap = 4096.0f;
// MFMA operands are read this many MFMAs before their use (LDS latency under
// the load of four waves reading at once is several MFMAs long).
constexpr int kPPAhead = 5;
constexpr int kPPAheadS = 8;
// Query blocks per work item of the block-window pipeline (and the most
// window blocks it takes: one wave pair per block of a window).
constexpr int kPipeBlocks = 16;
constexpr int kPipePairs = kPPWaves / 2;

template <int D, int ACT, int IN>
struct PP {
  // IN_BF16: K, V and Q tiles are bf16 rows loaded as they are.  IN_MX8
  // (D = 128, softmax): e4m3 code rows plus one E8M0 scale byte per 32
  // elements; the scores take the codes on the block-scaled fp8 MFMA and V is
  // converted exactly to a bf16 tile in LDS for O += V P.
  static constexpr bool kMx8 = IN == IN_MX8 || IN == IN_MX8P;
  // IN_MX8P: O += V P on the block-scaled fp8 MFMA as well (P and V
  // requantised with one E8M0 scale per 32 keys, see the kernel).
  static constexpr bool kPv8 = IN == IN_MX8P;
  static constexpr int kNT = 64 * kPPWaves;
  static constexpr int kRowBytes = 2 * D;  // one bf16 row in LDS
  static constexpr int kTileBytes = 64 * kRowBytes;
  static constexpr int kKsOff = 2 * kTileBytes;  // GELU: 64 fp32 key scales after K and V
  static constexpr int kStageBytes = 2 * kTileBytes + (ACT != ACT_SOFTMAX ? 256 : 0);
  static constexpr int kRing = 4;
  static constexpr int kQChunks = D / 16;
  static constexpr int kOTiles = D / 32;
  static constexpr int kLdRow = kMx8 ? D : 2 * D;  // bytes of one loaded row (codes: 1 per element)
  static constexpr int kLdTile = 64 * kLdRow;
  static constexpr int kSegsLd = kLdTile / 1024;
  static constexpr int kRowsPerSeg = 1024 / kLdRow;
  static constexpr int kChunksPerRow = kLdRow / 16;
  static constexpr int kDmaJobs = 2 * kSegsLd / kPPWaves;  // 1 KB loads per wave per tile
  // (every wave also loads a scale row per tile: GELU key scales, MX8 K or V scales)
  static constexpr int kVmemPerTile = kDmaJobs + (ACT != ACT_SOFTMAX || kMx8 ? 1 : 0);
  static constexpr int kStoresPerWave = 2 * kOTiles;  // 16-byte output stores per lane of an item
  static_assert((2 * kSegsLd) % kPPWaves == 0, "tile segments must split evenly over the waves");
  static_assert(!kMx8 || (D == 128 && ACT == ACT_SOFTMAX), "the fp8 tile stream takes D = 128 softmax");
  // MX8 LDS layout: K codes and V codes of tiles s, s+1, s+2 (3 stages each)
  // with their scale rows (4 bytes per key), the converted V of tiles s-1 and
  // s (bf16; fp8 P V: dim-major requantised codes, D rows of 64 bytes, plus 8
  // scale bytes per tile), and two staged Q blocks (codes + scale rows).
  // 256-byte aligned pieces.
  static constexpr int kMxKc = 0;
  static constexpr int kMxKs = kMxKc + 3 * kLdTile;
  static constexpr int kMxVc = kMxKs + 3 * 256;
  static constexpr int kMxVs = kMxVc + 3 * kLdTile;
  static constexpr int kMxVb = kMxVs + 3 * 256;
  static constexpr int kMxVtBytes = 64 * D;  // fp8 P V: one requantised V^T tile
  static constexpr int kMxVts = kMxVb + 2 * kMxVtBytes;
  static constexpr int kMxQc = kMxVb + (kPv8 ? 2 * kMxVtBytes + 256 : 2 * kTileBytes);
  static constexpr int kMxQs = kMxQc + 2 * kLdTile;
  static constexpr int kMxBytes = kMxQs + 2 * 256;
};

// Position in the tile stream: tile t of the k-th item of this workgroup
// (k == n: past the end), the end of the item's tiles and its key count.
// Windows: this wave computes tiles [wlo, whi] of the item, and its first
// query row is r0 (sample-local).  Block-window pipeline: the item's first
// tile is wlo, its query blocks are [r0, whi).  Wave-uniform.
struct Cur {
  int k, t, te, lk;
  int wlo, whi, r0;
};

// Window modes of the tile stream.
enum { kWinNone = 0, kWinBlock = 1, kWinSliding = 2, kWinPipe = 3 };

// Block-window pipeline, tile t of cursor cu for wave pair p: the query block
// the pair works on (the first block >= t in the pair's residue class mod 4),
// whether it sees tile t, and whether t is that block's first or last tile.
struct PipeStep {
  int b;
  bool act, first, last;
};
__device__ __forceinline__ PipeStep pipe_step(const Cur& cu, int p, int nb) {
  PipeStep r;
  r.b = cu.t + ((p - cu.t) & (kPipePairs - 1));
  r.act = r.b < cu.t + nb && r.b >= cu.r0 && r.b < cu.whi;
  r.first = r.act && cu.t == max(r.b - nb + 1, 0);
  r.last = r.act && cu.t == r.b;
  return r;
}

__device__ __forceinline__ int ntiles_of(int lk) { return (lk + 63) >> 6; }

// Where the tile loads of a cursor read: key row r of the item's head at
// kb + r * row_bytes (values at vb + ...), GELU key scales at ksc[r * H];
// query row r at qb + r * row_bytes (lq rows).
struct Src {
  const unsigned char* kb;
  const unsigned char* vb;
  const float* ksc;
  const unsigned char* qb;
  const unsigned char* ksb;  // MX8: scale rows of key row 0 (K and V) and query row 0
  const unsigned char* vsb;
  const unsigned char* qsb;
  int lq;
};

typedef int i32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const i32x4v lds_i32x4;

struct PPCtx {
  const WorkItem* items;
  lds_i32x4* cache;       // LDS copy of this workgroup's first kPPItemCache records (2 x 16 B each)
  const unsigned char* q;
  const unsigned char* k;
  const unsigned char* v;
  const unsigned char* qs;  // MX8 scale bytes
  const unsigned char* ks;
  const unsigned char* vs;
  const float* kscale;
  __bf16* out;
  // optional natural log-sum-exp per (query row, head) (softmax): the
  // pointer's halves, held in VGPRs (see lse_ptr)
  unsigned lse_lo, lse_hi;
  int H;
  int G, pos, n;          // item k of this workgroup is item_index(k), k < n
  unsigned row_bytes;  // bytes between a head's input rows (bf16: 2 H D; MX8 codes: H D)
};

// Round k deals items [kG, kG + G) to positions 0..G-1, in reverse order on odd rounds.
__device__ __forceinline__ int item_index(const PPCtx& c, int k) {
  return k * c.G + ((k & 1) ? c.G - 1 - c.pos : c.pos);
}

// Record of the k-th item, wave-uniform.
__device__ __forceinline__ WorkItem load_record(const PPCtx& c, int k) {
  WorkItem w;
  if (k < kPPItemCache) {
    const i32x4v u = c.cache[2 * k], x = c.cache[2 * k + 1];
    w = WorkItem{u[0], u[1], u[2], u[3], x[0], x[1], x[2], x[3]};
  } else {
    // (rare: more than kPPItemCache items per workgroup) waited for here, so
    // that no load is pending where the two paths meet -- the compiler would
    // otherwise wait there for every load in flight, tile prefetches included
    w = c.items[item_index(c, k)];
    wait_vmcnt(0);
  }
  w.h = __builtin_amdgcn_readfirstlane(w.h);
  w.q0 = __builtin_amdgcn_readfirstlane(w.q0);
  w.qbeg = __builtin_amdgcn_readfirstlane(w.qbeg);
  w.lq = __builtin_amdgcn_readfirstlane(w.lq);
  w.kbeg = __builtin_amdgcn_readfirstlane(w.kbeg);
  w.lk = __builtin_amdgcn_readfirstlane(w.lk);
  return w;
}

template <int D, int IN>
__device__ __forceinline__ Src make_src(const PPCtx& c, const WorkItem& w) {
  constexpr size_t kElt = IN == IN_MX8 ? 1 : 2;  // bytes per element
  const size_t krow = size_t(w.kbeg) * c.H + w.h, qrow = size_t(w.qbeg) * c.H + w.h;
  Src r;
  r.kb = uniform_ptr(c.k + krow * (kElt * D));
  r.vb = uniform_ptr(c.v + krow * (kElt * D));
  r.ksc = c.kscale ? uniform_ptr(c.kscale + krow) : nullptr;
  r.qb = uniform_ptr(c.q + qrow * (kElt * D));
  r.ksb = r.vsb = r.qsb = nullptr;
  if constexpr (IN == IN_MX8) {
    r.ksb = uniform_ptr(c.ks + krow * (D / kMxBlock));
    r.vsb = uniform_ptr(c.vs + krow * (D / kMxBlock));
    r.qsb = uniform_ptr(c.qs + qrow * (D / kMxBlock));
  }
  r.lq = w.lq;
  return r;
}

// The log-sum-exp output pointer (null: none).  Its halves pass through an
// empty asm that puts them in VGPRs: the tile loop's scalar registers are
// fully used, and a pointer kept there spilled others to VGPR lanes (more
// v_readlane/v_writelane in the loop even when no log-sum-exp is asked for).
__device__ __forceinline__ float* lse_ptr(const PPCtx& c) {
  return reinterpret_cast<float*>((uint64_t(c.lse_hi) << 32) | c.lse_lo);
}

// Rows [32*wave, 32*wave + 32) of an item with no keys: the output is zero
// (and the log-sum-exp over no keys -inf).
template <int D>
__device__ __forceinline__ void write_zero_rows(const PPCtx& c, const WorkItem& it, int wave, int lane) {
  const int qrow = it.q0 + 32 * wave + (lane & 31);
  if (qrow >= it.lq) return;
  if ((c.lse_lo | c.lse_hi) != 0u && lane < 32) lse_ptr(c)[size_t(it.qbeg + qrow) * c.H + it.h] = -__builtin_huge_valf();
  __bf16* orow = c.out + (size_t(it.qbeg + qrow) * c.H + it.h) * D + (D / 2) * (lane >> 5);
  bf16x8 z;
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = (__bf16)0.0f;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) *reinterpret_cast<bf16x8*>(orow + 8 * c) = z;
}

// Move the loading cursor to the next tile of the stream.  Items without keys
// are skipped (their rows of this wave are written as zeros on the way).  Past
// the end the cursor keeps the source and key count of the last item it
// visited and points at its tile 0, so the loads it still issues read rows
// that exist (and are never used).
//
// With a block window of nb blocks (self-attention, 64-token blocks counted
// from the sample's first token) an item covers the key tiles from nb - 1
// blocks before its first query block to its last query block, and a wave
// computes the tiles its own query block sees (techfeed.io summary of "GEM
// Training: ...", section "BlockAttention").  With a sliding window of wt
// tokens (query i sees keys i-wt+1 .. i) the tiles run from the one holding
// key q0-wt+1 to the one holding the item's last query.
template <int D, int WMODE, int IN>
__device__ __forceinline__ void advance(const PPCtx& c, Cur& cu, Src& src, int wave, int lane, int nb, int wt) {
  if (cu.k >= c.n) return;
  if (++cu.t < cu.te) return;
  while (++cu.k < c.n) {
    const WorkItem w = load_record(c, cu.k);
    int t_lo = 0, t_end = ntiles_of(w.lk);
    if constexpr (WMODE == kWinBlock) {
      t_lo = max(0, w.q0 / kBlock - nb + 1);
      t_end = min(t_end, (min(w.q0 + kPPRows, w.lq) + kBlock - 1) / kBlock);
      const int r0 = w.q0 + 32 * wave, wblk = r0 / kBlock;
      cu.wlo = wblk - nb + 1;
      cu.whi = r0 < w.lq ? wblk : -1;
    } else if constexpr (WMODE == kWinPipe) {
      // query blocks [c0b, ce) and the key tiles from nb - 1 blocks before c0b
      const int c0b = w.q0 / kBlock, ce = min(c0b + kPipeBlocks, (w.lq + kBlock - 1) / kBlock);
      t_lo = max(0, c0b - nb + 1);
      t_end = min(t_end, ce);
      cu.wlo = t_lo;
      cu.whi = ce;
      cu.r0 = c0b;
    } else if constexpr (WMODE == kWinSliding) {
      t_lo = max(0, w.q0 - wt + 1) / kBlock;
      t_end = min(t_end, (min(w.q0 + kPPRows, w.lq) + kBlock - 1) / kBlock);
      const int r0 = w.q0 + 32 * wave;
      cu.r0 = r0;
      cu.wlo = max(0, r0 - wt + 1) / kBlock;
      cu.whi = r0 < w.lq ? min(r0 + 31, w.lq - 1) / kBlock : -1;
    }
    if (t_end > t_lo) {
      cu.t = t_lo;
      cu.te = t_end;
      cu.lk = w.lk;
      src = make_src<D, IN>(c, w);
      return;
    }
    write_zero_rows<D>(c, w, wave, lane);
  }
  cu.t = 0;  // past the end: tile 0 of the last item visited
}

// ---- The tile stream's own work enumeration (no plan launch) --------------
// Every workgroup reads the B+1 offsets, checks them, and computes the same
// item order the plan kernel's counting sort gives in effect -- items sorted
// by the key tiles they walk, most first -- with a deterministic order inside
// a cost bucket (by wave, then lane, then run), so that every workgroup finds
// the same positions without talking to the others.  It keeps the records of
// its own positions (dealt in alternating rounds) in the LDS item cache and
// writes them to the workspace item list; workgroup 0 writes the header.  One
// thread per sample (B + 1 <= 512 offsets), sample b on lane b / 8 of wave
// b % 8: a few samples spread over all eight waves rank their runs in parallel
// (the ranking loop takes one pass per distinct cost in a wave).  A sample has
// at most kMaxRuns runs of equal cost (the host checks the window against bm).
constexpr int kMaxRuns = 4;

// Exclusive prefix sum over the wave's 64 lanes on the DPP network (no LDS
// trips): row_shr 1, 2, 4, 8 scan each row of 16 lanes (a lane without a
// source adds 0), row_bcast 15 and 31 carry the row totals into the rows above.
__device__ __forceinline__ int wave_excl_scan(int x) {
  int v = x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 (rows 1, 3)
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 (rows 2, 3)
  return v - x;
}

// Returns the number of items of the call (every workgroup gets the same), or
// -1 if the offsets are invalid.  `lds` is scratch of at least
// (9 * kCostBuckets + 16) ints (the tile ring, not yet in use).
__device__ int enumerate_items(const AttnArgs& a, int* lds, WorkItem* cache, int G, int pos) {
  const int tid = threadIdx.x, wave = tid >> 6;
  static_assert(kPPWaves == 8, "sample b sits on lane b / 8 of wave b % 8");
  int* s_cnt = lds;                          // [8][kCostBuckets]: item counts per wave, then wave bases
  int* s_start = lds + 8 * kCostBuckets;     // [kCostBuckets]: first position of each bucket
  int* s_wsum = s_start + kCostBuckets;      // [8 + 1]: block scan of the bucket totals
  // this thread's sample: offsets checked as the plan kernel checks them (the
  // loads are issued first, so that their latency covers the zeroing below)
  const int b = (tid & 63) * kPPWaves + wave;
  int q = 0, k = 0, q1 = 0, k1 = 0;
  if (b <= a.B) {
    q = a.qo[b];
    k = a.ko[b];
    if (b < a.B) {
      q1 = a.qo[b + 1];
      k1 = a.ko[b + 1];
    }
  }
  for (int i = tid; i < 8 * kCostBuckets; i += kPPWaves * 64) s_cnt[i] = 0;
  int bad = 0, qb = 0, lq = 0, kb = 0, lk = 0;
  if (b <= a.B) {
    if (b == 0 && (q != 0 || k != 0)) bad = 1;
    if (b == a.B && (q != a.total_q || k != a.total_kv)) bad = 1;
    if (a.self_check && q != k) bad = 1;
    if (b < a.B) {
      if (q1 < q || k1 < k) bad = 1;
      qb = q;
      lq = q1 - q;
      kb = k;
      lk = k1 - k;
    }
  }
  if (__syncthreads_or(bad)) {
    if (blockIdx.x == 0 && tid == 0) {
      WsHeader* hdr = const_cast<WsHeader*>(a.hdr);
      hdr->items_off = int32_t(reinterpret_cast<const char*>(a.items) - reinterpret_cast<const char*>(a.hdr));
      hdr->n_items = 0;
      hdr->n_slots = 0;
      hdr->status = JA_EOFFSETS;
      if (a.status_out) *a.status_out = JA_EOFFSETS;
    }
    return -1;
  }
  // runs of equal cost: (bucket, items = run x H, first query tile, run length)
  int eb[kMaxRuns], en[kMaxRuns], eq[kMaxRuns], er[kMaxRuns];
  int ne = 0;
  {
    const int nqt = (b < a.B && lq > 0) ? (lq + a.bm - 1) / a.bm : 0;
    int qt = 0;
#pragma unroll
    for (int e = 0; e < kMaxRuns; ++e) {
      eb[e] = en[e] = eq[e] = er[e] = 0;
      if (qt < nqt) {
        const int run = cost_run(a, qt, nqt);
        eb[e] = cost_bucket(a, qt, lq, lk);
        en[e] = run * a.H;
        eq[e] = qt;
        er[e] = run;
        atomicAdd(&s_cnt[wave * kCostBuckets + eb[e]], en[e]);
        ne = e + 1;
        qt += run;
      }
    }
  }
  __syncthreads();
  // per bucket: the waves' exclusive bases (in place) and the total; then the
  // buckets' start positions, most tiles first (thread t: descending ranks 2t, 2t+1)
  int tot[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int beta = kCostBuckets - 1 - (2 * tid + j);
    int run = 0;
#pragma unroll
    for (int w = 0; w < kPPWaves; ++w) {
      const int c = s_cnt[w * kCostBuckets + beta];
      s_cnt[w * kCostBuckets + beta] = run;
      run += c;
    }
    tot[j] = run;
  }
  {
    const int pair = tot[0] + tot[1];
    const int inc = wave_excl_scan(pair) + pair;
    if ((tid & 63) == 63) s_wsum[wave] = inc;
    __syncthreads();
    int wbase = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kPPWaves; ++w) {
      const int t = s_wsum[w];
      if (w < wave) wbase += t;
      all += t;
    }
    const int excl = wbase + inc - pair;
    s_start[kCostBuckets - 1 - 2 * tid] = excl;
    s_start[kCostBuckets - 2 - 2 * tid] = excl + tot[0];
    if (tid == 0) s_wsum[kPPWaves] = all;
  }
  __syncthreads();
  const int n_all = s_wsum[kPPWaves];
  // positions of this lane's runs: bucket start + wave base + the items of
  // lower lanes (and earlier runs of this lane) in the same bucket, one
  // bucket of the wave at a time
  int pe[kMaxRuns];
#pragma unroll
  for (int e = 0; e < kMaxRuns; ++e) pe[e] = e < ne ? s_start[eb[e]] + s_cnt[wave * kCostBuckets + eb[e]] : 0;
  unsigned pend = (1u << ne) - 1u;
  while (true) {
    const unsigned long long bal = __ballot(pend != 0u);
    if (bal == 0ull) break;
    int fb = -1;
#pragma unroll
    for (int e = kMaxRuns - 1; e >= 0; --e)
      if ((pend >> e) & 1u) fb = eb[e];
    const int beta = __builtin_amdgcn_readlane(fb, int(__builtin_ctzll(bal)));
    int mine = 0, off[kMaxRuns];
    unsigned took = 0u;
#pragma unroll
    for (int e = 0; e < kMaxRuns; ++e) {
      off[e] = mine;
      if (((pend >> e) & 1u) && eb[e] == beta) {
        mine += en[e];
        took |= 1u << e;
      }
    }
    // (pe[e] holds the bucket's start plus this wave's base for it)
    const int pre = wave_excl_scan(mine);
#pragma unroll
    for (int e = 0; e < kMaxRuns; ++e)
      if ((took >> e) & 1u) pe[e] += pre + off[e];
    pend &= ~took;
  }
  // this workgroup's positions p_k = k G + (k odd ? G-1-pos : pos) inside each run's range
#pragma unroll
  for (int e = 0; e < kMaxRuns; ++e) {
    if (e < ne) {
      const int P = pe[e], n = en[e];
      for (int k = P / G; k * G <= P + n - 1; ++k) {
        const int p = k * G + ((k & 1) ? G - 1 - pos : pos);
        if (p >= P && p < P + n && p < n_all) {
          const int i = p - P, h = i / er[e], qt = eq[e] + i % er[e];
          const WorkItem w{b, h, qt * a.bm, 0, qb, lq, kb, lk};
          if (k < kPPItemCache) cache[k] = w;
          const_cast<WorkItem*>(a.items)[p] = w;  // the workspace list (read back by diagnostics)
        }
      }
    }
  }
  if (blockIdx.x == 0 && tid == 0) {
    WsHeader* hdr = const_cast<WsHeader*>(a.hdr);
    hdr->items_off = int32_t(reinterpret_cast<const char*>(a.items) - reinterpret_cast<const char*>(a.hdr));
    hdr->n_items = n_all;
    hdr->n_slots = 0;
    hdr->status = JA_OK;
    if (a.status_out) *a.status_out = JA_OK;
  }
  __syncthreads();
  return n_all;
}

// QPF (cross-attention): the Q of the item starting on the next tile is loaded
// into the Q registers as soon as this step's scores have consumed them, and
// waited for only before that item's scores.  With the short K/V of
// cross-attention almost every step starts an item, and loading Q at the item
// start left every wave waiting for HBM once per step.
template <int D, int ACT, int WMODE, bool QPF, int IN>
__global__ __launch_bounds__(64 * kPPWaves, 1) void attn_pp_kernel(AttnArgs a) {
  using K = PP<D, ACT, IN>;
  constexpr int kQChunks = K::kQChunks, kOTiles = K::kOTiles, kRowBytes = K::kRowBytes;
  constexpr bool kPipe = WMODE == kWinPipe;
  constexpr bool kMx8 = K::kMx8, kPv8 = K::kPv8;
  constexpr bool kLateEpi = QPF;  // an item's output after the next item's scores
  // LDS: a ring of kRing stages of (K, V[, key scales]).  The pipeline instead
  // keeps K in 3 stages (tiles s, s+1, s+2: K_{s-1} is dead once the scores
  // of tile s-1 are taken), V in 4 (s-1 .. s+2) and two Q blocks (the block
  // starting on the next tile, alternating by tile parity).
  constexpr int kPipeV = 3 * K::kTileBytes, kPipeQ = 7 * K::kTileBytes;
  // MX8: see PP::kMx*.
  // (the ring is also the scratch of the in-kernel item enumeration)
  constexpr int kTileRing = kMx8 ? K::kMxBytes : (kPipe ? 9 * K::kTileBytes : K::kRing * K::kStageBytes);
  constexpr int kEnumBytes = 4 * (9 * kCostBuckets + 16);
  constexpr int kRingBytes = kTileRing > kEnumBytes ? kTileRing : kEnumBytes;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kRingBytes];
  __shared__ WorkItem cache[kPPItemCache];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const bool late = wave >= 4;  // VALU phase before the MFMA phase

  PPCtx c;
  c.items = a.items;
  c.cache = (lds_i32x4*)(cache);
  c.q = reinterpret_cast<const unsigned char*>(a.q);
  c.k = reinterpret_cast<const unsigned char*>(a.k);
  c.v = reinterpret_cast<const unsigned char*>(a.v);
  c.qs = a.qs;
  c.ks = a.ks;
  c.vs = a.vs;
  c.kscale = a.kscale;
  c.out = reinterpret_cast<__bf16*>(a.out);
  c.lse_lo = unsigned(reinterpret_cast<uintptr_t>(a.lse));
  c.lse_hi = unsigned(reinterpret_cast<uintptr_t>(a.lse) >> 32);
  asm volatile("" : "+v"(c.lse_lo), "+v"(c.lse_hi));
  c.H = a.H;
  // (the grid is a multiple of 8 and workgroup w runs on XCD w % 8: positions
  // [x G/8, (x+1) G/8) are the workgroups of XCD x)
  c.G = gridDim.x;
  c.pos = int(blockIdx.x % kXcds) * (c.G / kXcds) + int(blockIdx.x) / kXcds;
  // (the bf16 pipeline's runs share few key tiles: dealing consecutive runs
  // to one XCD only concentrates their loads there, so positions follow the
  // workgroup id and spread over the XCDs.  MX8 keeps the XCD grouping: the
  // heads of a token share their 128-byte lines of scale bytes, and
  // consecutive items are the heads of one sample)
  if constexpr (WMODE == kWinPipe && !kMx8) c.pos = int(blockIdx.x);
  int n_all;
  if (a.inplan) {
    // (softmax only: no key RMS factors are needed from a plan launch)
    n_all = enumerate_items(a, reinterpret_cast<int*>(ring), cache, c.G, c.pos);
    if (n_all < 0) return;
  } else {
    n_all = a.hdr->n_items;
  }
  {
    const int full = n_all / c.G;  // complete rounds
    c.n = full + (item_index(c, full) < n_all ? 1 : 0);
  }
  c.row_bytes = (kMx8 ? 1u : 2u) * unsigned(a.H) * D;  // bytes between a head's rows
  const unsigned srow = unsigned(a.H) * (D / kMxBlock);  // MX8: scale bytes between rows
  if (c.n == 0) return;
  if (!a.inplan) {
    for (int k = tid; k < min(c.n, kPPItemCache); k += K::kNT) cache[k] = a.items[item_index(c, k)];
    __syncthreads();
  }

  // Stream cursors: tile s (scores), s+1, s+2 (being loaded); only the
  // loading cursor carries the addresses of its item.
  const int nb = a.window_blocks, wt = a.window_tokens;
  Cur c0{-1, 0, 0, 0, 0, 0, 0};
  Src src{};
  advance<D, WMODE, IN>(c, c0, src, wave, lane, nb, wt);
  if (c0.k >= c.n) return;
  const Src src0 = src;
  Cur c1 = c0;
  advance<D, WMODE, IN>(c, c1, src, wave, lane, nb, wt);
  const Src src1 = src;
  Cur c2 = c1;
  advance<D, WMODE, IN>(c, c2, src, wave, lane, nb, wt);

  // Loads of the loading cursor's tile into LDS (K at byte kdst of the ring, V
  // at vdst).  Job j moves 1 KB segment wave + 8j of K|V; rows of a ragged tile
  // are clamped to its last key.
  auto tile_job = [&](const Cur& cu, const Src& sr, int kdst, int vdst, int j) __attribute__((always_inline)) {
    const int key0 = 64 * cu.t;
    const int lim = min(63, cu.lk - 1 - key0);
    const int sg = wave + kPPWaves * j;
    const bool is_v = sg >= K::kSegsLd;
    const int seg = is_v ? sg - K::kSegsLd : sg;
    const unsigned char* tile = (is_v ? sr.vb : sr.kb) + size_t(key0) * c.row_bytes;
    const int row = seg * K::kRowsPerSeg + lane / K::kChunksPerRow;
    const int phys = lane % K::kChunksPerRow;
    int ch;
    if constexpr (kMx8) ch = phys ^ swz_c<D>(row);
    else ch = phys ^ (is_v ? swz_v<D>(row) : swz_k<D>(row));
    const unsigned off = __umul24(unsigned(min(row, lim)), c.row_bytes) + 16u * unsigned(ch);
    lds_dma16(tile, off, lds_addr_of(ring) + (is_v ? vdst : kdst) + seg * 1024);
  };
  // Pipeline: the 64 query rows of block bq of the loading cursor's item into
  // Q slot `slot` (rows past the sample repeat its last row), laid out like a
  // K tile.  Waves past the block's 1 KB segments issue nothing.
  auto q_block_job = [&](const Src& sr, int bq, int slot) __attribute__((always_inline)) {
    // (the lane id is read here by volatile asm, so that the lane offsets are
    // formed at this point instead of being hoisted out of the stream loop and
    // kept live -- or spilled -- across it)
    int lid;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lid));
#pragma unroll
    for (int j = 0; j < (K::kSegsLd + kPPWaves - 1) / kPPWaves; ++j) {
      const int seg = wave + kPPWaves * j;
      if (seg < K::kSegsLd) {
        const int r0 = kBlock * bq;
        const int lim = min(63, sr.lq - 1 - r0);
        const int row = seg * K::kRowsPerSeg + lid / K::kChunksPerRow;
        const int ch = (lid % K::kChunksPerRow) ^ (kMx8 ? swz_c<D>(row) : swz_k<D>(row));
        const unsigned off = __umul24(unsigned(min(row, lim)), c.row_bytes) + 16u * unsigned(ch);
        const int qdst = kMx8 ? K::kMxQc + slot * K::kLdTile : kPipeQ + slot * K::kTileBytes;
        lds_dma16(sr.qb + size_t(r0) * c.row_bytes, off, lds_addr_of(ring) + qdst + seg * 1024);
      }
    }
    if constexpr (kMx8) {
      // the block's scale rows (4 bytes per query row), by wave 0
      if (wave == 0) {
        const int r0 = kBlock * bq;
        const unsigned r = unsigned(min(lid, sr.lq - 1 - r0));
        lds_dma4(sr.qsb + size_t(r0) * srow, r * srow, lds_addr_of(ring) + K::kMxQs + slot * 256);
      }
    }
  };
  // Pipeline: stage the Q block that starts on the loading cursor's tile, when
  // that tile is not its item's first (the first tile's blocks load Q
  // directly), into the Q slot of the tile's parity.
  auto q_stage = [&](const Cur& cu, const Src& sr) __attribute__((always_inline)) {
    if constexpr (kPipe) {
      const int bq = cu.t + nb - 1;
      if (cu.k < c.n && cu.t > cu.wlo && bq < cu.whi) q_block_job(sr, bq, cu.t & 1);
    }
  };
  // MX8: the K (even waves) or V (odd waves) scale rows of the loading
  // cursor's tile into the scale slot of stream tile s (every wave issues one
  // load per tile, so the waits count the same loads on every wave).
  auto mx_scales = [&](const Cur& cu, const Src& sr, int s) __attribute__((always_inline)) {
    if constexpr (kMx8) {
      const int key0 = 64 * cu.t;
      const unsigned r = unsigned(min(lane, cu.lk - 1 - key0));
      const bool is_v = wave & 1;
      lds_dma4((is_v ? sr.vsb : sr.ksb) + size_t(key0) * srow, r * srow,
               lds_addr_of(ring) + (is_v ? K::kMxVs : K::kMxKs) + (s % 3) * 256);
    }
  };
  auto tile_scales = [&](const Cur& cu, const Src& sr, int st) __attribute__((always_inline)) {
    if constexpr (ACT != ACT_SOFTMAX) {
      const int key0 = 64 * cu.t;
      const unsigned r = unsigned(min(lane, cu.lk - 1 - key0));
      lds_dma4(sr.ksc + size_t(key0) * a.H, r * unsigned(a.H) * 4u, lds_addr_of(ring) + st * K::kStageBytes + K::kKsOff);
    }
  };

  // Lane-constant LDS byte offsets of the MFMA operand reads.
  const int kp = key_perm(l32);
  int k_off[kQChunks];
#pragma unroll
  for (int cc = 0; cc < kQChunks; ++cc) k_off[cc] = kp * kRowBytes + 16 * ((kQChunks * g + cc) ^ swz_k<D>(kp));
  const int v_row = (8 * g + ((lane & 15) >> 2)) * kRowBytes;
  int v_col[kOTiles];
#pragma unroll
  for (int t = 0; t < kOTiles; ++t) {
    const int col = dim_perm<D>(t, 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    v_col[t] = 16 * ((col >> 3) ^ swz_v<D>((lane & 15) >> 2)) + 8 * ((col & 7) >> 2);
  }
  const float c2s = a.score_scale;  // softmax: log2(e)/sqrt(D); GELU: 1/sqrt(D)

  // LDS byte offsets of the K and V tiles of stream tile s.
  // (MX8: k_at is the K code tile, vc_at the V code tile the loads fill, v_at
  // the converted bf16 V tile that O += V P reads)
  auto k_at = [&](int s) __attribute__((always_inline)) {
    if constexpr (kMx8) return K::kMxKc + (s % 3) * K::kLdTile;
    return kPipe ? (s % 3) * K::kTileBytes : (s % K::kRing) * K::kStageBytes;
  };
  auto v_at = [&](int s) __attribute__((always_inline)) {
    if constexpr (kPv8) return K::kMxVb + (s & 1) * K::kMxVtBytes;
    if constexpr (kMx8) return K::kMxVb + (s & 1) * K::kTileBytes;
    return kPipe ? kPipeV + (s % 4) * K::kTileBytes : (s % K::kRing) * K::kStageBytes + K::kTileBytes;
  };
  auto vc_at = [&](int s) __attribute__((always_inline)) {
    if constexpr (kMx8) return K::kMxVc + (s % 3) * K::kLdTile;
    return v_at(s);
  };
  const int pair = wave >> 1;
  // First query row (sample-local) of this wave in the scores' item.
  auto wave_row0 = [&](const Cur& cu, int q0) __attribute__((always_inline)) {
    if constexpr (kPipe) return kBlock * pipe_step(cu, pair, nb).b + 32 * (wave & 1);
    else return q0 + 32 * wave;
  };

  // Q fragments of the scores' item: lane holds dims [(D/2)g, (D/2)g + D/2) of
  // query row q0 + 32*wave + l32 (rows past the sample load its last row).
  // MX8: qc[c] holds the 64-element chunk c of the row as the fp8 MFMA's B
  // operand (lane-half g: elements 64c+16g+[0,16) and 64c+32+16g+[0,16)), qsc[c]
  // the scale byte of 32-element block 2c+g.
  constexpr int kMxC = D / 64;
  bf16x8 qf[kMx8 ? 1 : kQChunks];
  i32x8 qc[kMx8 ? kMxC : 1];
  int qsc[kMx8 ? kMxC : 1];
  auto load_q = [&](const Cur& cu) __attribute__((always_inline)) {
    const WorkItem it = load_record(c, cu.k);
    const int qrow = min(wave_row0(cu, it.q0) + l32, it.lq - 1);
    const size_t row = size_t(it.qbeg + qrow) * a.H + it.h;
    if constexpr (kMx8) {
      const unsigned char* src = c.q + row * D;
      const unsigned sw = *reinterpret_cast<const unsigned*>(c.qs + row * (D / kMxBlock));
#pragma unroll
      for (int cc = 0; cc < kMxC; ++cc) {
        const u32x4 w0 = *reinterpret_cast<const u32x4*>(src + 64 * cc + 16 * g);
        const u32x4 w1 = *reinterpret_cast<const u32x4*>(src + 64 * cc + 32 + 16 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qc[cc][i] = int(w0[i]);
          qc[cc][4 + i] = int(w1[i]);
        }
        qsc[cc] = int((sw >> (8 * (2 * cc + g))) & 0xFFu);
      }
    } else {
      const __bf16* src_q = reinterpret_cast<const __bf16*>(a.q) + row * D + (D / 2) * g;
#pragma unroll
      for (int cc = 0; cc < kQChunks; ++cc) qf[cc] = *reinterpret_cast<const bf16x8*>(src_q + 8 * cc);
    }
  };
  float rq = 1.f;  // GELU: RMS factor of the query row times 1/sqrt(D)
  auto q_rms = [&]() __attribute__((always_inline)) {
    if constexpr (ACT != ACT_SOFTMAX) {
      float ss = 0.f;
#pragma unroll
      for (int cc = 0; cc < kQChunks; ++cc)
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fmaf(float(qf[cc][j]), float(qf[cc][j]), ss);
      ss = sum_halves(ss);
      rq = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.eps) * c2s;
    }
  };

  // Prologue: tiles 0 and 1 in flight, Q of the first item (pipeline: and of
  // the block starting on tile 1).
#pragma unroll
  for (int j = 0; j < K::kDmaJobs; ++j) tile_job(c0, src0, k_at(0), vc_at(0), j);
  tile_scales(c0, src0, 0);
  mx_scales(c0, src0, 0);
#pragma unroll
  for (int j = 0; j < K::kDmaJobs; ++j) tile_job(c1, src1, k_at(1), vc_at(1), j);
  tile_scales(c1, src1, 1);
  mx_scales(c1, src1, 1);
  q_stage(c1, src1);
  load_q(c0);
  wait_vmcnt(0);  // (nothing may be pending on the loop's entry edge, see below)
  bool q_fresh = true;  // Q was (re)loaded for c0's item: GELU needs its RMS factor

  f32x16 o[kOTiles];
#pragma unroll
  for (int t = 0; t < kOTiles; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  // O restarts at zero with the next item: its first P V takes C = 0 instead
  // of the 64 accumulator registers being cleared (the epilogue sets this)
  bool o_zero = false;
  // softmax diagnostics (a.stats), kept in vector registers (made so by the
  // asm): wave-uniform scalars would add to the scalar register spills
  unsigned st_tiles, st_first, st_later;
  asm volatile("v_mov_b32 %0, 0" : "=v"(st_tiles));
  asm volatile("v_mov_b32 %0, 0" : "=v"(st_first));
  asm volatile("v_mov_b32 %0, 0" : "=v"(st_later));
  float m = -__builtin_huge_valf(), l = 0.f;
  f32x16 sc[2];      // score tile: S^T halves (keys 32*st + 16*(i/8) + 8g + i%8)
  bf16x8 pb[kPv8 ? 1 : 4];  // P of the previous tile, 16-key chunks kc
  // fp8 P V: P of the previous tile as e4m3 codes, the fp8 MFMA's B operand
  // (bytes 0-15: the keys of sc[0], 16-31: those of sc[1], in register order),
  // and its two scale bytes (keys 0-31, 32-63)
  i32x8 pq;
  unsigned psc = 0;
  int pv_k = c0.k;   // item of tile s-1
  bool pv_last = false;
  bool pv_act = true;  // this wave computed tile s-1 (block windows)
  int pv_nvalid = 64;  // keys of tile s-1 inside its sample
  int pv_key0 = 0, pv_r0 = 0;  // sliding window: tile s-1's first key, this wave's first row
  int pv_row0 = 0;   // pipeline: first row of this wave's block at tile s-1

  // Softmax / GELU of the score tile `sc` (nvalid keys; sliding window: keys
  // key0.. of the tile against rows r0.. of this wave), written to pb as bf16.
  auto vphase = [&](int nvalid, int stage, int key0, int r0) __attribute__((always_inline)) {
    const bool ragged = nvalid < 64;
    if constexpr (ACT == ACT_SOFTMAX) {
      if (ragged) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kk = 32 * st + 16 * (i >> 3) + 8 * g + (i & 7);
            if (kk >= nvalid) sc[st][i] = -__builtin_huge_valf();
          }
      }
      if constexpr (WMODE == kWinSliding) {
        // key j is allowed for row i when i - wt < j <= i; only a tile that
        // reaches past the wave's first row or before its last row's window
        // start has disallowed keys
        if (key0 + 63 > r0 || key0 <= r0 + 31 - wt) {
          const int row = r0 + l32;
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int j = key0 + 32 * st + 16 * (i >> 3) + 8 * g + (i & 7);
              if (j > row || j <= row - wt) sc[st][i] = -__builtin_huge_valf();
            }
        }
      }
      // p = 2^(s c - m c) into pb (bf16); returns this lane's sum of the fp32
      // p, by plain adds: a dot-product sum of the bf16 pairs competes with
      // the other wave's MFMAs for the SIMD and cost a fifth of the step,
      // while the adds hide behind them.  (The bf16 rounding of each weight
      // is unbiased, and l differs from the sum of the rounded weights by far
      // less than that rounding.)
      // (fp8 P V: p in fp32 into pf; the sum is of the fp32 p, for the
      // reference check only -- l takes the sum of the quantised weights)
      float pf[kPv8 ? 32 : 1];
      auto exps = [&](float mc) __attribute__((always_inline)) {
        float part[4] = {0.f, 0.f, 0.f, 0.f};  // (four chains)
        if constexpr (kPv8) {
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            pf[i] = fast_exp2(fmaf(sc[i >> 4][i & 15], c2s, -mc));
            part[i & 3] += pf[i];
          }
        } else {
#pragma unroll
          for (int kc = 0; kc < 4; ++kc)
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
              const float e0 = fast_exp2(fmaf(sc[kc >> 1][8 * (kc & 1) + j], c2s, -mc));
              const float e1 = fast_exp2(fmaf(sc[kc >> 1][8 * (kc & 1) + j + 1], c2s, -mc));
              pb[kc][j] = (__bf16)e0;
              pb[kc][j + 1] = (__bf16)e1;
              part[j / 2] += e0 + e1;
            }
        }
        return (part[0] + part[1]) + (part[2] + part[3]);
      };
      // Lazy reference max: the exponentials are taken against the current
      // reference m without looking for the tile's max first.  While every
      // lane's sum stays at most 2^kPartLog2 (so each p does), nothing moves;
      // otherwise (and on an item's first tile) the tile's max is found, m
      // moves up to it, O and l are rescaled and the exponentials are taken
      // again.  Softmax is unchanged by the choice of reference.
      // (a row may have no allowed key yet -- a sliding window's first tiles
      // -- and keeps m = -inf; its exponentials are then taken against 0)
      const bool fresh = __any(m == -__builtin_huge_valf());
      float part = 0.f;
      if (!fresh) part = exps(m * c2s);
      const bool moved = fresh || __any(!(part <= kPartCap));
      if (a.stats) {
        // diagnostics: tiles, first-tile max passes, later rescales (per wave
        // and tile; added to the caller's counters once, at the wave's end)
        ++st_tiles;
        if (moved) ++(fresh ? st_first : st_later);
      }
      if (moved) {
        float mt = -__builtin_huge_valf();
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sc[st][i]);
        mt = max_halves(mt);
        const float m_new = fmaxf(m, mt);
        const float alpha = m == -__builtin_huge_valf() ? 0.f : fast_exp2((m - m_new) * c2s);
        l *= alpha;
        if (!o_zero) {
#pragma unroll
          for (int t = 0; t < kOTiles; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
        }
        m = m_new;
        part = exps(m == -__builtin_huge_valf() ? 0.f : m * c2s);
      }
      if constexpr (kPv8) {
        // P to e4m3 with one E8M0 scale per 32 keys (row, key block kb = the
        // registers of sc[kb], shared by the two lane halves): 2^(floor(log2
        // max) - 7), so every scaled weight is below 256 (no saturation
        // needed); l adds the quantised weights, so the weights O uses are
        // normalised exactly.
        float lq = 0.f;
        psc = 0;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          float amax = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) amax = fmaxf(amax, pf[16 * kb + i]);
          amax = max_halves(amax);
          const int sb = max(int((__float_as_uint(amax) >> 23) & 0xFFu) - 7, 0);
          const float scl = sb ? __uint_as_float(unsigned(sb) << 23) : __uint_as_float(0x00400000u);
#pragma unroll
          for (int wd = 0; wd < 4; ++wd) {
            const float* pw = pf + 16 * kb + 4 * wd;
            s16x2 cw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, pw[0], pw[1], scl, false);
            cw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(cw, pw[2], pw[3], scl, true);
            const unsigned u = __builtin_bit_cast(unsigned, cw);
            pq[4 * kb + wd] = int(u);
            const f32x2 d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(u, scl, false);
            const f32x2 d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(u, scl, true);
            lq += (d0[0] + d0[1]) + (d1[0] + d1[1]);
          }
          psc |= unsigned(sb) << (8 * kb);
        }
        part = lq;
      }
      l += part;
    } else {
      // (keys past the sample in a ragged tile need no mask: their V rows
      // are zero, see the top of the step, and their weights are finite)
      const float* ksl = reinterpret_cast<const float*>(ring + stage * K::kStageBytes + K::kKsOff);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const int kk = 32 * (kc >> 1) + 16 * ((kc & 1)) + 8 * g + j;
          const float g0 = gelu_act<ACT>(sc[kc >> 1][8 * (kc & 1) + j] * rq * ksl[kk]);
          const float g1 = gelu_act<ACT>(sc[kc >> 1][8 * (kc & 1) + j + 1] * rq * ksl[kk + 1]);
          pb[kc][j] = (__bf16)g0;
          pb[kc][j + 1] = (__bf16)g1;
        }
    }
  };

  // Output rows of the k-th item: O / l (softmax) or O / Lk (GELU), then reset
  // (O by the next P V, see o_zero).  Softmax with a log-sum-exp output: each
  // row also gets ln(sum_j exp(s_j / sqrt(D))) = (m c + log2 l) ln 2, m being
  // the reference max of the raw scores s and c = log2(e)/sqrt(D) (both lane
  // halves hold the same m and l bit for bit and store the same value).
  // Returns whether this wave issued its kStoresPerWave output stores.  (The
  // log-sum-exp store is not counted: the next wait then lets one op fewer
  // run on -- the first load of the next tile -- which is safe; an exact
  // count would cost the wait a run-time switch at every step.)
  auto epilogue = [&](int k, int prow0) __attribute__((always_inline)) {
    const WorkItem it = load_record(c, k);
    const int row0 = kPipe ? prow0 : it.q0 + 32 * wave;
    const int qrow = row0 + l32;
    float scale;
    if constexpr (ACT == ACT_SOFTMAX) {
      const float l_tot = sum_halves(l);
      scale = l_tot > 0.f ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
      if ((c.lse_lo | c.lse_hi) != 0u && qrow < it.lq)
        lse_ptr(c)[size_t(it.qbeg + qrow) * a.H + it.h] = (m * c2s + __log2f(l_tot)) * 0.69314718055994531f;
    } else {
      scale = __builtin_amdgcn_rcpf(float(it.lk));
    }
    if (qrow < it.lq) {
      // wave-uniform row base (scalar registers) + 32-bit lane offset: no
      // 64-bit lane address stays live across the stream loop
      unsigned char* ob = const_cast<unsigned char*>(
          uniform_ptr(reinterpret_cast<const unsigned char*>(a.out) + (size_t(it.qbeg + row0) * a.H + it.h) * size_t(2 * D)));
      // (out is bf16 whatever the input format: 2 H D bytes between a head's rows)
      const unsigned loff = unsigned(l32) * (2u * unsigned(a.H) * D) + unsigned(D * g);
#pragma unroll
      for (int t = 0; t < kOTiles; ++t)
#pragma unroll
        for (int i = 0; i < 16; i += 8) {
          bf16x8 ov;
#pragma unroll
          for (int j = 0; j < 8; ++j) ov[j] = (__bf16)(o[t][i + j] * scale);
          store_global16(ob + loff + 2 * (16 * t + i), ov);
        }
    }
    o_zero = true;
    m = -__builtin_huge_valf();
    l = 0.f;
    return row0 < it.lq;  // (lane 0 stores)
  };

  bool stores_pending = false;  // the output stores of the last step follow its tile loads
  bool q_ahead = false;         // QPF: the last step loaded the next item's Q after its tile loads
  for (int s = 0;; ++s) {
    // Tile s has landed once only the loads of tile s+1 (and the output
    // stores issued after them, and a Q prefetched after them) can still be
    // pending; so has the pipeline's Q block of the last step (issued before
    // them).
    wait_vmcnt(K::kVmemPerTile + (stores_pending ? K::kStoresPerWave : 0) + (q_ahead ? kQChunks : 0));
    lds_barrier();
    const int st_s = s % K::kRing, st_prev = (s + K::kRing - 1) % K::kRing, st_pf = (s + 2) % K::kRing;
    if constexpr (ACT != ACT_SOFTMAX) {
      // GELU: the V rows of tile s (landed above) past the sample's last key,
      // which the loads filled with copies of the last key, to zero.  O += V P
      // reads them in the next step (after its barrier), and a zero row makes
      // the weight of a key past the sample irrelevant, so the activation
      // needs no mask (GELU keeps no row sum, and its weights stay finite).
      const int nv = c0.lk - kBlock * c0.t;
      if (c0.k < c.n && nv < kBlock) {
        unsigned char* vz = ring + v_at(s);
        constexpr int kChunks = kRowBytes / 16;
#pragma unroll
        for (int e = tid; e < kBlock * kChunks; e += K::kNT)
          if (e / kChunks >= nv) *reinterpret_cast<u32x4*>(vz + 16 * e) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    // Q block starting on tile s+2 (read in step s+1): issued before this
    // step's tile loads, so the next step's wait covers it.
    q_stage(c2, src);

    // ---- late waves' VALU phase, then O += V_{s-1} P_{s-1}.
    auto head = [&]() __attribute__((always_inline)) {
      if (late && s > 0 && pv_act) vphase(pv_nvalid, st_prev, pv_key0, pv_r0);
      // The MFMA phase runs at raised wave priority: the SIMD's other wave is
      // in its VALU phase, and the matrix core should get the next MFMA as
      // soon as it can take one.
      __builtin_amdgcn_s_setprio(2);
      if (s > 0) {
        if (kPv8 && (WMODE == kWinNone || pv_act)) {
          // fp8 O^T += V^T P^T: one 32x32x64 MFMA per output tile t over all 64
          // keys.  A row r is head dim dim_perm(t, r) (the output layout of
          // the bf16 product), its bytes the requantised V^T codes of the keys
          // in the order of P's registers; lane half g gives the scale of key
          // block g of its row, P's scale of key block g.
          const unsigned char* vt = ring + v_at(s - 1);
          const unsigned vsw = *reinterpret_cast<const unsigned*>(ring + K::kMxVts + ((s - 1) & 1) * 8 + 4 * g);
          const int psg = int((psc >> (8 * g)) & 0xFFu);
          i32x8 aop[kOTiles];
#pragma unroll
          for (int t = 0; t < kOTiles; ++t) {
            const int d = dim_perm<D>(t, l32);
            const u32x4 w0 = *reinterpret_cast<const u32x4*>(vt + d * 64 + 16 * (g ^ vt_swz(d)));
            const u32x4 w1 = *reinterpret_cast<const u32x4*>(vt + d * 64 + 16 * ((2 + g) ^ vt_swz(d)));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              aop[t][j] = int(w0[j]);
              aop[t][4 + j] = int(w1[j]);
            }
          }
          const f32x16 zero{};
#pragma unroll
          for (int t = 0; t < kOTiles; ++t) {
            const int sa = int((vsw >> (8 * (dim_perm<D>(t, l32) / kMxBlock))) & 0xFFu);
            o[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop[t], pq, o_zero ? zero : o[t], 0, 0, 0, sa, 0, psg);
          }
          o_zero = false;
        } else if (WMODE == kWinNone || pv_act) {
          // 4*kOTiles MFMAs (16-key chunk kc, output tile t), the V^T operand
          // read kAhead MFMAs early: one wave issues them alone, so the LDS
          // transpose-read latency is not hidden by a second wave.
          const unsigned char* vs = ring + v_at(s - 1);  // (s > 0)
          auto vread = [&](int i) __attribute__((always_inline)) {
            const int kc = i / kOTiles, t = i % kOTiles;
            const unsigned char* p0 = vs + v_row + kc * 16 * kRowBytes + v_col[t];
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 4 * kRowBytes));
            const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
            u32x4 w;
            w[0] = lo2[0];
            w[1] = lo2[1];
            w[2] = hi2[0];
            w[3] = hi2[1];
            return __builtin_bit_cast(bf16x8, w);
          };
          constexpr int kN = 4 * kOTiles, kAhead = kN < kPPAhead ? kN : kPPAhead;
          // (one copy per value of `fresh`: the first chunk's MFMAs of an item
          // take C = 0)
          auto pv_tile = [&](auto fresh) __attribute__((always_inline)) {
            bf16x8 vop[kAhead];
#pragma unroll
            for (int i = 0; i < kAhead; ++i) vop[i] = vread(i);
#pragma unroll
            for (int i = 0; i < kN; ++i) {
              const bf16x8 op = vop[i % kAhead];
              if (i + kAhead < kN) vop[i % kAhead] = vread(i + kAhead);
              if (decltype(fresh)::value && i < kOTiles)
                o[i % kOTiles] = mfma_32x32x16(op, pb[i / kOTiles], f32x16{});
              else
                o[i % kOTiles] = mfma_32x32x16(op, pb[i / kOTiles], o[i % kOTiles]);
            }
            // keep the reads kAhead MFMAs early (the scheduler would sink them)
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2 * kAhead, 0);
#pragma unroll
            for (int i = 0; i < kN; ++i) {
              __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
              if (i + kAhead < kN) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
            }
          };
          if (o_zero)
            pv_tile(std::true_type{});
          else
            pv_tile(std::false_type{});
          o_zero = false;
        }
        // Output of an item whose last tile was s-1 (cross-attention: after
        // this step's scores, below).  These stores are newer than the loads
        // of tile s+1 (issued in the previous step), so the next step's wait
        // for that tile can let them run on.
        if constexpr (!kLateEpi)
          if (pv_last) stores_pending = epilogue(pv_k, pv_row0);
      }
    };
    // A new item starts with tile s: its Q is loaded and waited for here, in
    // one branch (once per item).  A load that may still be pending where
    // branches meet would make the compiler wait for all later loads -- the
    // tile loads it does not know about -- at every step's scores.
    if (s > 0 && c0.k < c.n && c0.k != pv_k) {
      if constexpr (!QPF) {
        load_q(c0);
        wait_vmcnt(0);
      }
      q_fresh = true;
    }
    stores_pending = false;
    head();
    if (c0.k >= c.n) {
      if constexpr (kLateEpi)
        if (s > 0 && pv_last) epilogue(pv_k, pv_row0);
      break;
    }
    if (q_fresh) {
      // QPF: the item's Q was loaded at the end of the last step, after every
      // other load and store still in flight (the compiler adds its own wait
      // for the Q registers here as well)
      if constexpr (QPF) wait_vmcnt(kLateEpi ? 0 : (stores_pending ? K::kStoresPerWave : 0));
      q_rms();
      q_fresh = false;
    }
    // Loads of tile s+2 (into the stage that held tile s-2, last read in the
    // previous step): between the MFMAs of the second score half, or all at
    // once for a wave that skips the tile.
    PipeStep ps{0, false, false, false};
    if constexpr (kPipe) ps = pipe_step(c0, pair, nb);
    // this wave computes tile s
    const bool act = WMODE == kWinNone || (kPipe ? ps.act : (c0.t >= c0.wlo && c0.t <= c0.whi));
    const int pf_k = k_at(s + 2), pf_v = vc_at(s + 2);
    if (!act) {
#pragma unroll
      for (int j = 0; j < K::kDmaJobs; ++j) tile_job(c2, src, pf_k, pf_v, j);
    } else if constexpr (kMx8) {
      // Block-scaled fp8 scores: four 32x32x64 MFMAs (key half st, 64-element
      // chunk c of D), A = the key row's codes from LDS (laid out like the query
      // operand), its scale byte from the tile's scale rows.  All operands are
      // read before the first MFMA; the tile loads go between the MFMAs of the
      // second half.
      const unsigned char* ks = ring + k_at(s);
      const unsigned char* kss = ring + K::kMxKs + (s % 3) * 256;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[st][i] = 0.f;
      i32x8 kop[2 * kMxC];
#pragma unroll
      for (int i = 0; i < 2 * kMxC; ++i) {
        const int krow = 32 * (i / kMxC) + kp, cc = i % kMxC;
        const u32x4 w0 = *reinterpret_cast<const u32x4*>(ks + krow * D + 16 * ((4 * cc + g) ^ swz_c<D>(krow)));
        const u32x4 w1 = *reinterpret_cast<const u32x4*>(ks + krow * D + 16 * ((4 * cc + 2 + g) ^ swz_c<D>(krow)));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kop[i][j] = int(w0[j]);
          kop[i][4 + j] = int(w1[j]);
        }
      }
      const unsigned ksw0 = *reinterpret_cast<const unsigned*>(kss + 4 * kp);
      const unsigned ksw1 = *reinterpret_cast<const unsigned*>(kss + 4 * (32 + kp));
#pragma unroll
      for (int i = 0; i < 2 * kMxC; ++i) {
        const int st = i / kMxC, cc = i % kMxC;
        const int kscl = int(((st ? ksw1 : ksw0) >> (8 * (2 * cc + g))) & 0xFFu);
        sc[st] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop[i], qc[cc], sc[st], 0, 0, 0, kscl, 0, qsc[cc]);
        constexpr int kPer = kMxC / K::kDmaJobs > 0 ? kMxC / K::kDmaJobs : 1;
        if (i >= kMxC && (i - kMxC) % kPer == kPer - 1) tile_job(c2, src, pf_k, pf_v, (i - kMxC) / kPer);
      }
      // keep the operand reads ahead of the MFMAs
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, 4 * kMxC + 2, 1);
#pragma unroll
      for (int i = 0; i < 2 * kMxC; ++i) __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 1);
    } else {
      const unsigned char* ks = ring + k_at(s);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[st][i] = 0.f;
      // 2 x kQChunks MFMAs (score half i / kQChunks, D chunk i % kQChunks), the
      // K operand read kAhead MFMAs early.  (LDS reads are not moved across
      // the asm of the tile loads, so the reads are placed early in source
      // order.)
      constexpr int kNS = 2 * kQChunks, kAhead = kNS < kPPAheadS ? kNS : kPPAheadS;
      auto kread = [&](int i) __attribute__((always_inline)) {
        return *reinterpret_cast<const bf16x8*>(ks + (i / kQChunks) * 32 * kRowBytes + k_off[i % kQChunks]);
      };
      bf16x8 kop[kAhead];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) kop[i] = kread(i);
#pragma unroll
      for (int i = 0; i < kNS; ++i) {
        const bf16x8 op = kop[i % kAhead];
        if (i + kAhead < kNS) kop[i % kAhead] = kread(i + kAhead);
        sc[i / kQChunks] = mfma_32x32x16(op, qf[i % kQChunks], sc[i / kQChunks]);
        constexpr int kPer = kQChunks / K::kDmaJobs;
        if (i >= kQChunks && (i - kQChunks) % kPer == kPer - 1) tile_job(c2, src, pf_k, pf_v, (i - kQChunks) / kPer);
      }
      // keep the reads kAhead MFMAs early and the MFMAs in order
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, kAhead, 1);
#pragma unroll
      for (int i = 0; i < kNS; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 1);
        if (i + kAhead < kNS) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 1);
      }
    }
    // Cross-attention (every step ends an item): the output of the item whose
    // last tile was s-1 after this step's scores, whose MFMAs keep the matrix
    // core busy while its first instructions wait for O += V P just issued.
    if constexpr (kLateEpi)
      if (s > 0 && pv_last) stores_pending = epilogue(pv_k, pv_row0);
    tile_scales(c2, src, st_pf);
    mx_scales(c2, src, s + 2);
    if constexpr (QPF) {
      // the scores above have consumed Q: load the next item's (one branch,
      // waited for by count, see above)
      q_ahead = c1.k != c0.k && c1.k < c.n;
      if (q_ahead) load_q(c1);
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (kPipe) {
      // This wave's next block starts on tile s+1 of the same item: its Q was
      // staged in LDS (in the previous step) and replaces the fragments the
      // scores above have consumed.
      const PipeStep pn = pipe_step(c1, pair, nb);
      if (c1.k == c0.k && pn.first && c1.t > c1.wlo) {
        const int row = 32 * (wave & 1) + l32;
        if constexpr (kMx8) {
          const unsigned char* qs = ring + K::kMxQc + (c1.t & 1) * K::kLdTile;
          const unsigned sw = *reinterpret_cast<const unsigned*>(ring + K::kMxQs + (c1.t & 1) * 256 + 4 * row);
#pragma unroll
          for (int cc = 0; cc < kMxC; ++cc) {
            const u32x4 w0 = *reinterpret_cast<const u32x4*>(qs + row * D + 16 * ((4 * cc + g) ^ swz_c<D>(row)));
            const u32x4 w1 = *reinterpret_cast<const u32x4*>(qs + row * D + 16 * ((4 * cc + 2 + g) ^ swz_c<D>(row)));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              qc[cc][j] = int(w0[j]);
              qc[cc][4 + j] = int(w1[j]);
            }
            qsc[cc] = int((sw >> (8 * (2 * cc + g))) & 0xFFu);
          }
        } else {
          const unsigned char* qs = ring + kPipeQ + (c1.t & 1) * K::kTileBytes;
#pragma unroll
          for (int cc = 0; cc < kQChunks; ++cc)
            qf[cc] = *reinterpret_cast<const bf16x8*>(qs + row * kRowBytes + 16 * ((kQChunks * g + cc) ^ swz_k<D>(row)));
        }
      }
    }
    if constexpr (kPv8) {
      // V of tile s (landed at the top of this step) requantised along the
      // keys for the fp8 O += V P, into the V^T slot the next step reads.
      // Wave w takes keys 32 kb .. +32 (kb = w / 4) and head dims 32 b .. +32
      // (b = w % 4); lane (kg, dg) 4 keys x 4 dims.  The new scale of (kb, b)
      // is the largest of the 32 keys' MX scales of block b, so a code only
      // moves down by the difference of exponents (exact unless it then falls
      // below e4m3's smallest subnormal), rounded to nearest even.  A 4 x 4
      // byte transpose turns 4 key rows into 4 dim rows of 4 keys each.
      const int kb = wave >> 2, b = wave & 3, kg = lane & 7, dg = lane >> 3;
      const unsigned char* vcs = ring + vc_at(s);
      const unsigned char* vss = ring + K::kMxVs + (s % 3) * 256;
      unsigned r[4];
      int e[4], emax = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = 32 * kb + 4 * kg + i;
        r[i] = *reinterpret_cast<const unsigned*>(vcs + k * D + 16 * ((2 * b + (dg >> 2)) ^ swz_c<D>(k)) + 4 * (dg & 3));
        e[i] = int((*reinterpret_cast<const unsigned*>(vss + 4 * k) >> (8 * b)) & 0xFFu);
        emax = max(emax, e[i]);
      }
      emax = max(emax, __shfl_xor(emax, 1, 64));
      emax = max(emax, __shfl_xor(emax, 2, 64));
      emax = max(emax, __shfl_xor(emax, 4, 64));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float down = __uint_as_float(unsigned(max(127 - (emax - e[i]), 0)) << 23);  // 2^(e - emax)
        const f32x2 x0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r[i], down, false);
        const f32x2 x1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r[i], down, true);
        s16x2 cw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, x0[0], x0[1], 1.0f, false);
        cw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(cw, x1[0], x1[1], 1.0f, true);
        r[i] = __builtin_bit_cast(unsigned, cw);
      }
      // byte j of r[i] is (key i, dim j) -> col[j] byte i
      const unsigned lo01 = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u), hi01 = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);
      const unsigned lo23 = __builtin_amdgcn_perm(r[3], r[2], 0x05010400u), hi23 = __builtin_amdgcn_perm(r[3], r[2], 0x07030602u);
      const unsigned col[4] = {__builtin_amdgcn_perm(lo23, lo01, 0x05040100u), __builtin_amdgcn_perm(lo23, lo01, 0x07060302u),
                               __builtin_amdgcn_perm(hi23, hi01, 0x05040100u), __builtin_amdgcn_perm(hi23, hi01, 0x07060302u)};
      // keys 32 kb + 16 a + 8 g' + r sit at position 32 kb + 16 g' + 8 a + r of a
      // V^T row (P's register order): bits 1 and 2 of the key group swap
      const int pos = 32 * kb + 4 * ((kg & 1) | ((kg & 2) << 1) | ((kg & 4) >> 1));
      unsigned char* vt = ring + v_at(s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * b + 4 * dg + i;
        *reinterpret_cast<unsigned*>(vt + d * 64 + 16 * ((pos >> 4) ^ vt_swz(d)) + (pos & 15)) = col[i];
      }
      if (lane == 0) ring[K::kMxVts + (s & 1) * 8 + 4 * kb + b] = (unsigned char)emax;
    } else if constexpr (kMx8) {
      // V of tile s (landed at the top of this step) to bf16, exactly (4-bit
      // e4m3 significands times a power of two), by every thread: 16 codes of
      // one row each, into the bf16 slot O += V P reads in the next step.
      // (that slot last held tile s-2, read in the previous step)
      const int row = tid >> 3, j16 = tid & 7;
      const unsigned char* vcs = ring + vc_at(s);
      const u32x4 w = *reinterpret_cast<const u32x4*>(vcs + row * D + 16 * (j16 ^ swz_c<D>(row)));
      const unsigned sw = *reinterpret_cast<const unsigned*>(ring + K::kMxVs + (s % 3) * 256 + 4 * row);
      const float scl = e8m0_to_float(sw >> (8 * (j16 >> 1)));
      u32x4 o0, o1;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        o0[2 * i] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], scl, false));
        o0[2 * i + 1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], scl, true));
        o1[2 * i] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 + i], scl, false));
        o1[2 * i + 1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 + i], scl, true));
      }
      unsigned char* vb = ring + v_at(s) + row * kRowBytes;
      *reinterpret_cast<u32x4*>(vb + 16 * ((2 * j16) ^ swz_v<D>(row))) = o0;
      *reinterpret_cast<u32x4*>(vb + 16 * ((2 * j16 + 1) ^ swz_v<D>(row))) = o1;
    }
    const bool s_last = kPipe ? ps.last : c0.t == c0.te - 1;
    const int nvalid = min(64, c0.lk - 64 * c0.t);
    if (!late && act) vphase(nvalid, st_s, 64 * c0.t, c0.r0);
    pv_k = c0.k;
    pv_act = act;
    pv_last = s_last;
    pv_nvalid = nvalid;
    pv_key0 = 64 * c0.t;
    pv_r0 = c0.r0;
    if constexpr (kPipe) pv_row0 = kBlock * ps.b + 32 * (wave & 1);
    c0 = c1;
    c1 = c2;
    advance<D, WMODE, IN>(c, c2, src, wave, lane, nb, wt);
  }
  if (a.stats && lane == 0 && st_tiles) {
    atomicAdd(a.stats, (unsigned long long)st_tiles);
    atomicAdd(a.stats + 1, (unsigned long long)st_first);
    atomicAdd(a.stats + 2, (unsigned long long)st_later);
  }
}

}  // namespace

template <int D, int ACT>
hipError_t launch_none(bool cross, dim3 gd, dim3 bd, hipStream_t st, const AttnArgs& a, const KTiming& tm) {
  if (cross) return launch1(attn_pp_kernel<D, ACT, kWinNone, true, IN_BF16>, gd, bd, st, a, tm);
  return launch1(attn_pp_kernel<D, ACT, kWinNone, false, IN_BF16>, gd, bd, st, a, tm);
}

template <int D>
hipError_t launch_d(int act, bool cross, dim3 gd, dim3 bd, hipStream_t st, const AttnArgs& a, const KTiming& tm) {
  if (a.window_tokens > 0)  // (softmax only)
    return launch1(attn_pp_kernel<D, ACT_SOFTMAX, kWinSliding, false, IN_BF16>, gd, bd, st, a, tm);
  if (a.window_blocks > 0 && a.window_blocks <= kPipePairs)  // (softmax only)
    return launch1(attn_pp_kernel<D, ACT_SOFTMAX, kWinPipe, false, IN_BF16>, gd, bd, st, a, tm);
  if (a.window_blocks > 0)  // (softmax only)
    return launch1(attn_pp_kernel<D, ACT_SOFTMAX, kWinBlock, false, IN_BF16>, gd, bd, st, a, tm);
  if (act == ACT_SOFTMAX) return launch_none<D, ACT_SOFTMAX>(cross, gd, bd, st, a, tm);
  if (act == ACT_GELU_POLY) return launch_none<D, ACT_GELU_POLY>(cross, gd, bd, st, a, tm);
  return launch_none<D, ACT_GELU>(cross, gd, bd, st, a, tm);
}

// MX8 inputs (D = 128, softmax self-attention): full, or block windows of up
// to four blocks.  (The IN_MX8P form -- P V on the fp8 MFMA -- is not
// instantiated: it faulted the GPU on its first run, cause not found.)
hipError_t launch_mx8(dim3 gd, dim3 bd, hipStream_t st, const AttnArgs& a, const KTiming& tm) {
  if (a.window_blocks > 0)
    return launch1(attn_pp_kernel<128, ACT_SOFTMAX, kWinPipe, false, IN_MX8>, gd, bd, st, a, tm);
  return launch1(attn_pp_kernel<128, ACT_SOFTMAX, kWinNone, false, IN_MX8>, gd, bd, st, a, tm);
}

int pp_rows() { return kPPRows; }
int pp_item_cache() { return kPPItemCache; }
int pp_enum_max_runs() { return kMaxRuns; }
int pp_enum_max_offsets() { return 64 * kPPWaves; }
int pp_pipe_rows() { return kBlock * kPipeBlocks; }
int pp_pipe_max_blocks() { return kPipePairs; }

bool pp_takes_mx8(int D, int act, bool self, int window_blocks) {
  return D == 128 && act == ACT_SOFTMAX && self && window_blocks <= kPipePairs;
}

// in: IN_BF16 or IN_MX8 (the MX form only where pp_takes_mx8 holds).
hipError_t launch_attn_pp(int D, int act, bool cross, int in, const AttnArgs& a, int num_cu, int64_t max_items,
                          int64_t grid_cap, const KTiming& tm, hipStream_t st) {
  // One workgroup per CU (the tile ring takes most of the LDS), a multiple of the XCD count.
  const dim3 gd(static_cast<unsigned>(persistent_grid(num_cu, max_items, grid_cap))), bd(64 * kPPWaves);
  if (in != IN_BF16) return launch_mx8(gd, bd, st, a, tm);
  if (D == 32) return launch_d<32>(act, cross, gd, bd, st, a, tm);
  if (D == 64) return launch_d<64>(act, cross, gd, bd, st, a, tm);
  return launch_d<128>(act, cross, gd, bd, st, a, tm);
}

}  // namespace ja
