// Internal definitions shared by the host launcher and the device kernels of
// libjagged_attn.  Not part of the public ABI (include/jagged_attn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct ja_io;

namespace ja {

constexpr int kBlock = 64;        // token block of block-aligned attention
constexpr int kMxBlock = 32;      // elements per E8M0 scale along D
constexpr int kWaveSize = 64;
constexpr int kThreads = 256;     // threads of the split-merge kernel
constexpr int kPmaRows = 32;      // query rows per key-split work item

// GELU scores: tanh form (exp + rcp) or the ALU-only polynomial (ja_gelu_poly.h).
enum Act { ACT_SOFTMAX = 0, ACT_GELU = 1, ACT_GELU_POLY = 2 };
// IN_MX: MX-fp8 decoded to bf16 on load; IN_MX8 (D = 128): fp8 codes stay fp8
// for block-scaled fp8 MFMA on QK^T, V is converted to bf16 in LDS; IN_MX8P:
// as IN_MX8, with P V on the fp8 MFMA too (P and V requantised along the keys).
enum In { IN_F32 = 0, IN_BF16 = 1, IN_MX = 2, IN_MX8 = 3, IN_MX8P = 4 };

// ---------------------------------------------------------------------------
// Workspace layout (caller-owned device memory; every section 256-B aligned)
//   [0, 256)            WsHeader
//   sample_nsplit[B]    key-split count per sample (1 = written directly)
//   sample_pbase[B]     first partial slot of the sample
//   items[max_items]    WorkItem
//   part_o[max_slots][32][D] float, part_ml[max_slots][32] float2
//   kscale[total_kv][H] float     RMS factor of every key row (ping-pong GELU only)
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;           // workgroup w runs on XCD w % 8 (round-robin dispatch)

struct WsHeader {
  int32_t status;              // JA_OK or JA_EOFFSETS, written by the plan kernel
  int32_t n_items;             // work items for the attention kernel
  int32_t n_slots;             // partial slots in use
  int32_t items_off;           // byte offset of the item list from the header (read back by tests)
  int32_t xcd_begin[kXcds + 1];  // items [xcd_begin[x], xcd_begin[x+1]) run on XCD x
                                 // (sample order; not used with cost order)
  int32_t pad[64 - 4 - (kXcds + 1)];
};

// One unit of attention work: sample b, head h, first query row q0 and key
// split, with the sample's offsets copied in so that a kernel needs a single
// 32-byte read (no dependent loads) to start the item.
struct WorkItem {
  int32_t b, h, q0, split;
  int32_t qbeg, lq, kbeg, lk;
};

struct WsLayout {
  size_t nsplit_off, pbase_off, items_off, part_o_off, part_ml_off, kscale_off, total;
  int64_t max_items, max_slots;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Work decomposition chosen on the host from the arguments alone.
struct Schedule {
  int bm;        // query rows per work item
  int kvc;       // key chunk per work item (0 = whole sample)
  int grid_cap;  // upper bound on work items
};

struct PlanArgs {
  const int32_t* qo;
  const int32_t* ko;
  int B, H;
  int32_t total_q, total_kv;
  int bm, kvc, self_check;
  int window_blocks;   // 0 = no window (used for the per-item cost estimate)
  int window_tokens;   // sliding window in tokens (0 = none)
  int cost_order;      // 1: items sorted by key tiles, most first (xcd_begin unused)
  int64_t max_items, max_slots;
  WsHeader* hdr;
  int32_t* status_out;  // optional copy of the status word (caller's device memory), or null
  int32_t* nsplit;
  int32_t* pbase;
  WorkItem* items;
  // Side job of the same launch (GELU scores on the tile stream): the RMS
  // factor (mean over D of k^2 + eps)^(-1/2) of each of krms_rows bf16 key
  // rows of krms_d elements into krms_out, by workgroups 1.. (0 rows: none).
  const void* krms_k;
  int64_t krms_rows;
  int krms_d;
  float krms_eps;
  float* krms_out;
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* qs;  // MX scales (IN_MX only)
  const uint8_t* ks;
  const uint8_t* vs;
  void* out;
  const int32_t* qo;
  const int32_t* ko;
  const WsHeader* hdr;
  const WorkItem* items;
  const int32_t* nsplit;
  const int32_t* pbase;
  float* part_o;
  float2* part_ml;
  const float* kscale;  // RMS factor per key row and head (ping-pong GELU), else null
  int H;
  int window_blocks;  // 0 = no window
  int window_tokens;  // sliding window in tokens (0 = none)
  int kvc;
  int dealt;          // items come sorted by cost, most first, and are dealt in alternating rounds
  float score_scale;  // softmax: log2(e)/sqrt(D); GELU: 1/sqrt(D)
  float eps;
  unsigned long long* stats;  // optional softmax counters (tile stream): tiles, max passes, rescales
  float* lse;                  // optional softmax log-sum-exp per query row and head (natural log)
  // Tile stream without a plan launch (inplan = 1): every workgroup checks the
  // offsets and enumerates its own items; workgroup 0 writes the header (and
  // status_out).  B + 1 <= 512 offsets, bm query rows per item.
  int inplan;
  int B, bm, self_check;
  int32_t total_q, total_kv;
  int32_t* status_out;
};

// Events that time one kernel from its own dispatch packet (hipExtLaunchKernel
// writes the dispatch's start and end timestamps into them; null: untimed).
struct KTiming {
  hipEvent_t start;
  hipEvent_t stop;
};

// Launch geometry shared by the persistent kernels: at most `cap` workgroups
// (0: no cap), a multiple of the XCD count and at least one per XCD.
inline int64_t persistent_grid(int64_t slots, int64_t max_items, int64_t cap) {
  int64_t grid = slots;
  const int64_t need = ((max_items + kXcds - 1) / kXcds) * kXcds;
  if (grid > need) grid = need;
  if (cap > 0 && grid > cap) grid = cap;
  grid = (grid / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  return grid;
}

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  float* dq;
  float* dk;
  float* dv;
  const WsHeader* hdr_q;    // plan over query tiles
  const WorkItem* items_q;
  const WsHeader* hdr_k;    // plan over key tiles (swapped offsets)
  const WorkItem* items_k;
  float2* stats;            // per (query row, head): log2-sum-exp of the scores, D_i
  const float* lse_in;      // optional (softmax): the forward's natural log-sum-exp per (query row, head)
  const void* o_in;         // with lse_in: the forward's output (input dtype), for D_i = dO_i . O_i
  float* rq;                // GELU: RMS factor per (query row, head)
  float* rk;                // GELU: RMS factor per (key row, head)
  int H;
  int window_blocks;
  int window_tokens;
  float c2;                 // log2(e) / sqrt(D)
  float inv_sqrt_d;
  float eps;                // GELU: RMSNorm epsilon
};

struct CombineArgs {
  void* out;
  const int32_t* qo;
  const int32_t* ko;
  const WsHeader* hdr;
  const int32_t* nsplit;
  const int32_t* pbase;
  const float* part_o;
  const float2* part_ml;
  float* lse;  // optional log-sum-exp output (softmax)
  int B, H, act;
};

// The forward on a given workspace (ja_api.cpp): validation, plan and
// attention launches on io.stream; the workspace is `workspace_bytes` of
// device memory (the caller's, or the library's own scratch).
int fwd_impl(const void* q, const void* k, const void* v, const int32_t* q_offsets, const int32_t* kv_offsets,
             int B, int H, int D, int variant, int act, int window, void* out, const ::ja_io& io, void* workspace,
             size_t workspace_bytes);

// Debug mode (environment variable JA_DEBUG set to anything but "0", read
// once per process): every entry point that launches work synchronises its
// stream before returning and reports the device status (offset errors,
// launch and runtime faults) as its own return value.
bool debug_sync();

// Debug mode: synchronise `stream` and return the status word(s) at the given
// device addresses (NULL entries are skipped); JA_EHIP if the stream failed.
int debug_status(hipStream_t stream, const void* st0, const void* st1);

}  // namespace ja
