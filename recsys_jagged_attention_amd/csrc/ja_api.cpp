// C ABI of libjagged_attn: argument validation, schedule choice, workspace
// layout and launches on the caller's stream.  No allocation, no host read
// of the offsets, no synchronisation on the forward path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "ja_internal.h"
#include "jagged_attn.h"

namespace ja {
hipError_t launch_plan(const PlanArgs& a, hipStream_t st);
hipError_t launch_plan_pair(const PlanArgs& a, const PlanArgs& b, hipStream_t st);
hipError_t launch_attn_mfma(int D, int in, int shape, int act, const AttnArgs& a, int num_cu,
                            int64_t max_items, int64_t grid_cap, const KTiming& tm, hipStream_t st);
hipError_t launch_combine(int D, const CombineArgs& a, hipStream_t st);
hipError_t launch_attn_f32(int D, int act, int window_mode, const AttnArgs& a, int grid, const KTiming& tm,
                           hipStream_t st);
hipError_t launch_attn_pp(int D, int act, bool cross, int in, const AttnArgs& a, int num_cu, int64_t max_items,
                          int64_t grid_cap, const KTiming& tm, hipStream_t st);
bool pp_takes_mx8(int D, int act, bool self, int window_blocks);
hipError_t launch_attn_bwd(int D, bool bf16, int act, int wmode, const BwdArgs& a, int64_t rows_q, int64_t rows_k,
                           int grid_q, int grid_k, hipStream_t st);
hipError_t launch_attn_bwd_mfma(int D, int act, int wmode, const BwdArgs& a, int grid_q, int grid_k,
                                hipStream_t st);
hipError_t launch_bwd_rms(int D, bool bf16, const BwdArgs& a, int64_t rows_q, int64_t rows_k, hipStream_t st);
hipError_t launch_mx_quant(bool bf16, const void* x, int64_t n_blocks, uint8_t* codes, uint8_t* scales,
                           hipStream_t st);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
int pp_rows();
int pp_pipe_rows();
int pp_pipe_max_blocks();
int pp_item_cache();
int pp_enum_max_runs();
int pp_enum_max_offsets();

namespace {

constexpr int kShapeQTiled = 0, kShapeWindow = 1, kShapeKvSplit = 2, kShapeFullSelf = 3, kShapeF32 = 4,
              kShapePingPong = 5;
constexpr int kMaxGrid = 1 << 20;

struct Plan {
  int shape;
  int bm;
  int kvc;
  WsLayout ws;
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device.  Cached per device id for the first
// kMaxCachedDevices ids (relaxed atomics: concurrent first calls on one device
// may both query it and store the same value); other ids are queried each call.
constexpr int kMaxCachedDevices = 64;
hipError_t device_cus(int* cus) {
  static std::atomic<int> cache[kMaxCachedDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxCachedDevices) {
    const int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) {
      *cus = n;
      return hipSuccess;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n < 1) return hipErrorInvalidDevice;
  if (dev >= 0 && dev < kMaxCachedDevices) cache[dev].store(n, std::memory_order_relaxed);
  *cus = n;
  return hipSuccess;
}

// Key chunk for the key-split shape: about 2048 work items per call, a
// power of two between 512 and 8192 keys (long samples are split, short ones
// are not), so skewed K/V lengths still spread over every CU.
int choose_kvc(int H, int32_t total_kv) {
  const int64_t target = cdiv(int64_t(H) * total_kv, 2048);
  int kvc = 512;
  while (kvc < target && kvc < 8192) kvc <<= 1;
  return kvc;
}

int validate(int B, int H, int D, int variant, int act, int window, int dtype, int32_t total_q,
             int32_t total_kv) {
  if (B < 1 || H < 1 || total_q < 0 || total_kv < 0) return JA_EINVAL;
  if (variant < JA_SELF || variant > JA_SLIDING) return JA_EINVAL;
  if (act < JA_SOFTMAX || act > JA_GELU_POLY) return JA_EINVAL;
  if (dtype < JA_F32 || dtype > JA_MXFP8_E4M3) return JA_EINVAL;
  if (window < 0) return JA_EINVAL;
  if ((variant == JA_SELF || variant == JA_SLIDING) && total_q != total_kv) return JA_EINVAL;
  if (variant == JA_SLIDING) {
    if (window < 1) return JA_EINVAL;
    if (act != JA_SOFTMAX || dtype == JA_MXFP8_E4M3) return JA_EUNSUPPORTED;
  } else if (window > 0 && variant != JA_SELF) {
    return JA_EINVAL;
  }
  if (D != 32 && D != 64 && D != 128) return JA_EUNSUPPORTED;
  if (variant == JA_SELF && window > 0 && (window % kBlock != 0 || act != JA_SOFTMAX)) return JA_EUNSUPPORTED;
  if (int64_t(B) * H > (int64_t(1) << 30) || H > 4096) return JA_EUNSUPPORTED;
  return JA_OK;
}

Plan make_plan(int B, int H, int D, int variant, int act, int window, int dtype, int32_t total_q,
               int32_t total_kv) {
  Plan p{};
  if (dtype == JA_F32) {
    p.shape = kShapeF32;
    p.bm = 64;
  } else if ((dtype == JA_BF16 && variant != JA_PMA) ||
             (dtype == JA_MXFP8_E4M3 && variant == JA_SELF && pp_takes_mx8(D, act, true, window / kBlock))) {
    // bf16 self (with or without window) and cross, and MX self-attention at
    // D = 128 (full, or windows of up to four blocks): one tile stream, 8 waves x 32 rows
    p.shape = kShapePingPong;
    p.bm = pp_rows();
    // block windows of at most one 64-token block per wave pair: pipelined runs of query blocks
    if (variant == JA_SELF && window > 0 && window / kBlock <= pp_pipe_max_blocks()) p.bm = pp_pipe_rows();
  } else if (window > 0) {
    p.shape = kShapeWindow;
    p.bm = 128;  // two 64-token query blocks
  } else if (variant == JA_PMA) {
    p.shape = kShapeKvSplit;
    p.bm = kPmaRows;
    p.kvc = choose_kvc(H, total_kv);
  } else if (variant == JA_SELF && act == JA_SOFTMAX) {
    p.shape = kShapeFullSelf;
    p.bm = 256;  // eight waves x 32 query rows
  } else {
    p.shape = kShapeQTiled;
    p.bm = 128;  // four waves x 32 query rows
  }
  WsLayout& w = p.ws;
  w.max_items = int64_t(H) * (cdiv(total_q, p.bm) + B);
  w.max_slots = 0;
  if (p.kvc > 0) {
    w.max_slots = int64_t(H) * (cdiv(total_kv, p.kvc) + B);
    w.max_items += w.max_slots;
  }
  size_t off = align256(sizeof(WsHeader));
  w.nsplit_off = off;
  off = align256(off + sizeof(int32_t) * size_t(B));
  w.pbase_off = off;
  off = align256(off + sizeof(int32_t) * size_t(B));
  w.items_off = off;
  off = align256(off + sizeof(WorkItem) * size_t(w.max_items));
  w.part_o_off = off;
  off = align256(off + sizeof(float) * size_t(w.max_slots) * kPmaRows * D);
  w.part_ml_off = off;
  off = align256(off + sizeof(float2) * size_t(w.max_slots) * kPmaRows);
  w.kscale_off = off;
  if (p.shape == kShapePingPong && act != JA_SOFTMAX) off = align256(off + sizeof(float) * size_t(total_kv) * H);
  w.total = off;
  return p;
}

}  // namespace

// The forward on a given workspace (the caller's, or the library's own
// scratch): validation, plan launch, attention launch [, split merge].
int fwd_impl(const void* q, const void* k, const void* v, const int32_t* q_offsets, const int32_t* kv_offsets,
             int B, int H, int D, int variant, int act, int window, void* out, const ja_io& io, void* workspace,
             size_t workspace_bytes) {
  const int st = validate(B, H, D, variant, act, window, io.dtype, io.total_q, io.total_kv);
  if (st != JA_OK) return st;
  if (!q_offsets || !kv_offsets) return JA_EINVAL;
  if (io.max_workgroups < 0) return JA_EINVAL;
  // fp8 P V is switched off: its kernel (attn_pp_kernel<.., IN_MX8P>) faulted
  // the GPU on its first run and the cause has not been found, so no call
  // launches it.
  if (io.fp8_pv) return JA_EUNSUPPORTED;
  // the log-sum-exp output: softmax only, written by the tile-stream, fp32 and
  // key-split (PMA) shapes
  if (io.lse != nullptr) {
    if (act != JA_SOFTMAX || (reinterpret_cast<uintptr_t>(io.lse) & 3)) return JA_EINVAL;
    const int shape = make_plan(B, H, D, variant, act, window, io.dtype, io.total_q, io.total_kv).shape;
    if (shape != kShapePingPong && shape != kShapeF32 && shape != kShapeKvSplit) return JA_EUNSUPPORTED;
  }
  // Empty tensors may come with null data pointers: no kernel reads q or
  // writes out without query rows, nor reads k or v without key rows.
  const bool has_q = io.total_q > 0, has_kv = io.total_kv > 0;
  if ((has_q && (!q || !out)) || (has_kv && (!k || !v))) return JA_EINVAL;
  if (io.dtype == JA_MXFP8_E4M3 && ((has_q && !io.q_scale) || (has_kv && (!io.k_scale || !io.v_scale))))
    return JA_EINVAL;
  const Plan p = make_plan(B, H, D, variant, act, window, io.dtype, io.total_q, io.total_kv);
  if (workspace == nullptr || workspace_bytes < p.ws.total) return JA_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
       reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(workspace)) & 15)
    return JA_EINVAL;
  if ((reinterpret_cast<uintptr_t>(io.status) & 3) || (reinterpret_cast<uintptr_t>(io.softmax_stats) & 7))
    return JA_EINVAL;
  int num_cu = 0;
  if (device_cus(&num_cu) != hipSuccess) return JA_EHIP;

  hipStream_t stream = reinterpret_cast<hipStream_t>(io.stream);
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
  int32_t* nsplit = reinterpret_cast<int32_t*>(ws + p.ws.nsplit_off);
  int32_t* pbase = reinterpret_cast<int32_t*>(ws + p.ws.pbase_off);
  WorkItem* items = reinterpret_cast<WorkItem*>(ws + p.ws.items_off);
  float* part_o = reinterpret_cast<float*>(ws + p.ws.part_o_off);
  float2* part_ml = reinterpret_cast<float2*>(ws + p.ws.part_ml_off);

  PlanArgs pa{};
  pa.qo = q_offsets;
  pa.ko = kv_offsets;
  pa.B = B;
  pa.H = H;
  pa.total_q = io.total_q;
  pa.total_kv = io.total_kv;
  pa.bm = p.bm;
  pa.kvc = p.kvc;
  pa.self_check = variant == JA_SELF || variant == JA_SLIDING;
  pa.window_blocks = variant == JA_SLIDING ? 0 : window / kBlock;
  pa.window_tokens = variant == JA_SLIDING ? window : 0;
  pa.cost_order = p.shape == kShapePingPong || p.shape == kShapeKvSplit || p.shape == kShapeWindow;
  pa.max_items = p.ws.max_items;
  pa.max_slots = p.ws.max_slots;
  pa.hdr = hdr;
  pa.status_out = io.status;
  pa.nsplit = nsplit;
  pa.pbase = pbase;
  pa.items = items;
  const float rms_eps = io.rms_eps > 0.f ? io.rms_eps : 1e-6f;
  float* ksc = nullptr;
  if (p.shape == kShapePingPong && act != JA_SOFTMAX) {
    // the key RMS factors are computed by extra workgroups of the plan launch
    ksc = reinterpret_cast<float*>(ws + p.ws.kscale_off);
    pa.krms_k = k;
    pa.krms_rows = int64_t(io.total_kv) * H;
    pa.krms_d = D;
    pa.krms_eps = rms_eps;
    pa.krms_out = ksc;
  }
  // The softmax tile stream enumerates its own items (no plan launch) when
  // every sample fits one thread of the workgroup, a sample has at most
  // pp_enum_max_runs() runs of equal cost, and each workgroup's items fit its
  // LDS item cache.
  const int64_t cap = io.max_workgroups;
  bool inplan = false;
  if (p.shape == kShapePingPong && act == JA_SOFTMAX && B + 1 <= pp_enum_max_offsets()) {
    const int span = pa.window_blocks > 0 ? (pa.window_blocks - 1) * kBlock
                                          : (pa.window_tokens > 0 ? pa.window_tokens - 1 : 0);
    const int64_t qt_mid = cdiv(span, p.bm);
    const int64_t grid = persistent_grid(num_cu, p.ws.max_items, cap);
    inplan = qt_mid + 2 <= pp_enum_max_runs() && p.ws.max_items <= int64_t(pp_item_cache()) * grid;
  }
  if (!inplan && launch_plan(pa, stream) != hipSuccess) return JA_EHIP;

  AttnArgs aa{};
  aa.q = q;
  aa.k = k;
  aa.v = v;
  aa.qs = io.q_scale;
  aa.ks = io.k_scale;
  aa.vs = io.v_scale;
  aa.out = out;
  aa.qo = q_offsets;
  aa.ko = kv_offsets;
  aa.hdr = hdr;
  aa.items = items;
  aa.nsplit = nsplit;
  aa.pbase = pbase;
  aa.part_o = part_o;
  aa.part_ml = part_ml;
  aa.H = H;
  aa.window_blocks = variant == JA_SLIDING ? 0 : window / kBlock;
  aa.window_tokens = variant == JA_SLIDING ? window : 0;
  aa.kvc = p.kvc;
  aa.dealt = p.shape == kShapeKvSplit || p.shape == kShapeWindow;
  aa.eps = rms_eps;
  aa.kscale = ksc;
  aa.stats = reinterpret_cast<unsigned long long*>(io.softmax_stats);
  aa.lse = io.lse;
  aa.inplan = inplan ? 1 : 0;
  aa.B = B;
  aa.bm = p.bm;
  aa.self_check = pa.self_check;
  aa.total_q = io.total_q;
  aa.total_kv = io.total_kv;
  aa.status_out = io.status;
  const float inv_sqrt_d = 1.0f / std::sqrt(float(D));
  aa.score_scale = act == JA_SOFTMAX ? inv_sqrt_d * 1.4426950408889634f : inv_sqrt_d;

  // (the events are written by the attention kernel's own dispatch)
  const KTiming tm{reinterpret_cast<hipEvent_t>(io.ev_start), reinterpret_cast<hipEvent_t>(io.ev_stop)};
  hipError_t e;
  if (p.shape == kShapeF32) {
    // (a grid-stride loop over the items: capped like the persistent kernels)
    int64_t grid = std::min<int64_t>(p.ws.max_items > 0 ? p.ws.max_items : 1, kMaxGrid);
    if (cap > 0) grid = std::min(grid, std::max<int64_t>(kXcds, cap / kXcds * kXcds));
    e = launch_attn_f32(D, act, variant == JA_SLIDING ? 2 : (window > 0 ? 1 : 0), aa, int(grid), tm, stream);
  } else if (p.shape == kShapePingPong) {
    const int in = io.dtype == JA_BF16 ? IN_BF16 : IN_MX8;
    e = launch_attn_pp(D, act, variant == JA_CROSS, in, aa, num_cu, p.ws.max_items, cap, tm, stream);
  } else {
    const int in = io.dtype == JA_BF16 ? IN_BF16 : IN_MX;
    e = launch_attn_mfma(D, in, p.shape, act, aa, num_cu, p.ws.max_items, cap, tm, stream);
  }
  if (e != hipSuccess) return JA_EHIP;
  if (p.shape == kShapeKvSplit) {
    CombineArgs ca{};
    ca.out = out;
    ca.qo = q_offsets;
    ca.ko = kv_offsets;
    ca.hdr = hdr;
    ca.nsplit = nsplit;
    ca.pbase = pbase;
    ca.part_o = part_o;
    ca.part_ml = part_ml;
    ca.lse = io.lse;
    ca.B = B;
    ca.H = H;
    ca.act = act;
    if (launch_combine(D, ca, stream) != hipSuccess) return JA_EHIP;
  }
  return JA_OK;
}

namespace {

// Backward workspace: two plans of 64-row tiles (over the queries, and over
// the keys with the offsets swapped) and one (lse, D) pair per query row and head.
constexpr int kBwdRows = 64;        // rows per backward work item (VALU kernels, MFMA key side)
constexpr int kBwdRowsMfmaQ = 128;  // query rows per item of the MFMA dQ kernel (4 waves)
struct BwdLayout {
  size_t hdr_q, nsplit_q, pbase_q, items_q, hdr_k, nsplit_k, pbase_k, items_k, stats, rq, rk, total;
  int64_t max_q, max_k;
};

BwdLayout bwd_layout(int B, int H, int act, int32_t total_q, int32_t total_kv) {
  BwdLayout L{};
  L.max_q = int64_t(H) * (cdiv(total_q, kBwdRows) + B);
  L.max_k = int64_t(H) * (cdiv(total_kv, kBwdRows) + B);
  size_t off = 0;
  L.hdr_q = off;
  off = align256(off + sizeof(WsHeader));
  L.nsplit_q = off;
  off = align256(off + sizeof(int32_t) * size_t(B));
  L.pbase_q = off;
  off = align256(off + sizeof(int32_t) * size_t(B));
  L.items_q = off;
  off = align256(off + sizeof(WorkItem) * size_t(L.max_q));
  L.hdr_k = off;
  off = align256(off + sizeof(WsHeader));
  L.nsplit_k = off;
  off = align256(off + sizeof(int32_t) * size_t(B));
  L.pbase_k = off;
  off = align256(off + sizeof(int32_t) * size_t(B));
  L.items_k = off;
  off = align256(off + sizeof(WorkItem) * size_t(L.max_k));
  L.stats = off;
  off = align256(off + sizeof(float2) * size_t(total_q) * H);
  L.rq = L.rk = off;
  if (act != JA_SOFTMAX) {  // RMS factors of the query and key rows
    L.rq = off;
    off = align256(off + sizeof(float) * size_t(total_q) * H);
    L.rk = off;
    off = align256(off + sizeof(float) * size_t(total_kv) * H);
  }
  L.total = off;
  return L;
}

int validate_bwd(int B, int H, int D, int variant, int act, int window, int dtype, int32_t total_q,
                 int32_t total_kv) {
  const int st = validate(B, H, D, variant, act, window, dtype, total_q, total_kv);
  if (st != JA_OK) return st;
  if (act == JA_GELU_POLY || dtype == JA_MXFP8_E4M3) return JA_EUNSUPPORTED;
  return JA_OK;
}

}  // namespace
}  // namespace ja

namespace ja {

bool debug_sync() {
  // (a function-local static: initialised once, thread-safely)
  static const bool on = [] {
    const char* e = std::getenv("JA_DEBUG");
    return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
  }();
  return on;
}

int debug_status(hipStream_t stream, const void* st0, const void* st1) {
  if (hipStreamSynchronize(stream) != hipSuccess) return JA_EHIP;
  for (const void* p : {st0, st1}) {
    if (p == nullptr) continue;
    int32_t status = 0;
    if (hipMemcpy(&status, p, sizeof(status), hipMemcpyDeviceToHost) != hipSuccess) return JA_EHIP;
    if (status != JA_OK) return status;
  }
  return JA_OK;
}

}  // namespace ja

using namespace ja;

extern "C" {

int jagged_attn_version(void) { return 101; }

const char* jagged_attn_strerror(int status) {
  switch (status) {
    case JA_OK: return "ok";
    case JA_EINVAL: return "invalid argument";
    case JA_EUNSUPPORTED: return "unsupported argument combination";
    case JA_EWORKSPACE: return "workspace missing or too small";
    case JA_EHIP: return "HIP runtime error";
    case JA_EOFFSETS: return "invalid offsets (not starting at 0, decreasing, not ending at total, or self offsets differ)";
    default: return "unknown status";
  }
}

size_t jagged_attn_workspace_size(int B, int H, int D, int variant, int act, int window, int dtype,
                                  int32_t total_q, int32_t total_kv) {
  if (validate(B, H, D, variant, act, window, dtype, total_q, total_kv) != JA_OK) return 0;
  return make_plan(B, H, D, variant, act, window, dtype, total_q, total_kv).ws.total;
}

int jagged_attn_fwd(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                    const int32_t* kv_offsets, int B, int H, int D, int variant, int act, int window,
                    void* out, const ja_io* io) {
  if (io == nullptr) return JA_EINVAL;
  const int st = fwd_impl(q, k, v, q_offsets, kv_offsets, B, H, D, variant, act, window, out, *io, io->workspace,
                          io->workspace_bytes);
  if (st != JA_OK || !debug_sync()) return st;
  // (the workspace starts with the plan header, whose first word is the status)
  return debug_status(reinterpret_cast<hipStream_t>(io->stream), io->workspace, nullptr);
}

size_t jagged_attn_bwd_workspace_size(int B, int H, int D, int variant, int act, int window, int dtype,
                                      int32_t total_q, int32_t total_kv) {
  if (validate_bwd(B, H, D, variant, act, window, dtype, total_q, total_kv) != JA_OK) return 0;
  return bwd_layout(B, H, act, total_q, total_kv).total;
}

int jagged_attn_bwd(const void* q, const void* k, const void* v, const void* dout, const int32_t* q_offsets,
                    const int32_t* kv_offsets, int B, int H, int D, int variant, int act, int window, float* dq,
                    float* dk, float* dv, const ja_io* io) {
  if (io == nullptr) return JA_EINVAL;
  const int st = validate_bwd(B, H, D, variant, act, window, io->dtype, io->total_q, io->total_kv);
  if (st != JA_OK) return st;
  if (!q_offsets || !kv_offsets) return JA_EINVAL;
  // Empty tensors may come with null data pointers, as in the forward: no
  // kernel touches q, dout, dq without query rows, nor k, v, dk, dv without
  // key rows.
  if ((io->total_q > 0 && (!q || !dout || !dq)) || (io->total_kv > 0 && (!k || !v || !dk || !dv)))
    return JA_EINVAL;
  const BwdLayout L = bwd_layout(B, H, act, io->total_q, io->total_kv);
  if (io->workspace == nullptr || io->workspace_bytes < L.total) return JA_EWORKSPACE;
  for (const void* p : {q, k, v, dout, static_cast<const void*>(dq), static_cast<const void*>(dk),
                        static_cast<const void*>(dv), static_cast<const void*>(io->workspace)})
    if (!aligned16(p)) return JA_EINVAL;
  if (reinterpret_cast<uintptr_t>(io->status) & 3) return JA_EINVAL;
  // the forward's log-sum-exp and output: both or neither, softmax only
  if ((io->lse != nullptr) != (io->fwd_out != nullptr)) return JA_EINVAL;
  if (io->lse != nullptr &&
      (act != JA_SOFTMAX || (reinterpret_cast<uintptr_t>(io->lse) & 3) || !aligned16(io->fwd_out)))
    return JA_EINVAL;

  hipStream_t stream = reinterpret_cast<hipStream_t>(io->stream);
  unsigned char* ws = reinterpret_cast<unsigned char*>(io->workspace);
  const bool self = variant == JA_SELF || variant == JA_SLIDING;
  // bf16 inputs on the matrix cores; fp32 inputs on the fp32 VALU kernels
  const bool mfma = io->dtype == JA_BF16;
  const int wmode = variant == JA_SLIDING ? 2 : (variant == JA_SELF && window > 0 ? 1 : 0);
  // Two plans, in one launch: over query tiles, and over key tiles (the same
  // plan on swapped offsets).
  PlanArgs plans[2];
  for (int pass = 0; pass < 2; ++pass) {
    PlanArgs& pa = plans[pass];
    pa = PlanArgs{};
    pa.qo = pass == 0 ? q_offsets : kv_offsets;
    pa.ko = pass == 0 ? kv_offsets : q_offsets;
    pa.B = B;
    pa.H = H;
    pa.total_q = pass == 0 ? io->total_q : io->total_kv;
    pa.total_kv = pass == 0 ? io->total_kv : io->total_q;
    pa.bm = mfma && pass == 0 ? kBwdRowsMfmaQ : kBwdRows;
    pa.kvc = 0;
    pa.self_check = self;
    pa.max_items = pass == 0 ? L.max_q : L.max_k;
    pa.max_slots = 0;
    pa.hdr = reinterpret_cast<WsHeader*>(ws + (pass == 0 ? L.hdr_q : L.hdr_k));
    pa.status_out = io->status;  // (both plans check the same offsets)
    pa.nsplit = reinterpret_cast<int32_t*>(ws + (pass == 0 ? L.nsplit_q : L.nsplit_k));
    pa.pbase = reinterpret_cast<int32_t*>(ws + (pass == 0 ? L.pbase_q : L.pbase_k));
    pa.items = reinterpret_cast<WorkItem*>(ws + (pass == 0 ? L.items_q : L.items_k));
  }
  if (launch_plan_pair(plans[0], plans[1], stream) != hipSuccess) return JA_EHIP;
  BwdArgs ba{};
  ba.q = q;
  ba.k = k;
  ba.v = v;
  ba.dout = dout;
  ba.dq = dq;
  ba.dk = dk;
  ba.dv = dv;
  ba.hdr_q = reinterpret_cast<const WsHeader*>(ws + L.hdr_q);
  ba.items_q = reinterpret_cast<const WorkItem*>(ws + L.items_q);
  ba.hdr_k = reinterpret_cast<const WsHeader*>(ws + L.hdr_k);
  ba.items_k = reinterpret_cast<const WorkItem*>(ws + L.items_k);
  ba.stats = reinterpret_cast<float2*>(ws + L.stats);
  ba.lse_in = io->lse;
  ba.o_in = io->fwd_out;
  ba.rq = reinterpret_cast<float*>(ws + L.rq);
  ba.rk = reinterpret_cast<float*>(ws + L.rk);
  ba.eps = io->rms_eps > 0.f ? io->rms_eps : 1e-6f;
  ba.H = H;
  ba.window_blocks = variant == JA_SELF ? window / kBlock : 0;
  ba.window_tokens = variant == JA_SLIDING ? window : 0;
  const float inv_sqrt_d = 1.0f / std::sqrt(float(D));
  ba.inv_sqrt_d = inv_sqrt_d;
  ba.c2 = inv_sqrt_d * 1.4426950408889634f;
  const int grid_q = int(std::min<int64_t>(L.max_q > 0 ? L.max_q : 1, kMaxGrid));
  const int grid_k = int(std::min<int64_t>(L.max_k > 0 ? L.max_k : 1, kMaxGrid));
  if (io->ev_start && hipEventRecord(reinterpret_cast<hipEvent_t>(io->ev_start), stream) != hipSuccess)
    return JA_EHIP;
  if (mfma && act != JA_SOFTMAX &&
      launch_bwd_rms(D, true, ba, int64_t(io->total_q) * H, int64_t(io->total_kv) * H, stream) != hipSuccess)
    return JA_EHIP;
  const hipError_t e = mfma ? launch_attn_bwd_mfma(D, act == JA_SOFTMAX ? ACT_SOFTMAX : ACT_GELU, wmode, ba,
                                                   grid_q, grid_k, stream)
                           : launch_attn_bwd(D, io->dtype == JA_BF16, act == JA_SOFTMAX ? ACT_SOFTMAX : ACT_GELU,
                                             wmode, ba, int64_t(io->total_q) * H, int64_t(io->total_kv) * H, grid_q,
                                             grid_k, stream);
  if (e != hipSuccess) return JA_EHIP;
  if (io->ev_stop && hipEventRecord(reinterpret_cast<hipEvent_t>(io->ev_stop), stream) != hipSuccess)
    return JA_EHIP;
  if (debug_sync()) return debug_status(stream, ws + L.hdr_q, ws + L.hdr_k);
  return JA_OK;
}

int jagged_attn_mx_quantize(const void* x, int dtype, int64_t rows, int D, uint8_t* codes, uint8_t* scales,
                            void* stream) {
  if (dtype != JA_F32 && dtype != JA_BF16) return JA_EINVAL;
  if (rows < 0 || D <= 0 || D % kMxBlock != 0) return JA_EINVAL;
  // (no rows: nothing to do, and empty tensors may come with null pointers)
  if (rows > 0 && (x == nullptr || codes == nullptr || scales == nullptr)) return JA_EINVAL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return JA_EINVAL;
  if (rows > (int64_t(1) << 40) / D) return JA_EINVAL;  // (keeps the grid in range)
  if (rows == 0) return JA_OK;
  const int64_t n_blocks = rows * (D / kMxBlock);
  if (launch_mx_quant(dtype == JA_BF16, x, n_blocks, codes, scales, reinterpret_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return JA_EHIP;
  if (debug_sync()) return debug_status(reinterpret_cast<hipStream_t>(stream), nullptr, nullptr);
  return JA_OK;
}

int jagged_attn_check(const void* workspace, void* stream) {
  if (workspace == nullptr) return JA_EINVAL;
  if (hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return JA_EHIP;
  int32_t status = 0;
  if (hipMemcpy(&status, workspace, sizeof(status), hipMemcpyDeviceToHost) != hipSuccess) return JA_EHIP;
  return status;
}

}  // extern "C"
