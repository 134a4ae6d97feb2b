// Device-side work enumeration for jagged attention.
//
// The pages describe a GDPA tile scheduler that precomputes the valid tiles on
// the CPU, skips empty ones and balances skewed work across SMs (techfeed.io
// summary of "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale
// Ads Foundation Model", section "Generalized Dot-Product Attention（GDPA）").
// Here the enumeration runs on the GPU, on the caller's stream, so the host
// never reads the offsets.  One workgroup:
//  1. validates the offsets and sums the estimated cost of every sample;
//  2. writes the work items (zero-length samples produce none), head-major
//     within a sample so items that share K/V are adjacent, and
//  3. cuts the item list into 8 contiguous ranges of equal estimated cost, one
//     per XCD: an XCD's workgroups then share K/V through its own L2, and the
//     XCDs finish together despite skewed lengths.
// In cost order (the tile-stream kernel) step 2 instead places the items by a
// counting sort on their key tiles, most first, so that dealing them out in
// rounds gives every workgroup about the same number of tile steps; the items
// of one (sample, head) stay adjacent.
#include "ja_internal.h"
#include "ja_sched.h"
#include "jagged_attn.h"

namespace ja {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
static_assert(kCostBuckets == kPlanThreads, "one cost bucket per plan thread");

// Cost bucket of a key-split item of `keys` keys (one query tile): its key tiles.
__device__ inline int split_bucket(int keys) { return min((keys + kBlock - 1) / kBlock, kCostBuckets - 1); }

template <typename T>
__device__ inline T wave_inclusive_scan(T x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    T y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive scan of one value per thread over the 1024-thread block; returns
// the thread's exclusive prefix and the block total.
template <typename T>
__device__ T block_exclusive_scan(T x, T* s_warp, T* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const T inc = wave_inclusive_scan(x);
  if (lane == 63) s_warp[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const T w = lane < kPlanWaves ? s_warp[lane] : T(0);
    const T wi = wave_inclusive_scan(w);
    if (lane < kPlanWaves) s_warp[kPlanWaves + lane] = wi - w;
    if (lane == kPlanWaves - 1) s_warp[2 * kPlanWaves] = wi;
  }
  __syncthreads();
  const T r = inc - x + s_warp[kPlanWaves + wave];
  *total = s_warp[2 * kPlanWaves];
  __syncthreads();
  return r;
}

struct SampleWork {
  int cnt;      // work items
  int ns;       // key splits
  int nqt;      // query tiles
  int slots;    // partial slots
  double ck;    // estimated cost of one item (keys it touches + fixed overhead)
};

// Three running sums scanned together (one set of barriers): estimated cost,
// items and partial slots (integer sums in doubles are exact below 2^53).
struct Sums {
  double cost, items, slots;
};

__device__ inline Sums wave_inclusive_scan3(Sums x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double c = __shfl_up(x.cost, o, 64), i = __shfl_up(x.items, o, 64), s = __shfl_up(x.slots, o, 64);
    if (lane >= o) {
      x.cost += c;
      x.items += i;
      x.slots += s;
    }
  }
  return x;
}

// Exclusive scan of one Sums per thread over the block; returns the thread's
// exclusive prefix and the block total.
__device__ Sums block_exclusive_scan3(Sums x, Sums* s_warp, Sums* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const Sums inc = wave_inclusive_scan3(x);
  if (lane == 63) s_warp[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const Sums w = lane < kPlanWaves ? s_warp[lane] : Sums{0.0, 0.0, 0.0};
    const Sums wi = wave_inclusive_scan3(w);
    if (lane < kPlanWaves) s_warp[kPlanWaves + lane] = Sums{wi.cost - w.cost, wi.items - w.items, wi.slots - w.slots};
    if (lane == kPlanWaves - 1) s_warp[2 * kPlanWaves] = wi;
  }
  __syncthreads();
  const Sums base = s_warp[kPlanWaves + wave];
  *total = s_warp[2 * kPlanWaves];
  __syncthreads();
  return Sums{inc.cost - x.cost + base.cost, inc.items - x.items + base.items, inc.slots - x.slots + base.slots};
}

__device__ inline SampleWork sample_work(const PlanArgs& a, int lq, int lk) {
  SampleWork w{0, 1, 0, 0, 0.0};
  if (lq <= 0) return w;
  w.nqt = (lq + a.bm - 1) / a.bm;
  if (a.kvc > 0 && w.nqt == 1 && lk > a.kvc) w.ns = (lk + a.kvc - 1) / a.kvc;
  w.cnt = a.H * w.nqt * w.ns;
  w.slots = w.ns > 1 ? a.H * w.ns : 0;
  int keys = lk;
  if (w.ns > 1) keys = a.kvc;
  if (a.window_blocks > 0) keys = min(lk, a.window_blocks * kBlock);
  if (a.window_tokens > 0) keys = min(lk, a.window_tokens + a.bm - 1);
  w.ck = double(keys) + 64.0;
  return w;
}

// The header's item-list offset and status word (also copied to the caller's
// status word when one is given).
__device__ inline void set_status(const PlanArgs& a, int status) {
  a.hdr->items_off = int32_t(reinterpret_cast<const char*>(a.items) - reinterpret_cast<const char*>(a.hdr));
  a.hdr->status = status;
  if (a.status_out) *a.status_out = status;
}

__device__ inline void fail(const PlanArgs& a, int status) {
  set_status(a, status);
  a.hdr->n_items = 0;
  a.hdr->n_slots = 0;
  for (int x = 0; x <= kXcds; ++x) a.hdr->xcd_begin[x] = 0;
}

}  // namespace

// RMS factor of key row r (QK-RMSNorm of the keys as a per-key scale of the
// GELU scores: techfeed.io summary, GDPA section).  One thread per row.
template <int D>
__device__ void key_rms_row(const PlanArgs& a, int64_t r) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  const bf16x8* p = reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(a.krms_k) + r * D);
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const bf16x8 x = p[c];
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(float(x[j]), float(x[j]), ss);
  }
  a.krms_out[r] = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.krms_eps);
}

// One plan, by one workgroup.
__device__ __forceinline__ void plan_main(const PlanArgs& a) {
  __shared__ int s_bad;
  __shared__ int s_iwarp[3 * kPlanWaves];
  __shared__ Sums s_swarp[2 * kPlanWaves + 1];
  __shared__ int s_bucket[kCostBuckets];  // cost order: item count, then next free position
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_bad = 0;
  }
  for (int i = tid; i < kCostBuckets; i += kPlanThreads) s_bucket[i] = 0;
  __syncthreads();

  // Pass 1: validate; total items, partial slots and estimated cost.
  // Offsets start at 0, never decrease and end at the totals; self-attention
  // needs identical query and key offsets.  With at most one sample per
  // thread (B <= kPlanThreads) the sample and its scan prefix are kept for
  // pass 2.
  int bad = 0;
  Sums mine{0.0, 0.0, 0.0};
  SampleWork w0{0, 1, 0, 0, 0.0};
  int qb0 = 0, lq0 = 0, kb0 = 0, lk0 = 0;
  for (int b = tid; b <= a.B; b += kPlanThreads) {
    const int q = a.qo[b], k = a.ko[b];
    if (b == 0 && (q != 0 || k != 0)) bad = 1;
    if (b == a.B && (q != a.total_q || k != a.total_kv)) bad = 1;
    if (a.self_check && q != k) bad = 1;
    if (b < a.B) {
      const int q1 = a.qo[b + 1], k1 = a.ko[b + 1];
      if (q1 < q || k1 < k) bad = 1;
      const SampleWork w = sample_work(a, q1 - q, k1 - k);
      mine.cost += w.cnt * w.ck;
      mine.items += w.cnt;
      mine.slots += w.slots;
      if (a.cost_order && w.cnt > 0 && w.ns > 1) {
        // key splits (one query tile): ns - 1 chunks of kvc keys, then the rest
        atomicAdd(&s_bucket[split_bucket(a.kvc)], (w.ns - 1) * a.H);
        atomicAdd(&s_bucket[split_bucket(k1 - k - (w.ns - 1) * a.kvc)], a.H);
      } else if (a.cost_order && w.cnt > 0)
        for (int qt = 0; qt < w.nqt;) {
          const int run = cost_run(a, qt, w.nqt);
          atomicAdd(&s_bucket[cost_bucket(a, qt, q1 - q, k1 - k)], run * a.H * w.ns);
          qt += run;
        }
      if (b == tid) {
        w0 = w;
        qb0 = q;
        lq0 = q1 - q;
        kb0 = k;
        lk0 = k1 - k;
      }
    }
  }
  if (bad) atomicOr(&s_bad, 1);
  Sums total;
  const Sums prefix = block_exclusive_scan3(mine, s_swarp, &total);
  const double total_cost = total.cost;
  const long long total_items_ll = (long long)total.items, total_slots_ll = (long long)total.slots;
  if (s_bad || total_items_ll > a.max_items || total_slots_ll > a.max_slots) {
    if (tid == 0) fail(a, JA_EOFFSETS);
    return;
  }
  if (a.cost_order) {
    // first position of every bucket, the bucket with the most key tiles first
    // (each thread reads and writes only its own bucket)
    static_assert(kCostBuckets == kPlanThreads, "one bucket per thread");
    const int bk = kCostBuckets - 1 - tid;
    int unused;
    s_bucket[bk] = block_exclusive_scan(s_bucket[bk], s_iwarp, &unused);
    __syncthreads();
  }

  // Pass 2: per chunk of kPlanThreads samples, write items, splits, slot
  // bases and the XCD cut points.
  __shared__ int s_base[kPlanThreads];
  __shared__ int s_nqt[kPlanThreads];
  __shared__ int s_ns[kPlanThreads];
  __shared__ int s_qb[kPlanThreads], s_lq[kPlanThreads], s_kb[kPlanThreads], s_lk[kPlanThreads];
  int item_carry = 0, slot_carry = 0;
  double cost_carry = 0.0;
  for (int base = 0; base < a.B; base += kPlanThreads) {
    const int b = base + tid;
    SampleWork w = w0;
    int qb = qb0, lq = lq0, kb = kb0, lk = lk0;
    Sums pre = prefix, chunk = total;
    if (base > 0 || a.B > kPlanThreads) {  // more than one chunk: reload and rescan
      w = SampleWork{0, 1, 0, 0, 0.0};
      qb = lq = kb = lk = 0;
      if (b < a.B) {
        qb = a.qo[b];
        lq = a.qo[b + 1] - qb;
        kb = a.ko[b];
        lk = a.ko[b + 1] - kb;
        w = sample_work(a, lq, lk);
      }
      pre = block_exclusive_scan3(Sums{w.cnt * w.ck, double(w.cnt), double(w.slots)}, s_swarp, &chunk);
    }
    const int ibase = int(pre.items) + item_carry;
    const int sbase = int(pre.slots) + slot_carry;
    const double cbase = pre.cost + cost_carry;
    if (b < a.B) {
      a.nsplit[b] = w.ns;
      a.pbase[b] = sbase;
      // XCD x starts at the item holding cost x/8 of the total.
      for (int x = 1; x < kXcds; ++x) {
        const double target = total_cost * x / kXcds;
        if (w.cnt > 0 && target >= cbase && target < cbase + w.cnt * w.ck) {
          const int k = min(w.cnt - 1, int((target - cbase) / w.ck));
          a.hdr->xcd_begin[x] = ibase + k;
        }
      }
    }
    s_base[tid] = ibase;
    s_nqt[tid] = w.nqt;
    s_ns[tid] = w.ns;
    s_qb[tid] = qb;
    s_lq[tid] = lq;
    s_kb[tid] = kb;
    s_lk[tid] = lk;
    __syncthreads();
    // One thread per (sample, head) writes that head's items (query tile, then
    // split), so no thread divides per item.  Item order within a sample is
    // head-major: items that share K/V stay adjacent.
    const int nchunk = min(kPlanThreads, a.B - base);
    for (int p = tid; p < nchunk * a.H; p += kPlanThreads) {
      const int j = p / a.H, h = p - j * a.H;
      const int nq = s_nqt[j], nsj = s_ns[j];
      const int qbj = s_qb[j], lqj = s_lq[j], kbj = s_kb[j], lkj = s_lk[j];
      if (nq == 0) continue;
      if (a.cost_order && nsj > 1) {
        // key splits of the sample's one query tile: the full chunks, then the rest
        int ib = atomicAdd(&s_bucket[split_bucket(a.kvc)], nsj - 1);
        for (int sp = 0; sp < nsj - 1; ++sp) a.items[ib++] = WorkItem{base + j, h, 0, sp, qbj, lqj, kbj, lkj};
        ib = atomicAdd(&s_bucket[split_bucket(lkj - (nsj - 1) * a.kvc)], 1);
        a.items[ib] = WorkItem{base + j, h, 0, nsj - 1, qbj, lqj, kbj, lkj};
      } else if (a.cost_order) {
        // each run of equal cost takes consecutive places in its bucket
        for (int qt0 = 0; qt0 < nq;) {
          const int run = cost_run(a, qt0, nq);
          int ib = atomicAdd(&s_bucket[cost_bucket(a, qt0, lqj, lkj)], run * nsj);
          for (int qt = qt0; qt < qt0 + run; ++qt)
            for (int sp = 0; sp < nsj; ++sp) a.items[ib++] = WorkItem{base + j, h, qt * a.bm, sp, qbj, lqj, kbj, lkj};
          qt0 += run;
        }
      } else {
        int ib = s_base[j] + h * nq * nsj;
        for (int qt = 0; qt < nq; ++qt)
          for (int sp = 0; sp < nsj; ++sp) a.items[ib++] = WorkItem{base + j, h, qt * a.bm, sp, qbj, lqj, kbj, lkj};
      }
    }
    item_carry += int(chunk.items);
    slot_carry += int(chunk.slots);
    cost_carry += chunk.cost;
    __syncthreads();
  }
  if (tid == 0) {
    set_status(a, JA_OK);
    a.hdr->n_items = item_carry;
    a.hdr->n_slots = slot_carry;
    a.hdr->xcd_begin[0] = 0;
    a.hdr->xcd_begin[kXcds] = item_carry;
    if (total_cost <= 0.0)
      for (int x = 1; x < kXcds; ++x) a.hdr->xcd_begin[x] = 0;
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  if (blockIdx.x > 0) {
    // the key RMS side job: rows (blockIdx.x - 1) * kPlanThreads + tid
    const int64_t r = int64_t(blockIdx.x - 1) * kPlanThreads + threadIdx.x;
    if (r < a.krms_rows) {
      if (a.krms_d == 32) key_rms_row<32>(a, r);
      else if (a.krms_d == 64) key_rms_row<64>(a, r);
      else key_rms_row<128>(a, r);
    }
    return;
  }
  plan_main(a);
}

// Two independent plans in one launch (the backward's plans over query tiles
// and over key tiles): workgroup 0 takes the first, workgroup 1 the second.
__global__ __launch_bounds__(kPlanThreads) void plan_pair_kernel(PlanArgs a, PlanArgs b) {
  plan_main(blockIdx.x == 0 ? a : b);
}

hipError_t launch_plan_pair(const PlanArgs& a, const PlanArgs& b, hipStream_t st) {
  if (a.krms_rows > 0 || b.krms_rows > 0) return hipErrorInvalidValue;  // (no side job here)
  hipLaunchKernelGGL(plan_pair_kernel, dim3(2), dim3(kPlanThreads), 0, st, a, b);
  return hipGetLastError();
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t st) {
  const int64_t side = a.krms_rows > 0 ? (a.krms_rows + kPlanThreads - 1) / kPlanThreads : 0;
  hipLaunchKernelGGL(plan_kernel, dim3(unsigned(1 + side)), dim3(kPlanThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ja
