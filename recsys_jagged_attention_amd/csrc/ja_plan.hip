// Device-side work enumeration for jagged attention.
//
// The pages describe a GDPA tile scheduler that precomputes the valid tiles on
// the CPU, skips empty ones and balances skewed work across SMs (techfeed.io
// summary of "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale
// Ads Foundation Model", section "Generalized Dot-Product Attention（GDPA）").
// Here the enumeration runs on the GPU, on the caller's stream, so the host
// never reads the offsets: one workgroup validates the offsets, counts the
// work items of every sample (zero-length samples produce none), scans the
// counts and writes the item list the attention kernel walks.
#include "ja_internal.h"
#include "jagged_attn.h"

namespace ja {

namespace {

constexpr int kPlanThreads = 1024;

__device__ inline int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive scan of one value per thread over the whole 1024-thread block;
// returns the exclusive prefix and writes the block total to *total.
__device__ int block_exclusive_scan(int x, int* s_warp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = wave_inclusive_scan(x);
  if (lane == 63) s_warp[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kPlanThreads / 64 ? s_warp[lane] : 0;
    int wi = wave_inclusive_scan(w);
    if (lane < kPlanThreads / 64) s_warp[16 + lane] = wi - w;
    if (lane == kPlanThreads / 64 - 1) s_warp[32] = wi;
  }
  __syncthreads();
  int r = inc - x + s_warp[16 + wave];
  *total = s_warp[32];
  __syncthreads();
  return r;
}

}  // namespace

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int s_bad;
  __shared__ int s_warp[48];
  __shared__ int s_cnt[kPlanThreads];
  __shared__ int s_base[kPlanThreads];
  __shared__ int s_nqt[kPlanThreads];
  __shared__ int s_ns[kPlanThreads];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_bad = 0;
  __syncthreads();

  // 1. Validate: offsets start at 0, never decrease, end at the totals;
  //    self-attention needs identical query and key offsets.
  int bad = 0;
  for (int b = tid; b <= a.B; b += kPlanThreads) {
    const int q = a.qo[b], k = a.ko[b];
    if (b == 0 && (q != 0 || k != 0)) bad = 1;
    if (b == a.B && (q != a.total_q || k != a.total_kv)) bad = 1;
    if (b < a.B && (a.qo[b + 1] < q || a.ko[b + 1] < k)) bad = 1;
    if (a.self_check && q != k) bad = 1;
  }
  if (bad) atomicOr(&s_bad, 1);
  __syncthreads();
  if (s_bad) {
    if (tid == 0) {
      a.hdr->status = JA_EOFFSETS;
      a.hdr->n_items = 0;
      a.hdr->n_slots = 0;
    }
    return;
  }

  // 2./3. Per chunk of 1024 samples: count, scan, write the items.
  int64_t item_carry = 0, slot_carry = 0;
  for (int base = 0; base < a.B; base += kPlanThreads) {
    const int b = base + tid;
    int cnt = 0, ns = 1, nqt = 0, slots = 0;
    if (b < a.B) {
      const int lq = a.qo[b + 1] - a.qo[b];
      const int lk = a.ko[b + 1] - a.ko[b];
      if (lq > 0) {
        nqt = (lq + a.bm - 1) / a.bm;
        if (a.kvc > 0 && nqt == 1 && lk > a.kvc) ns = (lk + a.kvc - 1) / a.kvc;
        cnt = a.H * nqt * ns;
        slots = ns > 1 ? a.H * ns : 0;
      }
    }
    int items_total, slots_total;
    const int ibase = block_exclusive_scan(cnt, s_warp, &items_total);
    const int sbase = block_exclusive_scan(slots, s_warp, &slots_total);
    if (item_carry + items_total > a.max_items || slot_carry + slots_total > a.max_slots) {
      if (tid == 0) {
        a.hdr->status = JA_EOFFSETS;
        a.hdr->n_items = 0;
        a.hdr->n_slots = 0;
      }
      return;
    }
    if (b < a.B) {
      a.nsplit[b] = ns;
      a.pbase[b] = int(slot_carry) + sbase;
    }
    s_cnt[tid] = cnt;
    s_base[tid] = int(item_carry) + ibase;
    s_nqt[tid] = nqt;
    s_ns[tid] = ns;
    __syncthreads();
    // One wave per sample; its lanes write the sample's items (head-major,
    // then query tile, then key split) so items sharing K/V stay adjacent.
    const int nchunk = min(kPlanThreads, a.B - base);
    for (int j = wave; j < nchunk; j += kPlanThreads / 64) {
      const int c = s_cnt[j], ib = s_base[j], nq = s_nqt[j], nsj = s_ns[j];
      for (int t = lane; t < c; t += 64) {
        const int s = t % nsj;
        const int qt = (t / nsj) % nq;
        const int h = t / (nsj * nq);
        a.items[ib + t] = make_int4(base + j, h, qt * a.bm, s);
      }
    }
    item_carry += items_total;
    slot_carry += slots_total;
    __syncthreads();
  }
  if (tid == 0) {
    a.hdr->status = JA_OK;
    a.hdr->n_items = int(item_carry);
    a.hdr->n_slots = int(slot_carry);
  }
}

}  // namespace ja

namespace ja {
hipError_t launch_plan(const PlanArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}
}  // namespace ja
