// Cost model of the work items, shared by the plan kernel (ja_plan.hip) and
// the tile stream's own enumeration of its items (ja_attn_pp.hip): an item's
// cost is the number of 64-key tiles it walks, and the items are placed most
// costly first so that dealing them out in rounds balances skewed lengths
// (techfeed.io summary of "GEM Training: How Meta Doubled the Efficiency of
// Its LLM-Scale Ads Foundation Model", section "Generalized Dot-Product
// Attention（GDPA）": only valid tiles are scheduled and skew is balanced).
// A is any argument struct with bm (query rows per item), window_blocks and
// window_tokens.
#pragma once

#include "ja_internal.h"

namespace ja {

constexpr int kCostBuckets = 1024;  // bucket = key tiles walked, clamped

// Cost bucket of query tile qt of a sample: the key tiles the tile-stream
// kernel walks for that item (all of the sample's, or with a window those from
// the first one a query of the item sees to the item's last query block).
template <typename A>
__device__ inline int cost_bucket(const A& a, int qt, int lq, int lk) {
  int te = (lk + kBlock - 1) / kBlock, tl = 0;
  if (a.window_blocks > 0 || a.window_tokens > 0) {
    const int q0 = qt * a.bm;
    te = min(te, (min(q0 + a.bm, lq) + kBlock - 1) / kBlock);
    tl = a.window_blocks > 0 ? max(0, q0 / kBlock - a.window_blocks + 1) : max(0, q0 - a.window_tokens + 1) / kBlock;
  }
  return min(max(te - tl, 0), kCostBuckets - 1);
}

// Length of the run of query tiles from qt on that share qt's cost bucket,
// found without visiting them one by one: without a window every item walks
// the same tiles; with one, the full items past the window's clamp at the
// sample's first key walk the same number, and the first and last items are
// runs of their own.  A sample thus has at most qt_mid + 2 runs.
template <typename A>
__device__ inline int cost_run(const A& a, int qt, int nqt) {
  if (a.window_blocks <= 0 && a.window_tokens <= 0) return nqt - qt;
  const int span = a.window_blocks > 0 ? (a.window_blocks - 1) * kBlock : a.window_tokens - 1;
  const int qt_mid = (span + a.bm - 1) / a.bm;  // first query tile whose window is unclamped
  return (qt >= qt_mid && qt < nqt - 1) ? nqt - 1 - qt : 1;
}

}  // namespace ja
