// jagged_attn_fwd without a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops and
// harnesses that forbid allocation).  The workspace -- plan header, work
// items, key-split partials, GELU key scales -- lives in a file-scope device
// array instead; each GPU the library runs on holds its own copy of it until
// the process ends.
//
// In host code the array's name is only a host-side stand-in: its device
// address on the current GPU is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// ever passed to kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "ja_internal.h"
#include "jagged_attn.h"

namespace ja {

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // the most any call may use
constexpr int kMaxScratchDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (looked up on the
// device's first call; later calls read the cached address).
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return JA_EHIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return JA_EUNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return JA_EHIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return JA_OK;
}

}  // namespace

}  // namespace ja

extern "C" int jagged_attn_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                                       const int32_t* kv_offsets, int B, int H, int D, int variant, int act,
                                       int window, void* out, const ja_io* io) {
  if (io == nullptr) return JA_EINVAL;
  if (io->workspace != nullptr || io->workspace_bytes != 0) return JA_EINVAL;
  const size_t need =
      jagged_attn_workspace_size(B, H, D, variant, act, window, io->dtype, io->total_q, io->total_kv);
  if (need == 0)  // invalid arguments: let the validation report which (no workspace is touched)
    return ja::fwd_impl(q, k, v, q_offsets, kv_offsets, B, H, D, variant, act, window, out, *io, nullptr, 0);
  if (need > ja::kScratchBytes) return JA_EWORKSPACE;
  void* ws = nullptr;
  const int st = ja::scratch_on_current_device(&ws);
  if (st != JA_OK) return st;
  // Nothing in the workspace needs to start at zero: the plan kernel writes
  // the header, the items and the split table of this call before any other
  // kernel reads them, and partials are written before they are merged.
  const int fst = ja::fwd_impl(q, k, v, q_offsets, kv_offsets, B, H, D, variant, act, window, out, *io, ws,
                               ja::kScratchBytes);
  if (fst != JA_OK || !ja::debug_sync()) return fst;
  return ja::debug_status(reinterpret_cast<hipStream_t>(io->stream), ws, nullptr);
}
