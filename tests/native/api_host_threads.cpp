// Host-side stress test of the C ABI's argument validation, workspace sizing,
// per-device CU cache and launch sequencing, built with g++ under a sanitizer
// (ThreadSanitizer, or AddressSanitizer + UBSan) by tests/test_host_sanitizers.py.
//
// ja_api.cpp is compiled as plain host code and linked against the stubs
// below instead of the HIP runtime and the kernel files: hipGetDevice reports
// a per-thread device id (including one past the library's cache of 64 ids),
// hipDeviceGetAttribute a CU count derived from that id, and every launch stub
// checks that it received that device's CU count.  Nothing here touches a GPU.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "ja_internal.h"
#include "jagged_attn.h"

namespace {
thread_local int t_device = 0;
std::atomic<long> g_launches{0};
std::atomic<int> g_errors{0};

int cus_of(int dev) { return 200 + dev; }

void expect_cus(int num_cu) {
  if (num_cu != cus_of(t_device)) {
    std::fprintf(stderr, "device %d: launch saw %d CUs, expected %d\n", t_device, num_cu, cus_of(t_device));
    g_errors.fetch_add(1);
  }
  g_launches.fetch_add(1, std::memory_order_relaxed);
}
}  // namespace

// ---- HIP runtime stubs (the functions ja_api.cpp calls) --------------------
extern "C" {
hipError_t hipGetDevice(int* dev) {
  *dev = t_device;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int dev) {
  if (attr != hipDeviceAttributeMultiprocessorCount) return hipErrorInvalidValue;
  *v = cus_of(dev);
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipMemcpy(void* dst, const void*, size_t n, hipMemcpyKind) {
  std::memset(dst, 0, n);  // (a status word of JA_OK)
  return hipSuccess;
}
}

// ---- kernel launcher stubs --------------------------------------------------
namespace ja {
int pp_rows() { return 256; }
int pp_pipe_rows() { return 1024; }
int pp_pipe_max_blocks() { return 4; }
int pp_item_cache() { return 256; }
int pp_enum_max_runs() { return 4; }
int pp_enum_max_offsets() { return 512; }
hipError_t launch_plan(const PlanArgs& a, hipStream_t) {
  if (!a.hdr || !a.items || a.max_items < 0) g_errors.fetch_add(1);
  return hipSuccess;
}
hipError_t launch_plan_pair(const PlanArgs& a, const PlanArgs& b, hipStream_t st) {
  launch_plan(a, st);
  return launch_plan(b, st);
}
hipError_t launch_attn_mfma(int, int, int, int, const AttnArgs&, int num_cu, int64_t, int64_t, const KTiming&,
                            hipStream_t) {
  expect_cus(num_cu);
  return hipSuccess;
}
bool pp_takes_mx8(int D, int act, bool self, int window_blocks) {
  return D == 128 && act == 0 && self && window_blocks <= 4;
}
hipError_t launch_attn_pp(int, int, bool, int, const AttnArgs&, int num_cu, int64_t, int64_t, const KTiming&,
                          hipStream_t) {
  expect_cus(num_cu);
  return hipSuccess;
}
hipError_t launch_attn_f32(int, int, int, const AttnArgs&, int grid, const KTiming&, hipStream_t) {
  if (grid < 1) g_errors.fetch_add(1);
  g_launches.fetch_add(1, std::memory_order_relaxed);
  return hipSuccess;
}
hipError_t launch_combine(int, const CombineArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_attn_bwd(int, bool, int, int, const BwdArgs&, int64_t, int64_t, int, int, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_attn_bwd_mfma(int, int, int, const BwdArgs&, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_rms(int, bool, const BwdArgs&, int64_t, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_mx_quant(bool, const void*, int64_t, uint8_t*, uint8_t*, hipStream_t) { return hipSuccess; }
}  // namespace ja

namespace {
// One thread's share: argument errors, sizes and whole forward calls on its device.
void worker(int tid, int iters, unsigned char* ws, size_t ws_bytes) {
  t_device = (tid % 4 == 3) ? 70 : tid % 4;  // ids 0..2 are cached, 70 is past the cache
  const uintptr_t dev_ptr = 4096;            // never dereferenced: the launches are stubs
  const void* p = reinterpret_cast<const void*>(dev_ptr);
  const int32_t* off = reinterpret_cast<const int32_t*>(dev_ptr);
  for (int i = 0; i < iters; ++i) {
    const int B = 1 + (i + tid) % 50, H = 1 + i % 8, D = 32 << (i % 3);
    const int32_t tq = 100 + i, tk = 100 + i;
    const int variant = i % 4, act = variant == JA_SLIDING ? JA_SOFTMAX : i % 3;
    const int window = variant == JA_SLIDING ? 1 + i % 300 : 0;
    const int dtype = i % 2 ? JA_BF16 : JA_F32;
    const size_t need = jagged_attn_workspace_size(B, H, D, variant, act, window, dtype, tq, tk);
    if (need == 0 || need > ws_bytes) {
      std::fprintf(stderr, "workspace size %zu for B=%d H=%d D=%d variant=%d\n", need, B, H, D, variant);
      g_errors.fetch_add(1);
      continue;
    }
    ja_io io{};
    io.dtype = dtype;
    io.total_q = tq;
    io.total_kv = tk;
    io.workspace = ws;
    io.workspace_bytes = ws_bytes;
    io.max_workgroups = i % 5 == 0 ? 16 : 0;
    int rc = jagged_attn_fwd(p, p, p, off, off, B, H, D, variant, act, window, const_cast<void*>(p), &io);
    if (rc != JA_OK) {
      std::fprintf(stderr, "fwd returned %d (%s)\n", rc, jagged_attn_strerror(rc));
      g_errors.fetch_add(1);
    }
    // argument errors return before any launch
    if (jagged_attn_fwd(p, p, p, off, off, 0, H, D, variant, act, window, const_cast<void*>(p), &io) != JA_EINVAL)
      g_errors.fetch_add(1);
    if (jagged_attn_fwd(p, p, p, off, off, B, H, 48, variant, act, window, const_cast<void*>(p), &io) !=
        JA_EUNSUPPORTED)
      g_errors.fetch_add(1);
    io.workspace_bytes = need - 1;
    if (jagged_attn_fwd(p, p, p, off, off, B, H, D, variant, act, window, const_cast<void*>(p), &io) !=
        JA_EWORKSPACE)
      g_errors.fetch_add(1);
    io.workspace_bytes = ws_bytes;
    io.max_workgroups = -1;
    if (jagged_attn_fwd(p, p, p, off, off, B, H, D, variant, act, window, const_cast<void*>(p), &io) != JA_EINVAL)
      g_errors.fetch_add(1);
    if (jagged_attn_check(ws, nullptr) != JA_OK) g_errors.fetch_add(1);
  }
}
}  // namespace

int main(int argc, char** argv) {
  const int threads = argc > 1 ? std::atoi(argv[1]) : 8;
  const int iters = argc > 2 ? std::atoi(argv[2]) : 200;
  std::vector<std::vector<unsigned char>> bufs(threads);
  std::vector<std::thread> pool;
  for (int t = 0; t < threads; ++t) {
    bufs[t].resize((size_t(1) << 24) + 256);
    unsigned char* base = bufs[t].data();
    unsigned char* ws = base + ((256 - (reinterpret_cast<uintptr_t>(base) & 255)) & 255);
    pool.emplace_back(worker, t, iters, ws, size_t(1) << 24);
  }
  for (auto& th : pool) th.join();
  std::printf("threads %d iterations %d launches %ld errors %d\n", threads, iters, g_launches.load(),
              g_errors.load());
  return g_errors.load() == 0 && g_launches.load() > 0 ? 0 : 1;
}
