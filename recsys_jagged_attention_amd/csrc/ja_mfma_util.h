// Device helpers shared by the MFMA attention kernels (gfx950): operand index
// permutations, LDS chunk swizzles, direct-to-LDS loads, wait counters and the
// LDS barrier.  Everything here is wave-level plumbing; the attention math
// lives in the kernels.
#pragma once

#include <stdint.h>

#include "ja_device.h"

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

// 16 bytes per lane from global memory (SGPR base + 32-bit lane offset) into
// LDS at M0 + 16*lane.  Issued as inline asm on purpose: the compiler does not
// track it, so it neither drains the prefetch with a conservative vmcnt(0)
// before every later LDS read nor keeps 64-bit lane addresses live.  Completion
// is ordered by wait_vmcnt() + lds_barrier() below, both volatile asm with a
// memory clobber: the compiler keeps volatile asm in program order, so a load
// can neither move above the barrier that frees its target nor below the wait
// that consumes it, while MFMAs and LDS reads may be scheduled around it (no
// memory clobber here).  No compiler-generated code in these kernels reads M0
// (checked in the generated ISA).
__device__ __forceinline__ void lds_dma16(const void* sbase, unsigned voff, unsigned lds_addr) {
  // the base and the LDS address are wave-uniform: make that explicit for the "s" operands
  const uintptr_t p = reinterpret_cast<uintptr_t>(sbase);
  // (readfirstlane returns int: convert through unsigned so nothing is sign-extended)
  const uint64_t hi = unsigned(__builtin_amdgcn_readfirstlane(unsigned(p >> 32)));
  const uint64_t lo = unsigned(__builtin_amdgcn_readfirstlane(unsigned(p)));
  const uint64_t pu = (hi << 32) | lo;
  const unsigned lu = unsigned(__builtin_amdgcn_readfirstlane(lds_addr));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(reinterpret_cast<const void*>(pu)), "s"(lu) : "m0");
}

// 4 bytes per lane into LDS at M0 + 4*lane (same contract as lds_dma16).
__device__ __forceinline__ void lds_dma4(const void* sbase, unsigned voff, unsigned lds_addr) {
  const uintptr_t p = reinterpret_cast<uintptr_t>(sbase);
  const uint64_t hi = unsigned(__builtin_amdgcn_readfirstlane(unsigned(p >> 32)));
  const uint64_t lo = unsigned(__builtin_amdgcn_readfirstlane(unsigned(p)));
  const uint64_t pu = (hi << 32) | lo;
  const unsigned lu = unsigned(__builtin_amdgcn_readfirstlane(lds_addr));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(reinterpret_cast<const void*>(pu)), "s"(lu) : "m0");
}

// Online softmax keeps exponentials below 2^kLazyLog2 (see the tile loop).
constexpr float kLazyLog2 = 8.0f;

// A wave-uniform pointer made explicit (scalar registers), through unsigned
// halves so that nothing is sign-extended.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uintptr_t u = reinterpret_cast<uintptr_t>(p);
  const uint64_t hi = unsigned(__builtin_amdgcn_readfirstlane(unsigned(u >> 32)));
  const uint64_t lo = unsigned(__builtin_amdgcn_readfirstlane(unsigned(u)));
  return reinterpret_cast<const T*>((hi << 32) | lo);
}

// 16-byte store through a pointer marked global.  A pointer rebuilt from
// integers (as above) has lost its address space, and the compiler would emit
// a flat store; flat operations count on the LDS counter too and may complete
// out of order with LDS reads, so while one is pending every wait for an LDS
// read must drain all of them (lgkmcnt(0)) instead of waiting by count.
__device__ __forceinline__ void store_global16(void* p, bf16x8 v) {
  *reinterpret_cast<__attribute__((address_space(1))) bf16x8*>(reinterpret_cast<uintptr_t>(p)) = v;
}

// 16-byte chunk swizzle of an fp8 code tile (D bytes per row) for the fp8
// MFMA operand reads: rows sharing a bank set get distinct chunk slots.
template <int D>
__device__ __forceinline__ int swz_c(int row) {
  return (row / (256 / D)) % (D / 16);
}

__device__ __forceinline__ float e8m0_to_float(unsigned e) {
  e &= 0xFFu;
  return e == 0 ? __uint_as_float(0x00400000u) : (e == 255u ? __builtin_nanf("") : __uint_as_float(e << 23));
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// 16-byte chunk swizzle of a requantised V^T tile (head-dim rows of 64 key
// bytes): the 16 lanes of an fp8 P V operand read -- head dims r%4 + 4*bit2 +
// 64*bit6 of dim_perm -- land on 16 distinct bank groups.
__device__ __forceinline__ int vt_swz(int d) { return (((d >> 6) & 1) << 1) | ((d >> 2) & 1); }

__device__ __forceinline__ unsigned lds_addr_of(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) unsigned char*)(p)));
}

// Wait until at most n of this wave's VMEM instructions are outstanding.
__device__ __forceinline__ void wait_vmcnt(int n) {
  // s_waitcnt encoding (gfx9): vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
#define JA_VMCNT(k) case k: __builtin_amdgcn_s_waitcnt(((k) & 15) | (((k) >> 4) << 14) | 0x0F70); break;
  switch (n) {
    JA_VMCNT(0) JA_VMCNT(1) JA_VMCNT(2) JA_VMCNT(3) JA_VMCNT(4) JA_VMCNT(5) JA_VMCNT(6) JA_VMCNT(7)
    JA_VMCNT(8) JA_VMCNT(9) JA_VMCNT(10) JA_VMCNT(11) JA_VMCNT(12) JA_VMCNT(13) JA_VMCNT(14)
    JA_VMCNT(15) JA_VMCNT(16) JA_VMCNT(17) JA_VMCNT(18) JA_VMCNT(19) JA_VMCNT(20) JA_VMCNT(21)
    JA_VMCNT(22) JA_VMCNT(23) JA_VMCNT(24)
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
#undef JA_VMCNT
}

// Workgroup barrier for LDS hand-offs that does not drain outstanding global
// loads (a __syncthreads() fence would wait for the prefetch too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace
}  // namespace ja
