// HBM -> LDS copies and the waits around them (gfx950), shared by the
// kernels that stream tiles through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_device.h"

namespace mla {

__device__ __forceinline__ uint32_t lds_addr(const MLA_LDS void* p) { return (uint32_t)(size_t)p; }

// Wave-wide HBM -> LDS copy of 16 bytes per lane: lane i's data lands at
// lds_base + 16 * i (the base travels in M0, which is saved and restored so
// the compiler's own use of M0 is untouched; one wait state separates the M0
// write from the load that reads it).  Issued through asm so that the
// compiler does not turn later LDS reads into waits for every outstanding
// copy; completion is tracked with explicit s_waitcnt vmcnt.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base)
      : "memory");
}

// Same copy with a wave-uniform 64-bit base in SGPRs plus a 32-bit per-lane
// byte offset (no per-lane address arithmetic).
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds_base) {
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);
  // readfirstlane returns int: widen each half through uint32_t (a sign
  // extension of the low half would overwrite the high half of the address)
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  base = (const void*)(((uint64_t)hi << 32) | (uint64_t)lo);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds_base)
      : "memory");
}

// Same copy where lane i's byte offset is (lc_i ^ x16) + lrow_i + row: a
// per-lane chunk offset (XORed with a wave-uniform swizzle) and row offset
// plus a wave-uniform row offset.
__device__ __forceinline__ void dma16xy(const void* base, uint32_t lc, uint32_t x16, uint32_t lrow, uint32_t row,
                                        uint32_t lds_base) {
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);
  x16 = __builtin_amdgcn_readfirstlane(x16);
  row = __builtin_amdgcn_readfirstlane(row);
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  base = (const void*)(((uint64_t)hi << 32) | (uint64_t)lo);
  uint32_t saved, off;
  asm volatile(
      "v_xor_b32 %1, %2, %3\n\t"
      "v_add3_u32 %1, %1, %4, %5\n\t"
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %7\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %6\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved), "=&v"(off)
      : "v"(lc), "s"(x16), "v"(lrow), "s"(row), "s"(base), "s"(lds_base)
      : "memory");
}

// Scalar (constant address space) load of a wave-uniform int: tracked by
// lgkmcnt, so it never waits on the outstanding HBM -> LDS copies.
__device__ __forceinline__ int load_uniform(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Wait until at most n groups of kPer copies (the ones issued last) are in
// flight, 0 <= n <= kMax.
template <int kPer, int kMax>
__device__ __forceinline__ void wait_groups(int n) {
  static_assert(kPer * kMax < 64, "vmcnt range");
  if constexpr (kMax >= 7) if (n >= 7) { wait_vmcnt<kPer * 7>(); return; }
  if constexpr (kMax >= 6) if (n == 6) { wait_vmcnt<kPer * 6>(); return; }
  if constexpr (kMax >= 5) if (n == 5) { wait_vmcnt<kPer * 5>(); return; }
  if constexpr (kMax >= 4) if (n == 4) { wait_vmcnt<kPer * 4>(); return; }
  if constexpr (kMax >= 3) if (n == 3) { wait_vmcnt<kPer * 3>(); return; }
  if constexpr (kMax >= 2) if (n == 2) { wait_vmcnt<kPer * 2>(); return; }
  if constexpr (kMax >= 1) if (n == 1) { wait_vmcnt<kPer>(); return; }
  wait_vmcnt<0>();
}

__device__ __forceinline__ void wg_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

}  // namespace mla
