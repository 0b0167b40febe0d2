// Shared definitions of the decode kernels: the work-unit decode, LDS-DMA
// copies and wait helpers.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace mla {

constexpr float kRefSlack = 64.0f;  // log2 headroom of the weights over the reference

// This workgroup's (request, split, row group): work_unit_of (launch.h).
__device__ __forceinline__ WorkUnit decode_work_unit(int B, int max_splits, int n_rg) {
  return work_unit_of(blockIdx.x, B, max_splits, n_rg);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// HBM -> LDS copy without VGPRs: each lane moves 16 (or 4) bytes from
// base + its own 32-bit offset to lds_base + lane * 16 (or 4); the base is a
// wave-uniform 64-bit address in SGPRs, so a page costs no vector ALU work.
// Issued through inline asm so the compiler does not serialise later LDS reads
// on it; completion is awaited explicitly with wait_vmcnt() and a barrier.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(off), "s"(base), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma16_lane(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(MLA_LDS const void*)p;
}

// Loads of values that stay constant for the whole kernel (lengths, the
// per-tensor scale) go through the constant address space so that uniform ones
// become scalar loads.
template <typename V>
__device__ __forceinline__ V load_const(const V* p, int64_t i) {
  return ((__attribute__((address_space(4))) const V*)p)[i];
}

}  // namespace mla
