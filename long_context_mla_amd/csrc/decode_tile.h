// Shared definitions of the decode kernels: the staged page tile, its LDS
// swizzle, LDS-DMA copies and wait helpers.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace mla {

constexpr int kRows = 32;           // query rows per workgroup
constexpr float kRefSlack = 64.0f;  // log2 headroom of the weights over the reference
constexpr int kMaxRestarts = 4;

template <int CACHE>
struct Tile {
  static constexpr int ELEM = CACHE == kFp8 ? 1 : 2;
  static constexpr int ROW_BYTES = kD * ELEM;
  static constexpr int PAGE_BYTES = kPage * ROW_BYTES;
  // FP8 pages are small enough for four LDS buffers, which lets P V of a page
  // run one iteration after its scores (one barrier per page) with two pages
  // in flight.  BF16 pages fit twice: scores and P V of a page in the same
  // iteration, one page in flight.
  static constexpr bool PIPE = CACHE == kFp8;
  static constexpr int NBUF = PIPE ? 4 : 2;
  static constexpr int DIST = PIPE ? 2 : 1;          // pages in flight ahead of the current one
  static constexpr int LOADS = PAGE_BYTES / 4096;  // 16-byte LDS-DMA loads per wave per page
  static constexpr int PART = LOADS / 3;           // loads issued at each of three points
  static constexpr int PSTRIDE = kPage * 2 + 16;   // bytes per P row in LDS
  static constexpr int KBATCH = 9;                 // BF16 K reads issued before their math
};

// LDS layout of a staged BF16 page: token t's 16-byte chunk c (of NCH = 72 per
// row) sits in chunk slot t * NCH + slot(t, c), the row rotated by 3 * (t / 2)
// chunks, so that the 16-token operand reads of QK^T and the 8-token
// transposed reads of PV hit distinct LDS banks.  The HBM -> LDS copy applies
// the inverse mapping when it picks each lane's source chunk.  (FP8 pages use
// their own grouped layout, defined with their kernel.)
struct SwzBf16 {
  static constexpr int NCH = 72;
  __device__ static __forceinline__ int rot(int t) {  // in [0, NCH)
    const int r = 3 * (t >> 1);
    return r >= NCH ? r - NCH : r;  // t < 64 keeps r < 2 * NCH
  }
  __device__ static __forceinline__ int slot(int t, int c) {
    const int v = c + rot(t);
    return v >= NCH ? v - NCH : v;
  }
  __device__ static __forceinline__ int chunk_of_slot(int t, int s) {
    const int v = s - rot(t);
    return v < 0 ? v + NCH : v;
  }
};

// Workgroup -> (request, split, row group) through decode_item (launch.h).
// Grid size: decode_grid_size(B, max_splits, n_rg).
struct WorkUnit {
  int b, split, rg;
  bool valid;
};
__device__ __forceinline__ WorkUnit decode_work_unit(int B, int max_splits, int n_rg) {
  const int v = (int)decode_item(blockIdx.x, B, max_splits, n_rg);
  const int u = v / n_rg;
  WorkUnit w;
  w.rg = v - u * n_rg;
  w.valid = u < B * max_splits;
  w.split = w.valid ? u / B : 0;
  w.b = w.valid ? u - w.split * B : 0;
  return w;
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
