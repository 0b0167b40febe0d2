// Measured-peak microbenchmarks for MI355X (gfx950): what the hardware
// actually sustains, so that the decode kernel's roofline fraction can be
// quoted against measured as well as vendor peaks.  Not part of the decode
// path; built into its own library (libmla_peaks.so).
//
//  * peak_stream_read: every thread streams 16-byte loads over a buffer larger
//    than the 256 MB last-level cache (a plain HBM read).
//  * peak_stream_pages: 36,864-byte pages (64 tokens x 576 FP8 bytes) picked
//    through a page list, copied HBM -> LDS with LDS-DMA the way the decode
//    kernel stages its cache, with DEPTH pages in flight per wave ring; the
//    bandwidth as a function of the bytes in flight per compute unit.
//  * peak_latency: one lane chasing a random cycle of pointers 4 KB apart
//    (dependent loads, idle memory latency).
//  * peak_mfma: independent v_mfma_f32_16x16x32_bf16 chains on every SIMD; also
//    the shader clock over the run (s_memtime against the 100 MHz s_memrealtime).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla_peaks.h"
#include "decode_tile.h"

namespace mla {
namespace {

constexpr int kStreamUnroll = 8;

__global__ __launch_bounds__(256) void peak_stream_read_kernel(const u32x4* src, int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * kStreamUnroll;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x * kStreamUnroll + threadIdx.x; base < n16; base += stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int k = 0; k < kStreamUnroll; ++k) {
      const int64_t i = base + (int64_t)k * blockDim.x;
      v[k] = i < n16 ? __builtin_nontemporal_load(&src[i]) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kStreamUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// One page = 36,864 bytes; wave w of the workgroup copies bytes
// [w * 9216, (w + 1) * 9216) of each page into its own ring of DEPTH slots of
// 9 KB (nine 1 KB LDS-DMA instructions per page), so the waves never wait for
// one another.  Workgroup g takes list entries [g * ppw, min((g + 1) * ppw, n)).
constexpr int kPageBytes = 36864;
constexpr int kSlotBytes = 9216;
constexpr int kLoadsPerSlot = 9;

template <int DEPTH>
__global__ __launch_bounds__(256) void peak_stream_pages_kernel(const uint8_t* src, const int32_t* ids, int n,
                                                                int ppw, int num_pages, uint32_t* sink) {
  static_assert(DEPTH >= 1 && DEPTH <= 4, "four 9 KB slots per wave at most");
  // always four slots per wave (144 KB): one workgroup per compute unit
  // whatever DEPTH, so the bytes in flight per unit are 4 waves x DEPTH x 9 KB
  __shared__ __attribute__((aligned(16))) uint8_t ring[4][4][kSlotBytes];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int first = blockIdx.x * ppw;
  const int cnt = max(0, min(n, first + ppw) - first);
  const uint32_t off = (uint32_t)(wave * kSlotBytes + lane * 16);
  auto issue = [&](int i) {
    const int pg = min(max(ids[first + i], 0), num_pages - 1);
    const uint8_t* base = src + (int64_t)pg * kPageBytes;
    const uint32_t dst = lds_addr(&ring[wave][i % DEPTH][0]);
#pragma unroll
    for (int j = 0; j < kLoadsPerSlot; ++j) lds_dma16(base + j * 1024, off, dst + j * 1024);
  };
  for (int i = 0; i < DEPTH && i < cnt; ++i) issue(i);
  uint32_t acc = 0;
  for (int i = 0; i < cnt; ++i) {
    if (i + DEPTH <= cnt)
      wait_vmcnt<(DEPTH - 1) * kLoadsPerSlot>();  // the pages issued after page i may stay in flight
    else
      wait_vmcnt<0>();
    acc ^= *reinterpret_cast<const uint32_t*>(&ring[wave][i % DEPTH][lane * 16]);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the slot may be overwritten now
    if (i + DEPTH < cnt) issue(i + DEPTH);
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ __launch_bounds__(64) void peak_latency_kernel(const uint32_t* chain, int64_t n, int steps,
                                                          uint32_t* out, uint64_t* ticks) {
  if (threadIdx.x != 0) return;
  uint32_t j = 0;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (int s = 0; s < steps; ++s) j = (uint32_t)min((int64_t)__builtin_nontemporal_load(&chain[j]), n - 1);
  const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
  out[0] = j;
  ticks[0] = t1 - t0;
}

template <int WPS>
__global__ __launch_bounds__(256 * WPS) void peak_mfma_kernel(int iters, float* sink, uint64_t* clocks) {
  const int lane = threadIdx.x & 63;
  const float fa = 1.0f + lane * 1e-3f, fb = 1.0f - lane * 1e-3f;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(fa * (e + 1) * 1e-2f);
    b[e] = static_cast<__bf16>(fb * (8 - e) * 1e-2f);
  }
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  sink[gid] = s;
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = c1 - c0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace
}  // namespace mla

extern "C" {

int mla_peak_stream_read(const void* src, int64_t bytes, uint32_t* sink, int grid, void* stream) {
  if (!src || !sink) return 1;
  if (bytes < 16 || (bytes & 15) || grid < 1) return 2;
  hipLaunchKernelGGL(mla::peak_stream_read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const mla::u32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int mla_peak_stream_pages(const void* src, int num_pages, const int32_t* page_ids, int n, int pages_per_wg,
                          int depth, uint32_t* sink, void* stream) {
  if (!src || !page_ids || !sink) return 1;
  if (num_pages < 1 || n < 1 || pages_per_wg < 1) return 2;
  if (depth < 1 || depth > 4) return 3;
  const int grid = (n + pages_per_wg - 1) / pages_per_wg;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* p = static_cast<const uint8_t*>(src);
  switch (depth) {
    case 1: hipLaunchKernelGGL(mla::peak_stream_pages_kernel<1>, dim3(grid), dim3(256), 0, s, p, page_ids, n, pages_per_wg, num_pages, sink); break;
    case 2: hipLaunchKernelGGL(mla::peak_stream_pages_kernel<2>, dim3(grid), dim3(256), 0, s, p, page_ids, n, pages_per_wg, num_pages, sink); break;
    case 3: hipLaunchKernelGGL(mla::peak_stream_pages_kernel<3>, dim3(grid), dim3(256), 0, s, p, page_ids, n, pages_per_wg, num_pages, sink); break;
    default: hipLaunchKernelGGL(mla::peak_stream_pages_kernel<4>, dim3(grid), dim3(256), 0, s, p, page_ids, n, pages_per_wg, num_pages, sink); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int mla_peak_latency(const uint32_t* chain, int64_t n, int steps, uint32_t* out, uint64_t* ticks, void* stream) {
  if (!chain || !out || !ticks) return 1;
  if (n < 1 || n > 4294967296LL || steps < 1) return 2;
  hipLaunchKernelGGL(mla::peak_latency_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), chain, n,
                     steps, out, ticks);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int mla_peak_mfma(int grid, int waves_per_simd, int iters, float* sink, uint64_t* clocks, void* stream) {
  if (!sink || !clocks) return 1;
  if (grid < 1 || iters < 1) return 2;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (waves_per_simd == 1)
    hipLaunchKernelGGL(mla::peak_mfma_kernel<1>, dim3(grid), dim3(256), 0, s, iters, sink, clocks);
  else if (waves_per_simd == 2)
    hipLaunchKernelGGL(mla::peak_mfma_kernel<2>, dim3(grid), dim3(512), 0, s, iters, sink, clocks);
  else
    return 3;
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
