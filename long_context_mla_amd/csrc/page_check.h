// The KV page-tag check of one request, for a workgroup of THREADS threads:
// shared by kv_check_pages (a launch of its own) and by the decode launch that
// carries the check in extra workgroups.  The check itself is described with
// kv_check_pages in the C header ("Smaller, faster, safer: running Kimi and GLM
// at scale", section "Protecting a shared KV cache").
#pragma once

#include "../../include/mla_decode.h"
#include "device_common.h"
#include "launch.h"

namespace mla {

constexpr int kCheckUnroll = 4;

// Status bits of one block of kCheckUnroll page-map entries per thread
// (entries base + u * THREADS + tid); pg / rec / tag are their loaded map
// entries, recorded pages and recorded tags.
template <int THREADS>
__device__ inline int check_block(const CheckArgs& a, int base, int n, const int (&pg)[kCheckUnroll],
                                  const int (&rec)[kCheckUnroll], const uint32_t (&tag)[kCheckUnroll]) {
  uint32_t cur[kCheckUnroll];
#pragma unroll
  for (int u = 0; u < kCheckUnroll; ++u) cur[u] = a.page_tags[min(max(pg[u], 0), a.num_pages - 1)];
  int bits = 0;
#pragma unroll
  for (int u = 0; u < kCheckUnroll; ++u) {
    const bool read = base + u * THREADS + (int)threadIdx.x < n;
    const bool outside = pg[u] < 0 || pg[u] >= a.num_pages;
    bits |= (read && pg[u] != rec[u]) ? MLA_PAGE_WRONG_PAGE : 0;
    bits |= (read && outside) ? MLA_PAGE_OUT_OF_RANGE : 0;
    bits |= (read && !outside && cur[u] != tag[u]) ? MLA_PAGE_STALE_TAG : 0;
  }
  return bits;
}

// Checks request b with the whole workgroup and returns its status bits to
// every thread.  L is the request's length, read by the caller.  s_bits: LDS
// scratch of THREADS / 64 ints.  Every load is issued from an index clamped
// into the row (and the tag gather from a page clamped into the pool), and the
// results of lanes past the request's pages are masked afterwards.  The first
// block of entries is loaded before the length is tested (clamped to the
// row's width instead), so one pass waits for two memory latencies.
template <int THREADS>
__device__ inline int check_request(const CheckArgs& a, int b, int L, int* s_bits) {
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)b * a.max_blocks;
  int pg[kCheckUnroll], rec[kCheckUnroll];
  uint32_t tag[kCheckUnroll];
#pragma unroll
  for (int u = 0; u < kCheckUnroll; ++u) {
    const int j = min(u * THREADS + tid, a.max_blocks - 1);
    pg[u] = a.block_table[row + j];
    rec[u] = a.expected_pages[row + j];
    tag[u] = a.expected_tags[row + j];
  }
  // keeps the compiler from sinking these loads behind the length test
#pragma unroll
  for (int u = 0; u < kCheckUnroll; ++u) asm volatile("" ::"v"(pg[u]), "v"(rec[u]), "v"(tag[u]));
  int bits = 0;
  if (L < 0 || L > a.max_blocks * kPage) {
    bits = MLA_PAGE_BAD_LEN;
  } else {
    const int n = (L + kPage - 1) / kPage;
    if (n > 0) bits = check_block<THREADS>(a, 0, n, pg, rec, tag);
    for (int base = THREADS * kCheckUnroll; base < n; base += THREADS * kCheckUnroll) {
#pragma unroll
      for (int u = 0; u < kCheckUnroll; ++u) {
        const int j = min(base + u * THREADS + tid, n - 1);
        pg[u] = a.block_table[row + j];
        rec[u] = a.expected_pages[row + j];
        tag[u] = a.expected_tags[row + j];
      }
      bits |= check_block<THREADS>(a, base, n, pg, rec, tag);
    }
  }
  // or over the workgroup: per bit a wave ballot, one LDS word per wave
  int wave_bits = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (__ballot(bits & (1 << k))) wave_bits |= 1 << k;
  if ((tid & 63) == 0) s_bits[tid >> 6] = wave_bits;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < THREADS / 64; ++w) s |= s_bits[w];
  return s;
}

}  // namespace mla
