// kv_check_pages: the KV page-tag check that runs as a batch of its own before
// decode reads the cache ("Smaller, faster, safer: running Kimi and GLM at
// scale", section "Protecting a shared KV cache": each physical page carries a
// tag that changes whenever the page is handed out again, the server keeps the
// (page, tag) pairs each request expects, and a request whose pairs do not
// match is aborted rather than allowed to read another request's page).
//
// One workgroup per request.  Each thread takes every 1024th logical page the
// request reads, four at a time: the page-map entry, the recorded page and the
// recorded tag of all four are loaded together (coalesced across the wave),
// then the four current tags are gathered.  The status bits are or-ed over
// the workgroup (wave ballots, one LDS word per wave) and thread 0 writes the
// request's status and checked length.
// The traffic is 12 bytes per page plus one gathered tag: the kernel is bound
// by the latency of its dependent loads (the kernel arguments, then the length
// and the first block of the row in parallel, then the tag gather), not by
// bandwidth.
#include "../../include/mla_decode.h"
#include "device_common.h"
#include "launch.h"

namespace mla {

constexpr int kCheckThreads = 1024;
constexpr int kCheckUnroll = 4;

// Status bits of one block of kCheckUnroll page-map entries per thread
// (entries base + u * kCheckThreads + tid); pg / rec / tag are their loaded
// map entries, recorded pages and recorded tags.
__device__ inline int check_block(const CheckArgs& a, int base, int n, const int (&pg)[kCheckUnroll],
                                  const int (&rec)[kCheckUnroll], const uint32_t (&tag)[kCheckUnroll]) {
  uint32_t cur[kCheckUnroll];
#pragma unroll
  for (int u = 0; u < kCheckUnroll; ++u) cur[u] = a.page_tags[min(max(pg[u], 0), a.num_pages - 1)];
  int bits = 0;
#pragma unroll
  for (int u = 0; u < kCheckUnroll; ++u) {
    const bool read = base + u * kCheckThreads + (int)threadIdx.x < n;
    const bool outside = pg[u] < 0 || pg[u] >= a.num_pages;
    bits |= (read && pg[u] != rec[u]) ? MLA_PAGE_WRONG_PAGE : 0;
    bits |= (read && outside) ? MLA_PAGE_OUT_OF_RANGE : 0;
    bits |= (read && !outside && cur[u] != tag[u]) ? MLA_PAGE_STALE_TAG : 0;
  }
  return bits;
}

__global__ __launch_bounds__(kCheckThreads) void kv_check_pages_kernel(CheckArgs a) {
  __shared__ int s_bits[kCheckThreads / 64];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)b * a.max_blocks;
  // Every load is issued from an index clamped into the row (and the tag
  // gather from a page clamped into the pool), and the results of lanes past
  // the request's pages are masked afterwards.  The first block of entries is
  // loaded before the length arrives (clamped to the row's width instead), so
  // the kernel waits for two memory latencies, not three.
  const int L = a.seq_lens[b];  // read before the barrier: checked_lens may be seq_lens
  int pg[kCheckUnroll], rec[kCheckUnroll];
  uint32_t tag[kCheckUnroll];
#pragma unroll
  for (int u = 0; u < kCheckUnroll; ++u) {
    const int j = min(u * kCheckThreads + tid, a.max_blocks - 1);
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
    if (n > 0) bits = check_block(a, 0, n, pg, rec, tag);
    for (int base = kCheckThreads * kCheckUnroll; base < n; base += kCheckThreads * kCheckUnroll) {
#pragma unroll
      for (int u = 0; u < kCheckUnroll; ++u) {
        const int j = min(base + u * kCheckThreads + tid, n - 1);
        pg[u] = a.block_table[row + j];
        rec[u] = a.expected_pages[row + j];
        tag[u] = a.expected_tags[row + j];
      }
      bits |= check_block(a, base, n, pg, rec, tag);
    }
  }
  // or over the workgroup: per bit a wave ballot, one LDS word per wave
  int wave_bits = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (__ballot(bits & (1 << k))) wave_bits |= 1 << k;
  if ((tid & 63) == 0) s_bits[tid >> 6] = wave_bits;
  __syncthreads();
  if (tid == 0) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < kCheckThreads / 64; ++w) s |= s_bits[w];
    a.status[b] = s;
    a.checked_lens[b] = s ? 0 : L;
  }
}

hipError_t launch_kv_check(const CheckArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(kv_check_pages_kernel, dim3(a.B), dim3(kCheckThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
