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
#include "page_check.h"

namespace mla {

constexpr int kCheckThreads = 1024;

__global__ __launch_bounds__(kCheckThreads) void kv_check_pages_kernel(CheckArgs a) {
  __shared__ int s_bits[kCheckThreads / 64];
  const int b = blockIdx.x;
  const int L = a.seq_lens[b];  // read before any barrier: checked_lens may be seq_lens
  const int s = check_request<kCheckThreads>(a, b, L, s_bits);
  if (threadIdx.x == 0) {
    a.status[b] = s;
    a.checked_lens[b] = s ? 0 : L;
  }
}

hipError_t launch_kv_check(const CheckArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(kv_check_pages_kernel, dim3(a.B), dim3(kCheckThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
