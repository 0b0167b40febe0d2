// mla_decode_combine: merge split-KV partial outputs with their log-sum-exp, the
// online-softmax merge the pages describe for partial attention outputs written
// by peers ("vLLM x AgentX: Optimizing for Real-World Agentic Serving", section
// "Model-specific parallelism / Kimi K3"), here applied to the splits of one GPU.
//
// One workgroup per (request, row, 128-dim chunk): 32 lanes x float4 cover the
// chunk and 8 groups of 32 lanes stride over the splits; an LDS reduction folds
// the 8 groups.  Split weights are exp(lse_s - max_s lse_s).
#include "device_common.h"
#include "launch.h"

namespace mla {

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int chunk = blockIdx.x & 3;
  const int br = blockIdx.x >> 2;  // b * R + r
  const int b = br / a.R;
  const int r = br - b * a.R;
  const int t = threadIdx.x;
  const int c4 = t & 31;  // float4 index inside the 128-dim chunk
  const int g = t >> 5;   // split group
  __shared__ f32x4 s_acc[8][32];
  __shared__ float s_w[8];

  int L = min(max(a.seq_lens[b], 0), a.max_blocks * kPage);
  const int n_pages = (L + kPage - 1) / kPage;
  const int n_b = min(a.max_splits, (n_pages + a.pps - 1) / a.pps);
  const int64_t lse_base = (int64_t)b * a.max_splits * a.R + r;

  float M = -INFINITY;
  for (int s = 0; s < n_b; ++s) M = fmaxf(M, a.lse_part[lse_base + (int64_t)s * a.R]);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.0f;
  if (M != -INFINITY) {
    for (int s = g; s < n_b; s += 8) {
      const float ls = a.lse_part[lse_base + (int64_t)s * a.R];
      if (ls == -INFINITY) continue;
      const float w = expf(ls - M);
      const f32x4 o = *reinterpret_cast<const f32x4*>(
          a.o_part + ((lse_base + (int64_t)s * a.R) * kDV) + chunk * 128 + c4 * 4);
      acc += w * o;
      wsum += w;
    }
  }
  s_acc[g][c4] = acc;
  if (c4 == 0) s_w[g] = wsum;
  __syncthreads();
  if (g == 0) {
    f32x4 tot = s_acc[0][c4];
    float wt = s_w[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) {
      tot += s_acc[k][c4];
      wt += s_w[k];
    }
    const float inv = wt > 0.0f ? 1.0f / wt : 0.0f;
    uint16_t* dst = a.out + (int64_t)br * kDV + chunk * 128 + c4 * 4;
    const uint32_t lo = float_to_bf16(tot[0] * inv) | (uint32_t(float_to_bf16(tot[1] * inv)) << 16);
    const uint32_t hi = float_to_bf16(tot[2] * inv) | (uint32_t(float_to_bf16(tot[3] * inv)) << 16);
    u32x2 v = {lo, hi};
    *reinterpret_cast<u32x2*>(dst) = v;
    if (chunk == 0 && c4 == 0) a.lse[br] = wt > 0.0f ? M + logf(wt) : -INFINITY;
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const dim3 grid(a.B * a.R * 4), block(256);
  hipLaunchKernelGGL(combine_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
