// mla_decode_combine: merge split-KV partial outputs with their log-sum-exp, the
// online-softmax merge the pages describe for partial attention outputs written
// by peers ("vLLM x AgentX: Optimizing for Real-World Agentic Serving", section
// "Model-specific parallelism / Kimi K3"), here applied to the splits of one GPU.
//
// One workgroup per (request, row, 128-dim chunk).  The split weights
// exp(lse_s - max_s lse_s) are computed once, in parallel, into LDS; then 8
// groups of 32 lanes (one float4 of the chunk per lane) stride over the splits
// with several loads in flight, and an LDS reduction folds the 8 groups.
#include "device_common.h"
#include "launch.h"

namespace mla {

constexpr int kWeightChunk = 1024;  // split weights held in LDS at a time
constexpr int kHeldSplits = 128;   // splits whose partials a lane holds in registers at once

// Four consecutive bf16 partial values (8 bytes) as floats (exact).
__device__ __forceinline__ f32x4 load_bf16x4(const uint16_t* p) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  return f32x4{float_of(w.x << 16), float_of(w.x & 0xffff0000u), float_of(w.y << 16), float_of(w.y & 0xffff0000u)};
}

// The merge of one (request, row, chunk) when its n_b splits fit NK loads per
// lane (8 * NK >= n_b >= 1): lane group g = t / 32 loads splits g + 8k (the
// ones past n_b repeat split n_b - 1, a finite partial, and take weight 0),
// all before the block-wide max of the LSEs; then the weights go through LDS
// and the partials are summed from registers.
template <int NK>
__device__ __forceinline__ void merge_held(const uint16_t* o_b, int64_t o_stride, float ls, int n_b,
                                           float* s_w, float* s_red, f32x4& acc, float& wsum,
                                           float& M) {
  const int t = threadIdx.x;
  const int g = t >> 5;
  f32x4 o[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) o[k] = load_bf16x4(o_b + min(g + 8 * k, n_b - 1) * o_stride);
  M = wave_max(ls);
  if ((t & 63) == 0) s_red[t >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  if (t < 8 * NK) s_w[t] = (ls == -INFINITY) ? 0.0f : expf(ls - M);
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const float w = g + 8 * k < n_b ? s_w[g + 8 * k] : 0.0f;
    acc += w * o[k];
    wsum += w;
  }
}

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int chunk = blockIdx.x & 3;
  const int br = blockIdx.x >> 2;  // b * R + r
  const int b = br / a.R;
  const int r = br - b * a.R;
  const int t = threadIdx.x;
  const int c4 = t & 31;  // float4 index inside the 128-dim chunk
  const int g = t >> 5;   // split group
  __shared__ float s_w[kWeightChunk];
  __shared__ float s_red[4];
  __shared__ f32x4 s_acc[8][32];
  __shared__ float s_ws[8];

  const float* lse_b = a.lse_part + (int64_t)b * a.max_splits * a.R + r;
  const uint16_t* o_b = a.o_part + ((int64_t)b * a.max_splits * a.R + r) * kDV + chunk * 128 + c4 * 4;
  const int64_t o_stride = (int64_t)a.R * kDV;
  // Up to kHeldSplits splits (the usual case) each thread's split LSE is
  // loaded before the length is known (every entry below max_splits lies in
  // the buffer; the ones past the request's splits are masked once the length
  // arrives), and each lane's partials for the request's splits are all
  // loaded at once: two memory round trips instead of one per pass over the
  // splits.
  const bool held = a.max_splits <= kHeldSplits;
  float ls_held = -INFINITY;
  if (held && t < a.max_splits) ls_held = lse_b[(int64_t)t * a.R];

  const int L = min(max(a.seq_lens[b], 0), a.max_blocks * kPage);
  const int n_pages = (L + kPage - 1) / kPage;
  // a request the page check flagged merges no split: its rows come out 0 / -inf
  const int n_b = (a.status && a.status[b]) ? 0 : min(a.max_splits, (n_pages + a.pps - 1) / a.pps);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.0f;
  float M = -INFINITY;
  if (held) {
    // Each group of 32 lanes takes splits g, g + 8, ...: ceil(n_b / 8) loads
    // per lane, rounded up to a power of two so that each count is straight-line
    // code with every load in flight at once (the count is uniform over the
    // workgroup).  An empty request (n_b == 0) merges nothing.
    const float ls = t < n_b ? ls_held : -INFINITY;
    const int n_k = (n_b + 7) >> 3;
    if (n_k > 8)
      merge_held<16>(o_b, o_stride, ls, n_b, s_w, s_red, acc, wsum, M);
    else if (n_k > 4)
      merge_held<8>(o_b, o_stride, ls, n_b, s_w, s_red, acc, wsum, M);
    else if (n_k > 2)
      merge_held<4>(o_b, o_stride, ls, n_b, s_w, s_red, acc, wsum, M);
    else if (n_k > 1)
      merge_held<2>(o_b, o_stride, ls, n_b, s_w, s_red, acc, wsum, M);
    else if (n_k == 1)
      merge_held<1>(o_b, o_stride, ls, n_b, s_w, s_red, acc, wsum, M);
  } else {
    for (int s = t; s < n_b; s += 256) M = fmaxf(M, lse_b[(int64_t)s * a.R]);
    M = wave_max(M);
    if ((t & 63) == 0) s_red[t >> 6] = M;
    __syncthreads();
    M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));

    for (int s0 = 0; s0 < n_b; s0 += kWeightChunk) {
      const int s1 = min(n_b, s0 + kWeightChunk);
      __syncthreads();
      for (int s = s0 + t; s < s1; s += 256) {
        const float ls = lse_b[(int64_t)s * a.R];
        s_w[s - s0] = (ls == -INFINITY) ? 0.0f : expf(ls - M);
      }
      __syncthreads();
      int s = s0 + g;
      for (; s + 24 < s1; s += 32) {
        const f32x4 o0 = load_bf16x4(o_b + s * o_stride);
        const f32x4 o1 = load_bf16x4(o_b + (s + 8) * o_stride);
        const f32x4 o2 = load_bf16x4(o_b + (s + 16) * o_stride);
        const f32x4 o3 = load_bf16x4(o_b + (s + 24) * o_stride);
        const float w0 = s_w[s - s0], w1 = s_w[s + 8 - s0], w2 = s_w[s + 16 - s0], w3 = s_w[s + 24 - s0];
        acc += w0 * o0 + w1 * o1 + w2 * o2 + w3 * o3;
        wsum += (w0 + w1) + (w2 + w3);
      }
      for (; s < s1; s += 8) {
        const float w = s_w[s - s0];
        acc += w * load_bf16x4(o_b + s * o_stride);
        wsum += w;
      }
    }
  }
  s_acc[g][c4] = acc;
  if (c4 == 0) s_ws[g] = wsum;
  __syncthreads();
  if (g == 0) {
    f32x4 tot = s_acc[0][c4];
    float wt = s_ws[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) {
      tot += s_acc[k][c4];
      wt += s_ws[k];
    }
    const float inv = wt > 0.0f ? 1.0f / wt : 0.0f;
    uint16_t* dst = a.out + (int64_t)br * kDV + chunk * 128 + c4 * 4;
    const uint32_t lo = float_to_bf16(tot[0] * inv) | (uint32_t(float_to_bf16(tot[1] * inv)) << 16);
    const uint32_t hi = float_to_bf16(tot[2] * inv) | (uint32_t(float_to_bf16(tot[3] * inv)) << 16);
    *reinterpret_cast<u32x2*>(dst) = u32x2{lo, hi};
    if (chunk == 0 && c4 == 0) a.lse[br] = wt > 0.0f ? M + logf(wt) : -INFINITY;
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const dim3 grid(a.B * a.R * 4), block(256);
  hipLaunchKernelGGL(combine_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
