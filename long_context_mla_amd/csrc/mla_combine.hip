// mla_decode_combine: merge split-KV partial outputs with their log-sum-exp, the
// online-softmax merge the pages describe for partial attention outputs written
// by peers ("vLLM x AgentX: Optimizing for Real-World Agentic Serving", section
// "Model-specific parallelism / Kimi K3"), here applied to the splits of one GPU.
//
// One workgroup per (request, row, 128-dim chunk), 256 threads: 16 groups of
// 16 lanes, each lane one 16-byte piece (8 values) of the chunk.  Up to 512
// splits (the instantiation the launch picks) every lane loads all of its
// group's partials (splits g, g + 16, ...) at once, together with the split
// LSEs, before anything depends on them: one memory round trip.  The split
// weights exp(lse_s - max_s lse_s) go through LDS, each lane sums its splits
// from registers; the four groups of a wave are folded on the VALU (permlane
// swaps) and the four waves through LDS.  More splits than that stream
// through in blocks.
#include "device_common.h"
#include "launch.h"

namespace mla {

constexpr int kGroups = 16;                  // split groups per workgroup
constexpr int kWeightChunk = 1024;           // split weights held in LDS at a time (streaming)

// Eight consecutive bf16 partial values (16 bytes) added to acc with weight w (exact widening).
__device__ __forceinline__ void fma_bf16x8(f32x4 (&acc)[2], float w, u32x4 v) {
  acc[0] += w * f32x4{float_of(v.x << 16), float_of(v.x & 0xffff0000u), float_of(v.y << 16),
                      float_of(v.y & 0xffff0000u)};
  acc[1] += w * f32x4{float_of(v.z << 16), float_of(v.z & 0xffff0000u), float_of(v.w << 16),
                      float_of(v.w & 0xffff0000u)};
}

// Maximum over the 16 lanes of each row (DPP rotations within the row), then
// over the wave's four rows (permlane swaps), then over the four waves (LDS).
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  return fmaxf(v, float_of((uint32_t)__builtin_amdgcn_update_dpp(0, (int)bits_of(v), CTRL, 0xf, 0xf, false)));
}
__device__ __forceinline__ float row16_max(float v) {
  // row_ror:8, 4, 2, 1
  return dpp_max<0x121>(dpp_max<0x122>(dpp_max<0x124>(dpp_max<0x128>(v))));
}

__device__ __forceinline__ float block_max(float v, float* s_red) {
  v = group4_max(row16_max(v));
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
}

// Splits of request b that hold a partial: those that start before its last
// page.  A request the page check flagged merges none: its rows come out
// 0 / -inf.
__device__ __forceinline__ int request_splits(const CombineArgs& a, int b) {
  // both loads go out together (without a status the length is read twice)
  const int st = (a.status ? a.status : a.seq_lens)[b];
  const int raw = a.seq_lens[b];
  asm volatile("" :: "s"(st), "s"(raw));
  const int L = min(max(raw, 0), a.max_blocks * kPage);
  const int n_pages = (L + kPage - 1) / kPage;
  return (a.status && st != 0) ? 0 : min(a.max_splits, (n_pages + a.pps - 1) / a.pps);
}

// The merge when the request's n_b splits fit NK loads per lane
// (16 * NK >= n_b >= 1): group g loads splits g + 16k (the ones past n_b
// repeat split n_b - 1, a written partial, and are left out of the sums).
// ls0 / ls1 are this thread's split LSEs (splits t and t + 256; -inf at or
// past max_splits).  (Loading the partials before the request's length
// arrives, which a single request would allow, was slower: the loads are
// bound by the memory's rate, and the length then came back behind them.)
template <int NK>
__device__ __forceinline__ void merge_held(const uint16_t* o_b, int64_t o_stride, float ls0, float ls1, int n_b,
                                           float* s_w, float* s_red, f32x4 (&acc)[2], float& wsum, float& M) {
  const int t = threadIdx.x;
  const int g = t >> 4;
  u32x4 o[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k)
    o[k] = *reinterpret_cast<const u32x4*>(o_b + min(g + kGroups * k, n_b - 1) * o_stride);
  // masked only now, so that the partial loads above do not wait for the LSEs
  if (t >= n_b) ls0 = -INFINITY;
  if (t + 256 >= n_b) ls1 = -INFINITY;
  M = block_max(fmaxf(ls0, ls1), s_red);
  s_w[t] = ls0 == -INFINITY ? 0.0f : expf(ls0 - M);
  if (NK * kGroups > 256) s_w[t + 256] = ls1 == -INFINITY ? 0.0f : expf(ls1 - M);
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    if (g + kGroups * k < n_b) {
      const float w = s_w[g + kGroups * k];
      fma_bf16x8(acc, w, o[k]);
      wsum += w;
    }
  }
}

// ceil(n_b / 16) loads per lane rounded up to a power of two, so that each
// count is straight-line code with every load in flight at once (n_b is
// uniform over the workgroup; an empty request merges nothing).
template <int MAXK>
__device__ __forceinline__ void merge_held_any(const uint16_t* o_b, int64_t o_stride, float ls0, float ls1,
                                               int n_b, float* s_w, float* s_red, f32x4 (&acc)[2], float& wsum,
                                               float& M) {
  const int n_k = (n_b + kGroups - 1) / kGroups;
  if (MAXK >= 32 && n_k > 16)
    merge_held<(MAXK >= 32 ? 32 : 1)>(o_b, o_stride, ls0, ls1, n_b, s_w, s_red, acc, wsum, M);
  else if (MAXK >= 16 && n_k > 8)
    merge_held<(MAXK >= 16 ? 16 : 1)>(o_b, o_stride, ls0, ls1, n_b, s_w, s_red, acc, wsum, M);
  else if (MAXK >= 8 && n_k > 4)
    merge_held<(MAXK >= 8 ? 8 : 1)>(o_b, o_stride, ls0, ls1, n_b, s_w, s_red, acc, wsum, M);
  else if (n_k > 2)
    merge_held<4>(o_b, o_stride, ls0, ls1, n_b, s_w, s_red, acc, wsum, M);
  else if (n_k > 1)
    merge_held<2>(o_b, o_stride, ls0, ls1, n_b, s_w, s_red, acc, wsum, M);
  else if (n_k == 1)
    merge_held<1>(o_b, o_stride, ls0, ls1, n_b, s_w, s_red, acc, wsum, M);
}

// MAXK: the most partial loads a lane holds at once (splits up to 16 * MAXK
// are held).  The kernel's register count, and so how many workgroups share a
// compute unit, follows MAXK, so the launch picks the smallest that covers
// max_splits: a batch of many short merges keeps a full compute unit.
template <int MAXK>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int chunk = blockIdx.x & 3;
  const int br = blockIdx.x >> 2;  // b * R + r
  const int b = br / a.R;
  const int r = br - b * a.R;
  const int t = threadIdx.x;
  const int c = t & 15;  // 16-byte piece of the 128-dim chunk
  const int g = t >> 4;  // split group
  __shared__ float s_w[kWeightChunk];
  __shared__ float s_red[4];
  __shared__ f32x4 s_acc[4][16][2];
  __shared__ float s_ws[4];

  const float* lse_b = a.lse_part + (int64_t)b * a.max_splits * a.R + r;
  const uint16_t* o_b = a.o_part + ((int64_t)b * a.max_splits * a.R + r) * kDV + chunk * 128 + c * 8;
  const int64_t o_stride = (int64_t)a.R * kDV;
  // Up to 16 * MAXK splits (the usual case) the split LSEs are loaded before
  // the length is known: every entry below max_splits lies in the buffer, and
  // the ones past the request's splits are masked once the length arrives.
  const bool held = a.max_splits <= kGroups * MAXK;
  float ls0 = -INFINITY, ls1 = -INFINITY;
  if (held && t < a.max_splits) ls0 = lse_b[(int64_t)t * a.R];
  if (held && t + 256 < a.max_splits) ls1 = lse_b[(int64_t)(t + 256) * a.R];

  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  float wsum = 0.0f;
  float M = -INFINITY;
  const int n_b = request_splits(a, b);
  if (held) {
    merge_held_any<MAXK>(o_b, o_stride, ls0, ls1, n_b, s_w, s_red, acc, wsum, M);
  } else {
    float m = -INFINITY;
    for (int s = t; s < n_b; s += 256) m = fmaxf(m, lse_b[(int64_t)s * a.R]);
    M = block_max(m, s_red);
    for (int s0 = 0; s0 < n_b; s0 += kWeightChunk) {
      const int s1 = min(n_b, s0 + kWeightChunk);
      __syncthreads();
      for (int s = s0 + t; s < s1; s += 256) {
        const float ls = lse_b[(int64_t)s * a.R];
        s_w[s - s0] = (ls == -INFINITY) ? 0.0f : expf(ls - M);
      }
      __syncthreads();
      int s = s0 + g;
      for (; s + 3 * kGroups < s1; s += 4 * kGroups) {
        u32x4 o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = *reinterpret_cast<const u32x4*>(o_b + (s + kGroups * k) * o_stride);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float w = s_w[s + kGroups * k - s0];
          fma_bf16x8(acc, w, o[k]);
          wsum += w;
        }
      }
      for (; s < s1; s += kGroups) {
        const float w = s_w[s - s0];
        fma_bf16x8(acc, w, *reinterpret_cast<const u32x4*>(o_b + s * o_stride));
        wsum += w;
      }
    }
  }
  // fold the wave's four split groups on the VALU, then the four waves through LDS
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[0][i] = group4_sum(acc[0][i]);
    acc[1][i] = group4_sum(acc[1][i]);
  }
  wsum = group4_sum(wsum);
  const int wv = t >> 6;
  if ((t & 63) < 16) {
    s_acc[wv][c][0] = acc[0];
    s_acc[wv][c][1] = acc[1];
    if (c == 0) s_ws[wv] = wsum;
  }
  __syncthreads();
  if (t < 16) {
    f32x4 lo = s_acc[0][c][0], hi = s_acc[0][c][1];
    float wt = s_ws[0];
#pragma unroll
    for (int k = 1; k < 4; ++k) {
      lo += s_acc[k][c][0];
      hi += s_acc[k][c][1];
      wt += s_ws[k];
    }
    const float inv = wt > 0.0f ? 1.0f / wt : 0.0f;
    uint16_t* dst = a.out + (int64_t)br * kDV + chunk * 128 + c * 8;
    u32x4 v;
    v.x = float_to_bf16(lo[0] * inv) | (uint32_t(float_to_bf16(lo[1] * inv)) << 16);
    v.y = float_to_bf16(lo[2] * inv) | (uint32_t(float_to_bf16(lo[3] * inv)) << 16);
    v.z = float_to_bf16(hi[0] * inv) | (uint32_t(float_to_bf16(hi[1] * inv)) << 16);
    v.w = float_to_bf16(hi[2] * inv) | (uint32_t(float_to_bf16(hi[3] * inv)) << 16);
    *reinterpret_cast<u32x4*>(dst) = v;
    if (chunk == 0 && c == 0) a.lse[br] = wt > 0.0f ? M + logf(wt) : -INFINITY;
  }
}

// The merge for a batch of many rows over few splits (max_splits <= 64): one
// wave per row of the query matrix (request b, row r), lane l holding dims
// 8l .. 8l+7 of the 512, so that a split's partial row is one coalesced 1 KB
// load and the wave needs no LDS and no barrier.  Lane s holds split s's LSE;
// the partial loads go out kRowChunk splits at a time, each chunk's loads
// before the previous chunk is summed.  (The workgroup-per-row-chunk form
// above spreads one row's splits over 16 groups: for a batch of short merges
// most of its lanes idle and every workgroup is one dependent chain of loads.)
constexpr int kRowChunk = 8;
constexpr int kRowMaxSplits = 64;
constexpr int kRowsPerGroup = 4;  // waves (rows) per 256-thread workgroup

__device__ __forceinline__ float row16_sum(float v) {
  v += float_of((uint32_t)__builtin_amdgcn_update_dpp(0, (int)bits_of(v), 0x128, 0xf, 0xf, false));
  v += float_of((uint32_t)__builtin_amdgcn_update_dpp(0, (int)bits_of(v), 0x124, 0xf, 0xf, false));
  v += float_of((uint32_t)__builtin_amdgcn_update_dpp(0, (int)bits_of(v), 0x122, 0xf, 0xf, false));
  v += float_of((uint32_t)__builtin_amdgcn_update_dpp(0, (int)bits_of(v), 0x121, 0xf, 0xf, false));
  return v;
}

__global__ __launch_bounds__(256) void combine_rows_kernel(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar loads below
  const int64_t br = (int64_t)blockIdx.x * kRowsPerGroup + wv;  // b * R + r
  if (br >= (int64_t)a.B * a.R) return;
  const int b = (int)(br / a.R);
  const int r = (int)(br - (int64_t)b * a.R);
  const int64_t row0 = (int64_t)b * a.max_splits * a.R + r;  // (b, split 0, r)
  // the split LSEs go out before the length is known (every entry below
  // max_splits lies in the buffer); those past the request's splits are
  // masked once it arrives
  float ls = lane < a.max_splits ? a.lse_part[row0 + (int64_t)lane * a.R] : -INFINITY;
  const int n_b = request_splits(a, b);
  const uint16_t* src = a.o_part + row0 * kDV + 8 * lane;
  const int64_t stride = (int64_t)a.R * kDV;  // between the splits of one row
  const int nch = (n_b + kRowChunk - 1) / kRowChunk;
  u32x4 o[2][kRowChunk];
  auto load_chunk = [&](int c, u32x4 (&d)[kRowChunk]) {
#pragma unroll
    for (int k = 0; k < kRowChunk; ++k)
      d[k] = *reinterpret_cast<const u32x4*>(src + min(kRowChunk * c + k, n_b - 1) * stride);
  };
  if (nch > 0) load_chunk(0, o[0]);
  if (lane >= n_b) ls = -INFINITY;
  const float M = group4_max(row16_max(ls));
  const float w = ls == -INFINITY ? 0.0f : expf(ls - M);
  const float wsum = group4_sum(row16_sum(w));
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int c = 0; c < kRowMaxSplits / kRowChunk; ++c) {
    if (c < nch) {
      if (c + 1 < nch) load_chunk(c + 1, o[(c + 1) & 1]);
#pragma unroll
      for (int k = 0; k < kRowChunk; ++k) {
        const int sp = kRowChunk * c + k;
        if (sp < n_b) fma_bf16x8(acc, float_of(__builtin_amdgcn_readlane(bits_of(w), sp)), o[c & 1][k]);
      }
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  u32x4 v;
  v.x = float_to_bf16(acc[0][0] * inv) | (uint32_t(float_to_bf16(acc[0][1] * inv)) << 16);
  v.y = float_to_bf16(acc[0][2] * inv) | (uint32_t(float_to_bf16(acc[0][3] * inv)) << 16);
  v.z = float_to_bf16(acc[1][0] * inv) | (uint32_t(float_to_bf16(acc[1][1] * inv)) << 16);
  v.w = float_to_bf16(acc[1][2] * inv) | (uint32_t(float_to_bf16(acc[1][3] * inv)) << 16);
  *reinterpret_cast<u32x4*>(a.out + br * kDV + 8 * lane) = v;
  if (lane == 0) a.lse[br] = wsum > 0.0f ? M + logf(wsum) : -INFINITY;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.R;
  if (a.max_splits <= kRowMaxSplits && rows >= 1024) {
    // many rows over few splits: a wave per row (at least 256 workgroups)
    const dim3 grid((unsigned)((rows + kRowsPerGroup - 1) / kRowsPerGroup)), block(256);
    hipLaunchKernelGGL(combine_rows_kernel, grid, block, 0, stream, a);
    return hipGetLastError();
  }
  const dim3 grid(a.B * a.R * 4), block(256);
  if (a.max_splits <= kGroups * 4)
    hipLaunchKernelGGL(combine_kernel<4>, grid, block, 0, stream, a);
  else if (a.max_splits <= kGroups * 8)
    hipLaunchKernelGGL(combine_kernel<8>, grid, block, 0, stream, a);
  else if (a.max_splits <= kGroups * 16)
    hipLaunchKernelGGL(combine_kernel<16>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(combine_kernel<32>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
