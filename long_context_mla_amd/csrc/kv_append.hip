// kv_append_fp8: quantise new latent rows to OCP E4M3 and scatter them into the
// paged cache.  The cache is kept in FP8 e4m3 instead of BF16, which halves its
// size ("Smaller, faster, safer: running Kimi and GLM at scale", section
// "Quantizing the KV cache").  One 64-lane wave per new row: 72 chunks of eight
// bf16 values, a wave max for the per-token scale, then 8-byte code stores.
#include "device_common.h"
#include "launch.h"

namespace mla {

template <int SCALE>
__global__ __launch_bounds__(64) void kv_append_kernel(AppendArgs a) {
  const int row = blockIdx.x;  // b * n_new + j
  const int b = row / a.n_new;
  const int j = row - b * a.n_new;
  const int lane = threadIdx.x;
  const int pos = a.seq_lens[b] - a.n_new + j;
  if (pos < 0 || pos >= a.max_blocks * kPage) return;
  int page = a.block_table[(int64_t)b * a.max_blocks + pos / kPage];
  page = min(max(page, 0), a.num_pages - 1);
  const int slot = pos % kPage;

  // 72 chunks of 8 elements; lanes 0..7 take a second chunk
  const u32x4* src = reinterpret_cast<const u32x4*>(a.kv_new + (int64_t)row * kD);
  const int nchunk = lane < 8 ? 2 : 1;
  float x[2][8];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c < nchunk) {
      const u32x4 w = src[lane + 64 * c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[c][2 * e] = float_of(w[e] << 16);
        x[c][2 * e + 1] = float_of(w[e] & 0xffff0000u);
        amax = fmaxf(amax, fmaxf(fabsf(x[c][2 * e]), fabsf(x[c][2 * e + 1])));
      }
    }
  }
  float scale;
  if (SCALE == kScaleToken) {
    amax = wave_max(amax);
    scale = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
  } else {
    scale = a.kv_scale[0];
  }
  uint8_t* dst = a.cache + ((int64_t)page * kPage + slot) * kD;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c < nchunk) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo |= float_to_e4m3(__fdiv_rn(x[c][e], scale)) << (8 * e);
        hi |= float_to_e4m3(__fdiv_rn(x[c][4 + e], scale)) << (8 * e);
      }
      u32x2 v = {lo, hi};
      *reinterpret_cast<u32x2*>(dst + 8 * (lane + 64 * c)) = v;
    }
  }
  if (SCALE == kScaleToken && lane == 0) a.kv_scale[(int64_t)page * kPage + slot] = scale;
}

hipError_t launch_kv_append(const AppendArgs& a, int scale_mode, hipStream_t stream) {
  const dim3 grid(a.B * a.n_new), block(64);
  if (scale_mode == kScaleToken)
    hipLaunchKernelGGL(kv_append_kernel<kScaleToken>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(kv_append_kernel<kScaleTensor>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
