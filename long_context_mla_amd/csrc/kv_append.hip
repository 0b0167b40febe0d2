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
  // a page id outside the pool names no page: nothing is written (clamping it
  // would put the row into another request's page)
  const int page = a.block_table[(int64_t)b * a.max_blocks + pos / kPage];
  if (page < 0 || page >= a.num_pages) return;
  const int slot = pos % kPage;

  u32x2 codes[2];
  const float scale = encode_row_e4m3<SCALE == kScaleToken>(a.kv_new + (int64_t)row * kD, lane,
                                                            SCALE == kScaleToken ? 1.0f : a.kv_scale[0], codes);
  uint8_t* dst = a.cache + ((int64_t)page * kPage + slot) * kD;
  *reinterpret_cast<u32x2*>(dst + 8 * lane) = codes[0];
  if (lane < 8) *reinterpret_cast<u32x2*>(dst + 8 * (lane + 64)) = codes[1];
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
