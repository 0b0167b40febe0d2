// Internal launcher interface between the C-ABI layer (api.hip) and the kernels.
// Arguments reaching these functions have already been validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct AppendArgs {
  const uint16_t* kv_new;   // bf16 [B, n_new, 576]
  uint8_t* cache;           // e4m3 [num_pages, 64, 576]
  float* kv_scale;          // per token [num_pages, 64] (written) or per tensor [1] (read)
  const int32_t* block_table;
  const int32_t* seq_lens;
  int B, n_new, max_blocks, num_pages;
};

struct CheckArgs {
  const uint32_t* page_tags;       // [num_pages] current tag of each physical page
  const int32_t* block_table;      // [B, max_blocks] page map decode will read
  const int32_t* expected_pages;   // [B, max_blocks] recorded pages (block_table when none are kept)
  const uint32_t* expected_tags;   // [B, max_blocks] recorded tags
  const int32_t* seq_lens;         // [B]
  int32_t* status;                 // [B] written
  int32_t* checked_lens;           // [B] written; may be seq_lens
  int B, max_blocks, num_pages;
};

struct DecodeArgs {
  const uint16_t* q;        // bf16 [B, R, 576], R = n_q * H
  const uint8_t* cache;     // e4m3 or bf16 rows [num_pages, 64, 576]
  const float* kv_scale;
  const int32_t* block_table;
  const int32_t* seq_lens;
  uint16_t* o_part;         // bf16 [B, max_splits, R, 512]
  float* lse_part;          // fp32 [B, max_splits, R]
  uint16_t* out;            // bf16 [B, R, 512]
  float* lse;               // fp32 [B, R]
  int B, n_q, H, R, max_blocks, num_pages, pps, max_splits, n_rg;
  float sm_log2;            // softmax_scale * log2(e)
  // Rows appended in the same launch (FP8 cache only; n_new = 0: none): bf16
  // [B, n_new, 576] at positions seq_lens[b] - n_new .. seq_lens[b] - 1, and
  // the writable cache / per-token scales they go to.
  const uint16_t* kv_new;
  int n_new;
  uint8_t* cache_out;
  float* scale_out;
  int store_rows;           // 0: the appended rows serve this launch only, nothing is stored
  // The page-tag check carried in the same launch (status != null, FP8 only):
  // workgroups from check_from on each check request blockIdx.x - check_from
  // and write its status; the rows above are stored only into pages that pass.
  const uint32_t* page_tags;
  const int32_t* expected_pages;
  const uint32_t* expected_tags;
  int32_t* status;
  int check_from;
};

struct CombineArgs {
  const uint16_t* o_part;   // bf16 [B, max_splits, R, 512]
  const float* lse_part;
  const int32_t* seq_lens;
  uint16_t* out;
  float* lse;
  const int32_t* status;    // [B] or null: requests with a non-zero entry get out = 0, lse = -inf
  int B, R, max_blocks, pps, max_splits;
};

// Rows of the query matrix one decode workgroup owns: 64 on either cache.
int decode_rows_per_group(int cache_kind);
int decode_rows_fp8();

// Compute units of the part (256 in 8 XCDs).  A decode workgroup takes most of
// a CU's LDS, so workgroups 0 .. kCUs-1 of a launch are the ones that start
// together at its beginning.
constexpr int kCUs = 256;

// Workgroups of a decode launch (a 1-D grid): the B * max_splits work units
// (request, split) padded to a multiple of the 8 XCDs, n_rg row groups each.
__host__ __device__ inline int64_t decode_grid_size(int64_t B, int64_t max_splits, int64_t n_rg) {
  return (B * max_splits + 7) / 8 * 8 * n_rg;
}

// The item a decode workgroup works on: item v = (split * B + b) * n_rg + rg
// (split-major).  The hardware hands workgroup i to XCD i % 8 in order of i.
// Within full block k of 64 workgroups, XCD x takes the block's 8 consecutive
// items of chunk (x - k) mod 8, which start together there: the row groups of
// a unit (which read the same pages) and the same split of neighbouring
// requests (which read the same pages when they share a prefix) share one L2.
// The chunk an XCD takes turns with the block, so that requests of unequal
// length spread over all XCDs.  A one-request, one-row-group batch shares
// nothing and goes round robin, as does a last block of fewer than 64.
__host__ __device__ inline int64_t decode_item(int64_t i, int64_t B, int64_t max_splits, int64_t n_rg) {
  const int64_t grid = decode_grid_size(B, max_splits, n_rg);
  const int64_t full = (B > 1 || n_rg > 1) ? grid & ~(int64_t)63 : 0;
  if (i >= full) return i;
  const int64_t k = i >> 6, x = i & 7, t = (i >> 3) & 7;
  return (k << 6) | (((x - k) & 7) << 3) | t;
}

// Workgroup i of a decode launch -> (request b, split, row group rg) of item
// decode_item(i); valid is false for the grid's padding past B * max_splits
// units.  Shared by the kernels and the host-side tests of the map.
struct WorkUnit {
  int b, split, rg;
  bool valid;
};
__host__ __device__ inline WorkUnit work_unit_of(int64_t i, int B, int max_splits, int n_rg) {
  const int v = (int)decode_item(i, B, max_splits, n_rg);
  const int u = v / n_rg;
  WorkUnit w;
  w.rg = v - u * n_rg;
  w.valid = u < B * max_splits;
  w.split = w.valid ? u / B : 0;
  w.b = w.valid ? u - w.split * B : 0;
  return w;
}

hipError_t launch_kv_append(const AppendArgs& a, int scale_mode, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int cache_kind, int scale_mode, hipStream_t stream);
hipError_t launch_decode_fp8(const DecodeArgs& a, int scale_mode, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
hipError_t launch_kv_check(const CheckArgs& a, hipStream_t stream);

}  // namespace mla
