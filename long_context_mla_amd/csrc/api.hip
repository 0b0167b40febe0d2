// C-ABI entry points declared in include/mla_decode.h: host-side argument
// validation (before any HIP call), split planning, and kernel launches on the
// caller's stream.  No allocation, no synchronisation, no exceptions.  The one
// buffer the library owns is the split-partial scratch of
// mla_decode_paged_append_noalloc below, a static device array.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <functional>
#include <mutex>
#include <queue>
#include <vector>

#include "../../include/mla_decode.h"
#include "device_common.h"
#include "launch.h"

// Split partials of mla_decode_paged_append_noalloc: MLA_NOALLOC_MAX_PARTIAL_ROWS
// rows of 512 bf16 (o), then as many fp32 (lse), in the [B, max_splits, R]
// order of mla_decode_paged's partial buffers.  Every GPU the library runs on
// holds its own copy until the process ends.  Host code never uses this name
// as an address: scratch_partials() resolves each device's copy.
constexpr size_t kScratchOBytes = (size_t)MLA_NOALLOC_MAX_PARTIAL_ROWS * MLA_VALUE_DIM * 2;
constexpr size_t kScratchBytes = kScratchOBytes + (size_t)MLA_NOALLOC_MAX_PARTIAL_ROWS * 4;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int64_t kMaxGrid = 2147483647;

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// The device address of the current device's scratch, looked up once per
// device; the stream must belong to that device.
int scratch_partials(hipStream_t stream, void** o_partial, float** lse_partial) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return MLA_ERR_UNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = 0;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MLA_ERR_HIP;
    if (sdev != dev) return MLA_ERR_UNSUPPORTED;
  }
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_HIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *o_partial = p;
  *lse_partial = reinterpret_cast<float*>(static_cast<uint8_t*>(p) + kScratchOBytes);
  return MLA_OK;
}

hipError_t combine_launch(const void* o_partial, const float* lse_partial, const int32_t* seq_lens,
                          int B, int R, int max_blocks, int pps, int max_splits, void* out, float* lse,
                          const int32_t* status, hipStream_t stream) {
  mla::CombineArgs a;
  a.o_part = static_cast<const uint16_t*>(o_partial);
  a.lse_part = lse_partial;
  a.seq_lens = seq_lens;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.status = status;
  a.B = B;
  a.R = R;
  a.max_blocks = max_blocks;
  a.pps = pps;
  a.max_splits = max_splits;
  return mla::launch_combine(a, stream);
}

bool bad_stream_free_shape(int B, int n_q, int H) {
  return B < 0 || B > 65535 || n_q < 1 || n_q > MLA_MAX_QUERIES || H < 1 || H > MLA_MAX_HEADS;
}

int check_cache_mode(int cache_dtype, int scale_mode) {
  if (cache_dtype != MLA_CACHE_BF16 && cache_dtype != MLA_CACHE_FP8_E4M3) return MLA_ERR_UNSUPPORTED;
  if (scale_mode < MLA_SCALE_NONE || scale_mode > MLA_SCALE_PER_TOKEN) return MLA_ERR_UNSUPPORTED;
  if (cache_dtype == MLA_CACHE_BF16 && scale_mode != MLA_SCALE_NONE) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

// The checks and the launch shared by mla_decode_paged and
// mla_decode_paged_append (kv_new == nullptr, n_new == 0 for the former).
int decode_impl(const void* q, const void* kv_cache, int cache_dtype, const float* kv_scale,
                int scale_mode, const int32_t* block_table, const int32_t* seq_lens, int B, int n_q,
                int H, int max_blocks, int num_pages, float softmax_scale, int pages_per_split,
                int max_splits, void* o_partial, float* lse_partial, void* out, float* lse,
                const void* kv_new, int n_new, int store_rows, void* stream,
                const uint32_t* page_tags = nullptr, const int32_t* expected_pages = nullptr,
                const uint32_t* expected_tags = nullptr, int32_t* status = nullptr,
                bool use_scratch = false, bool dry = false) {
  if (int s = check_cache_mode(cache_dtype, scale_mode)) return s;
  if (bad_stream_free_shape(B, n_q, H)) return MLA_ERR_BAD_SHAPE;
  if (max_blocks < 1 || num_pages < 1 || pages_per_split < 1 || max_splits < 1) return MLA_ERR_BAD_SHAPE;
  if ((int64_t)max_blocks * MLA_PAGE_SIZE > 2147483647LL) return MLA_ERR_BAD_SHAPE;
  // split starts s * pages_per_split stay inside int
  if ((int64_t)pages_per_split * max_splits > 2147483647LL) return MLA_ERR_BAD_SHAPE;
  if (!std::isfinite(softmax_scale)) return MLA_ERR_BAD_SHAPE;
  const int R = n_q * H;
  const int rows = mla::decode_rows_per_group(cache_dtype == MLA_CACHE_FP8_E4M3 ? mla::kFp8 : mla::kBf16);
  const int n_rg = (R + rows - 1) / rows;
  if (mla::decode_grid_size(B, max_splits, n_rg) + (status ? B : 0) > kMaxGrid) return MLA_ERR_BAD_SHAPE;
  if (B == 0) return MLA_OK;
  if (!q || !kv_cache || !block_table || !seq_lens) return MLA_ERR_NULL_PTR;
  if (scale_mode != MLA_SCALE_NONE && !kv_scale) return MLA_ERR_NULL_PTR;
  if (max_splits == 1 && (!out || !lse)) return MLA_ERR_NULL_PTR;
  if (use_scratch) {
    // partials in the library's scratch, merged into out / lse in this call
    if (!out || !lse) return MLA_ERR_NULL_PTR;
    if (max_splits > 1) {
      if ((int64_t)B * max_splits * R > MLA_NOALLOC_MAX_PARTIAL_ROWS) return MLA_ERR_SCRATCH_LIMIT;
      if (int s = scratch_partials(static_cast<hipStream_t>(stream), &o_partial, &lse_partial)) return s;
    }
  } else if (max_splits > 1 && (!o_partial || !lse_partial)) {
    return MLA_ERR_NULL_PTR;
  }
  if (dry) return MLA_OK;  // the arguments pass; nothing launched
  mla::DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.cache = static_cast<const uint8_t*>(kv_cache);
  a.kv_scale = kv_scale;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.o_part = static_cast<uint16_t*>(o_partial);
  a.lse_part = lse_partial;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.B = B;
  a.n_q = n_q;
  a.H = H;
  a.R = R;
  a.max_blocks = max_blocks;
  a.num_pages = num_pages;
  a.pps = pages_per_split;
  a.max_splits = max_splits;
  a.n_rg = n_rg;
  a.sm_log2 = softmax_scale * mla::kLog2e;
  a.kv_new = static_cast<const uint16_t*>(kv_new);
  a.n_new = n_new;
  a.cache_out = static_cast<uint8_t*>(const_cast<void*>(kv_cache));
  a.scale_out = const_cast<float*>(kv_scale);
  a.store_rows = store_rows ? 1 : 0;
  a.page_tags = page_tags;
  a.expected_pages = expected_pages ? expected_pages : block_table;  // no record: the map is the record
  a.expected_tags = expected_tags;
  a.status = status;
  a.check_from = (int)mla::decode_grid_size(B, max_splits, n_rg);
  const int kind = cache_dtype == MLA_CACHE_FP8_E4M3 ? mla::kFp8 : mla::kBf16;
  hipError_t e = mla::launch_decode(a, kind, scale_mode, static_cast<hipStream_t>(stream));
  if (e == hipSuccess && use_scratch && max_splits > 1)
    e = combine_launch(o_partial, lse_partial, seq_lens, B, R, max_blocks, pages_per_split, max_splits,
                       out, lse, nullptr, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// Appends of more than this many rows per request are encoded and stored by
// their own kv_append launch before the decode: in the decode launch every
// row-group workgroup whose pages hold new rows encodes them into its LDS copy,
// which for a chunk of hundreds of rows costs more than a launch (a 512-row
// extend chunk over 16k tokens: 1,583 against 992 us per step).  Only where
// the rows are stored and no page check runs in the launch: the codes, scales
// and stored bytes are then the same, and the decode reads them back.
constexpr int kFusedAppendMax = 16;

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL_PTR: return "null pointer argument";
    case MLA_ERR_BAD_SHAPE: return "bad shape or size argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MLA_ERR_HIP: return "HIP launch error";
    case MLA_ERR_SCRATCH_LIMIT: return "split partials exceed the fixed scratch of the allocation-free call";
    default: return "unknown status";
  }
}

int kv_append_fp8(const void* kv_new, void* kv_cache, float* kv_scale, int scale_mode,
                  const int32_t* block_table, const int32_t* seq_lens, int B, int n_new,
                  int max_blocks, int num_pages, void* stream) {
  if (scale_mode != MLA_SCALE_PER_TENSOR && scale_mode != MLA_SCALE_PER_TOKEN) return MLA_ERR_UNSUPPORTED;
  if (B < 0 || n_new < 0 || max_blocks < 1 || num_pages < 1) return MLA_ERR_BAD_SHAPE;
  if ((int64_t)B * n_new > kMaxGrid) return MLA_ERR_BAD_SHAPE;
  if ((int64_t)max_blocks * MLA_PAGE_SIZE > 2147483647LL) return MLA_ERR_BAD_SHAPE;
  if (B == 0 || n_new == 0) return MLA_OK;
  if (!kv_new || !kv_cache || !kv_scale || !block_table || !seq_lens) return MLA_ERR_NULL_PTR;
  mla::AppendArgs a;
  a.kv_new = static_cast<const uint16_t*>(kv_new);
  a.cache = static_cast<uint8_t*>(kv_cache);
  a.kv_scale = kv_scale;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.B = B;
  a.n_new = n_new;
  a.max_blocks = max_blocks;
  a.num_pages = num_pages;
  const hipError_t e = mla::launch_kv_append(a, scale_mode, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int kv_check_pages(const uint32_t* page_tags, int num_pages, const int32_t* block_table,
                   const int32_t* expected_pages, const uint32_t* expected_tags,
                   const int32_t* seq_lens, int B, int max_blocks, int32_t* status,
                   int32_t* checked_lens, void* stream) {
  if (B < 0 || max_blocks < 1 || num_pages < 1) return MLA_ERR_BAD_SHAPE;
  if ((int64_t)max_blocks * MLA_PAGE_SIZE > 2147483647LL) return MLA_ERR_BAD_SHAPE;
  if (B == 0) return MLA_OK;
  if (!page_tags || !block_table || !expected_tags || !seq_lens || !status || !checked_lens)
    return MLA_ERR_NULL_PTR;
  mla::CheckArgs a;
  a.page_tags = page_tags;
  a.block_table = block_table;
  a.expected_pages = expected_pages ? expected_pages : block_table;  // no record: the map is the record
  a.expected_tags = expected_tags;
  a.seq_lens = seq_lens;
  a.status = status;
  a.checked_lens = checked_lens;
  a.B = B;
  a.max_blocks = max_blocks;
  a.num_pages = num_pages;
  const hipError_t e = mla::launch_kv_check(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_decode_paged(const void* q, const void* kv_cache, int cache_dtype, const float* kv_scale,
                     int scale_mode, const int32_t* block_table, const int32_t* seq_lens, int B,
                     int n_q, int H, int max_blocks, int num_pages, float softmax_scale,
                     int pages_per_split, int max_splits, void* o_partial, float* lse_partial,
                     void* out, float* lse, void* stream) {
  return decode_impl(q, kv_cache, cache_dtype, kv_scale, scale_mode, block_table, seq_lens, B, n_q, H,
                     max_blocks, num_pages, softmax_scale, pages_per_split, max_splits, o_partial,
                     lse_partial, out, lse, nullptr, 0, 1, stream);
}

int mla_decode_paged_append(const void* kv_new, int n_new, const void* q, void* kv_cache,
                            float* kv_scale, int scale_mode, const int32_t* block_table,
                            const int32_t* seq_lens, int B, int n_q, int H, int max_blocks,
                            int num_pages, float softmax_scale, int pages_per_split, int max_splits,
                            void* o_partial, float* lse_partial, void* out, float* lse, int store_rows,
                            void* stream) {
  if (scale_mode != MLA_SCALE_PER_TENSOR && scale_mode != MLA_SCALE_PER_TOKEN) return MLA_ERR_UNSUPPORTED;
  if (n_new < 0) return MLA_ERR_BAD_SHAPE;
  if (n_new > 0 && B > 0 && !kv_new) return MLA_ERR_NULL_PTR;
  if (store_rows && n_new > kFusedAppendMax && B > 0 && (int64_t)B * n_new <= kMaxGrid) {
    if (int s = decode_impl(q, kv_cache, MLA_CACHE_FP8_E4M3, kv_scale, scale_mode, block_table, seq_lens, B,
                            n_q, H, max_blocks, num_pages, softmax_scale, pages_per_split, max_splits,
                            o_partial, lse_partial, out, lse, nullptr, 0, 1, stream, nullptr, nullptr,
                            nullptr, nullptr, false, true))
      return s;
    if (int s = kv_append_fp8(kv_new, kv_cache, kv_scale, scale_mode, block_table, seq_lens, B, n_new,
                              max_blocks, num_pages, stream))
      return s;
    n_new = 0;
  }
  return decode_impl(q, kv_cache, MLA_CACHE_FP8_E4M3, kv_scale, scale_mode, block_table, seq_lens, B,
                     n_q, H, max_blocks, num_pages, softmax_scale, pages_per_split, max_splits,
                     o_partial, lse_partial, out, lse, n_new > 0 ? kv_new : nullptr, n_new, store_rows,
                     stream);
}

int mla_decode_paged_append_checked(const void* kv_new, int n_new, const void* q, void* kv_cache,
                                    float* kv_scale, int scale_mode, const int32_t* block_table,
                                    const int32_t* seq_lens, int B, int n_q, int H, int max_blocks,
                                    int num_pages, float softmax_scale, int pages_per_split,
                                    int max_splits, void* o_partial, float* lse_partial,
                                    const uint32_t* page_tags, const int32_t* expected_pages,
                                    const uint32_t* expected_tags, int32_t* status, void* stream) {
  if (scale_mode != MLA_SCALE_PER_TENSOR && scale_mode != MLA_SCALE_PER_TOKEN) return MLA_ERR_UNSUPPORTED;
  if (max_splits < 2) return MLA_ERR_UNSUPPORTED;  // the flagged rows are masked by the combine
  if (n_new < 0) return MLA_ERR_BAD_SHAPE;
  if (B > 0 && ((n_new > 0 && !kv_new) || !page_tags || !expected_tags || !status)) return MLA_ERR_NULL_PTR;
  return decode_impl(q, kv_cache, MLA_CACHE_FP8_E4M3, kv_scale, scale_mode, block_table, seq_lens, B,
                     n_q, H, max_blocks, num_pages, softmax_scale, pages_per_split, max_splits,
                     o_partial, lse_partial, nullptr, nullptr, n_new > 0 ? kv_new : nullptr, n_new, 1,
                     stream, page_tags, expected_pages, expected_tags, status);
}

int mla_decode_paged_append_noalloc(const void* kv_new, int n_new, const void* q, void* kv_cache,
                                    float* kv_scale, int scale_mode, const int32_t* block_table,
                                    const int32_t* seq_lens, int B, int n_q, int H, int max_blocks,
                                    int num_pages, float softmax_scale, int pages_per_split,
                                    int max_splits, void* out, float* lse, int store_rows,
                                    void* stream) {
  if (scale_mode != MLA_SCALE_PER_TENSOR && scale_mode != MLA_SCALE_PER_TOKEN) return MLA_ERR_UNSUPPORTED;
  if (n_new < 0) return MLA_ERR_BAD_SHAPE;
  if (n_new > 0 && B > 0 && !kv_new) return MLA_ERR_NULL_PTR;
  if (store_rows && n_new > kFusedAppendMax && B > 0 && (int64_t)B * n_new <= kMaxGrid) {
    if (int s = decode_impl(q, kv_cache, MLA_CACHE_FP8_E4M3, kv_scale, scale_mode, block_table, seq_lens, B,
                            n_q, H, max_blocks, num_pages, softmax_scale, pages_per_split, max_splits,
                            nullptr, nullptr, out, lse, nullptr, 0, 1, stream, nullptr, nullptr, nullptr,
                            nullptr, true, true))
      return s;
    if (int s = kv_append_fp8(kv_new, kv_cache, kv_scale, scale_mode, block_table, seq_lens, B, n_new,
                              max_blocks, num_pages, stream))
      return s;
    n_new = 0;
  }
  return decode_impl(q, kv_cache, MLA_CACHE_FP8_E4M3, kv_scale, scale_mode, block_table, seq_lens, B,
                     n_q, H, max_blocks, num_pages, softmax_scale, pages_per_split, max_splits, nullptr,
                     nullptr, out, lse, n_new > 0 ? kv_new : nullptr, n_new, store_rows, stream, nullptr,
                     nullptr, nullptr, nullptr, true);
}

int mla_decode_combine(const void* o_partial, const float* lse_partial, const int32_t* seq_lens,
                       int B, int n_q, int H, int max_blocks, int pages_per_split, int max_splits,
                       void* out, float* lse, const int32_t* status, void* stream) {
  if (bad_stream_free_shape(B, n_q, H)) return MLA_ERR_BAD_SHAPE;
  if (max_blocks < 1 || pages_per_split < 1 || max_splits < 1) return MLA_ERR_BAD_SHAPE;
  if ((int64_t)pages_per_split * max_splits > 2147483647LL) return MLA_ERR_BAD_SHAPE;
  if ((int64_t)B * n_q * H * 4 > kMaxGrid) return MLA_ERR_BAD_SHAPE;
  if (B == 0) return MLA_OK;
  if (!o_partial || !lse_partial || !seq_lens || !out || !lse) return MLA_ERR_NULL_PTR;
  const hipError_t e = combine_launch(o_partial, lse_partial, seq_lens, B, n_q * H, max_blocks,
                                      pages_per_split, max_splits, out, lse, status,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_decode_plan(int B, int n_q, int H, int max_seq_len, int64_t total_seq_len, int num_cus,
                    int cache_dtype, int* pages_per_split, int* max_splits) {
  if (!pages_per_split || !max_splits) return MLA_ERR_NULL_PTR;
  if (bad_stream_free_shape(B, n_q, H) || max_seq_len < 0 || total_seq_len < 0 || num_cus < 0)
    return MLA_ERR_BAD_SHAPE;
  if (cache_dtype != MLA_CACHE_BF16 && cache_dtype != MLA_CACHE_FP8_E4M3) return MLA_ERR_UNSUPPORTED;
  if (num_cus == 0) num_cus = 256;
  const int R = n_q * H;
  const int rows = mla::decode_rows_per_group(cache_dtype == MLA_CACHE_FP8_E4M3 ? mla::kFp8 : mla::kBf16);
  const int64_t n_rg = (R + rows - 1) / rows;
  const int64_t max_pages = (max_seq_len + MLA_PAGE_SIZE - 1) / MLA_PAGE_SIZE;
  // pages of the batch, counting a partial last page per request
  const int64_t total_pages = (total_seq_len + MLA_PAGE_SIZE - 1) / MLA_PAGE_SIZE + B;
  if (max_pages == 0) {
    *pages_per_split = 1;
    *max_splits = 1;
    return MLA_OK;
  }
  // one workgroup per CU, each with about the same number of pages
  int64_t pps = (total_pages * n_rg + num_cus - 1) / num_cus;
  if (pps < 1) pps = 1;
  if (pps > max_pages) pps = max_pages;
  int64_t splits = (max_pages + pps - 1) / pps;
  if (mla::decode_grid_size(B, splits, n_rg) > kMaxGrid) return MLA_ERR_BAD_SHAPE;
  *pages_per_split = (int)pps;
  *max_splits = (int)splits;
  return MLA_OK;
}

int mla_decode_plan_lens(const int32_t* seq_lens, int B, int n_q, int H, int num_cus, int cache_dtype,
                         int* pages_per_split, int* max_splits) {
  if (!pages_per_split || !max_splits || (B > 0 && !seq_lens)) return MLA_ERR_NULL_PTR;
  if (bad_stream_free_shape(B, n_q, H) || num_cus < 0) return MLA_ERR_BAD_SHAPE;
  if (cache_dtype != MLA_CACHE_BF16 && cache_dtype != MLA_CACHE_FP8_E4M3) return MLA_ERR_UNSUPPORTED;
  if (num_cus == 0) num_cus = 256;
  const int R = n_q * H;
  const int rows = mla::decode_rows_per_group(cache_dtype == MLA_CACHE_FP8_E4M3 ? mla::kFp8 : mla::kBf16);
  const int n_rg = (R + rows - 1) / rows;
  std::vector<int> pages(B);
  int max_pages = 0;
  for (int b = 0; b < B; ++b) {
    if (seq_lens[b] < 0) return MLA_ERR_BAD_SHAPE;
    pages[b] = (int)(((int64_t)seq_lens[b] + MLA_PAGE_SIZE - 1) / MLA_PAGE_SIZE);
    max_pages = std::max(max_pages, pages[b]);
  }
  if (max_pages == 0) {
    *pages_per_split = 1;
    *max_splits = 1;
    return MLA_OK;
  }
  // workgroups of a plan: every request takes at least one unit (an empty
  // one writes its zero output), n_rg workgroups per unit
  auto workgroups = [&](int pps) {
    int64_t u = 0;
    for (int b = 0; b < B; ++b) u += std::max(1, (pages[b] + pps - 1) / pps);
    return u * n_rg;
  };
  // Estimated duration of a plan, in page times.  Workgroup i goes to XCD
  // i % 8, in order of i, and works on item decode_item(i) (the kernels'
  // order); it waits there for the first of its num_cus / 8 compute units to
  // come free (one workgroup per unit at a time) and costs its pages plus a
  // small fixed start and end.  Workgroups past a request's last page exit at
  // once and are skipped.  (Fitted by measurement on MI355X.  The model sees
  // neither the L2 sharing of co-scheduled workgroups nor a page interval
  // that shortens as fewer units copy at once: on the batched workloads its
  // pick measured within 3-6 % of the fastest split length found by a sweep.)
  constexpr int64_t kFixedPages = 2;
  const int per_xcd = std::max(1, num_cus / 8);
  auto makespan = [&](int pps) {
    const int ms = (max_pages + pps - 1) / pps;
    using MinHeap = std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>>;
    std::vector<MinHeap> free_at(8);
    for (auto& h : free_at)
      for (int c = 0; c < per_xcd; ++c) h.push(0);
    int64_t end = 0;
    const int64_t grid = mla::decode_grid_size(B, ms, n_rg);
    for (int64_t i = 0; i < grid; ++i) {
      const int64_t u = mla::decode_item(i, B, ms, n_rg) / n_rg;
      if (u >= (int64_t)B * ms) continue;
      const int split = (int)(u / B), b = (int)(u - (int64_t)split * B);
      const int n = std::max(0, std::min(pages[b], (split + 1) * pps) - split * pps);
      if (n == 0 && !(split == 0 && pages[b] == 0)) continue;
      MinHeap& h = free_at[i & 7];
      const int64_t t = h.top() + kFixedPages + n;
      h.pop();
      h.push(t);
      end = std::max(end, t);
    }
    return end;
  };
  // candidates: the smallest split length that fits the workgroups into one,
  // two, three or four rounds of the compute units.  For a batch of several
  // requests with one row group each, only three or four rounds: there the
  // longer splits of one or two rounds measured 5-12 % slower than this model
  // puts them (32 requests of 60k-140k tokens: 498-502 us at 40-65 pages per
  // split, 521 us at 70, 557 us at 103), while among the others it ranked the
  // fastest plan first or within 3 %.
  int best = max_pages;
  int64_t best_t = makespan(max_pages);
  const int first_rounds = (B > 1 && n_rg == 1) ? 3 : 1;
  if (first_rounds > 1) best_t = INT64_MAX;
  for (int rounds = first_rounds; rounds <= 4; ++rounds) {
    int lo = 1, hi = max_pages;
    while (lo < hi) {
      const int mid = lo + (hi - lo) / 2;
      if (workgroups(mid) <= (int64_t)rounds * num_cus) hi = mid; else lo = mid + 1;
    }
    const int64_t t = makespan(lo);
    if (t < best_t || (t == best_t && lo > best)) {
      best = lo;
      best_t = t;
    }
  }
  const int ms = (max_pages + best - 1) / best;
  if (mla::decode_grid_size(B, ms, n_rg) > kMaxGrid) return MLA_ERR_BAD_SHAPE;
  *pages_per_split = best;
  *max_splits = ms;
  return MLA_OK;
}

}  // extern "C"
