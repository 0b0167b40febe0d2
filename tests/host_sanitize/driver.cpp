// Host-side driver for the sanitizer build of the C ABI (api.hip): argument
// validation, the split planners and the status strings, under
// AddressSanitizer and UndefinedBehaviorSanitizer.  No GPU is touched: every
// call here returns before any HIP call, and the kernel launchers are stubs
// that report failure if ever reached.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>
#include <random>
#include <vector>

#include "../../include/mla_decode.h"
#include "../../long_context_mla_amd/csrc/launch.h"

static int failures = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main() {
  void* p = reinterpret_cast<void*>(0x1000);  // never dereferenced on the host
  int32_t* ip = static_cast<int32_t*>(p);
  float* fp = static_cast<float*>(p);
  // validation: every case returns before a launch
  EXPECT(mla_decode_paged(nullptr, p, 1, fp, 1, ip, ip, 1, 1, 64, 10, 10, 0.07f, 1, 1, nullptr, nullptr, p, fp,
                          nullptr) == MLA_ERR_NULL_PTR);
  EXPECT(mla_decode_paged(p, p, 1, fp, 1, ip, ip, 1, MLA_MAX_QUERIES + 1, 64, 10, 10, 0.07f, 1, 1, nullptr,
                          nullptr, p, fp, nullptr) == MLA_ERR_BAD_SHAPE);
  EXPECT(mla_decode_paged(p, p, 7, fp, 1, ip, ip, 1, 1, 64, 10, 10, 0.07f, 1, 1, nullptr, nullptr, p, fp,
                          nullptr) == MLA_ERR_UNSUPPORTED);
  EXPECT(mla_decode_paged(p, p, 1, fp, 1, ip, ip, 1, 1, 64, 10, 10, 0.07f, 1 << 16, 1 << 15, p, fp, p, fp,
                          nullptr) == MLA_ERR_BAD_SHAPE);
  EXPECT(mla_decode_paged(p, p, 1, fp, 1, ip, ip, 0, 1, 64, 10, 10, 0.07f, 1, 1, nullptr, nullptr, nullptr,
                          nullptr, nullptr) == MLA_OK);
  EXPECT(mla_decode_paged_append_noalloc(p, 1, p, p, fp, 2, ip, ip, 1, 1, 64, 10, 10, 0.07f, 1,
                                         MLA_NOALLOC_MAX_PARTIAL_ROWS / 64 + 1, p, fp, 1, nullptr) ==
         MLA_ERR_SCRATCH_LIMIT);
  EXPECT(mla_decode_combine(p, fp, ip, 1, 1, 1, 1, 1 << 16, 1 << 15, p, fp, nullptr, nullptr) == MLA_ERR_BAD_SHAPE);
  EXPECT(kv_append_fp8(p, p, fp, 0, ip, ip, 1, 1, 1, 1, nullptr) == MLA_ERR_UNSUPPORTED);
  EXPECT(kv_check_pages(nullptr, 4, ip, nullptr, nullptr, ip, 1, 4, ip, ip, nullptr) == MLA_ERR_NULL_PTR);
  for (int s = -2; s <= 6; ++s) EXPECT(mla_status_string(s) != nullptr);

  // planners over random batches: every page covered, plans fit the grid
  std::mt19937 rng(7);
  for (int trial = 0; trial < 400; ++trial) {
    const int B = 1 + static_cast<int>(rng() % 70);
    const int n_q = 1 + static_cast<int>(rng() % (trial % 10 == 0 ? 600 : 8));
    const int H = 1 + static_cast<int>(rng() % 128);
    const int dtype = static_cast<int>(rng() % 2);
    const int cus = static_cast<int>(rng() % 300);
    std::vector<int32_t> lens(B);
    int64_t total = 0;
    int maxL = 0;
    for (auto& L : lens) {
      L = static_cast<int32_t>(rng() % (trial % 3 == 0 ? 200 : 150000));
      total += L;
      if (L > maxL) maxL = L;
    }
    int pps = 0, ms = 0;
    const int r1 = mla_decode_plan_lens(lens.data(), B, n_q, H, cus, dtype, &pps, &ms);
    EXPECT(r1 == MLA_OK || r1 == MLA_ERR_BAD_SHAPE);
    if (r1 == MLA_OK) {
      EXPECT(pps >= 1 && ms >= 1);
      EXPECT((int64_t)pps * ms >= (maxL + MLA_PAGE_SIZE - 1) / MLA_PAGE_SIZE);
    }
    const int r2 = mla_decode_plan(B, n_q, H, maxL, total, cus, dtype, &pps, &ms);
    EXPECT(r2 == MLA_OK || r2 == MLA_ERR_BAD_SHAPE);
  }
  std::vector<int32_t> bad = {5, -1};
  int pps = 0, ms = 0;
  EXPECT(mla_decode_plan_lens(bad.data(), 2, 1, 64, 0, 1, &pps, &ms) == MLA_ERR_BAD_SHAPE);
  EXPECT(mla_decode_plan_lens(bad.data(), 2, 1, 64, 0, 9, &pps, &ms) == MLA_ERR_UNSUPPORTED);
  // the kernels' workgroup -> work-unit map: every (request, split, row group)
  // exactly once, every field in range, only padding invalid
  for (int B : {1, 2, 3, 7, 16, 32, 64, 100}) {
    for (int ms : {1, 2, 4, 9, 40, 224}) {
      for (int n_rg : {1, 2, 4, 16}) {
        const int64_t grid = mla::decode_grid_size(B, ms, n_rg);
        std::vector<char> seen((size_t)B * ms * n_rg, 0);
        int64_t n_valid = 0;
        for (int64_t i = 0; i < grid; ++i) {
          const mla::WorkUnit w = mla::work_unit_of(i, B, ms, n_rg);
          if (!w.valid) continue;
          ++n_valid;
          const bool ok = w.b >= 0 && w.b < B && w.split >= 0 && w.split < ms && w.rg >= 0 && w.rg < n_rg;
          EXPECT(ok);
          if (!ok) continue;
          char& s = seen[((size_t)w.split * B + w.b) * n_rg + w.rg];
          EXPECT(s == 0);
          s = 1;
        }
        EXPECT(n_valid == (int64_t)B * ms * n_rg);
      }
    }
  }
  std::printf("host sanitizer driver: %d failures\n", failures);
  return failures ? 1 : 0;
}
