// mla_decode_paged, FP8 cache: split-KV decode attention with specialised
// waves.  Computes what mla_decode.hip describes (one 576-element latent row
// per token as key and value, "How to serve trillions of tokens for
// trillion-parameter coding agents", sections "First, understand the workload"
// and "Tensor parallel was the best parallelism strategy for maximum
// interactivity"; an e4m3 cache converted as it is read, "Smaller, faster,
// safer: running Kimi and GLM at scale", section "Quantizing the KV cache").
//
// gfx950 design: one 512-thread workgroup (8 waves, two per SIMD) per
// (request, split, group of 32 query rows), one per CU.  The two waves of a
// SIMD do different work on different pages, so that one's stalls (LDS
// latency, conversions, the softmax) are covered by the other's MFMAs:
//  * score waves 0..3: wave w copies tokens 16w..16w+15 of each page HBM ->
//    LDS (LDS-DMA), computes their scores S^T = K Q^T for all 32 rows
//    (query held in VGPRs), the softmax weights P (bf16, into LDS) and the sums;
//  * output waves 4..7: wave 4+j accumulates O[32 rows][128j .. 128j+127] +=
//    P V over the previous page, V being the first 512 columns of the same
//    staged rows (transposing LDS reads).
// One barrier per page separates "scores of page p" from "P V of page p".
// The two roles run separate loops with the same sequence of barriers, so the
// query (score waves) and the accumulators (output waves) never need registers
// at the same time.  Two waves per SIMD leave 256 registers per wave; the
// kernel uses VGPRs only (no AGPRs), so all 256 are available to either role.
//
// mla_decode_paged_append runs the same kernel with the step's new rows: the
// score wave that owns a new row's slot encodes it into its LDS copy of the
// page (as kv_append_fp8 would), and row group 0 writes it to the cache.
//
// Softmax: one fixed reference per row and split (the first page's maximum),
// weights 2^(y - m0); a weight above 2^64 restarts the split with a larger
// reference (all waves together).  The output divides by the sum of the bf16
// weights that P V used; the LSE uses the exact fp32 sum.
#include <type_traits>

#include "decode_tile.h"
#include "page_check.h"
#include "device_common.h"
#include "launch.h"

namespace mla {

// CHECKED: the launch also carries the page-tag check (a.status != null).
template <int SCALE, bool CHECKED>
__global__ __launch_bounds__(512, 1) void decode_fp8_kernel(DecodeArgs a) {
  using T = Tile<kFp8>;
  // LDS layout of a staged page (36 16-byte chunks per token): token t's
  // chunk c sits in 16-byte slot pslot(t, c).  Each 16-token quarter (the
  // tokens one score wave copies and reads) takes 576 consecutive slots, in
  // nine groups of 64: group c / 4 holds chunks 4(c / 4) .. +3 of the 16
  // tokens, four per token, the chunk's two low bits XORed with
  // F(t % 16) = {0, 2, 3, 1}[(t % 16) / 4].  One page copy instruction then
  // fills one group (lane l: token l / 4, chunk (l % 4) ^ F), and both the
  // QK^T operand reads (16 B: token, chunk) and the transposing P V reads
  // (8 B: 8 tokens of one chunk) hit distinct LDS banks.
  auto pswz = [](int tl) { return (0x78 >> (2 * ((tl >> 2) & 3))) & 3; };
  auto pslot = [&](int t, int c) {
    const int tl = t & 15;
    return (t >> 4) * 576 + (c >> 2) * 64 + tl * 4 + ((c & 3) ^ pswz(tl));
  };
  static_assert(T::NBUF == 4 && T::DIST == 2, "four page buffers, two pages in flight");
  __shared__ __attribute__((aligned(16))) uint8_t s_kv[T::NBUF][T::PAGE_BYTES];
  __shared__ __attribute__((aligned(16))) float s_scale[T::NBUF][kPage];
  __shared__ __attribute__((aligned(16))) uint8_t s_p[2][kRows * T::PSTRIDE];
  __shared__ float s_red[4][kRows];   // per-score-wave row maxima (first page, restarts)
  __shared__ float s_lsum[4][kRows];
  __shared__ float s_lnrm[4][kRows];
  __shared__ float s_m0[kRows];
  __shared__ __attribute__((aligned(16))) uint8_t s_flag[2][4];  // [page parity][score wave]

  // Workgroups past the decode's carry the page-tag check, one per request.
  // The attention above does not wait for them: flagged requests are masked
  // by mla_decode_combine (a later launch), and each row store below checks
  // the page it writes on its own.
  if (CHECKED && (int)blockIdx.x >= a.check_from) {
    CheckArgs c;
    c.page_tags = a.page_tags;
    c.block_table = a.block_table;
    c.expected_pages = a.expected_pages;
    c.expected_tags = a.expected_tags;
    c.seq_lens = a.seq_lens;
    c.status = a.status;
    c.checked_lens = nullptr;
    c.B = a.B;
    c.max_blocks = a.max_blocks;
    c.num_pages = a.num_pages;
    const int cb = (int)blockIdx.x - a.check_from;
    const int st = check_request<512>(c, cb, a.seq_lens[cb], reinterpret_cast<int*>(&s_red[0][0]));
    if (threadIdx.x == 0) a.status[cb] = st;
    return;
  }

  // One round trip for the launch arguments the first loads need: without
  // this the compiler fetches them in dependent batches.
  asm volatile("" :: "s"(a.q), "s"(a.block_table), "s"(a.seq_lens), "s"(a.n_rg), "s"(a.max_blocks));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool scorer = wave < 4;
  const int qw = wave & 3;  // index within the role
  const int m = lane & 15, g = lane >> 4;
  const WorkUnit wu = decode_work_unit(a.B, a.max_splits, a.n_rg);
  if (!wu.valid) return;
  const int b = wu.b, split = wu.split, rg = wu.rg;
  const int r0 = rg * kRows;
  const int p_begin = split * a.pps;
  const int64_t bt_row = (int64_t)b * a.max_blocks;
  constexpr int QBUF = T::NBUF - 1;
  constexpr int kQueryLoads = 9;  // 16-byte query copies per score wave (32 rows x 1,152 B / 4 waves)

  // Before anything waits, the score waves issue the two loads that depend on
  // the launch arguments alone, so that their latencies overlap the length's:
  //  * the split's first 64 page ids (bounded by the table row, not yet by the
  //    length), one per lane;
  //  * the query of the group's 32 rows, HBM -> LDS in one coalesced copy
  //    shared by the four score waves, into the page buffer that stays free
  //    until the third page copy.  Row r's 16-byte chunk c (72 per row) goes to
  //    slot r * 72 + (c ^ ((r / 2) % 8)), which makes the operand reads below
  //    free of bank conflicts.  Rows past R repeat row R - 1 (results dropped).
  // Every load of page ids is inline asm, awaited explicitly with the result
  // tied to the wait: a load the compiler tracks would make it wait for all
  // copies in flight before each later readlane of the ids.
  int ids = 0;
  if (scorer) {
    const int32_t* id_src = a.block_table + bt_row + min(p_begin + lane, a.max_blocks - 1);
    asm volatile("global_load_dword %0, %1, off" : "=v"(ids) : "v"(id_src) : "memory");
    const uint16_t* qbase = a.q + ((int64_t)b * a.R + r0) * kD;
    const int rmax = a.R - 1 - r0;
    const uint32_t qlds = lds_addr(&s_kv[QBUF][0]);
#pragma unroll
    for (int j = 0; j < kQueryLoads; ++j) {
      const int slot = (qw * 9 + j) * 64 + lane;  // 2304 slots = 32 rows x 72 chunks
      const int r = slot / 72;
      const int c = (slot - r * 72) ^ ((r >> 1) & 7);
      lds_dma16(qbase, (uint32_t)(min(r, rmax) * (kD * 2) + c * 16), qlds + (qw * 9 + j) * 1024);
    }
  }
  const int L = min(max(load_const(a.seq_lens, b), 0), a.max_blocks * kPage);
  const int n_pages = (L + kPage - 1) / kPage;

  if (p_begin >= n_pages) {
    // Nothing to read.  Only an empty request's first split reports it; the
    // combine never reads splits past a request's last page.
    if (scorer) wait_vmcnt<0>();  // the query copy lands before the workgroup ends
    if (n_pages == 0 && split == 0) {
      for (int e = threadIdx.x; e < kRows * kDV; e += 512) {
        const int r = r0 + e / kDV;
        if (r >= a.R) break;
        if (a.max_splits == 1)
          a.out[((int64_t)b * a.R + r) * kDV + e % kDV] = 0;
        else
          a.o_part[((int64_t)b * a.max_splits * a.R + r) * kDV + e % kDV] = 0;
      }
      for (int r = r0 + threadIdx.x; r < min(r0 + kRows, a.R); r += 512) {
        if (a.max_splits == 1)
          a.lse[(int64_t)b * a.R + r] = -INFINITY;
        else
          a.lse_part[(int64_t)b * a.max_splits * a.R + r] = -INFINITY;
      }
    }
    return;
  }
  const int p_end = split == a.max_splits - 1 ? n_pages : min(n_pages, p_begin + a.pps);
  const int n_it = p_end - p_begin;
  const float tscale = SCALE == kScaleTensor ? load_const(a.kv_scale, 0) : 1.0f;
  bool have_ref = false;
  int restarts = 0;
  // The four score waves' restart flags of page it, one byte each, read as one
  // word.  They are read right after the barrier that publishes them and
  // looked at only after the next block of MFMA work has been issued:
  // settle() ties the word to that point, so the LDS latency of the read is
  // not waited for at the barrier.
  auto flag_words = [&](int it) { return *reinterpret_cast<const uint32_t*>(&s_flag[it & 1][0]); };
  auto settle = [](uint32_t& f) {
    asm volatile("" : "+v"(f));
    f = __builtin_amdgcn_readfirstlane(f);  // uniform again for the branch on it
  };
  auto restart_asked = [&](uint32_t f) { return f != 0u && restarts < kMaxRestarts; };

  if (scorer) {
    // =====================================================================
    // score waves
    // =====================================================================
    const float coef = a.sm_log2 * tscale;
    // Page ids of the split, 64 at a time, one per lane; picked out with
    // readlane so the DMA issue never waits on a scalar load.  Ids past the
    // split are never used; every used one is clamped to the pool.  The first
    // chunk was requested at the start, before the wave's nine query copies:
    // loads complete in order, so waiting until nine remain waits for the ids
    // alone and the first pages' copies go out while the query still lands.
    // Later chunks, and the first again on a restart, wait for themselves.
    static_assert(kQueryLoads == 9, "the wait below counts the query copies");
    asm volatile("s_waitcnt vmcnt(9)" : "+v"(ids) :: "memory");
    int id_chunk = 0;
    auto reload_ids = [&](int chunk) {
      id_chunk = chunk;
      const int32_t* src = a.block_table + bt_row + min(p_begin + (chunk << 6) + lane, p_end - 1);
      asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(ids) : "v"(src) : "memory");
    };

    // causal limit of this lane's rows rb*16 + m: row i*H + h sees tokens
    // t < L - n_q + i + 1; lim_lo is the first token any real row of the group
    // masks, so earlier pages need no mask (rows past R only pad the group)
    int lim[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = r0 + rb * 16 + m;
      lim[rb] = row < a.R ? L - a.n_q + row / a.H + 1 : 0;
    }
    const int lim_lo = L - a.n_q + r0 / a.H + 1;

    constexpr int LPP = T::LOADS + (SCALE == kScaleToken ? 1 : 0);  // loads per page per wave
    // wave w copies tokens 16w .. 16w+15 (the rows its own QK^T reads): copy
    // instruction j fills slot group j of its quarter, lane l taking token
    // 16w + l/4's chunk 4j + ((l % 4) ^ F), at source byte goff + 64 j
    static_assert(T::LOADS == 9 && T::ROW_BYTES == 576, "nine copies of 16 tokens x 4 chunks");
    const uint32_t goff =
        (uint32_t)((qw * 16 + (lane >> 2)) * T::ROW_BYTES + ((lane & 3) ^ pswz(lane >> 2)) * 16);
    // Page p_begin + it (and its scales) HBM -> its LDS buffer, two pages
    // ahead of its use.  dma_page picks the page and copies the scales;
    // dma_load(j) issues this wave's j-th 16-byte load of it.  Inside the loop
    // the nine loads ride between the QK^T MFMAs: issued in one burst, the four
    // score waves' 36 loads back up the CU's address path and stall the wave.
    const uint8_t* dma_src = a.cache;
    uint32_t dma_dst = 0;
    auto dma_page = [&](int it) {
      if ((it >> 6) != id_chunk) reload_ids(it >> 6);
      const int pg = min(max(__builtin_amdgcn_readlane(ids, it & 63), 0), a.num_pages - 1);
      dma_src = a.cache + (int64_t)pg * T::PAGE_BYTES;
      dma_dst = lds_addr(&s_kv[it % T::NBUF][0]) + qw * T::LOADS * 1024;
      // the scales of the wave's own 16 tokens only: a row appended in this
      // launch overwrites its scale in LDS after the wave's wait, and another
      // wave's copy of the same word could still land after that
      if (SCALE == kScaleToken && lane < 16)
        lds_dma4(a.kv_scale + (int64_t)pg * kPage + qw * 16, lane * 4, lds_addr(&s_scale[it % T::NBUF][qw * 16]));
    };
    auto dma_load = [&](int j) { lds_dma16(dma_src + 64 * j, goff, dma_dst + j * 1024); };
    auto prologue = [&]() {
#pragma unroll
      for (int k = 0; k < T::DIST; ++k)
        if (k < n_it) {
          dma_page(k);
#pragma unroll
          for (int j = 0; j < T::LOADS; ++j) dma_load(j);
        }
    };
    prologue();

    // Query operands LDS -> VGPRs: lane (m, g) holds rows rb*16 + m and, for
    // k-block kb, dims 64(kb/2) + 16g + 8(kb%2) .. +8; k-blocks 2i and 2i+1
    // take the 16 consecutive dims of one 16-byte FP8 chunk of K.
    if (n_it >= 2)
      wait_vmcnt<2 * LPP>();
    else
      wait_vmcnt<LPP>();
    __syncthreads();  // (1) every score wave's share of the query is in LDS
    bf16x8 qop[2][kD / 32];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = rb * 16 + m;
#pragma unroll
      for (int kb = 0; kb < kD / 32; ++kb) {
        const int c = 8 * (kb >> 1) + 2 * g + (kb & 1);
        qop[rb][kb] = *reinterpret_cast<const bf16x8*>(&s_kv[QBUF][(row * 72 + (c ^ ((row >> 1) & 7))) * 16]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the query buffer may be overwritten

    float m0[2] = {-INFINITY, -INFINITY};   // log2-domain reference of this lane's rows
    float ymax[2] = {-INFINITY, -INFINITY};  // running max of score - reference
    float lsum[2] = {0.0f, 0.0f};           // this lane's share of the softmax sums (fp32 P)
    float lnrm[2] = {0.0f, 0.0f};           // the same over the bf16-rounded P that PV uses
    const int tok = qw * 16 + m;            // this lane's token in QK^T
    const uint32_t klane = (uint32_t)(pslot(tok, g) * 16);  // chunk 4i + g at + 1024 i
    constexpr int KB = kD / 32;
    u32x4 kraw[KB / 2];  // this wave's K bytes of the next page, read ahead

    // Rows appended in this launch that fall among this wave's 16 tokens of
    // page it: the wave encodes each one exactly as kv_append_fp8 does and
    // puts it over the row the copy brought (the cache still held the old
    // contents); row group 0 also writes it, and its per-token scale, to the
    // cache for later steps (unless the caller stores the rows itself).  Both row groups compute the same bytes, so it
    // does not matter which copy the other group's page read saw.
    auto patch_new_rows = [&](int it, uint8_t* kv) {
      const int t_first = (p_begin + it) * kPage + qw * 16;
      const int first_new = L - a.n_new;
      const int lo = max(first_new, t_first), hi = min(L, t_first + 16);
      for (int pos = lo; pos < hi; ++pos) {
        u32x2 codes[2];
        const float sc = encode_row_e4m3<SCALE == kScaleToken>(
            a.kv_new + ((int64_t)b * a.n_new + (pos - first_new)) * kD, lane, tscale, codes);
        const int t = pos & (kPage - 1);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int c8 = lane + 64 * c;  // 8-byte chunk of the row
          if (c == 0 || lane < 8)
            *reinterpret_cast<u32x2*>(kv + pslot(t, c8 >> 1) * 16 + 8 * (c8 & 1)) = codes[c];
        }
        if (SCALE == kScaleToken && lane == 0) s_scale[it % T::NBUF][t] = sc;
        bool store = rg == 0 && a.store_rows;
        if (CHECKED && store) {
          // the page check runs beside this launch: store only into a page
          // that is in the pool, is the recorded one and carries its tag
          const int64_t e = bt_row + pos / kPage;
          const int raw = load_const(a.block_table, e);
          const uint32_t cur = load_const(a.page_tags, min(max(raw, 0), a.num_pages - 1));
          store = raw >= 0 && raw < a.num_pages && raw == load_const(a.expected_pages, e) &&
                  cur == load_const(a.expected_tags, e);
        }
        if (store) {
          const int pg = min(max(load_const(a.block_table, bt_row + pos / kPage), 0), a.num_pages - 1);
          uint8_t* dst = a.cache_out + ((int64_t)pg * kPage + t) * kD;
          *reinterpret_cast<u32x2*>(dst + 8 * lane) = codes[0];
          if (lane < 8) *reinterpret_cast<u32x2*>(dst + 8 * (lane + 64)) = codes[1];
          if (SCALE == kScaleToken && lane == 0) a.scale_out[(int64_t)pg * kPage + t] = sc;
        }
      }
      // the row loads and stores are counted like the copies: let them all
      // finish so the later waits keep their meaning
      if (lo < hi) wait_vmcnt<0>();
    };

    // Wait for this wave's own share of page it, zero its rows past the end of
    // the request (they may hold anything, even NaN codes, and P V multiplies
    // them by zero weights), and read its K bytes.  Loads complete in order, so
    // the wait allows exactly the loads issued after page it's: the whole next
    // page (LPP) when one is in flight behind it, none at the end of the split.
    auto k_read = [&](int it, bool page_behind) {
      if (page_behind)
        wait_vmcnt<LPP>();
      else
        wait_vmcnt<0>();
      uint8_t* kv = s_kv[it % T::NBUF];
      const int nvalid = L - (p_begin + it) * kPage;
      if (nvalid < qw * 16 + 16) {
        // tokens tl0 .. 15 of this wave's quarter: slots tl0 * 4 .. 63 of each group
        const int tl0 = max(nvalid - qw * 16, 0);
        const int per = (16 - tl0) * 4;
        u32x4* q = reinterpret_cast<u32x4*>(kv) + qw * 576 + tl0 * 4;
        for (int e = lane; e < 9 * per; e += 64) {
          const int grp = e / per;
          q[grp * 64 + (e - grp * per)] = u32x4{0u, 0u, 0u, 0u};
        }
      }
      if (a.n_new > 0) patch_new_rows(it, kv);
#pragma unroll
      for (int i = 0; i < KB / 2; ++i) kraw[i] = *reinterpret_cast<const u32x4*>(kv + klane + 1024 * i);
    };
    // S^T[token][row] = K Q^T for this wave's 16 tokens, all 32 rows: one MFMA
    // pair per k-block with the conversions of the next k-block between them.
    static_assert(T::LOADS * 2 == kD / 32, "one page load per two k-blocks");
    auto qk = [&](f32x4 (&S)[2], auto dma_c) {
      constexpr bool dma = decltype(dma_c)::value;
      auto lo_word = [&](int kb) { const u32x4 w = kraw[kb >> 1]; return (kb & 1) ? w[2] : w[0]; };
      auto hi_word = [&](int kb) { const u32x4 w = kraw[kb >> 1]; return (kb & 1) ? w[3] : w[1]; };
      uint32_t d[2][4];
      d[0][0] = cvt_e4m3_lo(lo_word(0));
      d[0][1] = cvt_e4m3_hi(lo_word(0));
      d[0][2] = cvt_e4m3_lo(hi_word(0));
      d[0][3] = cvt_e4m3_hi(hi_word(0));
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 kop = bf16x8_of(d[kb & 1]);
        uint32_t (&nx)[4] = d[(kb + 1) & 1];
        if (kb == 0) mfma_vvv0_w(S[0], kop, qop[0][0]); else mfma_vvv_w(S[0], kop, qop[0][kb]);
        if constexpr (dma) {
          if ((kb & 1) == 0) dma_load(kb >> 1);
        }
        if (kb + 1 < KB) {
          nx[0] = cvt_e4m3_lo(lo_word(kb + 1));
          nx[1] = cvt_e4m3_hi(lo_word(kb + 1));
        }
        if (kb == 0) mfma_vvv0(S[1], kop, qop[1][0]); else mfma_vvv(S[1], kop, qop[1][kb]);
        if (kb + 1 < KB) {
          nx[2] = cvt_e4m3_lo(hi_word(kb + 1));
          nx[3] = cvt_e4m3_hi(hi_word(kb + 1));
        }
      }
      mfma_drain_s(S[0], S[1], bf16x8_of(d[(KB - 1) & 1]));
    };
    // softmax, part 1: y = score * coef - reference (log2 units), masked past
    // each row's causal limit, and the running maxima.  Lane holds tokens
    // 16w + 4g + i of rows rb*16 + m.
    float y[2][4];
    f32x4 sc = {1.0f, 1.0f, 1.0f, 1.0f};
    auto scores = [&](const f32x4 (&S)[2], int it) {
      const int tbase = (p_begin + it) * kPage;
      float cs[4];
      if (SCALE == kScaleToken) {
        sc = *reinterpret_cast<const f32x4*>(&s_scale[it % T::NBUF][qw * 16 + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) cs[i] = coef * sc[i];
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float mr = m0[rb] == -INFINITY ? 0.0f : m0[rb];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          y[rb][i] = __builtin_fmaf(S[rb][i], SCALE == kScaleToken ? cs[i] : coef, -mr);
      }
      if (tbase + kPage > lim_lo) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tbase + qw * 16 + 4 * g + i >= lim[rb]) y[rb][i] = -INFINITY;
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        ymax[rb] = max3f(max3f(ymax[rb], y[rb][0], y[rb][1]), y[rb][2], y[rb][3]);
    };
    // softmax, part 2: weights 2^y as bf16 P into LDS, the sums, and the flag
    // that asks for a restart when a weight would exceed 2^64
    auto weights = [&](int it) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(y[rb][i]);
        uint32_t pk[2];
        if (SCALE == kScaleToken) {
          // the per-token V scale rides on the weight; the sums stay unscaled
#pragma unroll
          for (int i = 0; i < 2; ++i) pk[i] = pack_bf16x2(e[2 * i] * sc[2 * i], e[2 * i + 1] * sc[2 * i + 1]);
        } else {
#pragma unroll
          for (int i = 0; i < 2; ++i) pk[i] = pack_bf16x2(e[2 * i], e[2 * i + 1]);
          lnrm[rb] = dot2_bf16_ones(pk[1], dot2_bf16_ones(pk[0], lnrm[rb]));
        }
        lsum[rb] += (e[0] + e[1]) + (e[2] + e[3]);
        *reinterpret_cast<u32x2*>(s_p[it & 1] + (rb * 16 + m) * T::PSTRIDE + (qw * 16 + 4 * g) * 2) =
            u32x2{pk[0], pk[1]};
      }
      const bool over = ymax[0] > kRefSlack || ymax[1] > kRefSlack;
      const bool any_over = __any(over);
      if (lane == 0) s_flag[it & 1][qw] = any_over ? 1 : 0;
    };

    for (;;) {
      k_read(0, n_it > 1);
      {
        // page 0 (the first page of an attempt)
        const bool next = T::DIST < n_it;
        f32x4 S[2];
        if (next) {
          dma_page(T::DIST);
          qk(S, std::true_type{});
        } else {
          qk(S, std::false_type{});
        }
        if (1 < n_it) k_read(1, next);
        scores(S, 0);
        if (!have_ref) {
          // the reference of each row is its maximum over the first page
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const float pm = group4_max(ymax[rb]);
            if (g == 0) s_red[qw][rb * 16 + m] = pm;
          }
          __syncthreads();  // (2) first-page maxima in LDS
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const int row = rb * 16 + m;
            m0[rb] = fmaxf(fmaxf(s_red[0][row], s_red[1][row]), fmaxf(s_red[2][row], s_red[3][row]));
            const float mr = m0[rb] == -INFINITY ? 0.0f : m0[rb];
#pragma unroll
            for (int i = 0; i < 4; ++i) y[rb][i] -= mr;
            ymax[rb] -= mr;
          }
          have_ref = true;
        }
        weights(0);
      }
      __syncthreads();  // (3) P and flags of page 0 are in LDS
      // Page it's flags are read after the barrier that ends it but looked at
      // only after the next page's QK^T MFMAs have been issued, so that the
      // LDS latency of the read stays off the page's critical path.  On a
      // restart that work (and a copy already issued) is simply dropped; the
      // output waves leave their loop after the same barrier.
      uint32_t fw = flag_words(0);
      bool again = false;
      auto page = [&](int it, auto dma_c) {  // false: leave for a restart
        constexpr bool dma = decltype(dma_c)::value;
        if constexpr (dma) dma_page(it + T::DIST);
        f32x4 S[2];
        qk(S, dma_c);
        settle(fw);
        if (restart_asked(fw)) return false;
        if (it + 1 < n_it) k_read(it + 1, dma);
        scores(S, it);
        weights(it);
        __syncthreads();  // (4) P and flags of page it are in LDS; page it - 1 is consumed
        fw = flag_words(it);
        return true;
      };
      int it = 1;
      bool ok = true;
      for (; ok && it + T::DIST < n_it; ++it) ok = page(it, std::true_type{});
      for (; ok && it < n_it; ++it) ok = page(it, std::false_type{});
      if (ok) settle(fw);
      again = !ok || restart_asked(fw);
      if (!again) break;
      // A weight would exceed 2^64: restart the split with a reference raised
      // to each row's running maximum.
      ++restarts;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float pm = group4_max(ymax[rb]);
        if (g == 0) s_red[qw][rb * 16 + m] = pm;
      }
      wait_vmcnt<0>();
      __syncthreads();  // (5) every copy landed, the maxima are in LDS
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int row = rb * 16 + m;
        const float pm = fmaxf(fmaxf(s_red[0][row], s_red[1][row]), fmaxf(s_red[2][row], s_red[3][row]));
        const float mr = m0[rb] == -INFINITY ? 0.0f : m0[rb];
        if (pm > -INFINITY) m0[rb] = fmaxf(m0[rb], mr + pm);
        ymax[rb] = -INFINITY;
        lsum[rb] = 0.0f;
        lnrm[rb] = 0.0f;
      }
      reload_ids(0);
      prologue();
    }
    // the sums of this wave's tokens for the output waves
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float ls = group4_sum(lsum[rb]);
      const float ln = SCALE == kScaleToken ? ls : group4_sum(lnrm[rb]);
      const int row = rb * 16 + m;
      if (g == 0) {
        s_lsum[qw][row] = ls;
        s_lnrm[qw][row] = ln;
        if (qw == 0) s_m0[row] = m0[rb];
      }
    }
    __syncthreads();  // (6) sums in LDS
  } else {
    // =====================================================================
    // output waves: the same barrier sequence, P V one page behind
    // =====================================================================
    f32x4 O[2][8];  // rows rb*16 + 4g + i, dims 128*qw + 16db + m (VGPRs)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) O[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    mfma_zero_o(O);
    // per-lane LDS offsets of the V reads: lane 2j+h of a 16-lane group
    // addresses token 8g+j (+32 kt) of its wave's dims; dims 128w + 64(db/4) +
    // 16(db%4) are chunk 8w + 4(db/4) + db%4, at pslot + 1024 (db/4) + 18432 kt
    uint32_t voff[4];
    {
      const int t = g * 8 + (m >> 1);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) voff[bb] = (uint32_t)(pslot(t, 8 * qw + bb) * 16 + 8 * (m & 1));
    }
    bf16x8 pv_p[2][2];  // [32-token half][row block]
    u32x2 pv_v[2][8];   // [32-token half][16-dim block]
    auto pv = [&](int it) {
      const uint8_t* kvp = s_kv[it % T::NBUF];
      const uint8_t* pp = s_p[it & 1];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int tok0 = kt * 32 + g * 8;
#pragma unroll
        for (int rbp = 0; rbp < 2; ++rbp)
          pv_p[kt][rbp] = *reinterpret_cast<const bf16x8*>(pp + (rbp * 16 + m) * T::PSTRIDE + tok0 * 2);
#pragma unroll
        for (int db = 0; db < 8; ++db)
          pv_v[kt][db] = lds_read_tr8(kvp + voff[db & 3] + kt * 32 * T::ROW_BYTES + 1024 * (db >> 2));
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        uint32_t d[2][4];
        d[0][0] = cvt_e4m3_lo(pv_v[kt][0].x);
        d[0][1] = cvt_e4m3_hi(pv_v[kt][0].x);
        d[0][2] = cvt_e4m3_lo(pv_v[kt][0].y);
        d[0][3] = cvt_e4m3_hi(pv_v[kt][0].y);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const bf16x8 vop = bf16x8_of(d[db & 1]);
          uint32_t (&nx)[4] = d[(db + 1) & 1];
          mfma_vvv_w(O[0][db], pv_p[kt][0], vop);
          if (db + 1 < 8) {
            nx[0] = cvt_e4m3_lo(pv_v[kt][db + 1].x);
            nx[1] = cvt_e4m3_hi(pv_v[kt][db + 1].x);
          }
          mfma_vvv(O[1][db], pv_p[kt][1], vop);
          if (db + 1 < 8) {
            nx[2] = cvt_e4m3_lo(pv_v[kt][db + 1].y);
            nx[3] = cvt_e4m3_hi(pv_v[kt][db + 1].y);
          }
        }
        mfma_drain_o(O, pv_p[kt][0], pv_p[kt][1], bf16x8_of(d[1]));
      }
    };

    __syncthreads();  // (1)
    for (;;) {
      if (!have_ref) {
        __syncthreads();  // (2)
        have_ref = true;
      }
      __syncthreads();  // (3)
      // Page it - 1's flags are looked at after P V of page it - 1 has been
      // issued; when they ask for a restart that P V is wasted work (its
      // operands are valid) and O is cleared below.
      uint32_t fo = flag_words(0);
      bool again = false;
      for (int it = 1; it < n_it; ++it) {
        pv(it - 1);
        settle(fo);
        if (restart_asked(fo)) {
          again = true;
          break;
        }
        __syncthreads();  // (4)
        fo = flag_words(it);
      }
      if (!again) {
        settle(fo);
        again = restart_asked(fo);
      }
      if (!again) {
        pv(n_it - 1);
        break;
      }
      ++restarts;
      __syncthreads();  // (5)
      mfma_zero_o(O);
    }

    __syncthreads();  // (6) the score waves' sums are in LDS; every page buffer is free
    // Row normalisation: lane r < 32 of each output wave computes row r's
    // factor into this wave's slice of s_red (free by now); wave 4 also writes
    // the row's LSE.  The output is a weighted mean with the bf16 weights P V
    // used; the LSE uses the fp32 weights.
    const bool single = a.max_splits == 1;
    const int64_t prow0 = single ? (int64_t)b * a.R + r0 : ((int64_t)b * a.max_splits + split) * a.R + r0;
    if (lane < kRows) {
      const int row = lane;
      const float lt = s_lsum[0][row] + s_lsum[1][row] + s_lsum[2][row] + s_lsum[3][row];
      const float ln = s_lnrm[0][row] + s_lnrm[1][row] + s_lnrm[2][row] + s_lnrm[3][row];
      s_red[qw][row] = ln > 0.0f ? tscale / ln : 0.0f;
      if (qw == 0 && r0 + row < a.R) {
        const float mr = s_m0[row] == -INFINITY ? 0.0f : s_m0[row];
        (single ? a.lse : a.lse_part)[prow0 + row] = lt > 0.0f ? (mr + __log2f(lt)) * kLn2 : -INFINITY;
      }
    }
    // O goes out through LDS so that each store moves 16 contiguous bytes:
    // this wave's 32 x 128 fp32 tile, rows 132 floats apart (conflict-free
    // writes of the MFMA layout), then 8 dims of one row per lane.  Only this
    // wave touches its tile, and a wave's LDS accesses complete in order.
    constexpr int SST = 132;
    float* tile = reinterpret_cast<float*>(&s_kv[0][0]) + qw * (kRows * SST);
#pragma unroll
    for (int rbp = 0; rbp < 2; ++rbp)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int db = 0; db < 8; ++db) tile[(rbp * 16 + 4 * g + i) * SST + 16 * db + m] = O[rbp][db][i];
    uint16_t* dst = (single ? a.out : a.o_part) + prow0 * kDV + qw * 128;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int row = k * 4 + (lane >> 4), c = lane & 15;  // 32 rows x 16 chunks of 8 dims
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(&tile[row * SST + 8 * c]);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(&tile[row * SST + 8 * c + 4]);
      const float inv = s_red[qw][row];
      if (r0 + row < a.R)
        *reinterpret_cast<u32x4*>(dst + (int64_t)row * kDV + 8 * c) =
            u32x4{pack_bf16x2(v0.x * inv, v0.y * inv), pack_bf16x2(v0.z * inv, v0.w * inv),
                  pack_bf16x2(v1.x * inv, v1.y * inv), pack_bf16x2(v1.z * inv, v1.w * inv)};
    }
  }
}

hipError_t launch_decode_fp8(const DecodeArgs& a, int scale_mode, hipStream_t stream) {
  const bool checked = a.status != nullptr;
  const dim3 grid((unsigned)(decode_grid_size(a.B, a.max_splits, a.n_rg) + (checked ? a.B : 0))), block(512);
  switch (scale_mode) {
    case kScaleTensor:
      if (checked)
        hipLaunchKernelGGL((decode_fp8_kernel<kScaleTensor, true>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((decode_fp8_kernel<kScaleTensor, false>), grid, block, 0, stream, a);
      break;
    case kScaleToken:
      if (checked)
        hipLaunchKernelGGL((decode_fp8_kernel<kScaleToken, true>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((decode_fp8_kernel<kScaleToken, false>), grid, block, 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((decode_fp8_kernel<kScaleNone, false>), grid, block, 0, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace mla
