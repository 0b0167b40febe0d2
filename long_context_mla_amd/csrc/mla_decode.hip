// mla_decode_paged: split-KV decode attention of n_q new tokens x H heads over a
// paged latent cache of one shared 576-element row per token (512 latent + 64
// rope; the row is both key and value).
//
// The pages fix the problem: one latent row of 576 elements per token per layer
// with no distinct keys and values ("How to serve trillions of tokens for
// trillion-parameter coding agents", sections "First, understand the workload"
// and "Tensor parallel was the best parallelism strategy for maximum
// interactivity"); a single latent head shared by all query heads, decode
// attention being memory-bound with cost growing with context ("vLLM x AgentX:
// Optimizing for Real-World Agentic Serving", section "Model-specific
// parallelism / Kimi K3"); an FP8 e4m3 cache converted as it is read ("Smaller,
// faster, safer: running Kimi and GLM at scale", section "Quantizing the KV
// cache"); physical pages reached through per-request page maps (same page,
// section "Protecting a shared KV cache").
//
// This file holds the kernel for a BF16 cache and the dispatch; FP8 caches go
// to the kernel in mla_decode_fp8.hip.
//
// BF16 kernel, gfx950 design.  One 256-thread workgroup (4 waves, one per
// SIMD) per (request, split, group of 32 query rows); one workgroup per CU.
//  * Pages stream HBM -> LDS with LDS-DMA (global_load_lds, no VGPRs), two
//    buffers, one page in flight.  Each lane picks its source chunk so that
//    the page lands in a rotated layout whose operand reads are free of bank
//    conflicts.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: wave w takes tokens 16w..16w+15
//    of the page for all 32 rows; the rows' query stays in registers as bf16
//    operands for the whole split.
//  * Softmax weights 2^(x - m0) use one reference per row, fixed from the
//    split's first page (the only page that exchanges row maxima).  O is never
//    rescaled: if a later score exceeds the reference by more than 2^64 the
//    split restarts from its first page with the larger reference.
//  * O += P V on MFMA: wave w takes output dims 128w..128w+127; V is the first
//    512 columns of the same staged page, read with transposing LDS loads
//    (ds_read_b64_tr_b16).
//  * Epilogue: O / l and the natural-log LSE, either final (one split) or as
//    bf16 split partials for mla_decode_combine.
#include <type_traits>

#include "decode_tile.h"
#include "device_common.h"
#include "launch.h"

namespace mla {

__global__ __launch_bounds__(256, 1) void decode_bf16_kernel(DecodeArgs a) {
  using T = Tile<kBf16>;
  using Z = SwzBf16;
  __shared__ __attribute__((aligned(16))) uint8_t s_kv[T::NBUF][T::PAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_p[2][kRows * T::PSTRIDE];
  __shared__ float s_red[4][kRows];   // per-wave row maxima (first page, restarts)
  __shared__ float s_lsum[4][kRows];
  __shared__ float s_lnrm[4][kRows];
  __shared__ float s_m0[kRows];
  __shared__ __attribute__((aligned(16))) int s_flag[2][4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, g = lane >> 4;
  const WorkUnit wu = decode_work_unit(a.B, a.max_splits, a.n_rg);
  if (!wu.valid) return;
  const int b = wu.b, split = wu.split, rg = wu.rg;
  const int L = min(max(load_const(a.seq_lens, b), 0), a.max_blocks * kPage);
  const int n_pages = (L + kPage - 1) / kPage;
  const int r0 = rg * kRows;
  const int p_begin = split * a.pps;

  if (p_begin >= n_pages) {
    // Nothing to read.  Only an empty request's first split reports it; the
    // combine never reads splits past a request's last page.
    if (n_pages == 0 && split == 0) {
      for (int e = threadIdx.x; e < kRows * kDV; e += 256) {
        const int r = r0 + e / kDV;
        if (r >= a.R) break;
        if (a.max_splits == 1)
          a.out[((int64_t)b * a.R + r) * kDV + e % kDV] = 0;
        else
          a.o_part[((int64_t)b * a.max_splits * a.R + r) * kDV + e % kDV] = 0;
      }
      for (int r = r0 + threadIdx.x; r < min(r0 + kRows, a.R); r += 256) {
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
  const float coef = a.sm_log2;

  // ---- the query of the group's 32 rows, HBM -> LDS in one coalesced copy
  // shared by the four waves, into the page buffer that stays free until the
  // second page copy.  Row r's 16-byte chunk c (72 per row) goes to slot
  // r * 72 + (c ^ ((r / 2) % 8)), which makes the operand reads below free of
  // bank conflicts.  Rows past R repeat row R - 1 (their results are dropped).
  constexpr int QBUF = T::NBUF - 1;
  const uint32_t qlds = lds_addr(&s_kv[QBUF][0]);
#pragma unroll
  for (int j = 0; j < 9; ++j) {
    const int slot = (wave * 9 + j) * 64 + lane;  // 2304 slots = 32 rows x 72 chunks
    const int r = slot / 72;
    const int c = (slot - r * 72) ^ ((r >> 1) & 7);
    const uint16_t* src = a.q + ((int64_t)b * a.R + min(r0 + r, a.R - 1)) * kD + c * 8;
    lds_dma16_lane(src, qlds + (wave * 9 + j) * 1024);
  }

  // Page ids of the split, 64 at a time, one per lane; picked out with readlane
  // so the DMA issue never waits on a scalar load.
  const int64_t bt_row = (int64_t)b * a.max_blocks;
  auto load_ids = [&](int first) {
    const int idx = first + lane;
    int pg = idx < p_end ? a.block_table[bt_row + idx] : 0;
    return min(max(pg, 0), a.num_pages - 1);
  };
  int id_chunk = 0;
  int ids = load_ids(p_begin);

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

  constexpr int LPP = T::LOADS;  // loads per page per wave
  // each lane's source offsets inside a page for its LOADS LDS chunk slots;
  // wave w copies tokens 16w .. 16w+15, the rows its own QK^T reads
  uint32_t goff[T::LOADS];
#pragma unroll
  for (int j = 0; j < T::LOADS; ++j) {
    const int slot = (wave * T::LOADS + j) * 64 + lane;
    const int t = slot / Z::NCH;
    goff[j] = t * T::ROW_BYTES + Z::chunk_of_slot(t, slot - t * Z::NCH) * 16;
  }
  // the page a DMA batch copies: uniform source base and LDS destination
  const uint8_t* dma_src = a.cache;
  uint32_t dma_dst = 0;
  auto dma_page = [&](int it) {  // select page p_begin + it for the following dma_part calls
    if ((it >> 6) != id_chunk) {
      id_chunk = it >> 6;
      ids = load_ids(p_begin + (id_chunk << 6));
    }
    const int pg = __builtin_amdgcn_readlane(ids, it & 63);
    dma_src = a.cache + (int64_t)pg * T::PAGE_BYTES;
    dma_dst = lds_addr(&s_kv[it % T::NBUF][0]) + wave * T::LOADS * 1024;
  };
  auto dma_part = [&](int part) {
#pragma unroll
    for (int j = 0; j < T::LOADS; ++j)
      if (j / T::PART == part || (part == 2 && j >= 3 * T::PART))
        lds_dma16(dma_src, goff[j], dma_dst + j * 1024);
  };
  auto prologue = [&]() {
#pragma unroll
    for (int k = 0; k < T::DIST; ++k)
      if (k < n_it) {
        dma_page(k);
        dma_part(0);
        dma_part(1);
        dma_part(2);
      }
  };
  prologue();

  // ---- query operands LDS -> AGPRs: lane (m, g) holds rows rb*16 + m, and
  // for k-block kb the 8 dims 64(kb/2) + 16g + 8(kb%2) .. +8: k-blocks are
  // paired so that a lane's slots of k-blocks 2i and 2i+1 are the 16
  // consecutive dims of one 16-byte FP8 chunk of K (both cache types use
  // this order).  The wait covers the query only, not the pages behind it.
  static_assert(T::DIST == 1, "one page copy is in flight behind the query");
  wait_vmcnt<LPP>();
  __syncthreads();
  bf16x8 qop[2][kD / 32];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = rb * 16 + m;
#pragma unroll
    for (int kb = 0; kb < kD / 32; ++kb) {
      const int c = 8 * (kb >> 1) + 2 * g + (kb & 1);
      qop[rb][kb] = to_agpr(*reinterpret_cast<const bf16x8*>(
          &s_kv[QBUF][(row * 72 + (c ^ ((row >> 1) & 7))) * 16]));
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the query buffer is free to be overwritten

  float m0[2] = {-INFINITY, -INFINITY};  // log2-domain reference of this lane's rows
  float ymax[2] = {-INFINITY, -INFINITY}; // running max of score - reference, this lane's tokens
  float lsum[2] = {0.0f, 0.0f};          // this lane's share of the softmax sums (fp32 P)
  float lnrm[2] = {0.0f, 0.0f};          // the same over the bf16-rounded P that PV uses
  f32x4 O[2][8];                          // rows rb*16 + 4g + i, dims 128*wave + 16db + m (VGPRs)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) O[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  mfma_zero_o(O);
  bool have_ref = false;
  int restarts = 0;

  const int tok = wave * 16 + m;  // this lane's token in QK^T

  // ---- P V over this wave's 128 dims for the page in buffer kvp, with its
  // weights in P buffer pp; mid() runs between the two 32-token halves
  auto pv = [&](const uint8_t* kvp, const uint8_t* pp, auto mid) {
    const int dim0 = wave * 128;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      if (kt == 1) mid();
      // P (rows x 32 tokens) and V operands of this half of the page are read
      // first, then converted and fed to the MFMAs; the lane's 8 contraction
      // slots are tokens tok0 .. tok0+7 in both
      const int tok0 = kt * 32 + g * 8;
      bf16x8 pop[2];
      u32x2 vraw[8][2];
#pragma unroll
      for (int rbp = 0; rbp < 2; ++rbp)
        pop[rbp] = *reinterpret_cast<const bf16x8*>(pp + (rbp * 16 + m) * T::PSTRIDE + tok0 * 2);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        // lane 4j+q of the group addresses token tok0+j (+4), elements dcol+4q .. +4
        const int dcol = dim0 + db * 16;
        const int c = (dcol >> 3) + ((m & 3) >> 1);
        const int t0 = tok0 + (m >> 2), t1 = t0 + 4;
        vraw[db][0] = lds_read_tr16(kvp + (t0 * Z::NCH + Z::slot(t0, c)) * 16 + 8 * (m & 1));
        vraw[db][1] = lds_read_tr16(kvp + (t1 * Z::NCH + Z::slot(t1, c)) * 16 + 8 * (m & 1));
      }
      __builtin_amdgcn_sched_barrier(0);  // reads ahead of the math
      {
        // convert two V blocks into distinct registers, then issue their four MFMAs
#pragma unroll
        for (int d0 = 0; d0 < 8; d0 += 2) {
          bf16x8 vop[2];
#pragma unroll
          for (int d = 0; d < 2; ++d)
            vop[d] = __builtin_bit_cast(bf16x8, u32x4{vraw[d0 + d][0].x, vraw[d0 + d][0].y,
                                                      vraw[d0 + d][1].x, vraw[d0 + d][1].y});
#pragma unroll
          for (int d = 0; d < 2; ++d)
#pragma unroll
            for (int rbp = 0; rbp < 2; ++rbp)
              O[rbp][d0 + d] = mfma_16x16x32_bf16(pop[rbp], vop[d], O[rbp][d0 + d]);
        }
      }
    }
  };
  auto no_mid = [] {};

  // ---- S^T[token][row] = K Q^T for this wave's 16 tokens of the page, all
  // 32 rows, K straight from LDS
  constexpr int KB = kD / 32;
  auto qk_bf16 = [&](const uint8_t* kv, f32x4 (&S)[2]) {
#pragma unroll
    for (int k0 = 0; k0 < KB; k0 += T::KBATCH) {
      u32x4 kr[T::KBATCH];
#pragma unroll
      for (int k = 0; k < T::KBATCH; ++k) {
        const int kb = k0 + k;
        const int c = 8 * (kb >> 1) + 2 * g + (kb & 1);  // dims 64(kb/2) + 16g + 8(kb&1) .. +8
        kr[k] = *reinterpret_cast<const u32x4*>(kv + (tok * Z::NCH + Z::slot(tok, c)) * 16);
      }
      __builtin_amdgcn_sched_barrier(0);  // reads ahead of the math
#pragma unroll
      for (int k = 0; k < T::KBATCH; ++k) {
        const bf16x8 kop = __builtin_bit_cast(bf16x8, kr[k]);
        if (k0 + k == 0)
          mfma_qk2_first(S[0], S[1], kop, qop[0][0], qop[1][0]);
        else
          mfma_qk2(S[0], S[1], kop, qop[0][k0 + k], qop[1][k0 + k]);
      }
    }
  };

  // ---- softmax, part 1: y = score * coef - reference (log2 units), masked
  // past each row's causal limit, and the running maxima.  Lane holds tokens
  // 16w + 4g + i of rows rb*16 + m.
  float y[2][4];
  auto scores = [&](const f32x4 (&S)[2], int it) {
    const int tbase = (p_begin + it) * kPage;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float mr = m0[rb] == -INFINITY ? 0.0f : m0[rb];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        y[rb][i] = __builtin_fmaf(S[rb][i], coef, -mr);
    }
    if (tbase + kPage > lim_lo) {
      // the page reaches a row's causal limit or the end of the request
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tbase + wave * 16 + 4 * g + i >= lim[rb]) y[rb][i] = -INFINITY;
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      ymax[rb] = max3f(max3f(ymax[rb], y[rb][0], y[rb][1]), y[rb][2], y[rb][3]);
  };
  // first page of the split: the reference of each row is its page max
  auto first_ref = [&]() {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float pm = group4_max(ymax[rb]);
      if (g == 0) s_red[wave][rb * 16 + m] = pm;
    }
    __syncthreads();
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
  };
  // ---- softmax, part 2: weights 2^y as bf16 P into LDS, the sums, and the
  // flag that asks for a restart when a weight would exceed 2^64
  auto weights = [&](int it) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(y[rb][i]);
      uint32_t pk[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) pk[i] = pack_bf16x2(e[2 * i], e[2 * i + 1]);
      lnrm[rb] = dot2_bf16_ones(pk[1], dot2_bf16_ones(pk[0], lnrm[rb]));
      lsum[rb] += (e[0] + e[1]) + (e[2] + e[3]);
      *reinterpret_cast<u32x2*>(s_p[it & 1] + (rb * 16 + m) * T::PSTRIDE + (wave * 16 + 4 * g) * 2) =
          u32x2{pk[0], pk[1]};
    }
    const bool over = ymax[0] > kRefSlack || ymax[1] > kRefSlack;
    const bool any_over = __any(over);
    if (lane == 0) s_flag[it & 1][wave] = any_over;
  };
  auto flagged = [&](int it) {
    const int4 f = *reinterpret_cast<const int4*>(&s_flag[it & 1][0]);
    return (f.x | f.y | f.z | f.w) && restarts < kMaxRestarts;
  };
  // A weight would exceed 2^64: restart the split with a reference raised to
  // each row's running maximum.  Every wave calls this together.
  auto restart = [&]() {
    ++restarts;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float pm = group4_max(ymax[rb]);
      if (g == 0) s_red[wave][rb * 16 + m] = pm;
    }
    wait_vmcnt<0>();
    __syncthreads();  // every DMA landed, every wave is past its reads, maxima in LDS
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
    mfma_zero_o(O);
    // (s_red is next written at a later restart, past further barriers; the
    // flags read after a restart are always written after it)
    id_chunk = 0;
    ids = load_ids(p_begin);
    prologue();
  };

  static_assert(!T::PIPE, "this kernel serves the BF16 cache; FP8 has its own");
  for (int it = 0; it < n_it; ++it) {
    wait_vmcnt<0>();
    __syncthreads();  // page it is in LDS; every wave is done with page it - 1
    const bool next = it + T::DIST < n_it;
    if (next) {
      dma_page(it + T::DIST);
      dma_part(0);
      dma_part(1);
      dma_part(2);
    }
    uint8_t* kv = s_kv[it % T::NBUF];
    const int nvalid = min(kPage, L - (p_begin + it) * kPage);
    if (nvalid < kPage) {
      // rows past the end of the request may hold anything (even NaN codes):
      // zero them so that their zero weights give zero products in PV
      u32x4* junk = reinterpret_cast<u32x4*>(kv + nvalid * T::ROW_BYTES);
      for (int e = threadIdx.x; e < (kPage - nvalid) * (T::ROW_BYTES / 16); e += 256)
        junk[e] = u32x4{0u, 0u, 0u, 0u};
    }
    f32x4 S[2];
    qk_bf16(kv, S);
    mfma_result_fence_v(S[0], S[1]);
    scores(S, it);
    if (!have_ref) first_ref();
    weights(it);
    __syncthreads();  // P of the page is in LDS
    if (flagged(it)) {
      restart();
      it = -1;
      continue;
    }
    pv(kv, s_p[it & 1], no_mid);
  }


  // ---- epilogue: softmax sums across lanes and token groups, then O / l
  mfma_result_fence_v16(O);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float ls = group4_sum(lsum[rb]);
    const float ln = group4_sum(lnrm[rb]);
    const int row = rb * 16 + m;
    if (g == 0) {
      s_lsum[wave][row] = ls;
      s_lnrm[wave][row] = ln;
      if (wave == 0) s_m0[row] = m0[rb];
    }
  }
  __syncthreads();
  const int dim0 = wave * 128;
#pragma unroll
  for (int rbp = 0; rbp < 2; ++rbp)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rbp * 16 + 4 * g + i;
      const int r = r0 + row;
      if (r >= a.R) continue;
      const float lt = s_lsum[0][row] + s_lsum[1][row] + s_lsum[2][row] + s_lsum[3][row];
      const float ln = s_lnrm[0][row] + s_lnrm[1][row] + s_lnrm[2][row] + s_lnrm[3][row];
      // the output is a weighted mean with the bf16 weights PV used; the LSE
      // uses the fp32 weights
      const float inv = ln > 0.0f ? 1.0f / ln : 0.0f;
      const float mr = s_m0[row] == -INFINITY ? 0.0f : s_m0[row];
      const float lse_nat = lt > 0.0f ? (mr + __log2f(lt)) * kLn2 : -INFINITY;
      if (a.max_splits == 1) {
        uint16_t* dst = a.out + ((int64_t)b * a.R + r) * kDV + dim0 + m;
#pragma unroll
        for (int db = 0; db < 8; ++db) __builtin_nontemporal_store(float_to_bf16(O[rbp][db][i] * inv), dst + db * 16);
        if (wave == 0 && m == 0) __builtin_nontemporal_store(lse_nat, a.lse + (int64_t)b * a.R + r);
      } else {
        const int64_t pr = ((int64_t)b * a.max_splits + split) * a.R + r;
        uint16_t* dst = a.o_part + pr * kDV + dim0 + m;
#pragma unroll
        for (int db = 0; db < 8; ++db) __builtin_nontemporal_store(float_to_bf16(O[rbp][db][i] * inv), dst + db * 16);
        if (wave == 0 && m == 0) __builtin_nontemporal_store(lse_nat, a.lse_part + pr);
      }
    }
}

int decode_rows_per_group(int cache_kind) { return cache_kind == kFp8 ? decode_rows_fp8() : kRows; }

hipError_t launch_decode(const DecodeArgs& a0, int cache_kind, int scale_mode, hipStream_t stream) {
  DecodeArgs a = a0;
  const int rows = decode_rows_per_group(cache_kind);
  a.n_rg = (a.R + rows - 1) / rows;
  if (cache_kind == kFp8) return launch_decode_fp8(a, scale_mode, stream);
  const dim3 grid((unsigned)decode_grid_size(a.B, a.max_splits, a.n_rg)), block(256);
  hipLaunchKernelGGL(decode_bf16_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
