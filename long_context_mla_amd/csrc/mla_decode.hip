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
// BF16 kernel, gfx950 design: the FP8 kernel's specialised waves on units of
// half a page.  A BF16 page (64 tokens x 1,152 bytes) is twice an FP8 page, so
// the kernel stages 32-token units of 36,864 bytes, the size of an FP8 page,
// and keeps the same LDS pipeline: four units' V parts, three units' rope
// parts, P of two units.  One 512-thread workgroup (8 waves, two per SIMD) per
// (request, split, group of 64 query rows): 64 rows are every head of one
// query token of the 64-head models, so each page is copied into LDS once per
// compute unit.
//  * score waves 0..3: wave w = 2*th + rh holds the query of rows
//    32rh .. 32rh+31 in VGPRs and computes S^T = K Q^T for tokens
//    16th .. 16th+15 of each unit on v_mfma_f32_16x16x32_bf16 (two 16-row
//    tiles, K straight from LDS), the softmax weights P (bf16, into LDS) and
//    the sums;
//  * output waves 4..7: wave 4+j accumulates O[64 rows][128j .. 128j+127] +=
//    P V over the previous unit on v_mfma_f32_32x32x16_bf16, V being the
//    first 512 columns of the same staged rows (transposing LDS reads), and
//    copies its ninth of every unit HBM -> LDS by LDS-DMA, two units ahead.
// Two barriers per unit: D separates "scores of unit u" from "P V of unit u",
// and M, once the score waves have issued QK^T of unit u + 1, starts P V of
// unit u beside their softmax.
//
// Softmax: one fixed reference per row and split (the first unit's maximum),
// weights 2^(y - m0).  A weight above 2^64 switches the split to a scan: the
// remaining units are scored (no weights, no P V) to find every row's maximum,
// and the split runs once more with that maximum as its reference.  The
// output divides by the sum of the bf16 weights that P V used; the LSE uses
// the exact fp32 sum.
#include <type_traits>

#include "decode_tile.h"
#include "device_common.h"
#include "launch.h"

namespace mla {

namespace {

constexpr int kRowsB = 64;              // query rows per workgroup
constexpr int kUnit = 32;               // tokens per staged unit (half a page)
constexpr int kUnitBytes = kUnit * kD * 2;  // 36,864
constexpr int kVBuf = 4;                // staged V parts (units)
constexpr int kRBuf = 3;                // staged rope parts (units)
constexpr int kVBytes = kUnit * 1024;   // V part of a unit: 32 tokens x 1,024 bytes
constexpr int kRBytes = kUnit * 128;    // rope part: 32 tokens x 128 bytes
constexpr int kPBytes = kRowsB * 64;    // P of a unit: 64 rows x 32 tokens bf16
constexpr int kLoads = 9;               // 1 KB LDS-DMA loads per output wave per unit

// LDS map (bytes)
constexpr int kOffV = 0;
constexpr int kOffR = kOffV + kVBuf * kVBytes;      // 131072
constexpr int kOffP = kOffR + kRBuf * kRBytes;      // 143360
constexpr int kOffRed = kOffP + 2 * kPBytes;        // 151552: fp32 [2][64]
constexpr int kOffLsum = kOffRed + 512;             // fp32 [2][64]
constexpr int kOffLnrm = kOffLsum + 512;            // fp32 [2][64]
constexpr int kOffM0 = kOffLnrm + 512;              // fp32 [64]
constexpr int kOffFlag = kOffM0 + 256;              // uint8 [2][4]
constexpr int kLdsBytes = kOffFlag + 16;
// The query of the group's 64 rows (73,728 bytes) is staged once at the start
// over buffers that stay free until unit 2's copy: rows 0..55 over V buffers
// 2 and 3, rows 56..63 over rope buffer 2 and the two P buffers.
constexpr int kQA = kOffV + 2 * kVBytes;            // 65536: 56 rows
constexpr int kQB = kOffR + 2 * kRBytes;            // 139264: 8 rows
constexpr int kQRowBytes = kD * 2;                  // 1152
static_assert(kQA + 56 * kQRowBytes <= kOffR && kQB + 8 * kQRowBytes <= kOffP + 2 * kPBytes, "query staging");
constexpr int kQLoads = 18;                         // 1 KB query copies per score wave (72 in all)
static_assert(kLdsBytes <= 163840, "LDS");
static_assert(4 * kRowsB * 272 <= kOffP, "the output tiles fit over the unit buffers");

// Staged unit layout.  Token t = 16q + m of the unit (quarter q < 2, m < 16),
// 16-byte chunk c of its 1,152-byte row (72 per row).  The V part (c < 64)
// sits in V-buffer slot
//   vslot(q, m, c) = q*1024 + (c/8)*128 + 8m + ((c%8) ^ swz(m)),  swz(m) = (m/2) % 8:
// eight chunks of a token side by side.  The rope part (c' = c - 64 < 8) sits
// in rope-buffer slot rslot(q, m, c') = q*128 + 8m + (c' ^ swz(m)).  Then
//  * one LDS-DMA instruction fills one group of 64 slots: eight tokens x eight
//    chunks (lane l brings token 8h + l/8, chunk 8i + ((l%8) ^ swz)); each
//    eight consecutive lanes read 128 contiguous bytes of one token;
//  * the QK^T operand reads (16 tokens, one chunk each, per 16 lanes) and the
//    transposing P V reads (four tokens x chunks b, b+2, b+4, b+6 per 32 lanes)
//    run without LDS bank conflicts (measured with the bank-conflict counter;
//    a dim tile of four adjacent chunks conflicted 2-way).
__device__ __forceinline__ int swz(int m) { return (m >> 1) & 7; }
__device__ __forceinline__ int vslot(int q, int m, int c) { return q * 1024 + (c >> 3) * 128 + 8 * m + ((c & 7) ^ swz(m)); }
__device__ __forceinline__ int rslot(int q, int m, int c) { return q * 128 + 8 * m + (c ^ swz(m)); }
// P of a unit: row r (64 bytes, 32 tokens) at r * 64, its 16-byte chunk cc
// (tokens 8cc .. 8cc+7) at position (cc ^ (r/4)) % 4: free of bank conflicts
// for the 16-byte writes and reads below.
__device__ __forceinline__ int pbyte(int r, int cc) { return r * 64 + 16 * ((cc ^ (r >> 2)) & 3); }
// Wave-relative 16-byte chunks (8 dims each) of P V dim tile dt: b, b+2, b+4,
// b+6 with b = dt%2 + 8(dt/2); tile dim M is dim M%8 of chunk tchunk(dt, M/8).
__device__ __forceinline__ int tchunk(int dt, int k) { return (dt & 1) + 8 * (dt >> 1) + 2 * k; }

// Keeps the compiler from moving memory accesses across this point.
__device__ __forceinline__ void phase_fence() { asm volatile("" ::: "memory"); }

__global__ __launch_bounds__(512, 1) void decode_bf16_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  uint8_t* const s_v = lds + kOffV;
  uint8_t* const s_rope = lds + kOffR;
  uint8_t* const s_p = lds + kOffP;
  float* const s_red = reinterpret_cast<float*>(lds + kOffRed);
  float* const s_lsum = reinterpret_cast<float*>(lds + kOffLsum);
  float* const s_lnrm = reinterpret_cast<float*>(lds + kOffLnrm);
  float* const s_m0 = reinterpret_cast<float*>(lds + kOffM0);
  uint8_t* const s_flag = lds + kOffFlag;  // [unit parity][score wave], one byte each

  // One round trip for the launch arguments the first loads need.
  asm volatile("" :: "s"(a.q), "s"(a.block_table), "s"(a.seq_lens), "s"(a.n_rg), "s"(a.max_blocks));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool scorer = wave < 4;
  const int m = lane & 15, g = lane >> 4;
  const WorkUnit wu = decode_work_unit(a.B, a.max_splits, a.n_rg);
  if (!wu.valid) return;
  const int b = wu.b, split = wu.split, rg = wu.rg;
  const int r0 = rg * kRowsB;
  const int p_begin = split * a.pps;
  const int64_t bt_row = (int64_t)b * a.max_blocks;
  const int cap = a.max_blocks * kPage;

  // The output waves' first 64 page ids of the split go out before the length
  // is known (bounded by the table row), one per lane.
  int ids = 0;
  const int rh = wave & 1, th = (wave >> 1) & 1;
  // The score waves copy the query of the group's 64 rows HBM -> LDS in 72
  // coalesced 1 KB LDS-DMA copies (the rows are contiguous in q): slot s
  // (16 bytes) of the staged query is row s / 72, chunk (s % 72) ^ ((row / 2) % 8).
  // Rows past R repeat row R - 1.
  auto copy_query = [&]() {
    const uint8_t* qbase = reinterpret_cast<const uint8_t*>(a.q + (int64_t)b * a.R * kD);
#pragma unroll
    for (int k = 0; k < kQLoads; ++k) {
      const int ii = kQLoads * wave + k;
      const int sl = ii * 64 + lane;
      const int r = sl / 72;
      const int c = (sl - r * 72) ^ ((r >> 1) & 7);
      const uint32_t dst = lds_addr(lds + (ii < 63 ? kQA + ii * 1024 : kQB + (ii - 63) * 1024));
      lds_dma16(qbase, (uint32_t)(min(r0 + r, a.R - 1) * kQRowBytes + c * 16), dst);
    }
  };
  const bool q_early = blockIdx.x < kCUs;
  if (!scorer) {
    const int32_t* id_src = a.block_table + bt_row + min(p_begin + lane, a.max_blocks - 1);
    asm volatile("global_load_dword %0, %1, off" : "=v"(ids) : "v"(id_src) : "memory");
  }
  // The launch's first round of workgroups (one per CU) issues the query
  // copies before the length is known, so that their latency overlaps the
  // length's (the test takes the whole table row as the length).  Later
  // workgroups wait for the length and skip the copies for a split past the
  // request's end: in a batch of mixed lengths most workgroups of the longest
  // request's split count have no pages, and their query copies, spread over
  // the launch, mostly missed in L2 (a 64-request pool read 986 MB per launch
  // with them, 851 MB without).
  const int L_test = q_early ? cap : min(max(load_const(a.seq_lens, b), 0), cap);
  if (scorer && p_begin < (L_test + kPage - 1) / kPage) copy_query();
  const int L = min(max(load_const(a.seq_lens, b), 0), cap);
  const int n_pages = (L + kPage - 1) / kPage;

  if (p_begin >= n_pages) {
    // Nothing to read.  Only an empty request's first split reports it; the
    // combine never reads splits past a request's last page.  (Every copy
    // lands before the workgroup ends.)
    wait_vmcnt<0>();
    if (n_pages == 0 && split == 0) {
      for (int e = threadIdx.x; e < kRowsB * kDV; e += 512) {
        const int r = r0 + e / kDV;
        if (r >= a.R) break;
        if (a.max_splits == 1)
          a.out[((int64_t)b * a.R + r) * kDV + e % kDV] = 0;
        else
          a.o_part[((int64_t)b * a.max_splits * a.R + r) * kDV + e % kDV] = 0;
      }
      for (int r = r0 + threadIdx.x; r < min(r0 + kRowsB, a.R); r += 512) {
        if (a.max_splits == 1)
          a.lse[(int64_t)b * a.R + r] = -INFINITY;
        else
          a.lse_part[(int64_t)b * a.max_splits * a.R + r] = -INFINITY;
      }
    }
    return;
  }
  const int p_end = split == a.max_splits - 1 ? n_pages : min(n_pages, p_begin + a.pps);
  const int t_begin = p_begin * kPage;                   // the split's first token
  const int n_u = (min(p_end * kPage, L) - t_begin + kUnit - 1) / kUnit;  // units with a valid token
  bool have_ref = false;   // the reference is fixed (first unit done, or a rerun)
  bool allow_scan = true;  // the first run may switch to a scan; the rerun cannot need one

  auto flag_word = [&](int u) { return *reinterpret_cast<const uint32_t*>(s_flag + 4 * (u & 1)); };
  auto settle = [](uint32_t& f) {
    asm volatile("" : "+v"(f));
    f = __builtin_amdgcn_readfirstlane(f);
  };

  if (scorer) {
    // =====================================================================
    // score waves: rows 32rh .. 32rh+31 (tiles rt = 0, 1 of 16 rows), tokens
    // 16th .. 16th+15 (quarter th) of each unit
    // =====================================================================
    // K-step kk (32 dims, 18 per token) of tile rt: A = K (lane l: token
    // m = l % 16, dims 32kk + 8g .. +8 = chunk 4kk + g of its row), B = Q^T
    // (lane l: row 32rh + 16rt + m, the same dims).  D = S^T: lane l holds row
    // 32rh + 16rt + m, tokens 4g .. 4g+3 of the quarter.  Even and odd k-steps
    // accumulate apart (four chains of 16-cycle MFMAs).
    bf16x8 qop[2][kD / 32];  // the rows' query operands, for the whole split
    wait_vmcnt<0>();  // this wave's query copies have landed
    __syncthreads();  // (Q) the query is staged
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int lr = 32 * rh + 16 * rt + m;
      const uint8_t* qrow = lds + (lr < 56 ? kQA + lr * kQRowBytes : kQB + (lr - 56) * kQRowBytes);
#pragma unroll
      for (int kk = 0; kk < kD / 32; ++kk)
        qop[rt][kk] = *reinterpret_cast<const bf16x8*>(qrow + (((4 * kk + g) ^ ((lr >> 1) & 7)) << 4));
    }
    const float coef = a.sm_log2;
    // causal limits of this lane's rows; lim_lo is the first token any real
    // row of the workgroup masks (rows past R pad the group)
    int lim[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int row = r0 + 32 * rh + 16 * rt + m;
      lim[rt] = row < a.R ? L - a.n_q + row / a.H + 1 : 0;
    }
    const int lim_lo = L - a.n_q + r0 / a.H + 1;
    // LDS byte offsets of this lane's K chunk of k-step kk within a V buffer
    // (kk < 16: kvl[kk % 2] plus (kk / 2) * 2 KB) and a rope buffer
    // (kk = 16, 17: krl[kk - 16])
    uint32_t kvl[2], krl[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      kvl[e] = (uint32_t)(vslot(th, m, 4 * e + g) * 16);
      krl[e] = (uint32_t)(rslot(th, m, 4 * e + g) * 16);
    }
    float m0[2] = {-INFINITY, -INFINITY};    // log2-domain reference of this lane's rows
    float ymax[2] = {-INFINITY, -INFINITY};  // running max of score - reference
    float lsum[2] = {0.0f, 0.0f};            // this lane's share of the softmax sums (fp32 P)
    float lnrm[2] = {0.0f, 0.0f};            // the same over the bf16-rounded P that P V uses
    constexpr int KS = kD / 32;  // 18 k-steps
    constexpr int KW = 9;        // K chunks held in registers at a time
    bf16x8 kraw[KW];
    auto k_read = [&](int u, int kk) {
      kraw[kk % KW] = kk < 16 ? *reinterpret_cast<const bf16x8*>(s_v + (u % kVBuf) * kVBytes + kvl[kk & 1] + (kk >> 1) * 2048)
                              : *reinterpret_cast<const bf16x8*>(s_rope + (u % kRBuf) * kRBytes + krl[kk & 1]);
    };
    f32x4 S[2];  // [row tile]: tokens 4g .. 4g+3 of the lane's row
    auto qk = [&](int u, auto hook) {
#pragma unroll
      for (int kk = 0; kk < KW; ++kk) k_read(u, kk);
      f32x4 acc[2][2];  // [row tile][k-step parity]
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const bf16x8 kop = kraw[kk % KW];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          if (kk < 2) mfma_vvv0(acc[rt][kk & 1], kop, qop[rt][kk]);
          else mfma_vvv(acc[rt][kk & 1], kop, qop[rt][kk]);
        }
        if (kk + KW < KS) k_read(u, kk + KW);
        hook(kk);
      }
      mfma_result_fence_v(acc[0][0], acc[0][1]);
      mfma_result_tie_v(acc[1][0], acc[1][1]);
      S[0] = acc[0][0] + acc[0][1];
      S[1] = acc[1][0] + acc[1][1];
    };
    auto no_hook = [](int) {};
    // softmax, part 1: y = score * coef - reference (log2 units), masked past
    // each row's causal limit, and the running maxima; S is overwritten with y
    auto scores = [&](int u) {
      const int tbase = t_begin + u * kUnit + 16 * th + 4 * g;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const float mr = m0[rt] == -INFINITY ? 0.0f : m0[rt];
#pragma unroll
        for (int i = 0; i < 4; ++i) S[rt][i] = __builtin_fmaf(S[rt][i], coef, -mr);
        if (t_begin + u * kUnit + kUnit > lim_lo) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tbase + i >= lim[rt]) S[rt][i] = -INFINITY;
        }
        ymax[rt] = max3f(ymax[rt], max3f(S[rt][0], S[rt][1], S[rt][2]), S[rt][3]);
      }
    };
    // softmax, part 2: weights 2^y as bf16 P into LDS, and the sums.  Lanes l
    // and l ^ 16 hold tokens 4g .. 4g+3 and the other four of one 8-token chunk
    // of the same two rows; one permlane16_swap per word leaves the even-g lane
    // with the whole chunk of row tile 0 and the odd-g lane with that of row
    // tile 1, each written as one 16-byte store.
    auto weights = [&](int u) {
      uint32_t pk[2][2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(S[rt][i]);
        pk[rt][0] = pack_bf16x2(e[0], e[1]);
        pk[rt][1] = pack_bf16x2(e[2], e[3]);
        lnrm[rt] = dot2_bf16_ones(pk[rt][1], dot2_bf16_ones(pk[rt][0], lnrm[rt]));
        lsum[rt] += (e[0] + e[1]) + (e[2] + e[3]);
      }
      const auto w0 = __builtin_amdgcn_permlane16_swap(pk[0][0], pk[1][0], false, false);
      const auto w1 = __builtin_amdgcn_permlane16_swap(pk[0][1], pk[1][1], false, false);
      const int row = 32 * rh + 16 * (g & 1) + m;
      const int cc = 2 * th + (g >> 1);
      *reinterpret_cast<u32x4*>(s_p + (u & 1) * kPBytes + pbyte(row, cc)) = u32x4{w0[0], w1[0], w0[1], w1[1]};
    };
    auto set_flag = [&](int u, bool over) {
      const bool any_over = __any(over);
      if (lane == 0) s_flag[4 * (u & 1) + wave] = any_over ? 1 : 0;
    };
    auto over_ref = [&]() { return ymax[0] > kRefSlack || ymax[1] > kRefSlack; };

    for (;;) {
      bool scan = false;
      __syncthreads();  // (A) unit 0 is staged
      qk(0, no_hook);
      scores(0);
      if (!have_ref) {
        // the reference of each row is its maximum over the first unit
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const float pm = group4_max(ymax[rt]);
          if (g == 0) s_red[th * 64 + 32 * rh + 16 * rt + m] = pm;
        }
        __syncthreads();  // (B) first-unit maxima in LDS
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const int row = 32 * rh + 16 * rt + m;
          m0[rt] = fmaxf(s_red[row], s_red[64 + row]);
          const float mr = m0[rt] == -INFINITY ? 0.0f : m0[rt];
          S[rt] -= mr;
          ymax[rt] -= mr;
        }
        have_ref = true;
      }
      weights(0);
      set_flag(0, over_ref());
      __syncthreads();  // (C) P and flags of unit 0 are in LDS
      uint32_t fw = flag_word(0);
      for (int u = 1; u < n_u; ++u) {
        qk(u, [&](int kk) {
          if (kk == 3) {  // unit u - 1's flags, read after the barrier, are looked at here
            settle(fw);
            if (allow_scan && fw != 0u) scan = true;
          }
          // (M) QK^T of unit u is issued: the output waves start P V of unit
          // u - 1, which then runs beside this wave's softmax
          if (kk == KS - 1) __syncthreads();
        });
        scores(u);
        if (!scan) weights(u);
        set_flag(u, over_ref());
        __syncthreads();  // (D) P and flags of unit u in LDS; unit u - 1 consumed
        fw = flag_word(u);
      }
      settle(fw);
      if (allow_scan && fw != 0u) scan = true;
      if (!scan) break;
      // A weight would exceed 2^64: every unit of the split has been scored
      // since; run it again with each row's maximum as the reference.
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const float pm = group4_max(ymax[rt]);
        if (g == 0) s_red[th * 64 + 32 * rh + 16 * rt + m] = pm;
      }
      __syncthreads();  // (E) maxima in LDS; every copy has landed
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int row = 32 * rh + 16 * rt + m;
        const float pm = fmaxf(s_red[row], s_red[64 + row]);
        const float mr = m0[rt] == -INFINITY ? 0.0f : m0[rt];
        if (pm > -INFINITY) m0[rt] = fmaxf(m0[rt], mr + pm);
        ymax[rt] = -INFINITY;
        lsum[rt] = 0.0f;
        lnrm[rt] = 0.0f;
      }
      allow_scan = false;
    }
    // the sums of this wave's tokens for the output waves
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const float ls = group4_sum(lsum[rt]);
      const float ln = group4_sum(lnrm[rt]);
      if (g == 0) {
        const int row = 32 * rh + 16 * rt + m;
        s_lsum[th * 64 + row] = ls;
        s_lnrm[th * 64 + row] = ln;
        if (th == 0) s_m0[row] = m0[rt];
      }
    }
    __syncthreads();  // (F) sums in LDS
    return;
  }

  // =======================================================================
  // output waves: the same barrier sequence, P V one unit behind, and the
  // unit copies
  // =======================================================================
  const int j = wave - 4;  // dims 128j .. 128j+127 (wave-relative chunks 0..15)

  // Page ids of the split, 64 at a time, one per lane; picked out with
  // readlane so the copy issue never waits on a scalar load.  Every used one
  // is clamped to the pool.
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(ids) :: "memory");
  int id_chunk = 0;
  auto reload_ids = [&](int chunk) {
    id_chunk = chunk;
    const int32_t* src = a.block_table + bt_row + min(p_begin + (chunk << 6) + lane, p_end - 1);
    asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(ids) : "v"(src) : "memory");
  };
  // This wave copies quarter q = j / 2 of every unit: V chunk groups
  // 4(j % 2) .. 4(j % 2) + 3 (two instructions each, tokens 0..7 and 8..15 of
  // the quarter) and half j % 2 of the rope part.  Source offsets of this
  // lane's 16 bytes within the quarter: V tokens 0..7 and 8..15 (plus 128
  // bytes per chunk group), and the rope.
  const int q = j >> 1;
  uint32_t goff[3];
  {
    const int t8 = lane >> 3;
    goff[0] = (uint32_t)(t8 * kQRowBytes + 16 * ((lane & 7) ^ swz(t8)));
    goff[1] = (uint32_t)((8 + t8) * kQRowBytes + 16 * ((lane & 7) ^ swz(8 + t8)));
    const int mr = 8 * (j & 1) + t8;
    goff[2] = (uint32_t)(mr * kQRowBytes + 1024 + 16 * ((lane & 7) ^ swz(mr)));
  }
  auto dma_unit = [&](int u) {
    const int pi = u >> 1;  // page of the split
    if ((pi >> 6) != id_chunk) reload_ids(pi >> 6);
    const int pg = min(max(__builtin_amdgcn_readlane(ids, pi & 63), 0), a.num_pages - 1);
    const uint8_t* src = a.cache + (int64_t)pg * (kPage * kD * 2) + (u & 1) * kUnitBytes + q * 16 * kQRowBytes;
    const uint32_t vdst = lds_addr(s_v + (u % kVBuf) * kVBytes + q * 16384);
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int grp = 4 * (j & 1) + gi;
#pragma unroll
      for (int h = 0; h < 2; ++h) lds_dma16(src + 128 * grp, goff[h], vdst + grp * 2048 + h * 1024);
    }
    lds_dma16(src, goff[2], lds_addr(s_rope + (u % kRBuf) * kRBytes + q * 2048 + (j & 1) * 1024));
  };
  // This wave's part of unit u has landed (the caller waited): zero the V
  // bytes of its tokens past the end of the request (they may hold anything,
  // even NaN bits, and P V multiplies them by zero weights).
  auto staged = [&](int u) {
    const int nvalid = L - (t_begin + u * kUnit);
    if (nvalid < 16 * q + 16) {
      const int tl0 = max(nvalid - 16 * q, 0);
      const int per = (16 - tl0) * 8;  // slots per chunk group
      u32x4* v = reinterpret_cast<u32x4*>(s_v + (u % kVBuf) * kVBytes) + q * 1024 + tl0 * 8;
      for (int e = lane; e < 4 * per; e += 64) {
        const int grp = 4 * (j & 1) + e / per;
        v[grp * 128 + (e % per)] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  // O^T = V^T P^T on v_mfma_f32_32x32x16_bf16.  O[rt][dt] is the 32 x 32 tile
  // of rows 32rt .. 32rt+31 and the 32 dims of chunks tchunk(dt, 0..3) of this
  // wave's sixteen; lane l holds row 32rt + l%32 and, in element i, tile dim
  // M = 8(i/4) + 4(l/32) + i%4.  A unit is two k-steps of 16 tokens, k-step s
  // being quarter s; k index 8u + e (u = l/32) of k-step s is token 16s + 8u + e,
  // so the P operand of lane l is chunk 2s + u of its row: one 16-byte read.
  f32x16 O[2][4];
  // V operand: two transposing 16-bit reads (tokens e = 0..3 and 4..7) per
  // (k-step, dim tile).  Lane 4j' + q' of 16-lane group G addresses token
  // 8(G/2) + 4r + j' of the quarter, dims 4(q' % 2) .. +3 of chunk
  // tchunk(dt, 2(G % 2) + q'/2): vo[dt][r] plus s * 16 KB and j * 4 KB.
  uint32_t vo[4][2];
  {
    const int jj = m >> 2, qq = m & 3;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        vo[dt][r] = (uint32_t)(vslot(0, 8 * (g >> 1) + 4 * r + jj, tchunk(dt, 2 * (g & 1) + (qq >> 1))) * 16 + 8 * (qq & 1));
  }
  // P operand: row 32rt + l%32, chunk 2s + l/32
  uint32_t po[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) po[s] = (uint32_t)pbyte(lane & 31, 2 * s + (lane >> 5));
  auto pv = [&](int u) {
    const uint8_t* vb = s_v + (u % kVBuf) * kVBytes + j * 4096;
    const uint8_t* pp = s_p + (u & 1) * kPBytes;
    u32x2 vr[2][4][2];  // [step][dim tile][token half]
    bf16x8 pb[2][2];    // [step][row tile]
    auto load = [&](int s) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 2; ++r) vr[s][dt][r] = lds_read_tr16(vb + vo[dt][r] + s * 16384);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) pb[s][rt] = *reinterpret_cast<const bf16x8*>(pp + po[s] + rt * 2048);
    };
    load(0);
    load(1);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      phase_fence();
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x8 vop = __builtin_bit_cast(bf16x8, u32x4{vr[s][dt][0].x, vr[s][dt][0].y, vr[s][dt][1].x, vr[s][dt][1].y});
        mfma32_w(O[0][dt], vop, pb[s][0]);
        mfma32_w(O[1][dt], vop, pb[s][1]);
      }
    }
    const bf16x8 last = __builtin_bit_cast(bf16x8, u32x4{vr[1][3][0].x, vr[1][3][0].y, vr[1][3][1].x, vr[1][3][1].y});
    mfma32_tie8(O, last, pb[1][0], pb[1][1]);
    phase_fence();
  };

  // Unit 0 goes out before the query barrier (its buffers are not the
  // query's), unit 1 only once unit 0 has landed.  A rerun sends unit 0 again
  // at the end of its first pass.
  auto first_units = [&]() { dma_unit(0); };
  first_units();
  __syncthreads();  // (Q)
  for (;;) {
    bool scan = false;
    mfma32_def_zero8(O);
    // unit 0 landed; unit 1 goes out
    wait_vmcnt<0>();
    if (n_u > 1) dma_unit(1);
    staged(0);
    __syncthreads();  // (A)
    if (!have_ref) {
      __syncthreads();  // (B) the score waves have read the query: its buffers are free
      have_ref = true;
    }
    if (n_u > 2) dma_unit(2);
    if (n_u > 1) {
      if (n_u > 2) wait_vmcnt<kLoads>(); else wait_vmcnt<0>();
      staged(1);
    }
    __syncthreads();  // (C)
    uint32_t fo = flag_word(0);
    for (int u = 1; u <= n_u; ++u) {
      // The copy of unit u + 2 (its buffers were last read by P V of unit
      // u - 2 and QK^T of unit u - 1, both before barrier D), issued while
      // this wave waits for barrier M; P V of unit u - 1 then runs beside the
      // score waves' softmax.  The last pass has no QK^T to wait for.
      if (u + 2 < n_u) dma_unit(u + 2);
      if (u < n_u) __syncthreads();  // (M)
      phase_fence();
      __builtin_amdgcn_s_setprio(1);
      if (!scan) pv(u - 1);
      __builtin_amdgcn_s_setprio(0);
      phase_fence();
      settle(fo);
      if (allow_scan && fo != 0u) scan = true;
      if (u == n_u) break;
      if (u + 1 < n_u) {
        if (u + 2 < n_u) wait_vmcnt<kLoads>(); else wait_vmcnt<0>();
        staged(u + 1);
      }
      __syncthreads();  // (D)
      fo = flag_word(u);
    }
    if (!scan) break;
    __syncthreads();  // (E)
    allow_scan = false;
    if (id_chunk != 0) reload_ids(0);
    first_units();
  }

  __syncthreads();  // (F) the score waves' sums are in LDS; every unit buffer is free
  // Normalisation: lane l owns rows 32rt + l%32; the output is a weighted mean
  // with the bf16 weights P V used, the LSE uses the fp32 weights (lanes
  // l < 32 of wave 4 write it).
  const bool single = a.max_splits == 1;
  const int64_t prow0 = single ? (int64_t)b * a.R + r0 : ((int64_t)b * a.max_splits + split) * a.R + r0;
  float inv[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = 32 * rt + (lane & 31);
    const float ln = s_lnrm[row] + s_lnrm[64 + row];
    inv[rt] = ln > 0.0f ? 1.0f / ln : 0.0f;
    if (j == 0 && lane < 32 && r0 + row < a.R) {
      const float lt = s_lsum[row] + s_lsum[64 + row];
      const float mr = s_m0[row] == -INFINITY ? 0.0f : s_m0[row];
      __builtin_nontemporal_store(lt > 0.0f ? (mr + __log2f(lt)) * kLn2 : -INFINITY, (single ? a.lse : a.lse_part) + prow0 + row);
    }
  }
  // Stores: lane l holds, per [rt][dt] and k = i/4, four consecutive bf16 of
  // row 32rt + l%32: dims 4(l/32) .. +3 of chunk tchunk(dt, k).  They go
  // through LDS (this wave's 64 rows x 256 bytes, rows 272 bytes apart) so
  // that each store moves 16 contiguous bytes per lane and 16 lanes fill one
  // row's 256 bytes; the global stores are non-temporal (every workgroup
  // writes its partials at about the same time).  Only this wave touches its
  // tile, and a wave's LDS accesses complete in order.
  mfma32_result_fence8(O);
  constexpr int kTileStride = 272;
  uint8_t* tile = lds + j * (kRowsB * kTileStride);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x16& o = O[rt][dt];
        *reinterpret_cast<u32x2*>(tile + (32 * rt + (lane & 31)) * kTileStride + 16 * tchunk(dt, k) + 8 * (lane >> 5)) =
            u32x2{pack_bf16x2(o[4 * k] * inv[rt], o[4 * k + 1] * inv[rt]),
                  pack_bf16x2(o[4 * k + 2] * inv[rt], o[4 * k + 3] * inv[rt])};
      }
  uint16_t* dst = (single ? a.out : a.o_part) + prow0 * kDV + j * 128;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int row = 4 * k + (lane >> 4), c = lane & 15;  // 64 rows x 16 chunks of 8 dims
    const u32x4 v = *reinterpret_cast<const u32x4*>(tile + row * kTileStride + 16 * c);
    if (r0 + row < a.R) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + (int64_t)row * kDV + 8 * c));
  }
}

}  // namespace

int decode_rows_per_group(int cache_kind) { return cache_kind == kFp8 ? decode_rows_fp8() : kRowsB; }

hipError_t launch_decode(const DecodeArgs& a0, int cache_kind, int scale_mode, hipStream_t stream) {
  DecodeArgs a = a0;
  const int rows = decode_rows_per_group(cache_kind);
  a.n_rg = (a.R + rows - 1) / rows;
  if (cache_kind == kFp8) return launch_decode_fp8(a, scale_mode, stream);
  const dim3 grid((unsigned)decode_grid_size(a.B, a.max_splits, a.n_rg)), block(512);
  hipLaunchKernelGGL(decode_bf16_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
