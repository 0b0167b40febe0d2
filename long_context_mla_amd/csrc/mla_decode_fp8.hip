// mla_decode_paged, FP8 cache: split-KV decode attention with specialised
// waves.  Computes what mla_decode.hip describes (one 576-element latent row
// per token as key and value, "How to serve trillions of tokens for
// trillion-parameter coding agents", sections "First, understand the workload"
// and "Tensor parallel was the best parallelism strategy for maximum
// interactivity"; an e4m3 cache converted as it is read, "Smaller, faster,
// safer: running Kimi and GLM at scale", section "Quantizing the KV cache").
//
// gfx950 design: one 512-thread workgroup (8 waves, two per SIMD) per
// (request, split, group of 64 query rows), one per CU.  64 rows cover every
// head of one query token of the 64-head models, so each page of a split is
// fetched into LDS once per compute unit: the per-unit fetch rate, not HBM,
// caps a page stream on this chip (about 30 GB/s per unit by LDS-DMA), and
// a page read by two 32-row workgroups costs its units twice the bytes.
//  * score waves 0..3: wave w = 2*th + rh holds the query of rows
//    32rh .. 32rh+31 in VGPRs (bf16 MFMA operands) and computes S^T = K Q^T for
//    tokens 32th .. 32th+31 of each page, the softmax weights P (bf16, into
//    LDS) and the sums;
//  * output waves 4..7: wave 4+j accumulates O[64 rows][128j .. 128j+127] +=
//    P V over the previous page, V being the first 512 columns of the same
//    staged rows (transposing LDS reads), and copies quarter j (tokens
//    16j .. 16j+15) of every page HBM -> LDS by LDS-DMA, two pages ahead.
// Two barriers per page: D separates "scores of page p" from "P V of page p",
// and M, once the score waves have issued QK^T of page p + 1, starts P V of
// page p, so that it runs beside their softmax.
//
// LDS: the V parts (first 512 bytes of each row) of four pages, the rope parts
// (last 64 bytes) of three (rope bytes are dead once the scores of their page
// are done, a page before its V bytes), P of two pages, and small arrays.
//
// mla_decode_paged_append runs the same kernel with the step's new rows: the
// output wave that copies a new row's slot encodes it into its LDS copy of the
// page (as kv_append_fp8 would), and row group 0 writes it to the cache.
//
// Softmax: one fixed reference per row and split (the first page's maximum),
// weights 2^(y - m0).  A weight above 2^64 switches the split to a scan: the
// remaining pages are scored (no weights, no P V) to find every row's maximum,
// and the split runs once more with that maximum as its reference, which no
// score can exceed.  The output divides by the sum of the bf16 weights that
// P V used; the LSE uses the exact fp32 sum.
#include <type_traits>

#include "decode_tile.h"
#include "page_check.h"
#include "device_common.h"
#include "launch.h"

namespace mla {

namespace {

constexpr int kRows8 = 64;       // query rows per workgroup
constexpr int kVBuf = 4;         // staged V parts (pages)
constexpr int kRBuf = 3;         // staged rope parts (pages)
constexpr int kVBytes = 32768;   // V part of a page: 64 tokens x 512 bytes
constexpr int kRBytes = 4096;    // rope part: 64 tokens x 64 bytes
constexpr int kPBytes = kRows8 * 128;  // P of a page: 64 rows x 64 tokens bf16
constexpr int kLoads = 9;        // 1 KB LDS-DMA loads per output wave per page (8 V + 1 rope)

// LDS map (bytes)
constexpr int kOffV = 0;
constexpr int kOffR = kOffV + kVBuf * kVBytes;      // 131072
constexpr int kOffP = kOffR + kRBuf * kRBytes;      // 143360
constexpr int kOffScale = kOffP + 2 * kPBytes;      // 159744: fp32 [4][64]
constexpr int kOffRed = kOffScale + kVBuf * 256;    // 160768: fp32 [2][64]
constexpr int kOffLsum = kOffRed + 512;             // fp32 [2][64]
constexpr int kOffLnrm = kOffLsum + 512;            // fp32 [2][64]
constexpr int kOffM0 = kOffLnrm + 512;              // fp32 [64]
constexpr int kOffFlag = kOffM0 + 256;              // uint32 [2]
constexpr int kLdsBytes = kOffFlag + 16;
// The query of the group's 64 rows (73,728 bytes) is staged once at the start
// over buffers that stay free until page 2's copy: rows 0..55 over V buffers
// 2 and 3, rows 56..63 over rope buffer 2 and P buffer 0.
constexpr int kQA = kOffV + 2 * kVBytes;            // 65536: 56 rows
constexpr int kQB = kOffR + 2 * kRBytes;            // 139264: 8 rows
constexpr int kQRowBytes = kD * 2;                  // 1152
static_assert(kQA + 56 * kQRowBytes <= kOffR && kQB + 8 * kQRowBytes <= kOffP + kPBytes, "query staging");
constexpr int kQLoads = 18;                         // 1 KB query copies per score wave (72 in all)
static_assert(kLdsBytes <= 163840, "LDS");
static_assert(4 * kRows8 * 272 <= kOffP, "the output tiles fit over the page buffers");

// Staged page layout.  Token t = 16q + m of the page (quarter q, m < 16).
// The V part of its row (16-byte chunks c < 32) sits in V-buffer slot
//   vslot(q, m, c) = q*512 + (c/8)*128 + 8m + ((c%8) ^ vswz(m)),  vswz(m) = (m/2) % 8:
// eight chunks of one token side by side (128 bytes).  The rope part (chunks
// 32..35, c' = c - 32) sits in rope-buffer slot
//   rslot(q, m, c') = q*64 + 8(m/2) + ((4(m%2) + c') ^ rswz(m)),  rswz(m) = (m/4) % 4:
// two tokens per 128 bytes.  Then
//  * one LDS-DMA instruction fills one group of 64 slots.  V group i of a
//    quarter holds tokens 8(i%2) .. +7 and chunks 8(i/2) .. +7 (lane l brings
//    token 8(i%2) + l/8, chunk 8(i/2) + ((l%8) ^ vswz)); the rope group holds
//    the quarter's 16 tokens (lane l brings token 2(l/8) + (l/4)%2, rope chunk
//    (l%4) ^ rswz).  Eight (four) consecutive lanes read one token's bytes.
//  * the QK^T operand reads (16 tokens of a quarter, one 16-byte chunk each,
//    per 16 lanes) and the transposing P V reads (8-byte halves of chunks x
//    and x ^ 2 of tokens 4u..4u+3 and 8+4u..8+4u+3 of a quarter) run without
//    LDS bank conflicts.  That was measured with the bank-conflict counter on
//    this chip: a layout with the four chunks of a 64-byte group side by side
//    (tokens 64 bytes apart) cost four stall cycles on every QK^T read, and
//    swizzles of two bits instead of three cost as much.
__device__ __forceinline__ int vswz(int m) { return (m >> 1) & 7; }
__device__ __forceinline__ int rswz(int m) { return (m >> 2) & 3; }
__device__ __forceinline__ int vslot(int q, int m, int c) { return q * 512 + (c >> 3) * 128 + 8 * m + ((c & 7) ^ vswz(m)); }
__device__ __forceinline__ int rslot(int q, int m, int c) { return q * 64 + 8 * (m >> 1) + ((4 * (m & 1) + c) ^ rswz(m)); }

// Keeps the compiler from moving memory accesses across this point (no
// instruction): it stops loads of a later phase from being hoisted over the
// MFMAs of an earlier one, where their registers would be live at once.
__device__ __forceinline__ void phase_fence() { asm volatile("" ::: "memory"); }

template <int SCALE, bool CHECKED>
__global__ __launch_bounds__(512, 1) void decode_fp8_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  uint8_t* const s_v = lds + kOffV;
  uint8_t* const s_rope = lds + kOffR;
  uint8_t* const s_p = lds + kOffP;
  float* const s_scale = reinterpret_cast<float*>(lds + kOffScale);
  float* const s_red = reinterpret_cast<float*>(lds + kOffRed);
  float* const s_lsum = reinterpret_cast<float*>(lds + kOffLsum);
  float* const s_lnrm = reinterpret_cast<float*>(lds + kOffLnrm);
  float* const s_m0 = reinterpret_cast<float*>(lds + kOffM0);
  uint8_t* const s_flag = lds + kOffFlag;  // [page parity][score wave], one byte each

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
    const int st = check_request<512>(c, cb, a.seq_lens[cb], reinterpret_cast<int*>(s_red));
    if (threadIdx.x == 0) a.status[cb] = st;
    return;
  }

  // One round trip for the launch arguments the first loads need.
  asm volatile("" :: "s"(a.q), "s"(a.block_table), "s"(a.seq_lens), "s"(a.n_rg), "s"(a.max_blocks));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool scorer = wave < 4;
  const int m = lane & 15, g = lane >> 4;
  const WorkUnit wu = decode_work_unit(a.B, a.max_splits, a.n_rg);
  if (!wu.valid) return;
  const int b = wu.b, split = wu.split, rg = wu.rg;
  const int r0 = rg * kRows8;
  const int p_begin = split * a.pps;
  const int64_t bt_row = (int64_t)b * a.max_blocks;
  const int cap = a.max_blocks * kPage;

  // The output waves' first 64 page ids of the split go out before the length
  // is known (bounded by the table row, not yet by the length), one per lane,
  // so that their latency overlaps the length's.
  int ids = 0;
  const int rh = wave & 1, th = (wave >> 1) & 1;
  // The score waves copy the query of the group's 64 rows HBM -> LDS in 72
  // coalesced 1 KB LDS-DMA copies (the rows are contiguous in q): slot s
  // (16 bytes) of the staged query is row s / 72, chunk (s % 72) ^ ((row / 2) % 8),
  // which makes the operand reads below free of bank conflicts.  Rows past R
  // repeat row R - 1.
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
  const int L_raw = load_const(a.seq_lens, b);
  const int L = min(max(L_raw, 0), cap);
  const int n_pages = (L + kPage - 1) / kPage;

  if (p_begin >= n_pages) {
    // Nothing to read.  Only an empty request's first split reports it; the
    // combine never reads splits past a request's last page.  (Every copy
    // lands before the workgroup ends.)
    wait_vmcnt<0>();
    if (n_pages == 0 && split == 0) {
      for (int e = threadIdx.x; e < kRows8 * kDV; e += 512) {
        const int r = r0 + e / kDV;
        if (r >= a.R) break;
        if (a.max_splits == 1)
          a.out[((int64_t)b * a.R + r) * kDV + e % kDV] = 0;
        else
          a.o_part[((int64_t)b * a.max_splits * a.R + r) * kDV + e % kDV] = 0;
      }
      for (int r = r0 + threadIdx.x; r < min(r0 + kRows8, a.R); r += 512) {
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
  bool have_ref = false;   // the reference is fixed (first page done, or a rerun)
  bool allow_scan = true;  // the first run may switch to a scan; the rerun cannot need one

  // The four score waves' overflow flags of page it, one byte each, read as
  // one word right after the barrier that publishes them and looked at only
  // after the next block of MFMA work has been issued: settle() ties the word
  // to that point, so the LDS latency of the read is not waited for at the
  // barrier.
  auto flag_word = [&](int it) { return *reinterpret_cast<const uint32_t*>(s_flag + 4 * (it & 1)); };
  auto settle = [](uint32_t& f) {
    asm volatile("" : "+v"(f));
    f = __builtin_amdgcn_readfirstlane(f);  // uniform again for the branch on it
  };

  if (scorer) {
    // =====================================================================
    // score waves: rows 32rh .. 32rh+31, tokens 32th .. 32th+31 of each page
    // =====================================================================
    // QK^T runs on v_mfma_f32_32x32x16_bf16: one 32 x 32 tile is this wave's
    // 32 tokens x 32 rows, and the 36 k-blocks of 16 dims alternate between two
    // accumulators (even and odd k-blocks), which keeps the matrix core busy
    // through the dependent-accumulation latency (about 44 cycles, longer than
    // one 32-cycle MFMA).  Lane l works on row 32rh + (l % 32) of the query and,
    // as the K operand, on token 32th + (l % 32) of the page; its k half is
    // sg = l / 32.  K-block 2p + e holds the dims 32p + 16sg + 8e .. +8 of the
    // lane: bytes 8e .. 8e+7 of the token's 16-byte chunk 2p + sg, and the
    // query's 16-byte chunk 4p + 2sg + e.
    const int sn = lane & 31, sg = lane >> 5;
    const int lr = 32 * rh + sn;  // this lane's row within the group
    bf16x8 qop[kD / 16];          // the row's 36 query operands, for the whole split
    wait_vmcnt<0>();  // this wave's query copies have landed
    __syncthreads();  // (Q) the query is staged
    {
      const uint8_t* qrow = lds + (lr < 56 ? kQA + lr * kQRowBytes : kQB + (lr - 56) * kQRowBytes);
#pragma unroll
      for (int kb = 0; kb < kD / 16; ++kb) {
        const int c = 4 * (kb >> 1) + 2 * sg + (kb & 1);
        qop[kb] = *reinterpret_cast<const bf16x8*>(qrow + ((c ^ ((lr >> 1) & 7)) << 4));
      }
    }
    const float coef = a.sm_log2 * tscale;
    // causal limit of this lane's row: row i*H + h sees tokens
    // t < L - n_q + i + 1; lim_lo is the first token any real row of the
    // workgroup masks, so earlier pages need no mask (rows past R pad the group)
    const int lim = r0 + lr < a.R ? L - a.n_q + (r0 + lr) / a.H + 1 : 0;
    const int lim_lo = L - a.n_q + r0 / a.H + 1;
    // LDS byte offsets of this lane's K chunk 2p + sg (token 32th + sn: quarter
    // tq, token tm of it): within a V buffer for p < 16 (kvl[p % 4], plus
    // (p / 4) * 2 KB) and within a rope buffer for p = 16, 17 (krl[p - 16])
    const int tq = 2 * th + (sn >> 4), tm = sn & 15;
    uint32_t kvl[4], krl[2];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) kvl[a4] = (uint32_t)(vslot(tq, tm, 2 * a4 + sg) * 16);
#pragma unroll
    for (int e = 0; e < 2; ++e) krl[e] = (uint32_t)(rslot(tq, tm, 2 * e + sg) * 16);
    float m0 = -INFINITY;    // log2-domain reference of this lane's row
    float ymax = -INFINITY;  // running max of score - reference
    float lsum = 0.0f;       // this lane's share of the softmax sum (fp32 P)
    float lnrm = 0.0f;       // the same over the bf16-rounded P that P V uses
    constexpr int KP = kD / 32;  // 18 16-byte chunks per token and k half
    constexpr int KW = 9;        // K chunks held in registers at a time
    u32x4 kraw[KW];              // chunk p of the page in kraw[p % KW]
    auto k_read = [&](int it, int p) {
      kraw[p % KW] = p < 16 ? *reinterpret_cast<const u32x4*>(s_v + (it % kVBuf) * kVBytes + kvl[p & 3] + (p >> 2) * 2048)
                            : *reinterpret_cast<const u32x4*>(s_rope + (it % kRBuf) * kRBytes + krl[p & 1]);
    };
    f32x16 S;  // S^T tile: element r is token 32th + 8(r/4) + 4sg + r%4 of the lane's row
    // QK^T of page it: chunk p feeds k-blocks 2p (even accumulator) and 2p + 1
    // (odd); each chunk's conversions ride between MFMAs, and once a chunk is
    // converted its register is refilled with chunk p + 9.  hook(p) runs at
    // the end of step p.
    auto qk = [&](int it, auto hook) {
#pragma unroll
      for (int p = 0; p < KW; ++p) k_read(it, p);
      f32x16 se, so;
      // operands of step p are converted during step p - 1, so no MFMA waits
      // for the conversions just before it
      uint32_t E[2][4], O[2][4];
      auto cvt_even = [&](uint32_t (&d)[4], const u32x4 w) {
        d[0] = cvt_e4m3_lo(w[0]);
        d[1] = cvt_e4m3_hi(w[0]);
        d[2] = cvt_e4m3_lo(w[1]);
        d[3] = cvt_e4m3_hi(w[1]);
      };
      auto cvt_odd = [&](uint32_t (&d)[4], const u32x4 w) {
        d[0] = cvt_e4m3_lo(w[2]);
        d[1] = cvt_e4m3_hi(w[2]);
        d[2] = cvt_e4m3_lo(w[3]);
        d[3] = cvt_e4m3_hi(w[3]);
      };
      cvt_even(E[0], kraw[0]);
      cvt_odd(O[0], kraw[0]);
#pragma unroll
      for (int p = 0; p < KP; ++p) {
        const bool more = p + 1 < KP;
        if (p == 0) mfma32_first_w(se, bf16x8_of(E[0]), qop[0]); else mfma32(se, bf16x8_of(E[p & 1]), qop[2 * p]);
        if (more) cvt_even(E[(p + 1) & 1], kraw[(p + 1) % KW]);
        if (p == 0) mfma32_first(so, bf16x8_of(O[0]), qop[1]); else mfma32(so, bf16x8_of(O[p & 1]), qop[2 * p + 1]);
        if (more) cvt_odd(O[(p + 1) & 1], kraw[(p + 1) % KW]);
        if (p + KW < KP) k_read(it, p + KW);
        hook(p);
      }
      mfma32_drain(se, so, bf16x8_of(O[(KP - 1) & 1]));
      S = se + so;
    };
    auto no_hook = [](int) {};
    // softmax, part 1: y = score * coef - reference (log2 units), masked past
    // the row's causal limit, and the running maximum; S is overwritten with y
    f32x4 sc[4] = {{1.f, 1.f, 1.f, 1.f}, {1.f, 1.f, 1.f, 1.f}, {1.f, 1.f, 1.f, 1.f}, {1.f, 1.f, 1.f, 1.f}};
    auto scores = [&](int it) {
      const int tbase = (p_begin + it) * kPage + 32 * th + 4 * sg;
      const float mr = m0 == -INFINITY ? 0.0f : m0;
#pragma unroll
      for (int jr = 0; jr < 4; ++jr) {
        if (SCALE == kScaleToken)
          sc[jr] = *reinterpret_cast<const f32x4*>(&s_scale[(it % kVBuf) * 64 + 32 * th + 8 * jr + 4 * sg]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[4 * jr + i] = __builtin_fmaf(S[4 * jr + i], SCALE == kScaleToken ? coef * sc[jr][i] : coef, -mr);
      }
      if ((p_begin + it) * kPage + kPage > lim_lo) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (tbase + 8 * (r >> 2) + (r & 3) >= lim) S[r] = -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 16; r += 2) ymax = max3f(ymax, S[r], S[r + 1]);
    };
    // softmax, part 2: weights 2^y as bf16 P into LDS (two 16-byte chunks per
    // lane: elements 8h .. 8h+7 are tokens 16h + 4sg + i and 16h + 8 + 4sg + i,
    // the k order P V reads them in), and the sums
    auto weights = [&](int it) {
      uint8_t* prow = s_p + (it & 1) * kPBytes + lr * 128;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = __builtin_amdgcn_exp2f(S[8 * h + i]);
        uint32_t pk[4];
        if (SCALE == kScaleToken) {
          // the per-token V scale rides on the weight; the sums stay unscaled
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pk[i] = pack_bf16x2(e[2 * i] * sc[2 * h + (i >> 1)][(2 * i) & 3], e[2 * i + 1] * sc[2 * h + (i >> 1)][(2 * i + 1) & 3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pk[i] = pack_bf16x2(e[2 * i], e[2 * i + 1]);
            lnrm = dot2_bf16_ones(pk[i], lnrm);
          }
        }
        lsum += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
        // 16-byte chunk 4th + 2h + sg of the row, swizzled by the row
        *reinterpret_cast<u32x4*>(prow + (((4 * th + 2 * h + sg) ^ ((lr >> 1) & 7)) << 4)) =
            u32x4{pk[0], pk[1], pk[2], pk[3]};
      }
    };
    auto set_flag = [&](int it, bool over) {
      const bool any_over = __any(over);
      if (lane == 0) s_flag[4 * (it & 1) + wave] = any_over ? 1 : 0;
    };
    // maximum / sum of the two k-half lanes of a row (lanes l and l ^ 32)
    auto pair_max = [](float v) {
      const auto b = __builtin_amdgcn_permlane32_swap(bits_of(v), bits_of(v), false, false);
      return fmaxf(float_of(b[0]), float_of(b[1]));
    };
    auto pair_sum = [](float v) {
      const auto b = __builtin_amdgcn_permlane32_swap(bits_of(v), bits_of(v), false, false);
      return float_of(b[0]) + float_of(b[1]);
    };

    for (;;) {
      bool scan = false;
      __syncthreads();  // (A) page 0 is staged
      qk(0, no_hook);
      scores(0);
      if (!have_ref) {
        // the reference of each row is its maximum over the first page
        const float pm = pair_max(ymax);
        if (sg == 0) s_red[th * 64 + lr] = pm;
        __syncthreads();  // (B) first-page maxima in LDS
        m0 = fmaxf(s_red[lr], s_red[64 + lr]);
        const float mr = m0 == -INFINITY ? 0.0f : m0;
#pragma unroll
        for (int r = 0; r < 16; ++r) S[r] -= mr;
        ymax -= mr;
        have_ref = true;
      }
      weights(0);
      set_flag(0, ymax > kRefSlack);
      __syncthreads();  // (C) P and flags of page 0 are in LDS
      uint32_t fw = flag_word(0);
      for (int it = 1; it < n_it; ++it) {
        qk(it, [&](int p) {
          if (p == 3) {  // page it - 1's flags, read after the barrier, are looked at here
            settle(fw);
            if (allow_scan && fw != 0u) scan = true;
          }
          // (M) QK^T of page it is issued: the output waves start P V of
          // page it - 1, which then runs beside this wave's softmax
          if (p == KP - 1) __syncthreads();
        });
        scores(it);
        if (!scan) weights(it);
        set_flag(it, ymax > kRefSlack);
        __syncthreads();  // (D) P and flags of page it in LDS; page it - 1 consumed
        fw = flag_word(it);
      }
      settle(fw);
      if (allow_scan && fw != 0u) scan = true;
      if (!scan) break;
      // A weight would exceed 2^64: every page of the split has been scored
      // since; run it again with each row's maximum as the reference.
      {
        const float pm = pair_max(ymax);
        if (sg == 0) s_red[th * 64 + lr] = pm;
      }
      __syncthreads();  // (E) maxima in LDS; every copy has landed
      {
        const float pm = fmaxf(s_red[lr], s_red[64 + lr]);
        const float mr = m0 == -INFINITY ? 0.0f : m0;
        if (pm > -INFINITY) m0 = fmaxf(m0, mr + pm);
        ymax = -INFINITY;
        lsum = 0.0f;
        lnrm = 0.0f;
      }
      allow_scan = false;
    }
    // the sums of this wave's tokens for the output waves
    {
      const float ls = pair_sum(lsum);
      const float ln = SCALE == kScaleToken ? ls : pair_sum(lnrm);
      if (sg == 0) {
        s_lsum[th * 64 + lr] = ls;
        s_lnrm[th * 64 + lr] = ln;
        if (th == 0) s_m0[lr] = m0;
      }
    }
    __syncthreads();  // (F) sums in LDS
    return;
  }

  // =======================================================================
  // output waves: the same barrier sequence, P V one page behind, and the
  // page copies
  // =======================================================================
  const int j = wave - 4;  // dims 128j .. 128j+127; copies quarter j
  constexpr int LPP = kLoads + (SCALE == kScaleToken ? 1 : 0);  // loads per page per wave

  // Page ids of the split, 64 at a time, one per lane; picked out with
  // readlane so the copy issue never waits on a scalar load.  Ids past the
  // split are never used; every used one is clamped to the pool.
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(ids) :: "memory");
  int id_chunk = 0;
  auto reload_ids = [&](int chunk) {
    id_chunk = chunk;
    const int32_t* src = a.block_table + bt_row + min(p_begin + (chunk << 6) + lane, p_end - 1);
    asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(ids) : "v"(src) : "memory");
  };
  // Source offsets (within a page) of this lane's 16 bytes of quarter j: V
  // groups i even and odd (plus 128 (i / 2) bytes), and the rope group.
  uint32_t goff[3];
  {
    const int t8 = lane >> 3, mr = 2 * t8 + ((lane >> 2) & 1);
    goff[0] = (uint32_t)((16 * j + t8) * kD + 16 * ((lane & 7) ^ vswz(t8)));
    goff[1] = (uint32_t)((16 * j + 8 + t8) * kD + 16 * ((lane & 7) ^ vswz(8 + t8)));
    goff[2] = (uint32_t)((16 * j + mr) * kD + 512 + 16 * ((lane & 3) ^ rswz(mr)));
  }
  // Pieces p0 .. p1-1 of the copy of page it: groups 0..7 of the V part, the
  // rope part, then (per-token scales) the scales.
  auto dma_parts = [&](int it, int p0, int p1) {
    if ((it >> 6) != id_chunk) reload_ids(it >> 6);
    const int pg = min(max(__builtin_amdgcn_readlane(ids, it & 63), 0), a.num_pages - 1);
    const uint8_t* src = a.cache + (int64_t)pg * (kPage * kD);
    const uint32_t vdst = lds_addr(s_v + (it % kVBuf) * kVBytes + j * 8192);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i >= p0 && i < p1) lds_dma16(src + 128 * (i >> 1), goff[i & 1], vdst + 1024 * i);
    if (8 >= p0 && 8 < p1) lds_dma16(src, goff[2], lds_addr(s_rope + (it % kRBuf) * kRBytes + j * 1024));
    // the scales of this wave's own 16 tokens: a row appended in this launch
    // overwrites its scale in LDS after this wave's wait
    if (9 >= p0 && 9 < p1 && SCALE == kScaleToken && lane < 16)
      lds_dma4(a.kv_scale + (int64_t)pg * kPage + 16 * j, lane * 4, lds_addr(&s_scale[(it % kVBuf) * 64 + 16 * j]));
  };
  auto dma_page = [&](int it) { dma_parts(it, 0, 10); };

  // Rows appended in this launch that fall in this wave's quarter of page it:
  // encoded exactly as kv_append_fp8 does and put over the bytes the copy
  // brought (the cache still held the old contents); row group 0 also writes
  // them, and their per-token scales, to the cache for later steps.  Rows go
  // to positions L_raw - n_new + r; a row past the cache's reach is skipped.
  auto patch_new_rows = [&](int it) {
    const int t_first = (p_begin + it) * kPage + 16 * j;
    const int64_t first_new = (int64_t)L_raw - a.n_new;
    const int lo = (int)max(first_new, (int64_t)t_first), hi = min(L, t_first + 16);
    for (int pos = lo; pos < hi; ++pos) {
      u32x2 codes[2];
      const float sc = encode_row_e4m3<SCALE == kScaleToken>(
          a.kv_new + ((int64_t)b * a.n_new + (pos - first_new)) * kD, lane, tscale, codes);
      const int t = pos & (kPage - 1), tm = t & 15;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int c8 = lane + 64 * c;  // 8-byte chunk of the row
        if (c == 0 || lane < 8) {
          const int c16 = c8 >> 1;
          uint8_t* dst = c16 < 32 ? s_v + (it % kVBuf) * kVBytes + vslot(j, tm, c16) * 16
                                  : s_rope + (it % kRBuf) * kRBytes + rslot(j, tm, c16 - 32) * 16;
          *reinterpret_cast<u32x2*>(dst + 8 * (c8 & 1)) = codes[c];
        }
      }
      if (SCALE == kScaleToken && lane == 0) s_scale[(it % kVBuf) * 64 + t] = sc;
      bool store = rg == 0 && a.store_rows;
      const int64_t e = bt_row + pos / kPage;
      const int raw = load_const(a.block_table, e);
      // never write through a page id outside the pool
      store = store && raw >= 0 && raw < a.num_pages;
      if (CHECKED && store) {
        // the page check runs beside this launch: store only for a length
        // inside the map and into the recorded page carrying its tag
        const uint32_t cur = load_const(a.page_tags, raw);
        store = L_raw >= 0 && L_raw <= cap && raw == load_const(a.expected_pages, e) &&
                cur == load_const(a.expected_tags, e);
      }
      if (store) {
        uint8_t* dst = a.cache_out + ((int64_t)raw * kPage + t) * kD;
        *reinterpret_cast<u32x2*>(dst + 8 * lane) = codes[0];
        if (lane < 8) *reinterpret_cast<u32x2*>(dst + 8 * (lane + 64)) = codes[1];
        if (SCALE == kScaleToken && lane == 0) a.scale_out[(int64_t)raw * kPage + t] = sc;
      }
    }
    // the row loads and stores are counted like the copies: let them all
    // finish so the later waits keep their meaning
    if (lo < hi) wait_vmcnt<0>();
  };
  // This wave's quarter of page it has landed (the caller waited): zero its
  // tokens past the end of the request (they may hold anything, even NaN
  // codes, and P V multiplies them by zero weights), then the new rows.
  auto staged = [&](int it) {
    const int nvalid = L - (p_begin + it) * kPage;
    if (nvalid < 16 * j + 16) {
      const int tl0 = max(nvalid - 16 * j, 0);
      const int per = (16 - tl0) * 8;  // slots per group of eight chunks
      u32x4* v = reinterpret_cast<u32x4*>(s_v + (it % kVBuf) * kVBytes) + j * 512 + tl0 * 8;
      for (int e = lane; e < 4 * per; e += 64) {
        const int grp = e / per;
        v[grp * 128 + (e - grp * per)] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (a.n_new > 0) patch_new_rows(it);
  };

  // O^T = V^T P^T on v_mfma_f32_32x32x16_bf16.  O[rt][dt] is the 32 x 32
  // tile of rows 32rt .. 32rt+31 and of the 32 dims of chunks ca(dt) and
  // ca(dt) ^ 2 of this wave's eight 16-dim chunks, ca(dt) = dt%2 + 4(dt/2)
  // (that pairing keeps the V reads below free of bank conflicts).  Lane l
  // holds row 32rt + l%32 and, in element i, tile dim M = 8(i/4) + 4(l/32) + i%4:
  // dim M%16 of chunk ca(dt) ^ 2(M/16).  A page is four k-steps of 16 tokens,
  // k-step s being quarter s of the staged page.  K index 8u + e (u = l/32,
  // e < 8) of k-step s is token 16s + 4u + e + 4(e/4), the order the score
  // waves write P in (chunk 2s + u of a row of P holds those eight tokens), so
  // the P operand of lane l is one 16-byte read.
  f32x16 O[2][4];
  // V operand: a transposing read per (k-step, dim tile).  Lane 2e + h of
  // 16-lane group G addresses k index 8(G/2) + e of the step, i.e. token
  // m = 4(G/2) + e + 4(e/4) of the quarter, 8-byte half h of chunk
  // 8j + (ca(dt) ^ 2(G%2)): vslot(s, m, that chunk), i.e. vo[dt] plus
  // s * 8 KB and j * 2 KB.
  uint32_t vo[4];
  {
    const int e = m >> 1, h = m & 1;
    const int mt = 4 * (g >> 1) + e + 4 * (e >> 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      vo[dt] = (uint32_t)(vslot(0, mt, ((dt & 1) + 4 * (dt >> 1)) ^ (2 * (g & 1))) * 16 + 8 * h);
  }
  // P operand: row 32rt + l%32, chunk 2s + l/32, stored at chunk position
  // (2s + l/32) ^ ((row / 2) % 8) (the row swizzle does not depend on rt).
  uint32_t po[4];
  {
    const int pr = lane & 31, sw = (pr >> 1) & 7;
#pragma unroll
    for (int st = 0; st < 4; ++st) po[st] = (uint32_t)(pr * 128 + (((2 * st + (lane >> 5)) ^ sw) << 4));
  }
  auto pv = [&](int it) {
    const uint8_t* vb = s_v + (it % kVBuf) * kVBytes;
    const uint8_t* pp = s_p + (it & 1) * kPBytes;
    u32x2 vr[2][4];    // [step parity][dim tile]: raw fp8 V operands
    bf16x8 pb[2][2];   // [step parity][row tile]: P operands
    auto load = [&](int st) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) vr[st & 1][dt] = lds_read_tr8(vb + vo[dt] + st * 8192 + j * 2048);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) pb[st & 1][rt] = *reinterpret_cast<const bf16x8*>(pp + po[st] + rt * 4096);
    };
    load(0);
    uint32_t d[2][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      // the next step's operands are read while this step's MFMAs run
      if (st + 1 < 4) load(st + 1);
      phase_fence();
      const u32x2 (&v)[4] = vr[st & 1];
      d[0][0] = cvt_e4m3_lo(v[0].x);
      d[0][1] = cvt_e4m3_hi(v[0].x);
      d[0][2] = cvt_e4m3_lo(v[0].y);
      d[0][3] = cvt_e4m3_hi(v[0].y);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x8 vop = bf16x8_of(d[dt & 1]);
        uint32_t (&nx)[4] = d[(dt + 1) & 1];
        const bool more = dt + 1 < 4;
        mfma32_w(O[0][dt], vop, pb[st & 1][0]);
        if (more) {
          nx[0] = cvt_e4m3_lo(v[dt + 1].x);
          nx[1] = cvt_e4m3_hi(v[dt + 1].x);
        }
        mfma32(O[1][dt], vop, pb[st & 1][1]);
        if (more) {
          nx[2] = cvt_e4m3_lo(v[dt + 1].y);
          nx[3] = cvt_e4m3_hi(v[dt + 1].y);
        }
      }
    }
    // the last MFMAs' operands stay held until the next statement
    mfma32_tie8(O, bf16x8_of(d[1]), pb[1][0], pb[1][1]);
    phase_fence();
  };

  // Page 0 goes out before the query barrier (its buffers are not the
  // query's), page 1 only once page 0 has landed: at the start every compute
  // unit asks for its first pages at once, and page 0 alone lands sooner
  // (measured 0.3-0.6 us per launch) than pages 0 and 1 together.  A rerun
  // sends page 0 again at the end of its first pass.
  auto first_pages = [&]() { dma_page(0); };
  first_pages();
  __syncthreads();  // (Q)
  for (;;) {
    bool scan = false;
    mfma32_def_zero8(O);
    // page 0 landed; page 1 goes out
    wait_vmcnt<0>();
    if (n_it > 1) dma_page(1);
    staged(0);
    __syncthreads();  // (A)
    if (!have_ref) {
      __syncthreads();  // (B) the score waves have read the query: its buffers are free
      have_ref = true;
    }
    if (n_it > 2) dma_page(2);
    if (n_it > 1) {
      if (n_it > 2) wait_vmcnt<LPP>(); else wait_vmcnt<0>();
      staged(1);
    }
    __syncthreads();  // (C)
    // Page it - 1's flags are looked at after P V of page it - 1 has been
    // issued; when they ask for a scan that P V is wasted work (its operands
    // are valid) and O is cleared before the rerun.
    // (The last page's P V runs in the last pass of the loop, before that
    // page's flags are looked at; a scan then throws it away with the rest.)
    uint32_t fo = flag_word(0);
    for (int it = 1; it <= n_it; ++it) {
      // The copy of page it + 2 (its buffers were last read by P V of page
      // it - 2 and QK^T of page it - 1, both before barrier D), issued while
      // this wave would wait anyway: P V of page it - 1 starts only at barrier
      // M, once the score waves have issued QK^T of page it.  QK^T then has
      // the matrix core to itself, and P V overlaps the score waves' softmax
      // instead of QK^T (measured 2-3 % per launch over interleaving the two;
      // neither a barrier with the 16x16x32 P V nor the 32x32x16 P V without
      // one gained).  The last pass (it = n_it) has no QK^T to wait for.
      if (it + 2 < n_it) dma_page(it + 2);
      if (it < n_it) __syncthreads();  // (M)
      phase_fence();
      __builtin_amdgcn_s_setprio(1);
      if (!scan) pv(it - 1);
      __builtin_amdgcn_s_setprio(0);
      phase_fence();
      settle(fo);
      if (allow_scan && fo != 0u) scan = true;
      if (it == n_it) break;
      if (it + 1 < n_it) {
        if (it + 2 < n_it) wait_vmcnt<LPP>(); else wait_vmcnt<0>();
        staged(it + 1);
      }
      __syncthreads();  // (D)
      fo = flag_word(it);
    }
    if (!scan) break;
    __syncthreads();  // (E)
    allow_scan = false;
    if (id_chunk != 0) reload_ids(0);
    first_pages();
  }

  __syncthreads();  // (F) the score waves' sums are in LDS; every page buffer is free
  // Normalisation: lane l owns rows 32rt + l%32; the output is a weighted
  // mean with the bf16 weights P V used, the LSE uses the fp32 weights (lanes
  // l < 32 of wave 4 write it).
  const bool single = a.max_splits == 1;
  const int64_t prow0 = single ? (int64_t)b * a.R + r0 : ((int64_t)b * a.max_splits + split) * a.R + r0;
  float inv[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = 32 * rt + (lane & 31);
    const float ln = s_lnrm[row] + s_lnrm[64 + row];
    inv[rt] = ln > 0.0f ? tscale / ln : 0.0f;
    if (j == 0 && lane < 32 && r0 + row < a.R) {
      const float lt = s_lsum[row] + s_lsum[64 + row];
      const float mr = s_m0[row] == -INFINITY ? 0.0f : s_m0[row];
      __builtin_nontemporal_store(lt > 0.0f ? (mr + __log2f(lt)) * kLn2 : -INFINITY, (single ? a.lse : a.lse_part) + prow0 + row);
    }
  }
  // Stores: lane l holds, per [rt][dt] and k = i/4, four consecutive bf16 of
  // row 32rt + l%32: dims 8(k%2) + 4(l/32) .. +3 of chunk ca(dt) ^ 2(k/2).
  // The global stores are non-temporal: every workgroup of a launch writes
  // its 64 KB at about the same time, and with ordinary stores the lines were
  // still dirty in L2 when the launch ended (measured 1.0 us per launch at
  // 100k tokens, the combine reading them back 0.5 us slower).  They go through LDS (this wave's 64 rows x 256 bytes, rows
  // 272 bytes apart: 16-byte reads of whole rows) so that each store moves 16
  // contiguous bytes per lane and 16 lanes fill one row's 256 bytes.  Only
  // this wave touches its tile, and a wave's LDS accesses complete in order.
  mfma32_result_fence8(O);
  constexpr int kTileStride = 272;
  uint8_t* tile = lds + j * (kRows8 * kTileStride);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x16& o = O[rt][dt];
        const int ch = ((dt & 1) + 4 * (dt >> 1)) ^ (2 * (k >> 1));
        *reinterpret_cast<u32x2*>(tile + (32 * rt + (lane & 31)) * kTileStride + 32 * ch + 16 * (k & 1) + 8 * (lane >> 5)) =
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

int decode_rows_fp8() { return kRows8; }

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
