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
// gfx950 design.  One 256-thread workgroup (4 waves, one per SIMD) per
// (request, split, group of 32 query rows); one workgroup per CU.
//  * Pages stream HBM -> LDS with LDS-DMA (global_load_lds, no VGPRs), NBUF
//    deep.  Each lane picks its source chunk so that the page lands in a
//    swizzled layout whose operand reads are free of bank conflicts.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: wave w takes tokens 16w..16w+15
//    of the page for all 32 rows; the rows' query stays in registers as bf16
//    operands for the whole split.  FP8 codes become bf16 in registers
//    (exact); scales are applied to the fp32 scores.
//  * Softmax weights 2^(x - m0) use one reference per row, fixed from the
//    split's first page (the only page that exchanges row maxima).  O is never
//    rescaled: if a later score exceeds the reference by more than 2^64 the
//    split restarts from its first page with the larger reference.
//  * O += P V on MFMA with the accumulators in AGPRs: wave w takes output dims
//    128w..128w+127; V is the first 512 columns of the same staged page, read
//    with transposing LDS loads (ds_read_b64_tr_b8 / _b16).
//  * Epilogue: O / l and the natural-log LSE, either final (one split) or as
//    split partials for mla_decode_combine.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace mla {

constexpr int kRows = 32;           // query rows per workgroup
constexpr float kRefSlack = 64.0f;  // log2 headroom of the weights over the reference
constexpr int kMaxRestarts = 4;

template <int CACHE>
struct Tile {
  static constexpr int ELEM = CACHE == kFp8 ? 1 : 2;
  static constexpr int ROW_BYTES = kD * ELEM;
  static constexpr int PAGE_BYTES = kPage * ROW_BYTES;
  static constexpr int NBUF = CACHE == kFp8 ? 3 : 2;
  static constexpr int LOADS = PAGE_BYTES / 4096;  // 16-byte LDS-DMA loads per wave per page
  static constexpr int PSTRIDE = kPage * 2 + 16;   // bytes per P row in LDS
  static constexpr int KBATCH = 9;                 // BF16 K reads issued before their math
};

// LDS layout of a staged page: token t's 16-byte chunk c (of NCH per row) sits
// in chunk slot t * NCH + slot(t, c).  FP8 rows (36 chunks) XOR the two low
// chunk bits with (t / 4) % 4; BF16 rows (72 chunks) rotate by 3 * (t / 2).
// Both make the 16-token operand reads of QK^T and the 8-token transposed
// reads of PV hit distinct LDS banks.  The HBM -> LDS copy applies the inverse
// mapping when it picks each lane's source chunk.
template <int CACHE>
struct Swz {
  static constexpr int NCH = CACHE == kFp8 ? 36 : 72;
  __device__ static __forceinline__ int rot(int t) {  // BF16 rotation, in [0, NCH)
    const int r = 3 * (t >> 1);
    return r >= NCH ? r - NCH : r;  // t < 64 keeps r < 2 * NCH
  }
  __device__ static __forceinline__ int slot(int t, int c) {
    if constexpr (CACHE == kFp8) return c ^ ((t >> 2) & 3);
    else { const int v = c + rot(t); return v >= NCH ? v - NCH : v; }
  }
  __device__ static __forceinline__ int chunk_of_slot(int t, int s) {
    if constexpr (CACHE == kFp8) return s ^ ((t >> 2) & 3);
    else { const int v = s - rot(t); return v < 0 ? v + NCH : v; }
  }
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// HBM -> LDS copy without VGPRs: each lane moves 16 (or 4) bytes from its own
// global address to lds_base + lane * 16 (or 4).  Issued through inline asm so
// the compiler does not serialise later LDS reads on it; completion is awaited
// explicitly with wait_vmcnt() followed by a barrier.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(g), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(MLA_LDS const void*)p;
}

// Loads of values that stay constant for the whole kernel (lengths, the
// per-tensor scale) go through the constant address space so that uniform ones
// become scalar loads.
template <typename V>
__device__ __forceinline__ V load_const(const V* p, int64_t i) {
  return ((__attribute__((address_space(4))) const V*)p)[i];
}

template <int CACHE, int SCALE>
__global__ __launch_bounds__(256, 1) void decode_split_kernel(DecodeArgs a) {
  using T = Tile<CACHE>;
  using Z = Swz<CACHE>;
  __shared__ __attribute__((aligned(16))) uint8_t s_kv[T::NBUF][T::PAGE_BYTES];
  __shared__ __attribute__((aligned(16))) float s_scale[T::NBUF][kPage];
  __shared__ __attribute__((aligned(16))) uint8_t s_p[kRows * T::PSTRIDE];
  __shared__ float s_max[4][kRows];
  __shared__ float s_lsum[4][kRows];
  __shared__ float s_lnrm[4][kRows];
  __shared__ float s_m0[kRows];
  __shared__ int s_flag[4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, g = lane >> 4;
  // Workgroup -> (split, row group): workgroups are handed to the 8 XCDs round
  // robin, so the row groups of one split (which read the same pages) are
  // placed on the same XCD back to back and share its L2.
  const int b = blockIdx.y;
  const int xcd = blockIdx.x & 7;
  const int kx = blockIdx.x >> 3;
  const int rg = kx % a.n_rg;
  const int split = (kx / a.n_rg) * 8 + xcd;
  if (split >= a.max_splits) return;
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
          a.o_part[((int64_t)b * a.max_splits * a.R + r) * kDV + e % kDV] = 0.0f;
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
  const float tscale = SCALE == kScaleTensor ? load_const(a.kv_scale, 0) : 1.0f;
  const float coef = a.sm_log2 * tscale;

  // ---- query operands of this lane's rows rb*16 + m (rb = 0, 1), and the
  // causal limit of each: row i*H + h sees tokens t < L - n_q + i + 1
  bf16x8 qop[2][kD / 32];
  int lim[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = r0 + rb * 16 + m;
    lim[rb] = row < a.R ? L - a.n_q + row / a.H + 1 : 0;
    const uint16_t* qrow = a.q + ((int64_t)b * a.R + min(row, a.R - 1)) * kD;
#pragma unroll
    for (int kb = 0; kb < kD / 32; ++kb) {
      // the dims of this lane's 8 slots of k-block kb: k-blocks are paired so
      // that a lane's slots of k-blocks 2i and 2i+1 are 16 consecutive dims
      // (one 16-byte FP8 chunk of K); both cache types use this order
      const int d0 = 64 * (kb >> 1) + 16 * g + 8 * (kb & 1);
      u32x4 w = *reinterpret_cast<const u32x4*>(qrow + d0);
      if (row >= a.R) w = u32x4{0u, 0u, 0u, 0u};
      qop[rb][kb] = __builtin_bit_cast(bf16x8, w);
    }
  }

  constexpr int LPP = T::LOADS + (SCALE == kScaleToken ? 1 : 0);  // loads per page per wave
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
  // each lane's source offsets inside a page for its LOADS LDS chunk slots
  uint32_t goff[T::LOADS];
#pragma unroll
  for (int j = 0; j < T::LOADS; ++j) {
    const int slot = (wave * T::LOADS + j) * 64 + lane;
    const int t = slot / Z::NCH;
    goff[j] = t * T::ROW_BYTES + Z::chunk_of_slot(t, slot - t * Z::NCH) * 16;
  }
  auto issue = [&](int p, int buf) {
    const int rel = p - p_begin;
    if ((rel >> 6) != id_chunk) {
      id_chunk = rel >> 6;
      ids = load_ids(p_begin + (id_chunk << 6));
    }
    const int pg = __builtin_amdgcn_readlane(ids, rel & 63);
    const uint8_t* src = a.cache + (int64_t)pg * T::PAGE_BYTES;
    const uint32_t dst = lds_addr(&s_kv[buf][0]) + wave * T::LOADS * 1024;
#pragma unroll
    for (int j = 0; j < T::LOADS; ++j) lds_dma16(src + goff[j], dst + j * 1024);
    if (SCALE == kScaleToken) lds_dma4(a.kv_scale + (int64_t)pg * kPage + lane, lds_addr(&s_scale[buf][0]));
  };
  auto prologue = [&]() {
#pragma unroll
    for (int k = 0; k < T::NBUF - 1; ++k)
      if (p_begin + k < p_end) issue(p_begin + k, k);
  };
  prologue();

  float m0[2] = {-INFINITY, -INFINITY};  // log2-domain reference of this lane's rows
  float lsum[2] = {0.0f, 0.0f};          // this lane's share of the softmax sums (fp32 P)
  float lnrm[2] = {0.0f, 0.0f};          // the same over the bf16-rounded P that PV uses
  f32x4 O[2][8];                          // rows rb*16 + 4g + i, dims 128*wave + 16db + m
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) O[i][j] = mfma_zero();
  bool have_ref = false;
  int restarts = 0;

  for (int p = p_begin, it = 0; p < p_end; ++p, ++it) {
    const int buf = it % T::NBUF;
    if (p + T::NBUF - 2 < p_end)
      wait_vmcnt<(T::NBUF - 2) * LPP>();
    else
      wait_vmcnt<0>();
    __syncthreads();  // page p is in LDS; every wave is done with page p-1
    if (p + T::NBUF - 1 < p_end) issue(p + T::NBUF - 1, (it + T::NBUF - 1) % T::NBUF);
    uint8_t* kv = s_kv[buf];
    const int tbase = p * kPage;
    const int nvalid = min(kPage, L - tbase);
    if (nvalid < kPage) {
      // rows past the end of the request may hold anything (even NaN codes):
      // zero them so that their zero weights give zero products in PV
      u32x4* junk = reinterpret_cast<u32x4*>(kv + nvalid * T::ROW_BYTES);
      for (int e = threadIdx.x; e < (kPage - nvalid) * (T::ROW_BYTES / 16); e += 256)
        junk[e] = u32x4{0u, 0u, 0u, 0u};
    }

    // ---- S^T[token][row] = K Q^T for tokens 16*wave .. +16 of the page
    f32x4 S[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    {
      constexpr int KB = kD / 32;
      const int tok = wave * 16 + m;
      if constexpr (CACHE == kFp8) {
        // chunk 4i + g of token tok sits at slot 4i + (g ^ f): a fixed per-lane
        // base plus 64 i; each 16-byte read feeds k-blocks 2i and 2i+1
        const uint8_t* kbase = kv + (tok * Z::NCH + Z::slot(tok, g)) * 16;
        u32x4 kraw[KB / 2];
#pragma unroll
        for (int i = 0; i < KB / 2; ++i) kraw[i] = *reinterpret_cast<const u32x4*>(kbase + 64 * i);
        __builtin_amdgcn_sched_barrier(0);  // reads ahead of the math
        // convert three k-blocks into distinct registers, then issue their six
        // MFMAs: consecutive MFMAs never wait on a register still being read
#pragma unroll
        for (int k0 = 0; k0 < KB; k0 += 3) {
          bf16x8 kop[3];
#pragma unroll
          for (int k = 0; k < 3; ++k) {
            const u32x4 w = kraw[(k0 + k) >> 1];
            kop[k] = e4m3x8_to_bf16x8(((k0 + k) & 1) ? u32x2{w[2], w[3]} : u32x2{w[0], w[1]});
          }
#pragma unroll
          for (int k = 0; k < 3; ++k) mfma_qk2(S[0], S[1], kop[k], qop[0][k0 + k], qop[1][k0 + k]);
        }
      } else {
#pragma unroll
        for (int k0 = 0; k0 < KB; k0 += T::KBATCH) {
          u32x4 kraw[T::KBATCH];
#pragma unroll
          for (int k = 0; k < T::KBATCH; ++k) {
            const int kb = k0 + k;
            const int c = 8 * (kb >> 1) + 2 * g + (kb & 1);  // dims 64(kb/2) + 16g + 8(kb&1) .. +8
            kraw[k] = *reinterpret_cast<const u32x4*>(kv + (tok * Z::NCH + Z::slot(tok, c)) * 16);
          }
          __builtin_amdgcn_sched_barrier(0);  // reads ahead of the math
#pragma unroll
          for (int k = 0; k < T::KBATCH; ++k)
            mfma_qk2(S[0], S[1], __builtin_bit_cast(bf16x8, kraw[k]), qop[0][k0 + k], qop[1][k0 + k]);
        }
      }
    }

    mfma_result_fence_v(S[0], S[1]);

    // ---- scores in log2 units (lane holds tokens 16w + 4g + i of rows rb*16 + m)
    float x[2][4];
    float pmax[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = wave * 16 + 4 * g + i;
      const float c = SCALE == kScaleToken ? coef * s_scale[buf][tl] : coef;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float v = S[rb][i] * c;
        if (tbase + tl >= lim[rb]) v = -INFINITY;
        x[rb][i] = v;
        pmax[rb] = fmaxf(pmax[rb], v);
      }
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      pmax[rb] = group4_max(pmax[rb]);
      if (g == 0) s_max[wave][rb * 16 + m] = pmax[rb];
    }
    if (!have_ref) {
      // first page of the split: the reference of each row is its page max
      __syncthreads();
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int row = rb * 16 + m;
        m0[rb] = fmaxf(fmaxf(s_max[0][row], s_max[1][row]), fmaxf(s_max[2][row], s_max[3][row]));
      }
      have_ref = true;
    }
    bool over = false;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      over |= pmax[rb] > m0[rb] + kRefSlack;
      const float mr = m0[rb] == -INFINITY ? 0.0f : m0[rb];
      uint32_t pb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = x[rb][i];
        const float e = __builtin_amdgcn_exp2f(v - mr);
        if (SCALE == kScaleToken) {
          const float w = v == -INFINITY ? 0.0f : e * s_scale[buf][wave * 16 + 4 * g + i];
          pb[i] = float_to_bf16(w);
          lsum[rb] += e;
        } else {
          pb[i] = float_to_bf16(e);
          lsum[rb] += e;
          lnrm[rb] += float_of(pb[i] << 16);
        }
      }
      u32x2 packed = {pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16)};
      *reinterpret_cast<u32x2*>(s_p + (rb * 16 + m) * T::PSTRIDE + (wave * 16 + 4 * g) * 2) = packed;
    }
    const bool any_over = __any(over);
    if (lane == 0) s_flag[wave] = any_over;
    __syncthreads();  // P of the page is in LDS

    if ((s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3]) && restarts < kMaxRestarts) {
      // A weight would exceed 2^64: restart the split with the larger reference.
      ++restarts;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int row = rb * 16 + m;
        const float pm = fmaxf(fmaxf(s_max[0][row], s_max[1][row]), fmaxf(s_max[2][row], s_max[3][row]));
        m0[rb] = fmaxf(m0[rb], pm);
        lsum[rb] = 0.0f;
        lnrm[rb] = 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) O[i][j] = mfma_zero();
      wait_vmcnt<0>();
      __syncthreads();  // every DMA landed and every wave is past its reads
      id_chunk = 0;
      ids = load_ids(p_begin);
      prologue();
      p = p_begin - 1;
      it = -1;
      continue;
    }

    // ---- O[row][dim] += P V over this wave's 128 dims
    {
      const int dim0 = wave * 128;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        // P (rows x 32 tokens) and V operands of this half of the page are read
        // first, then converted and fed to the MFMAs; the lane's 8 contraction
        // slots are tokens tok0 .. tok0+7 in both
        const int tok0 = kt * 32 + g * 8;
        bf16x8 pop[2];
        u32x2 vraw[8][CACHE == kFp8 ? 1 : 2];
#pragma unroll
        for (int rbp = 0; rbp < 2; ++rbp)
          pop[rbp] = *reinterpret_cast<const bf16x8*>(s_p + (rbp * 16 + m) * T::PSTRIDE + tok0 * 2);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const int dcol = dim0 + db * 16;
          if constexpr (CACHE == kFp8) {
            // lane 2j+h of the group addresses token tok0+j, bytes dcol+8h .. +8
            const int t = tok0 + (m >> 1);
            vraw[db][0] = lds_read_tr8(kv + (t * Z::NCH + Z::slot(t, dcol >> 4)) * 16 + 8 * (m & 1));
          } else {
            // lane 4j+q of the group addresses token tok0+j (+4), elements dcol+4q .. +4
            const int c = (dcol >> 3) + ((m & 3) >> 1);
            const int t0 = tok0 + (m >> 2), t1 = t0 + 4;
            vraw[db][0] = lds_read_tr16(kv + (t0 * Z::NCH + Z::slot(t0, c)) * 16 + 8 * (m & 1));
            vraw[db][CACHE == kFp8 ? 0 : 1] = lds_read_tr16(kv + (t1 * Z::NCH + Z::slot(t1, c)) * 16 + 8 * (m & 1));
          }
        }
        __builtin_amdgcn_sched_barrier(0);  // reads ahead of the math
        // convert two V blocks into distinct registers, then issue their four MFMAs
#pragma unroll
        for (int d0 = 0; d0 < 8; d0 += 2) {
          bf16x8 vop[2];
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            if constexpr (CACHE == kFp8)
              vop[d] = e4m3x8_to_bf16x8(vraw[d0 + d][0]);
            else
              vop[d] = __builtin_bit_cast(bf16x8, u32x4{vraw[d0 + d][0].x, vraw[d0 + d][0].y,
                                                        vraw[d0 + d][CACHE == kFp8 ? 0 : 1].x,
                                                        vraw[d0 + d][CACHE == kFp8 ? 0 : 1].y});
          }
#pragma unroll
          for (int d = 0; d < 2; ++d)
#pragma unroll
            for (int rbp = 0; rbp < 2; ++rbp)
              O[rbp][d0 + d] = mfma_16x16x32_bf16(pop[rbp], vop[d], O[rbp][d0 + d]);
        }
      }
    }
  }

  // ---- epilogue: softmax sums across lanes and token groups, then O / l
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float ls = group4_sum(lsum[rb]);
    const float ln = SCALE == kScaleToken ? ls : group4_sum(lnrm[rb]);
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
      const float inv = ln > 0.0f ? tscale / ln : 0.0f;
      const float mr = s_m0[row] == -INFINITY ? 0.0f : s_m0[row];
      const float lse_nat = lt > 0.0f ? (mr + __log2f(lt)) * kLn2 : -INFINITY;
      if (a.max_splits == 1) {
        uint16_t* dst = a.out + ((int64_t)b * a.R + r) * kDV + dim0 + m;
#pragma unroll
        for (int db = 0; db < 8; ++db) dst[db * 16] = float_to_bf16(O[rbp][db][i] * inv);
        if (wave == 0 && m == 0) a.lse[(int64_t)b * a.R + r] = lse_nat;
      } else {
        const int64_t pr = ((int64_t)b * a.max_splits + split) * a.R + r;
        float* dst = a.o_part + pr * kDV + dim0 + m;
#pragma unroll
        for (int db = 0; db < 8; ++db) dst[db * 16] = O[rbp][db][i] * inv;
        if (wave == 0 && m == 0) a.lse_part[pr] = lse_nat;
      }
    }
}

int decode_rows_per_group(int B, int R) {
  (void)B;
  (void)R;
  return kRows;
}

template <int CACHE>
static hipError_t launch_cache(const DecodeArgs& a, int scale_mode, hipStream_t stream) {
  const dim3 grid(((a.max_splits + 7) / 8) * 8 * a.n_rg, a.B), block(256);
  switch (scale_mode) {
    case kScaleTensor:
      hipLaunchKernelGGL((decode_split_kernel<CACHE, kScaleTensor>), grid, block, 0, stream, a);
      break;
    case kScaleToken:
      hipLaunchKernelGGL((decode_split_kernel<CACHE, kScaleToken>), grid, block, 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((decode_split_kernel<CACHE, kScaleNone>), grid, block, 0, stream, a);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a0, int cache_kind, int scale_mode, hipStream_t stream) {
  DecodeArgs a = a0;
  a.n_rg = (a.R + kRows - 1) / kRows;
  if (cache_kind == kFp8) return launch_cache<kFp8>(a, scale_mode, stream);
  return launch_cache<kBf16>(a, kScaleNone, stream);
}

}  // namespace mla
