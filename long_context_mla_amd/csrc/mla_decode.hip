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
// gfx950 design (one 256-thread workgroup per (request, split, row group), one
// workgroup per CU):
//  * Pages stream HBM -> LDS with global_load_lds (16 B per lane, no VGPRs),
//    NBUF-deep so later pages are in flight while the current one is used.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: the four waves split the 64
//    tokens (and, with 64 rows, the rows) of the page; each wave keeps its
//    32 query rows as bf16 MFMA operands in registers for the whole split.
//    FP8 codes become bf16 in registers (exact), scales are applied to the
//    fp32 scores.
//  * Online softmax in the log2 domain with a lazily moved reference max
//    (rescale only when the max grows by more than 2^8), row maxima exchanged
//    through LDS; P goes to LDS as bf16 (per-token scales folded in).
//  * O += P V on MFMA: the four waves split the 512 output dims; V is the first
//    512 columns of the same staged page.
//  * Epilogue: O / l and the natural-log LSE, either final (one split) or as
//    split partials for mla_decode_combine.
#include "device_common.h"
#include "launch.h"

namespace mla {

constexpr float kTau = 8.0f;  // log2 slack before the softmax reference max moves

template <int ROWS, int CACHE>
struct Tile {
  static constexpr int TW = 128 / ROWS;       // token groups of the QK^T phase
  static constexpr int TPW = kPage / TW;      // tokens per QK^T wave
  static constexpr int TB = TPW / 16;         // 16-token blocks per QK^T wave
  static constexpr int RBP = ROWS / 16;       // 16-row blocks per PV wave
  static constexpr int ELEM = CACHE == kFp8 ? 1 : 2;
  static constexpr int ROW_BYTES = kD * ELEM;
  static constexpr int PAGE_BYTES = kPage * ROW_BYTES;
  static constexpr int NBUF = CACHE == kFp8 ? 3 : 2;
  static constexpr int LOADS = PAGE_BYTES / 4096;  // 16-byte LDS-direct loads per wave per page
  static constexpr int PSTRIDE = kPage * 2 + 16;   // bytes per P row in LDS
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// HBM -> LDS copy without VGPRs: each lane moves `bytes` (16 or 4) from its own
// global address to lds_base + lane * bytes.  Issued through inline asm so the
// compiler does not serialise later LDS reads on it; completion is awaited
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

// Loads of values that stay constant for the whole kernel (page maps, lengths,
// the per-tensor scale) go through the constant address space so that uniform
// ones become scalar loads.
template <typename V>
__device__ __forceinline__ V load_const(const V* p, int64_t i) {
  return ((__attribute__((address_space(4))) const V*)p)[i];
}

template <int ROWS, int CACHE, int SCALE>
__global__ __launch_bounds__(256, 1) void decode_split_kernel(DecodeArgs a) {
  using T = Tile<ROWS, CACHE>;
  __shared__ __attribute__((aligned(16))) uint8_t s_kv[T::NBUF][T::PAGE_BYTES];
  __shared__ __attribute__((aligned(16))) float s_scale[T::NBUF][kPage];
  __shared__ __attribute__((aligned(16))) uint8_t s_p[ROWS * T::PSTRIDE];
  __shared__ float s_max[T::TW][ROWS];
  __shared__ float s_lsum[T::TW][ROWS];
  __shared__ float s_lnrm[T::TW][ROWS];
  __shared__ __attribute__((aligned(16))) float s_alpha[ROWS];
  __shared__ float s_mref[ROWS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.y;
  const int split = blockIdx.x / a.n_rg;
  const int rg = blockIdx.x - split * a.n_rg;
  const int L = min(max(load_const(a.seq_lens, b), 0), a.max_blocks * kPage);
  const int n_pages = (L + kPage - 1) / kPage;
  const int r0 = rg * ROWS;
  const int p_begin = split * a.pps;

  if (p_begin >= n_pages) {
    // Nothing to read.  Only an empty request's first split reports it; the
    // combine never reads splits past a request's last page.
    if (n_pages == 0 && split == 0) {
      for (int e = threadIdx.x; e < ROWS * kDV; e += 256) {
        const int r = r0 + e / kDV;
        if (r >= a.R) break;
        if (a.max_splits == 1)
          a.out[((int64_t)b * a.R + r) * kDV + e % kDV] = 0;
        else
          a.o_part[((int64_t)b * a.max_splits * a.R + r) * kDV + e % kDV] = 0.0f;
      }
      for (int r = r0 + threadIdx.x; r < min(r0 + ROWS, a.R); r += 256) {
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

  // ---- QK^T role: token group tw, row half rw (32 rows)
  const int tw = wave % T::TW;
  const int rw = wave / T::TW;
  bf16x8 qop[2][kD / 32];
  int lim[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = r0 + rw * 32 + rb * 16 + (lane & 15);
    lim[rb] = row < a.R ? L - a.n_q + row / a.H + 1 : 0;
    const u32x4* src = reinterpret_cast<const u32x4*>(
        a.q + ((int64_t)b * a.R + min(row, a.R - 1)) * kD + (lane >> 4) * 8);
#pragma unroll
    for (int kb = 0; kb < kD / 32; ++kb) {
      u32x4 w = src[kb * 4];
      if (row >= a.R) w = u32x4{0u, 0u, 0u, 0u};
      qop[rb][kb] = __builtin_bit_cast(bf16x8, w);
    }
  }

  constexpr int LPP = T::LOADS + (SCALE == kScaleToken ? 1 : 0);  // loads per page per wave
  auto issue = [&](int p, int buf) {
    int pg = load_const(a.block_table, (int64_t)b * a.max_blocks + p);
    pg = min(max(pg, 0), a.num_pages - 1);
    const uint8_t* src = a.cache + (int64_t)pg * T::PAGE_BYTES + lane * 16;
    const uint32_t dst = lds_addr(&s_kv[buf][0]) + wave * T::LOADS * 1024;
#pragma unroll
    for (int j = 0; j < T::LOADS; ++j) lds_dma16(src + (wave * T::LOADS + j) * 1024, dst + j * 1024);
    if (SCALE == kScaleToken) lds_dma4(a.kv_scale + (int64_t)pg * kPage + lane, lds_addr(&s_scale[buf][0]));
  };

#pragma unroll
  for (int k = 0; k < T::NBUF - 1; ++k)
    if (p_begin + k < p_end) issue(p_begin + k, k);

  float mref[2] = {-INFINITY, -INFINITY};  // log2-domain reference max of this lane's two rows
  float lsum[2] = {0.0f, 0.0f};            // this lane's share of the softmax sums (fp32 P)
  float lnrm[2] = {0.0f, 0.0f};            // the same over the bf16-rounded P that PV uses
  f32x4 O[T::RBP][8];
#pragma unroll
  for (int i = 0; i < T::RBP; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) O[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int p = p_begin; p < p_end; ++p) {
    const int it = p - p_begin;
    const int buf = it % T::NBUF;
    if (p + T::NBUF - 2 < p_end)
      wait_vmcnt<(T::NBUF - 2) * LPP>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if (p + T::NBUF - 1 < p_end) issue(p + T::NBUF - 1, (it + T::NBUF - 1) % T::NBUF);
    const uint8_t* kv = s_kv[buf];
    const int tbase = p * kPage;

    // ---- S^T[token][row] = K Q^T
    f32x4 S[T::TB][2];
#pragma unroll
    for (int tb = 0; tb < T::TB; ++tb)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) S[tb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < kD / 32; ++kb) {
#pragma unroll
      for (int tb = 0; tb < T::TB; ++tb) {
        const int tok = tw * T::TPW + tb * 16 + (lane & 15);
        const uint8_t* src = kv + tok * T::ROW_BYTES + (kb * 32 + (lane >> 4) * 8) * T::ELEM;
        bf16x8 kop;
        if constexpr (CACHE == kFp8)
          kop = e4m3x8_to_bf16x8(*reinterpret_cast<const u32x2*>(src));
        else
          kop = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) S[tb][rb] = mfma_16x16x32_bf16(kop, qop[rb][kb], S[tb][rb]);
      }
    }

    // ---- scores in log2 units, masks, partial row maxima
    float x[T::TB][2][4];
    float pmax[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int tb = 0; tb < T::TB; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tl = tw * T::TPW + tb * 16 + 4 * (lane >> 4) + i;
        const float c = SCALE == kScaleToken ? coef * s_scale[buf][tl] : coef;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          float v = S[tb][rb][i] * c;
          if (tbase + tl >= lim[rb]) v = -INFINITY;
          x[tb][rb][i] = v;
          pmax[rb] = fmaxf(pmax[rb], v);
        }
      }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      pmax[rb] = group4_max(pmax[rb]);
      if ((lane >> 4) == 0) s_max[tw][rw * 32 + rb * 16 + lane] = pmax[rb];
    }
    __syncthreads();

    // ---- move the reference max if needed, then P = 2^(x - ref) to LDS
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = rw * 32 + rb * 16 + (lane & 15);
      float pm = s_max[0][row];
#pragma unroll
      for (int t = 1; t < T::TW; ++t) pm = fmaxf(pm, s_max[t][row]);
      const float mnew = pm > mref[rb] + kTau ? pm : mref[rb];
      const float alpha = mnew == mref[rb] ? 1.0f : __builtin_amdgcn_exp2f(mref[rb] - mnew);
      lsum[rb] *= alpha;
      lnrm[rb] *= alpha;
      mref[rb] = mnew;
      if (tw == 0 && (lane >> 4) == 0) s_alpha[row] = alpha;
    }
#pragma unroll
    for (int tb = 0; tb < T::TB; ++tb)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float m0 = mref[rb] == -INFINITY ? 0.0f : mref[rb];
        uint32_t pb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = x[tb][rb][i];
          const float e = __builtin_amdgcn_exp2f(v - m0);
          if (SCALE == kScaleToken) {
            const int tl = tw * T::TPW + tb * 16 + 4 * (lane >> 4) + i;
            const float w = v == -INFINITY ? 0.0f : e * s_scale[buf][tl];
            pb[i] = float_to_bf16(w);
            lsum[rb] += e;
          } else {
            pb[i] = float_to_bf16(e);
            lsum[rb] += e;
            lnrm[rb] += float_of(pb[i] << 16);
          }
        }
        const int row = rw * 32 + rb * 16 + (lane & 15);
        const int tok0 = tw * T::TPW + tb * 16 + 4 * (lane >> 4);
        u32x2 packed = {pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16)};
        *reinterpret_cast<u32x2*>(s_p + row * T::PSTRIDE + tok0 * 2) = packed;
      }
    __syncthreads();

    // ---- O[row][dim] += P V over this wave's 128 dims
    {
      const int dim0 = wave * 128;
      bool rescale = false;
      f32x4 al[T::RBP];
#pragma unroll
      for (int rbp = 0; rbp < T::RBP; ++rbp) {
        al[rbp] = *reinterpret_cast<const f32x4*>(&s_alpha[rbp * 16 + 4 * (lane >> 4)]);
        rescale |= (al[rbp][0] != 1.0f) | (al[rbp][1] != 1.0f) | (al[rbp][2] != 1.0f) | (al[rbp][3] != 1.0f);
      }
      if (__any(rescale)) {
#pragma unroll
        for (int rbp = 0; rbp < T::RBP; ++rbp)
#pragma unroll
          for (int db = 0; db < 8; ++db) O[rbp][db] *= al[rbp];
      }
      const int nvalid = min(kPage, L - tbase);  // tokens past the end may hold anything
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        bf16x8 pop[T::RBP];
#pragma unroll
        for (int rbp = 0; rbp < T::RBP; ++rbp)
          pop[rbp] = *reinterpret_cast<const bf16x8*>(s_p + (rbp * 16 + (lane & 15)) * T::PSTRIDE +
                                                       (kt * 32 + (lane >> 4) * 8) * 2);
        const int tok0 = kt * 32 + (lane >> 4) * 8;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const int dim = dim0 + db * 16 + (lane & 15);
          bf16x8 vop;
          if constexpr (CACHE == kFp8) {
            uint32_t w0 = 0, w1 = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              uint32_t c0 = kv[(tok0 + j) * T::ROW_BYTES + dim];
              uint32_t c1 = kv[(tok0 + 4 + j) * T::ROW_BYTES + dim];
              if (tok0 + j >= nvalid) c0 = 0;
              if (tok0 + 4 + j >= nvalid) c1 = 0;
              w0 |= c0 << (8 * j);
              w1 |= c1 << (8 * j);
            }
            vop = e4m3x8_to_bf16x8(u32x2{w0, w1});
          } else {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint16_t* v16 = reinterpret_cast<const uint16_t*>(kv);
              uint32_t c0 = v16[(tok0 + 2 * j) * kD + dim];
              uint32_t c1 = v16[(tok0 + 2 * j + 1) * kD + dim];
              if (tok0 + 2 * j >= nvalid) c0 = 0;
              if (tok0 + 2 * j + 1 >= nvalid) c1 = 0;
              w[j] = c0 | (c1 << 16);
            }
            vop = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
          }
#pragma unroll
          for (int rbp = 0; rbp < T::RBP; ++rbp) O[rbp][db] = mfma_16x16x32_bf16(pop[rbp], vop, O[rbp][db]);
        }
      }
    }
  }

  // ---- epilogue: softmax sums across lanes and token groups, then O / l
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float ls = group4_sum(lsum[rb]);
    const float ln = SCALE == kScaleToken ? ls : group4_sum(lnrm[rb]);
    const int row = rw * 32 + rb * 16 + (lane & 15);
    if ((lane >> 4) == 0) {
      s_lsum[tw][row] = ls;
      s_lnrm[tw][row] = ln;
      if (tw == 0) s_mref[row] = mref[rb];
    }
  }
  __syncthreads();
  const int dim0 = wave * 128;
#pragma unroll
  for (int rbp = 0; rbp < T::RBP; ++rbp)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rbp * 16 + 4 * (lane >> 4) + i;
      const int r = r0 + row;
      if (r >= a.R) continue;
      float lt = 0.0f, ln = 0.0f;
#pragma unroll
      for (int t = 0; t < T::TW; ++t) {
        lt += s_lsum[t][row];
        ln += s_lnrm[t][row];
      }
      // the output is a weighted mean with the bf16 weights PV used; the LSE
      // uses the fp32 weights
      const float inv = ln > 0.0f ? tscale / ln : 0.0f;
      const float lse_nat = lt > 0.0f ? (s_mref[row] + __log2f(lt)) * kLn2 : -INFINITY;
      if (a.max_splits == 1) {
        uint16_t* dst = a.out + ((int64_t)b * a.R + r) * kDV + dim0 + (lane & 15);
#pragma unroll
        for (int db = 0; db < 8; ++db) dst[db * 16] = float_to_bf16(O[rbp][db][i] * inv);
        if (wave == 0 && (lane & 15) == 0) a.lse[(int64_t)b * a.R + r] = lse_nat;
      } else {
        const int64_t pr = ((int64_t)b * a.max_splits + split) * a.R + r;
        float* dst = a.o_part + pr * kDV + dim0 + (lane & 15);
#pragma unroll
        for (int db = 0; db < 8; ++db) dst[db * 16] = O[rbp][db][i] * inv;
        if (wave == 0 && (lane & 15) == 0) a.lse_part[pr] = lse_nat;
      }
    }
}

int decode_rows_per_group(int B, int R) {
  if (R <= 32) return 32;
  const int64_t groups64 = (R + 63) / 64;
  return (int64_t)B * groups64 >= 16 ? 64 : 32;
}

template <int ROWS, int CACHE>
static hipError_t launch_rows(const DecodeArgs& a, int scale_mode, hipStream_t stream) {
  const dim3 grid(a.max_splits * a.n_rg, a.B), block(256);
  switch (scale_mode) {
    case kScaleTensor:
      hipLaunchKernelGGL((decode_split_kernel<ROWS, CACHE, kScaleTensor>), grid, block, 0, stream, a);
      break;
    case kScaleToken:
      hipLaunchKernelGGL((decode_split_kernel<ROWS, CACHE, kScaleToken>), grid, block, 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((decode_split_kernel<ROWS, CACHE, kScaleNone>), grid, block, 0, stream, a);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a0, int cache_kind, int scale_mode, hipStream_t stream) {
  DecodeArgs a = a0;
  const int rows = decode_rows_per_group(a.B, a.R);
  a.n_rg = (a.R + rows - 1) / rows;
  if (cache_kind == kFp8) {
    return rows == 64 ? launch_rows<64, kFp8>(a, scale_mode, stream)
                      : launch_rows<32, kFp8>(a, scale_mode, stream);
  }
  return rows == 64 ? launch_rows<64, kBf16>(a, kScaleNone, stream)
                    : launch_rows<32, kBf16>(a, kScaleNone, stream);
}

}  // namespace mla
