/*
 * Measured-peak microbenchmarks for MI355X (gfx950) — C ABI of libmla_peaks.so.
 *
 * These are measurement tools, not part of the decode path: they give the
 * bandwidth, latency and matrix-core rate the hardware actually sustains, so
 * that a kernel's fraction of its roofline can be stated against measured
 * peaks as well as the vendor's (relative performance as a fraction of the
 * hardware's "speed of light": "How to serve trillions of tokens for
 * trillion-parameter coding agents", opening section).
 *
 * All pointers are device pointers; work is enqueued on `stream` (a
 * hipStream_t, NULL = default) and nothing is synchronised.  Return value:
 * 0 ok, 1 null pointer, 2 bad size, 3 unsupported parameter, 4 launch error.
 */
#ifndef MLA_PEAKS_H
#define MLA_PEAKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` (a multiple of 16) from `src` with 16-byte
 * non-temporal loads, `grid` workgroups of 256 threads; sink: uint32
 * [grid * 256] receives a checksum per thread. */
int mla_peak_stream_read(const void* src, int64_t bytes, uint32_t* sink, int grid, void* stream);

/* 36,864-byte pages src[page_ids[i]] (i < n; ids clamped to [0, num_pages))
 * copied HBM -> LDS by LDS-DMA, ceil(n / pages_per_wg) workgroups of 4 waves
 * (one per compute unit: 144 KB of LDS each), each wave keeping `depth`
 * (1..4) pages' worth of its 9 KB quarter in flight.  sink: uint32
 * [ceil(n / pages_per_wg) * 256]. */
int mla_peak_stream_pages(const void* src, int num_pages, const int32_t* page_ids, int n, int pages_per_wg,
                          int depth, uint32_t* sink, void* stream);

/* One lane follows `steps` dependent loads j = min(chain[j], n - 1) from
 * j = 0 over chain: uint32 [n]; out[0] = the final index, ticks[0] = elapsed
 * 100 MHz s_memrealtime ticks. */
int mla_peak_latency(const uint32_t* chain, int64_t n, int steps, uint32_t* out, uint64_t* ticks, void* stream);

/* `grid` workgroups of 4 * waves_per_simd (1 or 2) waves, each wave running
 * `iters` rounds of eight independent v_mfma_f32_16x16x32_bf16 chains
 * (16 x 16 x 32 x 2 flops each).  sink: float [grid * 256 * waves_per_simd];
 * clocks: uint64 [2 * grid], per workgroup the s_memtime (shader clock) and
 * s_memrealtime (100 MHz) ticks over its loop. */
int mla_peak_mfma(int grid, int waves_per_simd, int iters, float* sink, uint64_t* clocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PEAKS_H */
