/*
 * Paged MLA decode attention over an FP8 (e4m3) or BF16 latent KV cache — C ABI.
 *
 * The operation: decode attention for a few new query tokens per request over
 * a long cache of one shared latent row per token.  The row has 576 elements
 * (512 latent + 64 rope) and serves as both key and value: models like Kimi
 * have no distinct keys and values, and the row is 576 elements per token per
 * layer ("How to serve trillions of tokens for trillion-parameter coding
 * agents", sections "First, understand the workload" and "Tensor parallel was
 * the best parallelism strategy for maximum interactivity"); MLA keeps one
 * latent head shared by all query heads ("vLLM x AgentX: Optimizing for
 * Real-World Agentic Serving", section "Model-specific parallelism / Kimi K3").
 * The cache is stored as FP8 e4m3, half the bytes of BF16, and converted as
 * it is read ("Smaller, faster, safer: running Kimi and GLM at scale", section
 * "Quantizing the KV cache").  Requests reach physical cache pages through a
 * per-request page map ("Smaller, faster, safer", section "Protecting a shared
 * KV cache").  Split-KV partial outputs and their log-sum-exp are merged with
 * the online-softmax identity ("vLLM x AgentX", section "Model-specific
 * parallelism / Kimi K3").
 *
 * Definitions used by every call:
 *   D = 576 (row width), DV = 512 (value width = first 512 elements of the row),
 *   P = 64 tokens per physical page.
 *   Token t of request b lives in slot t % 64 of physical page
 *   block_table[b * max_blocks + t / 64].
 *   seq_lens[b] = L_b counts the tokens request b can see, including rows the
 *   step has just appended; its n_q queries are positions L_b-n_q .. L_b-1 and
 *   query i sees tokens t < L_b - n_q + i + 1 (causal among the new tokens).
 *   Query / output row r = i * H + h.
 *   E4M3 is the OCP E4M3FN encoding (bias 7, no infinities, max 448).
 *   Alignment: q, kv_cache, kv_new, o_partial and out must be 16-byte aligned
 *   (the kernels move 16-byte pieces); the other arrays need the alignment of
 *   their element type.
 *
 * Ownership and threading: the caller owns every buffer; the library never
 * allocates, frees or synchronises (the one buffer it owns, the static
 * scratch of mla_decode_paged_append_noalloc, is part of its code object).  All pointers except the scalar-out
 * arguments of mla_decode_plan are device pointers.  Work is enqueued on
 * `stream` (a hipStream_t; NULL = the default stream) and the calls return
 * before it runs.  The calls are re-entrant; calls that write the same buffers
 * must be ordered by the caller.
 *
 * Errors: host-detectable argument errors return a non-zero mla_status_t
 * before anything is launched.  A failed launch returns MLA_ERR_HIP.  No
 * exception or abort crosses the ABI.  Device-side contents (page ids,
 * lengths) are not checked on the host: for reads, page ids outside
 * [0, num_pages) are clamped into range and lengths are clamped to
 * [0, max_blocks * 64], so a bad table gives wrong numbers but never an
 * out-of-bounds access; a new row whose page id is outside [0, num_pages) is
 * not written anywhere (a clamped id would name another request's page).
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_HEAD_DIM 576
#define MLA_VALUE_DIM 512
#define MLA_PAGE_SIZE 64
#define MLA_MAX_HEADS 128
#define MLA_MAX_QUERIES 2048

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL_PTR = 1,
  MLA_ERR_BAD_SHAPE = 2,
  MLA_ERR_UNSUPPORTED = 3,
  MLA_ERR_HIP = 4,
  MLA_ERR_SCRATCH_LIMIT = 5
} mla_status_t;

/* Split-partial rows (B * max_splits * n_q * H) the fixed scratch of
 * mla_decode_paged_append_noalloc holds: 32 MiB of bf16 partials plus
 * 128 KiB of fp32 LSEs per GPU. */
#define MLA_NOALLOC_MAX_PARTIAL_ROWS 32768

/* Per-request result bits of kv_check_pages (0 = the request may read the cache). */
typedef enum {
  MLA_PAGE_OK = 0,
  MLA_PAGE_BAD_LEN = 1,      /* seq_lens[b] < 0 or > max_blocks * 64 */
  MLA_PAGE_OUT_OF_RANGE = 2, /* a page-map entry it reads is outside [0, num_pages) */
  MLA_PAGE_WRONG_PAGE = 4,   /* a page-map entry it reads differs from the recorded page */
  MLA_PAGE_STALE_TAG = 8     /* a page it reads carries another tag than the recorded one */
} mla_page_status_t;

typedef enum { MLA_CACHE_BF16 = 0, MLA_CACHE_FP8_E4M3 = 1 } mla_cache_dtype_t;

typedef enum {
  MLA_SCALE_NONE = 0,       /* BF16 cache: no scale */
  MLA_SCALE_PER_TENSOR = 1, /* one fp32 scale for the whole cache: kv_scale[0] */
  MLA_SCALE_PER_TOKEN = 2   /* one fp32 scale per cached token: kv_scale[page * 64 + slot] */
} mla_scale_mode_t;

/*
 * kv_append_fp8 — quantise new latent rows to E4M3 and write them into the
 * paged cache ("Smaller, faster, safer", section "Quantizing the KV cache":
 * the cache is stored in FP8 e4m3 instead of BF16).
 *
 *   kv_new      bf16 [B, n_new, 576], row-major.  Inputs must be finite.
 *   kv_cache    e4m3 codes [num_pages, 64, 576] (576 bytes per token row).
 *   kv_scale    PER_TOKEN: fp32 [num_pages, 64], written for each new row;
 *               PER_TENSOR: fp32 [1], read.
 *   block_table int32 [B, max_blocks]; seq_lens int32 [B] (after the append).
 *
 * Row j of request b goes to position p = seq_lens[b] - n_new + j.
 * PER_TOKEN: amax = max_d |x_d|; scale = fp32(amax / 448) (1.0 when amax = 0);
 * code_d = E4M3(fp32(x_d / scale)).  PER_TENSOR: code_d = E4M3(fp32(x_d / kv_scale[0])).
 * Divisions are correctly rounded fp32; E4M3() rounds to nearest, ties to the
 * even code, saturating to +-448.  Positions p < 0 or p >= max_blocks * 64,
 * and rows whose page id is outside [0, num_pages), are skipped.
 * B = 0 or n_new = 0 is a no-op.
 */
int kv_append_fp8(const void* kv_new, void* kv_cache, float* kv_scale, int scale_mode,
                  const int32_t* block_table, const int32_t* seq_lens, int B, int n_new,
                  int max_blocks, int num_pages, void* stream);

/*
 * mla_decode_paged — split-KV decode attention over the paged latent cache.
 *
 * MLA keeps one latent head that every query head attends to; when the cache
 * of a request is cut by sequence, each part computes a partial attention
 * output with its log-sum-exp, and the parts are merged with online softmax
 * ("vLLM x AgentX: Optimizing for Real-World Agentic Serving", section
 * "Model-specific parallelism / Kimi K3", where the parts sit on different
 * GPUs).  Here the parts are splits of one request's pages on one GPU:
 * for row r of request b and split s over its visible tokens T_s,
 *   lse_s = ln sum_{t in T_s} exp(c q_r.k_t),
 *   o_s   = sum_{t in T_s} exp(c q_r.k_t - lse_s) v_t,
 * with k_t the whole 576-element row, v_t its first 512 elements and
 * c = softmax_scale; mla_decode_combine merges the splits.
 *
 *   q           bf16 [B, n_q, H, 576]: the query already absorbed into the
 *               latent space (latent 512 | rope 64).
 *   kv_cache    MLA_CACHE_FP8_E4M3: e4m3 codes [num_pages, 64, 576];
 *               MLA_CACHE_BF16: bf16 [num_pages, 64, 576].
 *   kv_scale    see mla_scale_mode_t (NULL allowed for MLA_SCALE_NONE).
 *   softmax_scale  multiplies q.K before the softmax.
 *   pages_per_split, max_splits  the split-KV plan (mla_decode_plan gives one):
 *               split s of request b covers pages [s*pps, (s+1)*pps), except
 *               that split max_splits-1 also takes every page after it.
 *               pages_per_split * max_splits must not exceed 2^31 - 1.
 *   o_partial   bf16 [B, max_splits, n_q, H, 512]: per-split output,
 *               normalised by the split's own softmax sum (rounded to bf16:
 *               the partials are read back once, and their rounding is far
 *               inside the output tolerance).
 *   lse_partial fp32 [B, max_splits, n_q, H]: per-split natural log-sum-exp
 *               (-inf for a row that sees no token of the split).
 *   out         bf16 [B, n_q, H, 512];  lse  fp32 [B, n_q, H] (natural log).
 *
 * With max_splits == 1 the final out and lse are written directly and the
 * partial buffers may be NULL.  With max_splits > 1 only the partials are
 * written (splits past a request's last page are left untouched) and
 * mla_decode_combine must run next; out and lse may then be NULL.
 * Supported: 1 <= H <= 128, 1 <= n_q <= 2048: a decode step's few new
 * tokens, or an extend / prefill chunk of up to 2048 new tokens, causal among
 * themselves, over the cached context (each group of 64 query rows is a
 * workgroup of its own that reads the pages of its split).  A row that sees no token gets out = 0 and lse = -inf.
 */
int mla_decode_paged(const void* q, const void* kv_cache, int cache_dtype, const float* kv_scale,
                     int scale_mode, const int32_t* block_table, const int32_t* seq_lens, int B,
                     int n_q, int H, int max_blocks, int num_pages, float softmax_scale,
                     int pages_per_split, int max_splits, void* o_partial, float* lse_partial,
                     void* out, float* lse, void* stream);

/*
 * mla_decode_paged_append — kv_append_fp8 followed by mla_decode_paged on an
 * FP8 cache, in one launch.  The new rows land in the cache's last page(s),
 * which the decode reads in the same step; each workgroup that reads such a
 * page encodes the rows itself (the same bytes kv_append_fp8 writes) and puts
 * them over what its page copy brought, and one of them writes them, with
 * their per-token scales, to the cache.  This saves the separate append
 * launch and the wait between the two on every decode step.
 *
 *   kv_new, n_new   bf16 [B, n_new, 576] as in kv_append_fp8 (n_new = 0:
 *                   plain decode); rows go to seq_lens[b] - n_new + j.
 *   kv_cache        e4m3 codes [num_pages, 64, 576], written for the new rows.
 *   kv_scale        PER_TOKEN: [num_pages, 64], written for the new rows;
 *                   PER_TENSOR: [1], read.
 *   the rest        as in mla_decode_paged (cache_dtype is MLA_CACHE_FP8_E4M3).
 *
 * After the call the cache and scales hold exactly what kv_append_fp8 would
 * have written, and out / lse (or the partials) are bit-identical to those of
 * mla_decode_paged on that cache.  A row whose position has no visible page
 * (seq_lens[b] - n_new + j < 0) is skipped, as in kv_append_fp8.  Errors as in
 * the two calls it replaces; MLA_ERR_UNSUPPORTED for MLA_SCALE_NONE.
 *
 *   store_rows      1: as above.  With more than 16 new rows per request the
 *                   rows are encoded and stored by a kv_append_fp8 launch on
 *                   the same stream, and the decode launch that follows reads
 *                   them back from the cache: every workgroup of the fused
 *                   launch would otherwise encode them all again.  Same
 *                   results; all arguments are checked before either launch.
 *                   0: the new rows take part in this launch's
 *                   attention but nothing is written to kv_cache / kv_scale;
 *                   the caller stores them with kv_append_fp8 (for instance on
 *                   another stream, after kv_check_pages, with the checked
 *                   lengths).  That append may run while this launch runs:
 *                   the launch puts its own encoding over whatever it reads
 *                   of the new rows' slots, so its results do not depend on
 *                   when the append lands.
 */
int mla_decode_paged_append(const void* kv_new, int n_new, const void* q, void* kv_cache,
                            float* kv_scale, int scale_mode, const int32_t* block_table,
                            const int32_t* seq_lens, int B, int n_q, int H, int max_blocks,
                            int num_pages, float softmax_scale, int pages_per_split, int max_splits,
                            void* o_partial, float* lse_partial, void* out, float* lse, int store_rows,
                            void* stream);

/*
 * mla_decode_paged_append_checked — mla_decode_paged_append (rows stored,
 * split partials written) with the KV page-tag check of kv_check_pages
 * carried in the same launch ("Smaller, faster, safer", section "Protecting a
 * shared KV cache").  B extra workgroups, placed after the decode's, each
 * check one request and write status[b] exactly as kv_check_pages does.  The
 * attention does not wait for them: it reads the unchecked lengths (page ids
 * are clamped, so it stays inside the cache), and the flagged requests are
 * masked afterwards by mla_decode_combine with the same status array, so no
 * flagged request returns data.  Each new row is stored only into a page
 * that passes the check on its own (in the pool, equal to the recorded page,
 * carrying the recorded tag), so nothing is written into a page that was
 * handed to another request.  (A flagged request can still store its rows
 * into its own pages that pass; kv_check_pages in front of the decode stores
 * none of a flagged request's rows.)
 *   page_tags, expected_pages (or NULL), expected_tags, status: as in
 *               kv_check_pages.
 *   the rest    as in mla_decode_paged_append with max_splits >= 2 (out and
 *               lse come from mla_decode_combine, which must get `status`).
 * Returns MLA_ERR_UNSUPPORTED for max_splits < 2 or MLA_SCALE_NONE,
 * MLA_ERR_NULL_PTR for a NULL check array with B > 0; otherwise as
 * mla_decode_paged_append.
 */
int mla_decode_paged_append_checked(const void* kv_new, int n_new, const void* q, void* kv_cache,
                                    float* kv_scale, int scale_mode, const int32_t* block_table,
                                    const int32_t* seq_lens, int B, int n_q, int H, int max_blocks,
                                    int num_pages, float softmax_scale, int pages_per_split,
                                    int max_splits, void* o_partial, float* lse_partial,
                                    const uint32_t* page_tags, const int32_t* expected_pages,
                                    const uint32_t* expected_tags, int32_t* status, void* stream);

/*
 * mla_decode_paged_append_noalloc — mla_decode_paged_append followed by
 * mla_decode_combine, with the split partials in a scratch array the library
 * holds, for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The call
 * makes no allocation of any kind; the caller passes only inputs and outputs.
 *
 *   arguments   as in mla_decode_paged_append, without o_partial and
 *               lse_partial; out bf16 [B, n_q, H, 512] and lse fp32
 *               [B, n_q, H] are always written (for max_splits == 1 directly
 *               by the decode launch, else by the merge launched after it on
 *               the same stream).
 *
 * Results are bit-identical to mla_decode_paged_append + mla_decode_combine
 * with the same pages_per_split / max_splits (the same kernels run).  The
 * scratch is a file-scope device array of MLA_NOALLOC_MAX_PARTIAL_ROWS partial
 * rows; each GPU holds its own copy from the first call on that device until
 * the process ends.  Nothing in it has to start at zero: the merge reads only
 * the partials the decode launch of the same call has written.  Every call on
 * one GPU shares that GPU's scratch, so calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race and
 * give wrong results; calls ordered on one stream are safe.  The stream must
 * belong to the current device.
 *
 * Returns MLA_ERR_SCRATCH_LIMIT when max_splits > 1 and
 * B * max_splits * n_q * H > MLA_NOALLOC_MAX_PARTIAL_ROWS (nothing launched),
 * MLA_ERR_NULL_PTR for a NULL out / lse with B > 0, MLA_ERR_UNSUPPORTED for a
 * stream of another device; otherwise as mla_decode_paged_append.
 */
int mla_decode_paged_append_noalloc(const void* kv_new, int n_new, const void* q, void* kv_cache,
                                    float* kv_scale, int scale_mode, const int32_t* block_table,
                                    const int32_t* seq_lens, int B, int n_q, int H, int max_blocks,
                                    int num_pages, float softmax_scale, int pages_per_split,
                                    int max_splits, void* out, float* lse, int store_rows,
                                    void* stream);

/*
 * mla_decode_combine — merge the split partials of mla_decode_paged
 * ("vLLM x AgentX", section "Model-specific parallelism / Kimi K3": partial
 * outputs and LSE statistics merged with online softmax).
 *
 * For each row, over the n_b = min(max_splits, ceil(ceil(L_b/64)/pps)) splits
 * request b used: M = max_s lse_s; w_s = exp(lse_s - M);
 * out = bf16(sum_s w_s o_s / sum_s w_s); lse = M + ln(sum_s w_s).
 * Same shapes as mla_decode_paged; pages_per_split and max_splits must be the
 * values that call used.
 *   status     int32 [B] from kv_check_pages, or NULL.  A request whose entry
 *              is non-zero merges no split: its rows get out = 0 and
 *              lse = -inf, whatever its partials hold.  This lets the page
 *              check run beside the decode launch (which then reads the
 *              unchecked lengths; page ids are clamped, so a bad page map
 *              still reads only inside the cache) and still keep a flagged
 *              request from returning data read from another page.
 */
int mla_decode_combine(const void* o_partial, const float* lse_partial, const int32_t* seq_lens,
                       int B, int n_q, int H, int max_blocks, int pages_per_split, int max_splits,
                       void* out, float* lse, const int32_t* status, void* stream);

/*
 * mla_decode_plan — host-only helper that picks pages_per_split and max_splits
 * so the split workgroups fill `num_cus` compute units (0 = 256) with about
 * equal work.  max_seq_len and total_seq_len are the largest and the summed
 * L_b of the batch; cache_dtype (mla_cache_dtype_t) selects the kernel the
 * plan is for (64 query rows per workgroup on FP8, 32 on BF16).  Writes
 * *pages_per_split >= 1 and *max_splits >= 1.  Touches no device.
 */
int mla_decode_plan(int B, int n_q, int H, int max_seq_len, int64_t total_seq_len, int num_cus,
                    int cache_dtype, int* pages_per_split, int* max_splits);

/*
 * mla_decode_plan_lens — host-only split plan from the batch's lengths.
 *   seq_lens   host int32 [B], the L_b of the coming launch (after its append).
 *   cache_dtype  mla_cache_dtype_t of the coming launch.
 * Chooses pages_per_split among the smallest values whose workgroups fit one,
 * two, three or four rounds of `num_cus` compute units (0 = 256), by the
 * shortest estimated duration when workgroup i waits for a free compute unit
 * of XCD i % 8 (one workgroup per unit at a time) and costs its pages plus a
 * fixed start-up of two pages.  Writes *pages_per_split >= 1 and *max_splits >= 1 (1 and 1 for an
 * all-empty batch).  Returns MLA_ERR_NULL_PTR for a NULL output (or NULL
 * seq_lens with B > 0), MLA_ERR_BAD_SHAPE for a negative length or a plan
 * whose grid would exceed 2^31 - 1 workgroups.  Touches no device.
 */
int mla_decode_plan_lens(const int32_t* seq_lens, int B, int n_q, int H, int num_cus, int cache_dtype,
                         int* pages_per_split, int* max_splits);

/*
 * kv_check_pages — the KV page-tag integrity check, a batch launch of its own
 * ahead of decode ("Smaller, faster, safer", section "Protecting a shared KV
 * cache": every physical page carries a tag that changes whenever the page is
 * handed out again; the server records the (page, tag) pairs each request
 * expects; before decode reads the cache the records are compared with the
 * current state, and a request that does not match is aborted).
 *   page_tags       uint32 [num_pages], the current tag of each physical page.
 *   block_table     int32 [B, max_blocks], the page map decode will read.
 *   expected_pages  int32 [B, max_blocks], the recorded pages, or NULL to take
 *                   the page map itself as the record.
 *   expected_tags   uint32 [B, max_blocks], the recorded tag of each entry.
 *   seq_lens        int32 [B].
 *   status          int32 [B] out: or of mla_page_status_t bits.
 *   checked_lens    int32 [B] out: seq_lens[b] where status[b] == 0, else 0.
 *                   It may be seq_lens itself (the lengths are then masked in
 *                   place); it must not overlap status or the other inputs.
 * Request b reads logical pages j < ceil(L / 64), L = seq_lens[b]; only those
 * entries are checked.  Per entry: the page-map entry against the recorded
 * page (MLA_PAGE_WRONG_PAGE), the entry against [0, num_pages)
 * (MLA_PAGE_OUT_OF_RANGE, and then no tag is read), else the page's current
 * tag against the recorded tag (MLA_PAGE_STALE_TAG).  A length outside
 * [0, max_blocks * 64] gives MLA_PAGE_BAD_LEN alone.  Passing checked_lens as
 * the seq_lens of kv_append_fp8, mla_decode_paged(_append) and
 * mla_decode_combine aborts the flagged requests within the step: none of
 * their pages is read or written, their output rows are 0 and their
 * log-sum-exp is -inf.  One workgroup of 1024 threads per request.
 * Returns MLA_ERR_BAD_SHAPE for B < 0, num_pages < 1, max_blocks < 1 or
 * max_blocks * 64 >= 2^31; MLA_ERR_NULL_PTR for a NULL required pointer with
 * B > 0; nothing is launched for B == 0.
 */
int kv_check_pages(const uint32_t* page_tags, int num_pages, const int32_t* block_table,
                   const int32_t* expected_pages, const uint32_t* expected_tags,
                   const int32_t* seq_lens, int B, int max_blocks, int32_t* status,
                   int32_t* checked_lens, void* stream);

/* Static text for a status code. */
const char* mla_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
