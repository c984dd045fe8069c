/*
 * sparse_attn.h -- C ABI of a gfx950 (MI355X) library for dynamic page- and
 * block-sparse attention over a paged KV cache.
 *
 * Method sources (web pages, cited by title and section):
 *  [UAE] "Universal Attention Engine - Declarative Sparse Attention for
 *        Production": "The Product" (sink tokens, local window, cache budget),
 *        "Content-Dependent Dynamic Routing (Novel)" (router
 *        top_k_blocks(q @ mean(k_blocks), k): block-granular routing, full
 *        attention on the selected blocks, only selected blocks loaded),
 *        "Key Design Decisions" 3 (decode optimised for bytes loaded, prefill
 *        for FLOPs), "Architecture" Layer 2/3 (gather-based sparse-KV decode,
 *        block-sparse prefill, PagedAttention-compatible layout).
 *  [TS]  "TileSparse: Arithmetic-Intensity-Aware Sparse Attention for
 *        Compute-Bound LLM Decoding" (README): "Motivation" (QK 2D sparsity;
 *        Tiered QK 2D sparsity with a Critical tier of alpha pages on all
 *        query heads and an Ambient tier of beta pages on h heads), "Two
 *        implementations, by design" (true per-head page-list Flash-decode),
 *        "Configuration" (critical_top_count, ambient_head_count).
 *  [STS] STS abstract on the page titled "Vortex: Efficient and Programmable
 *        Sparse Attention Serving for AI Agents" (token-and-head-wise masks
 *        built from draft-model attention scores).
 *  [CA]  CompactAttention abstract on the page titled "Causal Attention on
 *        CPU: A Cache-Aware and Load-Balanced Scheduling Kernel for Prefill"
 *        (2D block masks -> GQA-aware per-group KV block tables by Q-block union
 *        then intra-group union; KV read in place under chunked prefill).
 *
 * Conventions for every call below.
 *  - Memory: every tensor pointer is a DEVICE pointer owned by the caller.
 *    The library allocates no device memory; calls that need scratch take a
 *    caller-provided `workspace` of at least the size its *_workspace_size
 *    function returns (256-byte aligned).
 *  - Streams: all work is enqueued on `stream`; calls return without
 *    synchronising.  Calls sharing a workspace must be ordered by the caller.
 *  - Errors: arguments are validated on the host before anything is
 *    launched.  On error the call returns a non-SA_OK status, enqueues
 *    nothing, writes no output, records a message for sa_last_error_message()
 *    (thread-local) and never aborts.  A launch failure returns SA_ERR_DEVICE.
 *    Device data (page ids, list entries, lengths, given scores) is trusted:
 *    out-of-range page ids are undefined behaviour, unless debug validation
 *    is on (sa_set_debug_validate below).
 *  - Layout of the paged KV cache (sa_paged_kv), all row-major:
 *      k_pool      [n_phys_pages][n_kv_heads][page_size][d_qk]   (token-major page)
 *      v_pool      [n_phys_pages][n_kv_heads][d_v][page_size]    (page-transposed,
 *                  the PagedAttention value layout); NULL means V is the first
 *                  d_v dims of each K row (MLA latent cache, d_qk 576 / d_v 512)
 *      block_table [batch][max_pages] int32: logical page -> physical page
 *      seq_lens    [batch] int32: valid tokens per sequence; logical page p of
 *                  sequence b holds tokens [p*page_size, min((p+1)*page_size, len))
 *  - Supported shapes: page_size 16 or 64; (d_qk, d_v) = (64, 64) or (128, 128)
 *    with a V pool, (576, 512) without one; dtype bf16, or fp32 for the decode
 *    side (summary, select, decode) at d 64/128, or FP8 E4M3 pages (see
 *    sa_dtype) at d 128.  Anything else returns SA_ERR_UNSUPPORTED.
 */
#ifndef SPARSE_ATTN_H_
#define SPARSE_ATTN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  SA_ERR_INVALID_ARGUMENT = 1,
  SA_ERR_UNSUPPORTED = 2,
  SA_ERR_WORKSPACE_TOO_SMALL = 3,
  SA_ERR_DEVICE = 4,
  SA_ERR_DATA = 5                /* debug validation found invalid device data */
} sa_status;

/* SA_DTYPE_FP8_E4M3: k_pool and v_pool hold OCP FP8 E4M3 bytes, with one
 * fp32 scale per (physical page, KV head) for K (k_scale) and one for V
 * (v_scale): an element's value is its E4M3 value times its page's scale
 * ([UAE] "Key Design Decisions" 2 and "Milestones" Phase 3: quantized KV
 * cache).  Queries and outputs are then bf16.  Supported by sa_page_summary,
 * sa_select_pages (without refresh_newest_page), sa_prefill_block_mask and
 * sa_sparse_decode, at d_qk == d_v == 128 with a V pool. */
typedef enum { SA_DTYPE_BF16 = 0, SA_DTYPE_FP32 = 1, SA_DTYPE_FP8_E4M3 = 2 } sa_dtype;

/* Selection granularity.  PER_KV_HEAD: one list per KV head, scored with the
 * query summed over the head's query group (GQA) and query tokens.
 * PER_Q_HEAD: one list per query head ([TS] QK 2D sparsity, [STS] head-wise
 * masks). */
typedef enum { SA_SEL_PER_KV_HEAD = 0, SA_SEL_PER_Q_HEAD = 1 } sa_sel_mode;

typedef struct {
  const void* k_pool;
  const void* v_pool;            /* may be NULL (latent cache) */
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t n_phys_pages;
  int32_t n_kv_heads;
  int32_t page_size;
  int32_t d_qk;
  int32_t d_v;
  int32_t max_pages;             /* row stride of block_table */
  sa_dtype dtype;                /* element type of q, k_pool, v_pool and outputs (FP8: of the pools) */
  const float* k_scale;          /* FP8 only: [n_phys_pages][n_kv_heads] K scales (else NULL) */
  const float* v_scale;          /* FP8 only: [n_phys_pages][n_kv_heads] V scales (else NULL) */
} sa_paged_kv;

/* ------------------------------------------------------------------------
 * sa_page_summary -- per-page mean key, the block summary the router scores
 * against ([UAE] "Content-Dependent Dynamic Routing": mean(k_blocks)).
 *
 *   page_summary[phys][g][:] = mean over the page's valid tokens of k_pool[phys][g][j][:]
 *
 * Accumulated in float64, rounded once to fp32.  Written for logical pages
 * [0, n) of every sequence (n = ceil(seq_len/page_size)), or only the last
 * `last_pages` of them when last_pages > 0 (the pages a decode step's new
 * tokens touched).  Entries of other physical pages are left untouched.
 *   page_summary: out [n_phys_pages][n_kv_heads][d_qk] fp32.
 * ---------------------------------------------------------------------- */
sa_status sa_page_summary(const sa_paged_kv* kv, int32_t batch, int32_t last_pages,
                          float* page_summary, hipStream_t stream);

/* ------------------------------------------------------------------------
 * sa_select_pages -- per-selection-head page lists: forced sink pages and
 * local-window pages plus the top-k other pages by router score
 * ([UAE] "The Product" sink/local window, "Content-Dependent Dynamic
 * Routing" top_k_blocks; [TS] tiers; [STS] head-wise masks).
 *
 * Score of logical page p for selection head s of sequence b:
 *   score = fp32( sum_d Qbar[d] * page_summary[phys(b,p)][g(s)][d] ),
 *   Qbar = sum over the q_tokens query tokens and the query heads of s
 *          (PER_KV_HEAD: the n_q_heads/n_kv_heads heads of KV head s;
 *           PER_Q_HEAD: head s alone, KV head s / group) of q, in float64.
 * With `scores` given, those values are used as-is instead (q and
 * page_summary may then be NULL).
 * refresh_newest_page != 0 (router scores only, page_summary required):
 * first recompute page_summary for each sequence's newest page, all KV heads,
 * exactly as sa_page_summary(kv, batch, 1, page_summary) would (same bits),
 * then score with it; one call replaces the per-step pair of calls.
 * Forced pages F = [0, sink_pages) u [n - window_pages, n), clipped to [0, n).
 * The other pages are ranked by (score descending, logical index ascending),
 * NaN last, -0 == +0; the first k = min(top_k, n - |F|) are selected.
 *   untiered (critical_counts == NULL): list = ascending(F u selected)
 *   tiered: Critical = ascending(F u first min(critical_k, k) selected),
 *           Ambient  = ascending(the remaining selected); list = Critical
 *           then Ambient; critical_counts = |Critical|.
 *   q            [batch][q_tokens][n_q_heads][d_qk] (kv->dtype) or NULL
 *   page_summary [n_phys_pages][n_kv_heads][d_qk] fp32 or NULL (written only
 *                for the newest pages, and only with refresh_newest_page)
 *   scores       [batch][n_sel][scores_stride] fp32 or NULL, scores_stride >= max_pages
 *   page_lists   out [batch][n_sel][list_stride] int32 logical ids, entries
 *                past the count are left untouched;
 *                list_stride >= min(max_pages, sink_pages + window_pages + top_k)
 *   page_counts  out [batch][n_sel];  critical_counts out [batch][n_sel] or NULL
 *   scores_out   optional out [batch][n_sel][max_pages] fp32 router scores (NaN
 *                past each sequence's last page); ignored when scores given
 * n_sel = n_kv_heads (PER_KV_HEAD) or n_q_heads (PER_Q_HEAD).  max_pages <= 16384.
 * Unless scores_out is given, the page_summary rows of forced pages take no
 * part in the call (they are read only when no page of the sequence is
 * scored, and then ignored), so a summary update of forced pages (e.g. the
 * newest page inside the local window) may run concurrently with this call on
 * another stream.
 * ---------------------------------------------------------------------- */
size_t sa_select_pages_workspace_size(int32_t batch, int32_t n_sel, int32_t max_pages);

sa_status sa_select_pages(const sa_paged_kv* kv, int32_t batch,
                          const void* q, int32_t q_tokens, int32_t n_q_heads,
                          float* page_summary, int32_t refresh_newest_page,
                          const float* scores, int32_t scores_stride,
                          sa_sel_mode mode,
                          int32_t sink_pages, int32_t window_pages, int32_t top_k,
                          int32_t critical_k,
                          int32_t* page_lists, int32_t list_stride,
                          int32_t* page_counts, int32_t* critical_counts,
                          float* scores_out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * sa_sparse_decode -- split-K paged flash-decode over per-head page lists
 * ([UAE] gather-based sparse-KV decode; [TS] per-head page-list Flash-decode
 * and Tiered QK 2D sparsity).
 *
 * Query row (b, t, h) attends exactly the valid tokens of its pages:
 *   untiered: every page in its selection head's list;
 *   tiered (critical_counts != NULL): the first critical_counts[b][s] list
 *   entries (Critical, all heads) plus each later entry p (Ambient) whose
 *   ambient_head_mask[b][p] has bit h.
 *   o = softmax(sm_scale * q K^T) V over that token set, lse = log-sum-exp of
 *   the scaled logits; an empty set gives o = 0 and lse = -inf.  sm_scale
 *   must be finite and positive (SA_ERR_INVALID_ARGUMENT otherwise).
 * Each list is cut into num_splits contiguous chunks (sizes differ by at most
 * one); chunk partials (o_s, lse_s) are combined by an LSE merge.  The
 * workspace holds the partials: o_s in fp32, or in bf16 for a latent cache
 * (each o_s is a normalised average, so bf16 adds at most 2^-9 of its
 * magnitude before the merge), lse_s in fp32.
 *   q                 [batch][q_tokens][n_q_heads][d_qk]
 *   page_lists/counts as produced by sa_select_pages (logical page ids)
 *   ambient_head_mask [batch][max_pages][ceil(n_q_heads/32)] uint32 (tiered only)
 *   num_splits        0: the library chooses; otherwise 1..64
 *   out               [batch][q_tokens][n_q_heads][d_v] (kv->dtype)
 *   out_lse           [batch][q_tokens][n_q_heads] fp32 natural-log units, or NULL
 * Per-KV-head lists need q_tokens*group <= 16 at d 64/128 (one 16-row MFMA
 * tile per KV head); the latent path needs n_kv_heads == 1, per-KV-head
 * lists, page_size 64 and q_tokens in {1, 2, 4, 8, 16} (the query tokens of
 * one head share a 16-row tile and its Ambient bit).
 * ---------------------------------------------------------------------- */
size_t sa_sparse_decode_workspace_size(const sa_paged_kv* kv, int32_t batch, int32_t q_tokens,
                                       int32_t n_q_heads, int32_t list_stride, sa_sel_mode mode,
                                       int32_t num_splits);

sa_status sa_sparse_decode(const sa_paged_kv* kv, int32_t batch,
                           const void* q, int32_t q_tokens, int32_t n_q_heads,
                           const int32_t* page_lists, const int32_t* page_counts,
                           int32_t list_stride, sa_sel_mode mode,
                           const int32_t* critical_counts, const uint32_t* ambient_head_mask,
                           float sm_scale, int32_t num_splits,
                           void* out, float* out_lse,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * sa_sparse_decode_noalloc -- sa_sparse_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments, kernels and results
 * bit for bit, without `workspace`.  The split partials live in a static
 * device array of SA_NOALLOC_SCRATCH_BYTES inside the library, one copy per
 * GPU, held from the library's load until the process ends; its address is
 * looked up once per device, on the first call that needs it with that
 * device current.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine).
 *  - `stream` must belong to the current device.
 *  - A call whose partials need more than SA_NOALLOC_SCRATCH_BYTES (the size
 *    sa_sparse_decode_workspace_size reports for the same arguments) returns
 *    SA_ERR_WORKSPACE_TOO_SMALL and launches nothing; fewer splits need less.
 *  - Every call on one GPU shares that GPU's array and leaves its partials
 *    there.  Calls that overlap on one GPU (other streams, or other threads
 *    without ordering) race on it: the caller must order them.
 * ---------------------------------------------------------------------- */
#define SA_NOALLOC_SCRATCH_BYTES (64u << 20)

sa_status sa_sparse_decode_noalloc(const sa_paged_kv* kv, int32_t batch,
                                   const void* q, int32_t q_tokens, int32_t n_q_heads,
                                   const int32_t* page_lists, const int32_t* page_counts,
                                   int32_t list_stride, sa_sel_mode mode,
                                   const int32_t* critical_counts, const uint32_t* ambient_head_mask,
                                   float sm_scale, int32_t num_splits,
                                   void* out, float* out_lse, hipStream_t stream);

/* ------------------------------------------------------------------------
 * sa_select_decode -- the decode step's two calls in one launch: page
 * selection with router scores ([UAE] "The Product", "Content-Dependent
 * Dynamic Routing") and sparse decode over the selected pages ([UAE] "Key
 * Design Decisions" 3), for per-KV-head, untiered lists.
 *
 * Writes exactly what these two calls write, bit for bit:
 *   sa_select_pages(kv, batch, q, q_tokens, n_q_heads, page_summary,
 *                   refresh_newest_page, NULL, 0, SA_SEL_PER_KV_HEAD,
 *                   sink_pages, window_pages, top_k, 0, page_lists,
 *                   list_stride, page_counts, NULL, NULL, ...)
 *   sa_sparse_decode(kv, batch, q, q_tokens, n_q_heads, page_lists,
 *                    page_counts, list_stride, SA_SEL_PER_KV_HEAD, NULL, NULL,
 *                    sm_scale, 1, out, out_lse, ...)
 * One workgroup per (sequence, KV head) selects its list and decodes it
 * without waiting for the other lists' selections; no workspace is needed.
 * Arguments are those of the two calls.  Supported: bf16, a V pool, d_qk ==
 * d_v == 128, page_size 64, q_tokens * group <= 16, and max_pages +
 * list_stride small enough for the keys and the list to sit in LDS (about
 * 6,000 entries: 128K tokens of pages of 64 fit); anything else returns
 * SA_ERR_UNSUPPORTED (use the two calls).  Validation and errors as for the
 * two calls.
 * ---------------------------------------------------------------------- */
sa_status sa_select_decode(const sa_paged_kv* kv, int32_t batch,
                           const void* q, int32_t q_tokens, int32_t n_q_heads,
                           float* page_summary, int32_t refresh_newest_page,
                           int32_t sink_pages, int32_t window_pages, int32_t top_k,
                           int32_t* page_lists, int32_t list_stride, int32_t* page_counts,
                           float sm_scale, void* out, float* out_lse, hipStream_t stream);

/* ------------------------------------------------------------------------
 * sa_prefill_block_mask -- the 2D block mask of a prefill chunk by
 * block-level pattern discovery (block-sparse prefill brief on the Paperraft
 * page: instantaneous pattern discovery, max-based dynamic thresholding;
 * score form of the [UAE] router, "Content-Dependent Dynamic Routing"; the
 * mask feeds the [CA] Q-block / intra-group union of sa_block_sparse_prefill).
 *
 * For query head h and Q-block qb (queries [qb*block_q, min(+block_q, q_len))):
 *   qbar   = mean of the Q-block's query rows of head h (float64)
 *   n      = KV blocks holding a token at or before the Q-block's last
 *            position q_start + i_last and below seq_lens[seq] (causal blocks)
 *   s[kb]  = fp32(sm_scale * sum_d qbar[d] * page_summary[phys(kb)][g(h)][d]),  kb < n
 *   forced = block 0 and the diagonal blocks [block of q_start + i_first, n)
 *   top_k >= 0: keep the top_k other causal blocks by (score desc, index asc)
 *   top_k <  0: keep the other causal blocks with s >= fp32(max_kb<n s[kb] - max_gap)
 *   block_mask_out[h][qb][kb] = 1 for forced and kept blocks, else 0.
 *   q            [q_len][n_q_heads][d_qk] (kv->dtype)
 *   page_summary [n_phys_pages][n_kv_heads][d_qk] fp32 (sa_page_summary)
 *   block_mask_out out [n_q_heads][ceil(q_len/block_q)][n_kv_blocks] uint8
 * Needs a V-pool cache (d 64 or 128), at most 8 query heads per KV head,
 * n_kv_blocks covering q_start + q_len and <= max_pages, and
 * (group + 2) * n_kv_blocks * 4 bytes <= 144 KiB (e.g. 4 heads per KV head
 * and 4,096 blocks).  max_gap >= 0 (may be +inf) in threshold mode.
 * ---------------------------------------------------------------------- */
sa_status sa_prefill_block_mask(const sa_paged_kv* kv, int32_t seq,
                                const void* q, int32_t q_len, int32_t q_start, int32_t n_q_heads,
                                const float* page_summary, int32_t block_q, int32_t n_kv_blocks,
                                float sm_scale, int32_t top_k, float max_gap,
                                uint8_t* block_mask_out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * sa_block_sparse_prefill -- chunked-prefill attention with a 2D block mask
 * turned into GQA-union KV block tables ([CA]; [UAE] block-sparse prefill).
 *
 *   U_h[kb]  = OR over Q-blocks qb of block_mask[h][qb][kb]
 *   T_g[kb]  = OR over the query heads h of KV head g of U_h[kb]
 *   block_table_out[g][0..count) = ascending {kb : T_g[kb]}, block_counts_out[g] = count
 * then query i (position q_start + i) of head h attends, in place in the
 * paged pool row `seq`, every token j of the blocks in T_{g(h)} with
 * j <= q_start + i and j < seq_lens[seq]:  o = softmax(sm_scale q K^T) V
 * (sm_scale finite and positive).
 *   q          [q_len][n_q_heads][d_qk]
 *   block_mask [n_q_heads][ceil(q_len/block_q)][n_kv_blocks] uint8 (nonzero = keep);
 *              KV block kb is logical page kb (block size = page_size)
 *   block_table_out  out [n_kv_heads][n_kv_blocks] int32 (entries past the
 *              count are left untouched); block_counts_out out [n_kv_heads]
 *   out        [q_len][n_q_heads][d_v];  out_lse [q_len][n_q_heads] fp32 or NULL
 * Needs bf16, d_qk == d_v == 128, page_size 64, n_kv_blocks <= max_pages and
 * n_kv_blocks <= 4096 (262144 tokens).
 * ---------------------------------------------------------------------- */
size_t sa_block_sparse_prefill_workspace_size(const sa_paged_kv* kv, int32_t q_len,
                                              int32_t n_q_heads, int32_t n_kv_blocks);

sa_status sa_block_sparse_prefill(const sa_paged_kv* kv, int32_t seq,
                                  const void* q, int32_t q_len, int32_t q_start, int32_t n_q_heads,
                                  const uint8_t* block_mask, int32_t block_q, int32_t n_kv_blocks,
                                  int32_t* block_table_out, int32_t* block_counts_out,
                                  float sm_scale, void* out, float* out_lse,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * sa_page_value_summary -- per-page mean value row, the value counterpart of
 * sa_page_summary, for the mean correction below:
 *
 *   value_summary[phys][g][:] = mean over the page's valid tokens j of v_pool[phys][g][:][j]
 *
 * (FP8 pages: of the dequantised values, code * v_scale).  Accumulated in
 * float64, rounded once to fp32; pages [0, n) of every sequence, or the last
 * `last_pages` of them when last_pages > 0; other entries untouched.
 *   value_summary: out [n_phys_pages][n_kv_heads][d_v] fp32.
 * Needs a V-pool cache.
 * ---------------------------------------------------------------------- */
sa_status sa_page_value_summary(const sa_paged_kv* kv, int32_t batch, int32_t last_pages,
                                float* value_summary, hipStream_t stream);

/* ------------------------------------------------------------------------
 * sa_prefill_mean_correction -- adds the blocks a block-sparse prefill left
 * out back into its result, each as one mean term (block-sparse prefill
 * brief on the Paperraft page: a mean correction term that bounds the error
 * of the skipped blocks).  The pages give no formula; the reading taken:
 * for query i (position p = q_start + i) of head h, every logical block kb of
 * the sequence that is not in the group table T_{g(h)} and whose valid
 * tokens all lie at or before p (kb*page_size + n_b - 1 <= p, n_b its valid
 * tokens) adds the term
 *     weight n_b * exp(sm_scale * q_i . mu_b),  value nu_b
 * to the softmax, mu_b / nu_b the block's mean key / value
 * (sa_page_summary / sa_page_value_summary).  With (o, lse) the prefill's
 * result over T_{g(h)} (one term of weight exp(lse), value o):
 *     lse' = log(exp(lse) + sum_b n_b exp(z_b)),
 *     o'   = (exp(lse) o + sum_b n_b exp(z_b) nu_b) / exp(lse').
 * A row that no skipped block reaches keeps its (o, lse) bit for bit.
 *   q, seq, q_len, q_start, n_q_heads, sm_scale: as given to sa_block_sparse_prefill
 *   block_table, block_counts: its block_table_out / block_counts_out
 *   page_summary, value_summary: [n_phys_pages][n_kv_heads][128] fp32, valid
 *              for every page of sequence `seq` below q_start + q_len
 *   out [q_len][n_q_heads][128] bf16, out_lse [q_len][n_q_heads] fp32: the
 *              prefill's result, read and overwritten in place
 * The means are rounded to bf16 for the q . mu products and the nu sums
 * (fp32 accumulation).  Same shape limits as sa_block_sparse_prefill.
 *   workspace: device memory of at least
 *              sa_prefill_mean_correction_workspace_size(kv, n_kv_blocks) bytes
 *              (the skipped blocks and their packed means; overwritten;
 *              SA_ERR_WORKSPACE_TOO_SMALL if short).  Calls sharing one
 *              workspace must be ordered on one stream.
 * ---------------------------------------------------------------------- */
size_t sa_prefill_mean_correction_workspace_size(const sa_paged_kv* kv, int32_t n_kv_blocks);

sa_status sa_prefill_mean_correction(const sa_paged_kv* kv, int32_t seq,
                                     const void* q, int32_t q_len, int32_t q_start, int32_t n_q_heads,
                                     const int32_t* block_table, const int32_t* block_counts, int32_t n_kv_blocks,
                                     const float* page_summary, const float* value_summary, float sm_scale,
                                     void* out, float* out_lse, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * AutoTuner of the tiered selection (TileSparse README, "Motivation":
 * Critical pages with all query heads, Ambient pages with h heads, and an
 * online per-layer search of the tier/head configuration that maximises an
 * estimated attention-mass coverage; "Configuration": token_budget,
 * critical_top_count, ambient_head_count).  The pages do not define the
 * estimate; the reading taken is stated with each call.  Per-KV-head
 * selection only (selection head g = KV head g, query heads g*G .. g*G+G-1).
 *
 * sa_head_page_mass -- estimated attention mass of every (query head, page):
 *   est[b][t][h][p] = sm_scale * q[b][t][h] . page_summary[phys(b,p)][g(h)] + ln n_p
 *   head_mass[b][h][p] = sum over t < q_tokens of softmax over p < n_b of est
 * (a page stands in for its n_p valid tokens by its mean key; each head's
 * masses sum to q_tokens).  The mean keys are split into two bf16 halves on
 * MFMA, so the products are fp32-accurate; softmax in fp32.
 *   q            [batch][q_tokens][n_q_heads][d_qk] bf16 (bf16 or FP8 caches)
 *   page_summary [n_phys_pages][n_kv_heads][d_qk] fp32 (sa_page_summary)
 *   head_mass    out [batch][n_q_heads][max_pages] fp32; entries of pages past
 *                a sequence's end are left untouched
 *   workspace    >= sa_head_page_mass_workspace_size(...) bytes (page
 *                log-weights), overwritten
 * Needs d_qk 64, 128 or 576 and max_pages <= 4096.
 * ---------------------------------------------------------------------- */
size_t sa_head_page_mass_workspace_size(const sa_paged_kv* kv, int32_t batch, int32_t q_tokens,
                                        int32_t n_q_heads);

sa_status sa_head_page_mass(const sa_paged_kv* kv, int32_t batch, const void* q, int32_t q_tokens,
                            int32_t n_q_heads, const float* page_summary, float sm_scale, float* head_mass,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * sa_autotune_tiers -- coverage of each (alpha, h) of a search grid and the
 * configuration the AutoTuner keeps.
 *   budget B: (page, query head) entries per KV head beyond its forced pages;
 *   beta(alpha, h) = floor((B - alpha*G) / h), infeasible when alpha*G > B.
 * For sequence b and KV head g the configuration selects, exactly as
 * sa_select_pages with top_k = alpha + beta and critical_k = alpha would from
 * `scores`: the forced pages F and the first alpha ranked candidates
 * (Critical, all G heads) and the next beta (Ambient, each with the h heads
 * of largest head_mass on it, mass descending then head ascending).  Its
 * coverage = (sum of head_mass over those (head, page) pairs) / (q_tokens*G);
 * the layer's coverage is the mean over sequences and KV heads.
 *   head_mass  [batch][n_q_heads][max_pages] fp32 (sa_head_page_mass)
 *   scores     [batch][n_kv_heads][scores_stride] fp32 router scores
 *              (sa_select_pages scores_out), scores_stride >= max_pages
 *   alphas, ambient_heads: HOST arrays of 1..16 entries (alpha >= 0, h >= 1)
 *   coverage_out out [n_alphas][n_heads] fp32 (device), NaN where infeasible
 *   choice_out   out int32[3] (device): alpha index, h index, beta of the
 *                first configuration of largest coverage in row-major order
 *                (-1 each when none is feasible)
 *   workspace  >= sa_autotune_tiers_workspace_size(...) bytes, overwritten
 * Needs n_q_heads / n_kv_heads <= 128 and max_pages <= 4096.
 * ---------------------------------------------------------------------- */
size_t sa_autotune_tiers_workspace_size(const sa_paged_kv* kv, int32_t batch, int32_t n_heads);

sa_status sa_autotune_tiers(const sa_paged_kv* kv, int32_t batch, int32_t q_tokens, int32_t n_q_heads,
                            const float* head_mass, const float* scores, int32_t scores_stride,
                            int32_t sink_pages, int32_t window_pages, int32_t budget,
                            const int32_t* alphas, int32_t n_alphas, const int32_t* ambient_heads,
                            int32_t n_heads, float* coverage_out, int32_t* choice_out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * sa_ambient_head_mask -- the Ambient tier's head mask for tiered lists
 * (sa_select_pages with critical_counts): for every list entry of KV head g
 * past its Critical count, page p gets the bits of the `ambient_heads` query
 * heads of g with the largest head_mass[b][h][p] (mass descending, head
 * ascending); every other bit of ambient_mask_out is cleared.
 *   ambient_mask_out out [batch][max_pages][ceil(n_q_heads/32)] uint32, the
 *   layout sa_sparse_decode reads.
 * Needs n_q_heads / n_kv_heads <= 128.
 * ---------------------------------------------------------------------- */
sa_status sa_ambient_head_mask(const sa_paged_kv* kv, int32_t batch, int32_t n_q_heads, const float* head_mass,
                               const int32_t* page_lists, int32_t list_stride, const int32_t* page_counts,
                               const int32_t* critical_counts, int32_t ambient_heads,
                               uint32_t* ambient_mask_out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * sa_set_debug_validate -- opt-in device-side checks of the index data every
 * call trusts, for callers that must not trust it (the "raise a clear error"
 * convention of the TileSparse README, "Quick start"; [UAE] "Key Design
 * Decisions": the cache is read through page tables).
 *
 * With validation on, each call first runs check kernels on its stream that
 * read the device arrays it is about to trust, within their declared shapes,
 * and never dereference the values they check:
 *   seq_lens[b] in [0, max_pages * page_size] (all calls, seq for prefill);
 *   block_table[b][lp] in [0, n_phys_pages) for the sequence's pages (all
 *     calls that read pages or page summaries);
 *   page_counts in [0, list_stride], list entries in [0, n_pages(b)),
 *     critical_counts in [0, page_counts] (decode);
 *   given scores finite over each sequence's pages (selection).
 * The call then waits for the checks (it synchronises `stream`, so it cannot
 * be captured into a graph) and, on the first violation found, returns
 * SA_ERR_DATA with a message naming the entry, enqueues nothing more and
 * writes no output.  Off by default; the environment variable
 * SA_DEBUG_VALIDATE (any value but "0") turns it on at the first call.
 * Returns the previous setting (0 or 1).  Process-wide.
 * ---------------------------------------------------------------------- */
int sa_set_debug_validate(int on);

/* ------------------------------------------------------------------------ utilities */
const char* sa_status_string(sa_status s);
const char* sa_last_error_message(void);   /* thread-local; "" when the last call succeeded */
int sa_version(void);                      /* major*10000 + minor*100 + patch */

#ifdef __cplusplus
}
#endif
#endif /* SPARSE_ATTN_H_ */
