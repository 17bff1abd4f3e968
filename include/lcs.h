/*
 * lcs.h - C ABI of the verify / select / sparse-draft attention path of
 * verification-guided self-speculative decoding, for AMD MI355X (gfx950).
 *
 * The three calls follow the problem as the pages state it:
 *  - Vegas page ("The pith", "Core claim", Figure 6 caption "Collect-2-Query"):
 *    verification computes full attention for the k+1 verifier tokens over the
 *    whole KV cache and exposes the pre-softmax logits of two rows, the first
 *    draft token and the bonus token;  -> lcs_verify_attn
 *  - the same pages, plus the Sparse Glimpse page ("Core claim": sink, recent
 *    and top-ranked historical tokens per head) and the SSV page (NSA block
 *    selection, "What carries the argument"): the two rows are summed over
 *    heads and the top-k prefix positions (or blocks) are kept;  -> lcs_select_topk
 *  - drafting attends only to the selected entries (Vegas "The pith"), and the
 *    SSV page's grouped verifier rows load each shared block once
 *    ("overlap-aware grouped-query execution", section 4.2 exact merged
 *    schedule, per-row causal masks at absolute positions).  -> lcs_sparse_draft_attn
 *
 * Variants of the first two calls:
 *  - any set of collected rows, and selection over n rows by summed logits or
 *    by post-softmax weights (Vegas Figure 6 and Figure 7; Sparse Glimpse "Core
 *    claim")  -> lcs_verify_attn_rows, lcs_select_topk_rows
 *  - the head sum of the two rows done per KV head in the verify epilogue, one
 *    score row per KV head handed to the selector  -> lcs_verify_attn_scores,
 *    lcs_select_topk_scores
 *
 * Conventions common to every call
 *  - Every pointer argument is DEVICE memory owned by the caller, except the
 *    lcs_paged_kv struct itself (host memory, read during the call only).
 *    The library never allocates or frees device memory and keeps no state
 *    between calls beyond its loaded code objects (which include the static
 *    scratch array of lcs_sparse_draft_attn_noalloc).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream).  Outputs are valid once the stream has reached the call.
 *  - All shape and argument checks run on the host before anything is
 *    launched.  On failure the call returns a non-OK status, launches nothing
 *    and lcs_last_error() describes the problem.  LCS_E_HIP reports a launch
 *    failure from the HIP runtime.
 *  - Contents of device arrays (index lists, block tables, lengths) are not
 *    validated on the host.  Kernels skip, rather than read, any position or
 *    page id that falls outside the cache; such entries simply do not take
 *    part in the result.
 *  - Calls are thread-safe as long as concurrent calls use distinct
 *    workspaces and outputs.
 *  - bf16 inputs, fp32 accumulation, fp32 outputs.
 *
 * Paged KV layout (the pages name vLLM's PagedAttention but fix no layout):
 * K and V are separate bf16 arrays [num_pages][Hkv][page_size][d]; logical
 * position p of sequence b lives in page block_table[b][p / page_size] at slot
 * p % page_size.  A (page, head) run is page_size*d contiguous elements and a
 * (token, head) row is d contiguous elements.  Query head h uses KV head
 * h / (Hq / Hkv).
 */
#ifndef LCS_H
#define LCS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LCS_OK = 0,
  LCS_E_ARG = 1,          /* null pointer, negative size, bad enum, bad row index   */
  LCS_E_SHAPE = 2,        /* inconsistent sizes (Hq % Hkv, cap too small, ...)       */
  LCS_E_WORKSPACE = 3,    /* workspace smaller than the *_workspace_bytes query      */
  LCS_E_UNSUPPORTED = 4,  /* valid but not implemented (d not 64/128, n_q > 64, ...) */
  LCS_E_HIP = 5           /* the HIP runtime refused a launch                        */
} lcs_status;

typedef enum {
  LCS_SET_SHARED = 0,      /* Vegas: one set per sequence, used by every KV head     */
  LCS_SET_PER_KV_HEAD = 1, /* Sparse Glimpse: one set per (sequence, KV head)        */
  LCS_SET_BLOCK = 2        /* SSV / NSA: block ids, one block = one page              */
} lcs_set_mode;

typedef enum {
  LCS_SCORE_LOGIT_SUM = 0,      /* Vegas: pre-softmax logits of the collected rows    */
  LCS_SCORE_SOFTMAX_WEIGHT = 1  /* Sparse Glimpse: post-softmax weights of the rows   */
} lcs_score_kind;

typedef enum {
  LCS_BLOCK_MAX = 0,  /* a block scores the max of its positions' scores               */
  LCS_BLOCK_LSE = 1   /* a block scores the log-sum-exp of its positions' scores       */
} lcs_block_score;

typedef enum {
  LCS_GROUP_EXACT = 0,       /* SSV exact merged schedule: each row keeps its own blocks */
  LCS_GROUP_APPROXIMATE = 1  /* SSV approximate mode: every row sees the group's union   */
} lcs_group_mode;

typedef struct {
  const void* k;              /* device bf16 [num_pages][Hkv][page_size][d]            */
  const void* v;              /* device bf16 [num_pages][Hkv][page_size][d]            */
  const int32_t* block_table; /* device int32 [B][max_pages]                           */
  int32_t num_pages;          /* >= 1; num_pages*Hkv*page_size < 2^31                  */
  int32_t page_size;          /* power of two, 1..1024                                  */
  int32_t max_pages;          /* row length of block_table                              */
  int32_t Hkv;                /* KV heads, >= 1                                         */
  int32_t d;                  /* head dim: 64 or 128                                    */
} lcs_paged_kv;

/* ---------------------------------------------------------------------------
 * Dense verify attention with Collect-2-Query logits.
 *
 * Vegas page, "The pith" / "Core claim" and Figure 6: full attention for the
 * n_q = k+1 verifier queries (draft chain plus bonus token) over the whole
 * cache; only the pre-softmax logits of rows collect_row0 and collect_row1
 * (the first draft token and the bonus token: 0 and n_q-1) are written.
 *
 *  q            bf16 [B][n_q][Hq][d].  Row i of sequence b sits at cache
 *               position prefix_len[b] + i; the cache must already hold the
 *               K/V of all n_q verifier tokens.
 *  prefix_len   device int32 [B]; values above max_prefix_len are clamped.
 *  max_prefix_len  host bound on prefix_len, sizes the launch.
 *  tree_mask    device uint64 [B][n_q] or NULL.  NULL: row i sees verifier
 *               slots j <= i (a chain).  Otherwise row i sees slot j iff bit j
 *               of tree_mask[b][i] is set.  Every row sees the whole prefix.
 *  scale        softmax scale, finite and > 0 (1/sqrt(d) in the pages' models).
 *  out          fp32 [B][n_q][Hq][d]: softmax(scale q K^T) V.
 *  logits       fp32 [B][Hq][2][logits_ld]: scale*q.k of the two collected rows
 *               for columns p < prefix_len[b]; other columns are untouched.
 *               logits_ld >= max_prefix_len.  Rows 16-byte aligned (logits_ld a
 *               multiple of 4) take the fast write path; a row stride of 32 floats
 *               past a multiple of 64 (e.g. round_up(max_prefix_len, 64) + 32)
 *               spreads the rows' concurrent writes over the HBM channels, where a
 *               power-of-two stride makes them collide (B = 8 at 128K: 852 us
 *               against 876-886 us per call).
 *  lse          fp32 [B][n_q][Hq] natural-log sum-exp of the scaled logits, or NULL.
 *  workspace    device scratch of at least lcs_verify_workspace_bytes(...) bytes
 *               (no initialisation needed; contents are clobbered).
 * Limits: n_q in [1, 64]; Hq % Hkv == 0; Hq/Hkv <= 64; d in {64, 128}.
 * ------------------------------------------------------------------------- */
size_t lcs_verify_workspace_bytes(int32_t B, int32_t n_q, int32_t Hq,
                                  const lcs_paged_kv* kv, int32_t max_prefix_len);

lcs_status lcs_verify_attn(const lcs_paged_kv* kv, const void* q, int32_t B, int32_t n_q,
                           int32_t Hq, const int32_t* prefix_len, int32_t max_prefix_len,
                           const uint64_t* tree_mask, float scale, int32_t collect_row0,
                           int32_t collect_row1, float* out, float* logits, int64_t logits_ld,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Dense verify attention that collects any set of verifier rows.
 *
 * Vegas page, Figure 6 and its text: collecting more rows costs verification
 * time through memory-bandwidth contention, which is why the method keeps two;
 * Sparse Glimpse page, "Core claim": its importance signal comes from the last
 * verification queries.  This entry point collects the rows named by a mask so
 * that both choices, and all-row collection, can be run and measured.
 *
 *  collect_mask bit i set: verifier row i is collected.  With logits != NULL it
 *               must be non-zero and name rows below n_q only (LCS_E_ARG).
 *  logits       fp32 [B][Hq][n_c][logits_ld], n_c = popcount(collect_mask):
 *               slot c holds the c-th collected row in ascending row order,
 *               columns p < prefix_len[b] written, others untouched.  NULL:
 *               nothing is collected and collect_mask is ignored.
 * Every other argument, the workspace size and the limits are those of
 * lcs_verify_attn, whose result this reproduces bit for bit for the two rows
 * 0 < n_q-1 (collect_mask = 1 | 1 << (n_q-1)).
 * ------------------------------------------------------------------------- */
lcs_status lcs_verify_attn_rows(const lcs_paged_kv* kv, const void* q, int32_t B, int32_t n_q,
                                int32_t Hq, const int32_t* prefix_len, int32_t max_prefix_len,
                                const uint64_t* tree_mask, float scale, uint64_t collect_mask,
                                float* out, float* logits, int64_t logits_ld, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Dense verify attention that writes per-KV-head partial scores of the two
 * collected rows instead of their logits.
 *
 * Vegas page, "Core claim": the selector only needs the two rows' logits summed
 * over the query heads.  Summing the G heads of each KV group inside the verify
 * epilogue writes 2G times fewer bytes than the two logit rows (Figure 6 text:
 * the collection cost is memory traffic) and leaves one row per KV head for
 * lcs_select_topk_scores.
 *
 *  scores       fp32 [B][Hkv][scores_ld], scores_ld >= max_prefix_len:
 *               scores[b][g][p] = sum over the heads h of group g, ascending, of
 *               (l[h][row0][p] + l[h][row1][p]) in fp32 as acc = acc + (pair),
 *               l the scaled logits lcs_verify_attn would write (bit for bit);
 *               columns p < prefix_len[b] written, others untouched.
 * Every other argument is that of lcs_verify_attn (logits are not written).
 * Limits: n_q * Hq/Hkv <= 48, and Hq/Hkv <= d/32 * ceil(n_q * Hq/Hkv / 16)
 * (the staging area); else LCS_E_UNSUPPORTED.
 * ------------------------------------------------------------------------- */
lcs_status lcs_verify_attn_scores(const lcs_paged_kv* kv, const void* q, int32_t B, int32_t n_q,
                                  int32_t Hq, const int32_t* prefix_len, int32_t max_prefix_len,
                                  const uint64_t* tree_mask, float scale, int32_t collect_row0,
                                  int32_t collect_row1, float* out, float* scores, int64_t scores_ld,
                                  float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Verification-guided top-k selection.
 *
 * Vegas page, "Core claim" / "What carries the argument": the two collected
 * logit rows are combined across query heads and the top-k prefix positions
 * are kept.  Sparse Glimpse page, "Core claim": sink + recent + top-ranked
 * history, per head.  SSV page: hardware-aligned blocks.
 *
 * Score of prefix position p for a set:  sigma_p = sum over the set's query
 * heads h, ascending, of (logits[b][h][0][p] + logits[b][h][1][p]), summed in
 * that fixed fp32 order (acc = acc + (row0 + row1)); -0 counts as +0.
 *   SHARED:       one set per sequence over all Hq heads.
 *   PER_KV_HEAD:  one set per (sequence, KV head g) over heads g*G .. g*G+G-1.
 *   BLOCK:        per (sequence, KV head) like PER_KV_HEAD; a block c of
 *                 block_size positions scores max(sigma_p) over its p < L.
 * Rule (L = prefix_len[b]; items are positions, or blocks in BLOCK mode):
 *   if L items <= n_sink + top_k + n_recent: keep every item;
 *   else keep the sink window, the recent window, and the top_k items of the
 *   pool between them by (score descending, index ascending).
 *   In BLOCK mode the sink window is every block holding a position < n_sink
 *   and the recent window every block meeting [L - n_recent, L).
 * Output: indices [B][n_sets][cap] int32, ascending; counts [B][n_sets].
 * Entries past counts are untouched.  cap >= min(max items, window sizes + top_k).
 * The result is bit-identical to the same rule run on the CPU over the same
 * logits with the same fp32 summation order.
 *
 *  logits       fp32 [B][Hq][2][logits_ld] as written by lcs_verify_attn.
 *  block_size   BLOCK mode only: power of two in [4, 512]; ignored otherwise.
 *  workspace    at least lcs_select_workspace_bytes(...) bytes, no initialisation.
 *               A call leaves its histograms clean and marks them with the call's
 *               layout, so that the next call on the same workspace with the same
 *               layout skips clearing them; a workspace with other contents (first
 *               use, another layout, other data) fails the mark or the item count
 *               and the call rebuilds the histograms from its keys.  Calls that share
 *               a workspace must not overlap.
 * Limits: max_prefix_len < 2^24.
 * ------------------------------------------------------------------------- */
size_t lcs_select_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, lcs_set_mode mode,
                                  int32_t max_prefix_len, int32_t block_size);

lcs_status lcs_select_topk(const float* logits, int64_t logits_ld, int32_t B, int32_t Hq,
                           int32_t Hkv, const int32_t* prefix_len, int32_t max_prefix_len,
                           lcs_set_mode mode, int32_t top_k, int32_t n_sink, int32_t n_recent,
                           int32_t block_size, int32_t* indices, int32_t* counts, int32_t cap,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Selection handed to the draft as physical cache slots.
 *
 * Vegas page, "What carries the argument": the selector's output feeds the
 * drafting phase directly.  These two calls hand the set over as physical
 * slots of the paged cache, slot = block_table[b][p / page_size] * page_size
 * + p % page_size, so that the draft reads each selected K/V row without its
 * own block-table lookup (only the tail slots still go through the table).
 *
 * lcs_select_topk_physical: lcs_select_topk for SHARED and PER_KV_HEAD sets
 * (BLOCK returns LCS_E_UNSUPPORTED) that writes, in the same ascending order of
 * positions, the physical slot of each selected position through kv's block
 * table (kv->block_table [B][max_pages]; only the table and page geometry are
 * read).  Requires max_prefix_len <= max_pages * page_size and
 * num_pages * page_size < 2^31.  Workspace, counts and errors as lcs_select_topk.
 *
 * lcs_sparse_draft_attn_physical: lcs_sparse_draft_attn for SHARED and
 * PER_KV_HEAD lists whose entries are such physical slots (the result is that
 * of lcs_sparse_draft_attn on the positions they stand for, bit for bit).
 * Workspace as lcs_sparse_workspace_bytes.  A slot whose page is outside the
 * cache is skipped.
 * ------------------------------------------------------------------------- */
lcs_status lcs_select_topk_physical(const float* logits, int64_t logits_ld, int32_t B, int32_t Hq, int32_t Hkv,
                                    const int32_t* prefix_len, int32_t max_prefix_len, lcs_set_mode mode,
                                    int32_t top_k, int32_t n_sink, int32_t n_recent, const lcs_paged_kv* kv,
                                    int32_t* indices, int32_t* counts, int32_t cap, void* workspace,
                                    size_t workspace_bytes, void* stream);

lcs_status lcs_sparse_draft_attn_physical(const lcs_paged_kv* kv, const void* q, int32_t B, int32_t n_q,
                                          int32_t Hq, lcs_set_mode mode, const int32_t* indices,
                                          const int32_t* counts, int32_t cap, const int32_t* tail_begin,
                                          const int32_t* tail_len, int32_t max_tail_len, const uint64_t* tail_mask,
                                          float scale, float* out, float* lse, void* workspace,
                                          size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Block selection with a choice of block score.
 *
 * SSV page, Figure 3 overview (NSA token selection picks hardware-aligned
 * blocks): the pages print no block score.  LCS_BLOCK_MAX is the max of the
 * block's position scores (what lcs_select_topk uses in BLOCK mode, with which
 * this call agrees bit for bit); LCS_BLOCK_LSE is their log-sum-exp,
 *   beta_c = m + log(sum over p in block c, p < L, of exp(sigma_p - m)),
 *   m = the block's max, evaluated in fp32 (expf, logf),
 * which also rewards blocks holding several strong positions.  Sets are per
 * (sequence, KV head); every other argument, the output layout, the rule and
 * the workspace (lcs_select_workspace_bytes with LCS_SET_BLOCK) are those of
 * lcs_select_topk in BLOCK mode.  LSE keys go through expf / logf, so the
 * result matches the same rule on the CPU up to their rounding.
 * ------------------------------------------------------------------------- */
lcs_status lcs_select_topk_blocks(const float* logits, int64_t logits_ld, int32_t B, int32_t Hq, int32_t Hkv,
                                  const int32_t* prefix_len, int32_t max_prefix_len, lcs_block_score block_score,
                                  int32_t top_k, int32_t n_sink, int32_t n_recent, int32_t block_size,
                                  int32_t* indices, int32_t* counts, int32_t cap, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Top-k selection from per-KV-head partial scores (lcs_verify_attn_scores).
 *
 * Rule, modes, windows, outputs and workspace (lcs_select_workspace_bytes with
 * the model's Hq) as for lcs_select_topk, with the position score
 *   SHARED:       sigma_p = sum over g ascending of scores[b][g][p] (fp32);
 *   PER_KV_HEAD,
 *   BLOCK:        sigma_p = scores[b][g][p] for the set of KV head g,
 * so PER_KV_HEAD and BLOCK select exactly what lcs_select_topk selects on the
 * logits, and SHARED sums the same terms grouped by KV head first.
 *
 *  scores       fp32 [B][Hkv][scores_ld], scores_ld >= max_prefix_len.
 * ------------------------------------------------------------------------- */
lcs_status lcs_select_topk_scores(const float* scores, int64_t scores_ld, int32_t B, int32_t Hkv,
                                  const int32_t* prefix_len, int32_t max_prefix_len,
                                  lcs_set_mode mode, int32_t top_k, int32_t n_sink, int32_t n_recent,
                                  int32_t block_size, int32_t* indices, int32_t* counts, int32_t cap,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Top-k selection over n collected rows, scored by logits or softmax weights.
 *
 * The rule, modes, windows, outputs and workspace are those of lcs_select_topk;
 * only the per-head term of sigma_p changes, for a head h with n_rows rows:
 *   LCS_SCORE_LOGIT_SUM:      t = l[h][0][p]; t = t + l[h][c][p] for c = 1..n-1
 *                             (Vegas page, "Core claim", extended to n rows).
 *   LCS_SCORE_SOFTMAX_WEIGHT: t = sum over c ascending of
 *                             expf(l[h][c][p] - lse[b][row_c][h]), row_c the
 *                             c-th set bit of rows_mask (Sparse Glimpse page,
 *                             "Core claim": post-softmax weights of the last
 *                             verification queries).
 * and sigma_p = sum over the set's heads ascending of t, in fp32.  LOGIT_SUM is
 * bit-identical to the CPU rule in the same order (n_rows = 2 gives exactly
 * lcs_select_topk); SOFTMAX_WEIGHT matches it to within expf's rounding.
 *
 *  logits       fp32 [B][Hq][n_rows][logits_ld] (lcs_verify_attn_rows layout).
 *  n_rows       1..64.
 *  lse, n_q, rows_mask  SOFTMAX_WEIGHT only (else ignored, may be NULL / 0):
 *               lse fp32 [B][n_q][Hq] as written by the verify call, natural log;
 *               rows_mask names exactly n_rows rows below n_q (LCS_E_ARG).
 * ------------------------------------------------------------------------- */
lcs_status lcs_select_topk_rows(const float* logits, int64_t logits_ld, int32_t n_rows,
                                lcs_score_kind kind, const float* lse, int32_t n_q,
                                uint64_t rows_mask, int32_t B, int32_t Hq, int32_t Hkv,
                                const int32_t* prefix_len, int32_t max_prefix_len,
                                lcs_set_mode mode, int32_t top_k, int32_t n_sink, int32_t n_recent,
                                int32_t block_size, int32_t* indices, int32_t* counts, int32_t cap,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Sparse draft attention over the selected entries plus the recent tail.
 *
 * Vegas page, "The pith": drafting attends only to the selected prefix
 * positions.  SSV page, section 4.2 and Figure 5/6 text: verifier rows with
 * different block sets share block loads (merged schedule, per-row selection
 * unchanged) and each row keeps its own causal boundary.
 *
 *  q            bf16 [B][n_q][Hq][d]; n_q = 1 for a single-token draft step,
 *               several rows for grouped (tree) verification in BLOCK mode.
 *  mode, indices, counts, cap:
 *    SHARED       indices [B][1][cap] ascending token positions, counts [B][1]
 *    PER_KV_HEAD  indices [B][Hkv][cap], counts [B][Hkv]
 *    BLOCK        indices [B][n_q][Hkv][cap] ascending block ids (block = page,
 *                 page_size % 32 == 0), counts [B][n_q][Hkv]; a block covers
 *                 positions [c*page_size, (c+1)*page_size) below tail_begin[b].
 *    Listed positions must be < tail_begin[b] and distinct.
 *  tail_begin, tail_len  device int32 [B]: every row also sees the tail slots
 *               tail_begin[b] + j, j < tail_len[b] (the tokens written since the
 *               selection, the current one included), filtered by tail_mask.
 *  max_tail_len host bound on tail_len, sizes the launch; larger tail_len values are
 *               clamped to it.
 *  tail_mask    device uint64 [B][n_q] or NULL: row i sees tail slot j iff bit j
 *               is set (needs tail_len <= 64); NULL = every row sees the whole tail.
 *  out, lse     as for lcs_verify_attn.  A row that sees nothing gets out = 0
 *               and lse = -inf.
 * Limits: n_q in [1, 64]; d in {64, 128}.
 * ------------------------------------------------------------------------- */
size_t lcs_sparse_workspace_bytes(int32_t B, int32_t n_q, int32_t Hq, const lcs_paged_kv* kv,
                                  lcs_set_mode mode, int32_t cap, int32_t max_tail_len);

lcs_status lcs_sparse_draft_attn(const lcs_paged_kv* kv, const void* q, int32_t B, int32_t n_q,
                                 int32_t Hq, lcs_set_mode mode, const int32_t* indices,
                                 const int32_t* counts, int32_t cap, const int32_t* tail_begin,
                                 const int32_t* tail_len, int32_t max_tail_len,
                                 const uint64_t* tail_mask, float scale, float* out, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * NSA sparse verification: token compression, block plan, gated three-branch
 * attention.
 *
 * SSV page, Figure 3 overview: NSA attention runs a token-compression branch,
 * a token-selection branch and a sliding-window branch for every verifier
 * query; Figure 10 caption: the grouped-query kernel runs without grouping,
 * exact or approximate; Figure 3 text: reuse layers take the nearest refresh
 * layer's index, skip index derivation and go straight into one fused kernel.
 * The pages print no formula for the branches; this library's reading:
 *  - compression: compressed block i of (b, g) covers positions
 *    [i*cmp_stride, i*cmp_stride + cmp_len) and exists once it lies wholly in
 *    the prefix; its key (value) is the bf16 mean of the block's keys (values)
 *    (NSA learns this map; the mean is the parameter-free instance);
 *  - a verifier row attends, in three separate softmaxes, to (a) every
 *    compressed block of its sequence, (b) its selected blocks (exact) or the
 *    union of its group's blocks (approximate), clipped to the prefix, plus the
 *    tail slots it sees, and (c) the last `window` prefix positions plus the
 *    tail slots it sees;
 *  - out = g_cmp*o_a + g_slc*o_b + g_win*o_c with the caller's gates; a branch
 *    that sees nothing contributes 0 and reports lse = -inf.
 *
 * lcs_nsa_compress writes the compressed cache:
 *  k_cmp, v_cmp  bf16 [B][Hkv][max_cmp][d] (caller-owned, written): rows
 *                i < floor((L - cmp_len) / cmp_stride) + 1 (L = prefix_len[b],
 *                none if L < cmp_len, at most max_cmp) hold block means, the
 *                rest zero.
 *  cmp_len power of two in [1, 1024]; cmp_stride in [1, cmp_len].
 *
 * lcs_nsa_plan derives the block index of a layer ("refresh"): the union of
 * the n_q rows' block lists of every (b, g), ascending, with the rows that
 * selected each block (group EXACT) or every row (group APPROXIMATE), into the
 * caller's plan buffer of lcs_nsa_plan_bytes(B, n_q, Hkv, cap) bytes.
 *  indices, counts  as lcs_sparse_draft_attn's BLOCK mode: [B][n_q][Hkv][cap]
 *                   ascending distinct block ids, [B][n_q][Hkv].
 *
 * lcs_nsa_attn runs the three branches and the gating in one attention kernel
 * (plus its split-K combine); a "reuse" layer calls it with the plan of the
 * refresh layer, skipping lcs_nsa_plan.
 *  q            bf16 [B][n_q][Hq][d]; row i sits at tail slot i.
 *  plan, plan_bytes, cap  the plan written by lcs_nsa_plan with the same B,
 *               n_q, Hkv and cap (block = page, page_size % 32 == 0).
 *  tail_begin   device int32 [B]: the prefix length L (tail slot j is position
 *               L + j); tail_len [B] <= max_tail_len; tail_mask [B][n_q] or NULL
 *               as in lcs_sparse_draft_attn.
 *  gates        fp32 [B][n_q][Hq][3] (compression, selection, window).
 *  out          fp32 [B][n_q][Hq][d]; lse fp32 [B][n_q][Hq][3] per branch, or NULL.
 *  workspace    lcs_nsa_workspace_bytes(...) bytes (split-K partials), no init.
 * Limits: n_q in [1, 64]; d in {64, 128}; B*Hkv*max_cmp < 2^31.  Errors as for
 * the other calls (host checks, nothing launched on failure).
 * ------------------------------------------------------------------------- */
lcs_status lcs_nsa_compress(const lcs_paged_kv* kv, int32_t B, const int32_t* prefix_len, int32_t max_prefix_len,
                            int32_t cmp_len, int32_t cmp_stride, void* k_cmp, void* v_cmp, int32_t max_cmp,
                            void* stream);

size_t lcs_nsa_plan_bytes(int32_t B, int32_t n_q, int32_t Hkv, int32_t cap);

lcs_status lcs_nsa_plan(const lcs_paged_kv* kv, int32_t B, int32_t n_q, const int32_t* indices,
                        const int32_t* counts, int32_t cap, lcs_group_mode group, void* plan, size_t plan_bytes,
                        void* stream);

size_t lcs_nsa_workspace_bytes(int32_t B, int32_t n_q, int32_t Hq, const lcs_paged_kv* kv, int32_t cap,
                               int32_t max_tail_len, int32_t max_cmp, int32_t window);

lcs_status lcs_nsa_attn(const lcs_paged_kv* kv, const void* k_cmp, const void* v_cmp, int32_t max_cmp,
                        int32_t cmp_len, int32_t cmp_stride, int32_t window, const void* q, int32_t B, int32_t n_q,
                        int32_t Hq, const void* plan, size_t plan_bytes, int32_t cap, const int32_t* tail_begin,
                        const int32_t* tail_len, int32_t max_tail_len, const uint64_t* tail_mask,
                        const float* gates, float scale, float* out, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * lcs_sparse_draft_attn without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.
 *
 * Arguments, outputs, limits and results are those of lcs_sparse_draft_attn
 * (the same kernels run; outputs are bit-identical).  The split-K partials and
 * the block-union plan go to a static device array of the library, 32 MiB per
 * GPU, held from the first such call on a device until the process ends; the
 * call itself allocates and frees nothing.  A call whose workspace need
 * (lcs_sparse_workspace_bytes) exceeds 32 MiB returns LCS_E_WORKSPACE and
 * launches nothing.  Every call on one GPU uses that GPU's one array: calls
 * that overlap on a GPU (concurrent streams, threads) race and give undefined
 * results; calls ordered on one stream are safe.  Nothing in the array needs
 * to start at zero (every byte a call reads was written earlier in that call).
 * ------------------------------------------------------------------------- */
lcs_status lcs_sparse_draft_attn_noalloc(const lcs_paged_kv* kv, const void* q, int32_t B, int32_t n_q,
                                         int32_t Hq, lcs_set_mode mode, const int32_t* indices,
                                         const int32_t* counts, int32_t cap, const int32_t* tail_begin,
                                         const int32_t* tail_len, int32_t max_tail_len,
                                         const uint64_t* tail_mask, float scale, float* out, float* lse,
                                         void* stream);

/* Thread-local description of the last non-OK status returned on this thread. */
const char* lcs_last_error(void);

/* Library version string ("lcs <major>.<minor> gfx950"). */
const char* lcs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LCS_H */
