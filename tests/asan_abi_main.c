/* Drives every host-side error path and workspace query of the C ABI from plain C, for
 * a host build instrumented with AddressSanitizer.  No call reaches a launch: each one
 * is rejected (or is an empty batch) before anything touches a device. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lcs.h"

static int fails = 0;
#define EXPECT(call, status)                                                        \
  do {                                                                              \
    lcs_status st_ = (call);                                                        \
    if (st_ != (status)) {                                                          \
      printf("line %d: got %d want %d (%s)\n", __LINE__, (int)st_, (int)(status),  \
             lcs_last_error());                                                     \
      ++fails;                                                                      \
    }                                                                               \
    if (st_ != LCS_OK && strlen(lcs_last_error()) == 0) ++fails;                    \
  } while (0)

#define P(x) ((void*)(uintptr_t)(x))

int main(void) {
  lcs_paged_kv kv = {P(0x1000), P(0x2000), (const int32_t*)P(0x3000), 10, 16, 4, 2, 128};
  lcs_paged_kv bad_d = kv, bad_page = kv, big = kv;
  bad_d.d = 96;
  bad_page.page_size = 12;
  big.max_pages = 64;
  big.num_pages = 200;
  const int32_t* pl = (const int32_t*)P(0x5000);
  float* out = (float*)P(0x6000);
  float* lg = (float*)P(0x7000);
  void* ws = P(0x8000);

  /* verify */
  EXPECT(lcs_verify_attn(&bad_d, P(0x4000), 1, 5, 4, pl, 40, 0, 0.1f, 0, 4, out, lg, 40, 0, ws, 1 << 20, 0),
         LCS_E_UNSUPPORTED);
  EXPECT(lcs_verify_attn(&bad_page, P(0x4000), 1, 5, 4, pl, 40, 0, 0.1f, 0, 4, out, lg, 40, 0, ws, 1 << 20, 0),
         LCS_E_UNSUPPORTED);
  EXPECT(lcs_verify_attn(0, P(0x4000), 1, 5, 4, pl, 40, 0, 0.1f, 0, 4, out, lg, 40, 0, ws, 1 << 20, 0), LCS_E_ARG);
  EXPECT(lcs_verify_attn(&kv, P(0x4000), 1, 5, 3, pl, 40, 0, 0.1f, 0, 4, out, lg, 40, 0, ws, 1 << 20, 0),
         LCS_E_SHAPE);
  EXPECT(lcs_verify_attn(&kv, P(0x4000), 1, 65, 4, pl, 40, 0, 0.1f, 0, 4, out, lg, 40, 0, ws, 1 << 20, 0),
         LCS_E_UNSUPPORTED);
  EXPECT(lcs_verify_attn(&kv, 0, 1, 5, 4, pl, 40, 0, 0.1f, 0, 4, out, lg, 40, 0, ws, 1 << 20, 0), LCS_E_ARG);
  EXPECT(lcs_verify_attn(&kv, P(0x4000), 1, 5, 4, pl, 40, 0, 0.1f, 0, 9, out, lg, 40, 0, ws, 1 << 20, 0),
         LCS_E_ARG);
  EXPECT(lcs_verify_attn(&kv, P(0x4000), 1, 5, 4, pl, 40, 0, 0.1f, 0, 4, out, lg, 39, 0, ws, 1 << 20, 0),
         LCS_E_SHAPE);
  EXPECT(lcs_verify_attn(&kv, P(0x4000), 1, 5, 4, pl, 40, 0, 0.1f, 0, 4, out, lg, 40, 0, ws, 0, 0),
         LCS_E_WORKSPACE);
  EXPECT(lcs_verify_attn(&kv, 0, 0, 5, 4, 0, 40, 0, 0.1f, 0, 4, 0, 0, 40, 0, 0, 0, 0), LCS_OK);
  EXPECT(lcs_verify_attn_rows(&kv, P(0x4000), 1, 5, 4, pl, 40, 0, 0.1f, 0, out, lg, 40, 0, ws, 1 << 20, 0),
         LCS_E_ARG);
  EXPECT(lcs_verify_attn_rows(&kv, P(0x4000), 1, 5, 4, pl, 40, 0, 0.1f, 0xFFFFFFFFFFFFFFFFull, out, lg, 40, 0,
                              ws, 1 << 20, 0),
         LCS_E_ARG);
  EXPECT(lcs_verify_attn_scores(&kv, P(0x4000), 1, 5, 4, pl, 40, 0, 0.1f, 0, 4, out, 0, 40, 0, ws, 1 << 20, 0),
         LCS_E_ARG);
  EXPECT(lcs_verify_attn_scores(&big, P(0x4000), 1, 13, 8, pl, 40, 0, 0.1f, 0, 12, out, lg, 40, 0, ws, 1 << 20,
                                0),
         LCS_E_UNSUPPORTED);

  /* select */
  int32_t* idx = (int32_t*)P(0x3000);
  int32_t* cnt = (int32_t*)P(0x4000);
  EXPECT(lcs_select_topk(lg, 100, 1, 4, 2, pl, 100, (lcs_set_mode)7, 10, 4, 8, 0, idx, cnt, 22, ws, 1 << 24, 0),
         LCS_E_ARG);
  EXPECT(lcs_select_topk(0, 100, 1, 4, 2, pl, 100, LCS_SET_SHARED, 10, 4, 8, 0, idx, cnt, 22, ws, 1 << 24, 0),
         LCS_E_ARG);
  EXPECT(lcs_select_topk(lg, 100, 1, 5, 2, pl, 100, LCS_SET_SHARED, 10, 4, 8, 0, idx, cnt, 22, ws, 1 << 24, 0),
         LCS_E_SHAPE);
  EXPECT(lcs_select_topk(lg, 100, 1, 4, 2, pl, 100, LCS_SET_SHARED, 10, 4, 8, 0, idx, cnt, 21, ws, 1 << 24, 0),
         LCS_E_SHAPE);
  EXPECT(lcs_select_topk(lg, 100, 1, 4, 2, pl, 100, LCS_SET_BLOCK, 10, 4, 8, 12, idx, cnt, 22, ws, 1 << 24, 0),
         LCS_E_UNSUPPORTED);
  EXPECT(lcs_select_topk(lg, 100, 1, 4, 2, pl, 100, LCS_SET_SHARED, 10, 4, 8, 0, idx, cnt, 22, ws, 10, 0),
         LCS_E_WORKSPACE);
  EXPECT(lcs_select_topk_rows(lg, 100, 0, LCS_SCORE_LOGIT_SUM, 0, 0, 0, 1, 4, 2, pl, 100, LCS_SET_SHARED, 10, 4,
                              8, 0, idx, cnt, 22, ws, 1 << 24, 0),
         LCS_E_ARG);
  EXPECT(lcs_select_topk_rows(lg, 100, 3, LCS_SCORE_SOFTMAX_WEIGHT, out, 9, 0x3, 1, 4, 2, pl, 100,
                              LCS_SET_SHARED, 10, 4, 8, 0, idx, cnt, 22, ws, 1 << 24, 0),
         LCS_E_ARG);
  EXPECT(lcs_select_topk_scores(0, 100, 1, 2, pl, 100, LCS_SET_SHARED, 10, 4, 8, 0, idx, cnt, 22, ws, 1 << 24, 0),
         LCS_E_ARG);
  EXPECT(lcs_select_topk(0, 100, 0, 4, 2, 0, 100, LCS_SET_SHARED, 10, 4, 8, 0, 0, 0, 22, 0, 0, 0), LCS_OK);

  /* sparse draft */
  EXPECT(lcs_sparse_draft_attn(&kv, P(0x1000), 1, 1, 4, (lcs_set_mode)3, idx, cnt, 10, pl, pl, 4, 0, 0.1f, out,
                               0, ws, 1 << 24, 0),
         LCS_E_ARG);
  EXPECT(lcs_sparse_draft_attn(&kv, P(0x1000), 1, 65, 4, LCS_SET_SHARED, idx, cnt, 10, pl, pl, 4, 0, 0.1f, out,
                               0, ws, 1 << 24, 0),
         LCS_E_UNSUPPORTED);
  EXPECT(lcs_sparse_draft_attn(&kv, P(0x1000), 1, 1, 4, LCS_SET_SHARED, idx, cnt, 100000, pl, pl, 100, 0, 0.1f,
                               out, 0, ws, 0, 0),
         LCS_E_WORKSPACE);
  EXPECT(lcs_sparse_draft_attn(&kv, P(0x1000), 0, 1, 4, LCS_SET_SHARED, idx, cnt, 10, pl, pl, 4, 0, 0.1f, out, 0,
                               ws, 1 << 24, 0),
         LCS_OK);

  /* workspace queries and identification */
  if (lcs_verify_workspace_bytes(1, 9, 32, &kv, 32768) == 0) ++fails;
  if (lcs_verify_workspace_bytes(1, 9, 33, &kv, 32768) != 0) ++fails;
  if (lcs_select_workspace_bytes(1, 4, 2, LCS_SET_SHARED, 100, 0) == 0) ++fails;
  if (lcs_sparse_workspace_bytes(1, 1, 4, &kv, LCS_SET_SHARED, 10, 4) == 0) ++fails;
  /* sparse draft without a workspace: argument checks and the scratch-size refusal */
  EXPECT(lcs_sparse_draft_attn_noalloc(0, P(0x1000), 1, 1, 4, LCS_SET_SHARED, idx, cnt, 10, pl, pl, 4, 0, 0.1f,
                                       out, 0, 0),
         LCS_E_ARG);
  EXPECT(lcs_sparse_draft_attn_noalloc(&kv, P(0x1000), 0, 1, 4, LCS_SET_SHARED, idx, cnt, 10, pl, pl, 4, 0, 0.1f,
                                       out, 0, 0),
         LCS_OK);
  {
    lcs_paged_kv big = kv;
    big.page_size = 64;
    EXPECT(lcs_sparse_draft_attn_noalloc(&big, P(0x1000), 4, 64, 4, LCS_SET_BLOCK, idx, cnt, 100000, pl, pl, 4, 0,
                                         0.1f, out, 0, 0),
           LCS_E_WORKSPACE);
  }
  if (strncmp(lcs_version(), "lcs ", 4) != 0) ++fails;
  printf("%d failures\n", fails);
  return fails != 0;
}
