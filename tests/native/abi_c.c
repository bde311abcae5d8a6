/* The C ABI used from plain C99 (no C++ and no Python): the host-side calls of
 * libpkv.so -- version and status strings, shape checks and workspace sizes,
 * the split plan and the shared-prefix helper, the page allocator. Built and
 * run by tests/test_abi_c.py; exit status 0 when every check holds. No GPU
 * call is made. */
#include <stdio.h>
#include <string.h>

#include "pkv.h"

#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      return 1;                                                  \
    }                                                            \
  } while (0)

int main(void) {
  CHECK(pkv_version() > 0);
  CHECK(strlen(pkv_status_string(PKV_ERR_SHAPE)) > 0);

  /* the verify workload: 8 sequences x 8192 tokens, window 6, 32/8 heads */
  pkv_attn_shape s;
  memset(&s, 0, sizeof s);
  s.num_seqs = 8;
  s.num_q_heads = 32;
  s.num_kv_heads = 8;
  s.head_dim = 128;
  s.page_size = PKV_PAGE_SIZE;
  s.num_pages = 256;
  s.max_pages_per_seq = 32;
  s.total_q = 48;
  s.max_q_len = 6;
  s.scale = 0.08838835f;
  CHECK(pkv_attn_workspace_bytes(&s) > 0);
  int32_t lens[8];
  for (int b = 0; b < 8; ++b) lens[b] = 8192;
  CHECK(pkv_attn_plan(&s, lens) == PKV_OK);
  CHECK(s.total_pages == 256 && s.pages_per_split == 8);

  pkv_attn_shape bad = s;
  bad.head_dim = 96;
  CHECK(pkv_attn_workspace_bytes(&bad) == 0);
  CHECK(pkv_attn_plan(&bad, lens) == PKV_ERR_SHAPE);

  /* two sequences whose tables share their first page */
  pkv_attn_shape t = s;
  t.num_seqs = 2;
  t.max_pages_per_seq = 3;
  t.total_q = 2;
  t.max_q_len = 1;
  t.total_pages = 0;
  t.pages_per_split = 0;
  const int32_t table[6] = {4, 9, 1, 4, 7, -1};
  const int32_t tl[2] = {700, 400}, tq[2] = {1, 1};
  CHECK(pkv_shared_prefix_pages(table, tl, tq, &t) == 1);
  CHECK(pkv_attn_shared_workspace_bytes(&t, 1) > 0);

  /* accept shape: 8 sequences x 6 rows over 128256 logits */
  pkv_accept_shape a = {8, 128256, 48, 5};
  CHECK(pkv_accept_workspace_bytes(&a) > 0);
  CHECK(pkv_window_next(5, 5, 6) == 7 && pkv_window_next(5, 5, 2) == 4);

  /* the allocator: a prompt, then a second sharing its first page */
  pkv_pool* pool = pkv_pool_create(8);
  CHECK(pool != NULL);
  int32_t toks[600];
  for (int i = 0; i < 600; ++i) toks[i] = i;
  int32_t pages[3], n = 0, cached = 0;
  CHECK(pkv_pool_admit(pool, toks, 600, pages, 3, &n, &cached) == PKV_OK && n == 3 && cached == 0);
  int32_t pages2[2];
  CHECK(pkv_pool_admit(pool, toks, 300, pages2, 2, &n, &cached) == PKV_OK && n == 2 && cached == 256);
  CHECK(pages2[0] == pages[0]);
  int32_t st[4];
  CHECK(pkv_pool_stats(pool, st) == PKV_OK);
  CHECK(pkv_pool_release(pool, pages, 3) == PKV_OK && pkv_pool_release(pool, pages2, 2) == PKV_OK);
  pkv_pool_destroy(pool);
  printf("ok\n");
  return 0;
}
