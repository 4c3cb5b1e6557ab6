/* Host-side checks of libcsa2 under AddressSanitizer (host code only).
 *
 * Every call below is decided by the library's host code before any device
 * work: workspace sizing over a grid of shapes, and argument validation that
 * must fail (NULL pointers, bad dimensions, bad query batches, bad page
 * descriptors, bad flags, short workspaces).  The pointers passed are never
 * dereferenced by the library (they fail validation first), so nothing here
 * needs a GPU.  Exit status 0: every status was the documented one.
 * Built and run by tests/test_host_asan.py. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../include/csa2.h"

static int failures = 0;

static void expect(csa2_status got, csa2_status want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d (%s), expected %d; last error: %s\n", what, (int)got,
            csa2_status_string(got), (int)want, csa2_last_error());
    ++failures;
  }
}

static csa2_dims dims(int h, int hi, int di, int p, int k, int w, int g) {
  csa2_dims d;
  d.n_heads = h; d.d_latent = 512; d.d_rope = 64; d.idx_heads = hi; d.idx_dim = di;
  d.block = 8; d.pool_blocks = p; d.topk = k; d.swa = w; d.kv_group = g;
  return d;
}

#define FAKE(x) ((void*)(uintptr_t)(x))

int main(void) {
  static int64_t seq_base[4096];
  static int32_t n_visible[4096];
  csa2_queries q;
  memset(&q, 0, sizeof q);
  q.seq_base = seq_base;
  q.n_visible = n_visible;

  if (csa2_abi_version() != CSA2_ABI_VERSION) { fprintf(stderr, "abi version\n"); ++failures; }
  for (int s = -1; s <= 5; ++s)
    if (!csa2_status_string((csa2_status)s)) { fprintf(stderr, "status string %d\n", s); ++failures; }

  /* workspace sizing over a grid of shapes: every query succeeds, and the
   * Full workspace holds the pool workspace */
  const int heads[] = {16, 64, 128};
  const int nqs[] = {1, 3, 8, 64, 256, 4096};
  const int vis[] = {0, 1, 128, 129, 4096, 131072, 1048576, 2097152};
  const int tps[] = {1, 4, 64};
  for (int a = 0; a < 3; ++a)
    for (int b = 0; b < 6; ++b)
      for (int c = 0; c < 8; ++c)
        for (int t = 0; t < 3; ++t) {
          if (nqs[b] % tps[t]) continue;
          csa2_dims d = dims(heads[a], 64, 128, 2048, 512, 128, 16);
          q.n_q = nqs[b]; q.tokens_per_seq = tps[t]; q.max_visible = vis[c];
          size_t full = 0, pool = 0, re = 0, att = 0, step = 0;
          expect(csa2_index_full_workspace_size(&d, &q, &full), CSA2_OK, "full ws");
          expect(csa2_index_pool_workspace_size(&d, &q, &pool), CSA2_OK, "pool ws");
          expect(csa2_index_reindex_workspace_size(&d, &q, &re), CSA2_OK, "reindex ws");
          expect(csa2_attend_workspace_size(&d, &q, &att), CSA2_OK, "attend ws");
          expect(csa2_decode_step_workspace_size(&d, &q, &step), CSA2_OK, "step ws");
          if (full < pool || step < full + re) { fprintf(stderr, "workspace sizes inconsistent\n"); ++failures; }
        }

  /* bad dimensions */
  q.n_q = 8; q.tokens_per_seq = 1; q.max_visible = 131072;
  const csa2_dims bad[] = {dims(20, 64, 128, 2048, 512, 128, 16), dims(16, 0, 128, 2048, 512, 128, 16),
                           dims(16, 65, 128, 2048, 512, 128, 16), dims(16, 64, 96, 2048, 512, 128, 16),
                           dims(16, 64, 128, 0, 512, 128, 16), dims(16, 64, 128, 4096, 512, 128, 16),
                           dims(16, 64, 128, 8, 65, 128, 16), dims(16, 64, 128, 2048, 512, 2048, 16),
                           dims(16, 64, 128, 2048, 512, 128, 8)};
  for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
    size_t n = 0;
    expect(csa2_index_full_workspace_size(&bad[i], &q, &n), CSA2_ERR_INVALID_ARG, "bad dims");
  }
  /* bad query batches */
  csa2_dims d = dims(64, 64, 128, 2048, 512, 128, 16);
  {
    size_t n = 0;
    csa2_queries b = q;
    b.n_q = 0; expect(csa2_index_full_workspace_size(&d, &b, &n), CSA2_ERR_INVALID_ARG, "n_q 0");
    b = q; b.tokens_per_seq = 3; expect(csa2_index_full_workspace_size(&d, &b, &n), CSA2_ERR_INVALID_ARG, "tokens");
    b = q; b.max_visible = -1; expect(csa2_index_full_workspace_size(&d, &b, &n), CSA2_ERR_INVALID_ARG, "max_visible");
    b = q; b.reserved = 1; expect(csa2_index_full_workspace_size(&d, &b, &n), CSA2_ERR_INVALID_ARG, "reserved");
    b = q; b.seq_base = NULL; expect(csa2_index_full_workspace_size(&d, &b, &n), CSA2_ERR_INVALID_ARG, "seq_base");
    expect(csa2_index_full_workspace_size(&d, &q, NULL), CSA2_ERR_INVALID_ARG, "bytes NULL");
  }

  /* NULL pointers, flags and short workspaces */
  expect(csa2_index_scan(&d, &q, NULL, NULL, NULL, NULL, 0, NULL, 0, NULL), CSA2_ERR_INVALID_ARG, "scan NULL");
  expect(csa2_index_full(&d, &q, FAKE(0x1000), FAKE(0x2000), FAKE(0x3000), FAKE(0x4000), FAKE(0x5000), NULL, 0,
                         NULL, 0, NULL), CSA2_ERR_WORKSPACE, "full without workspace");
  expect(csa2_index_pool(&d, &q, FAKE(0x1000), 16384, FAKE(0x2000), FAKE(0x3000), FAKE(0x4000), (size_t)1 << 30,
                         2, NULL), CSA2_ERR_INVALID_ARG, "pool flags");
  expect(csa2_index_reindex(&d, &q, FAKE(0x1000), FAKE(0x2000), FAKE(0x3000), NULL, FAKE(0x5000), FAKE(0x6000),
                            FAKE(0x7000), NULL, FAKE(0x8000), (size_t)1 << 30, NULL), CSA2_ERR_INVALID_ARG,
         "reindex NULL pool");
  expect(csa2_attend(&d, &q, NULL, NULL, 1.0f, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL),
         CSA2_ERR_INVALID_ARG, "attend NULL");
  expect(csa2_encode_kv(-1, NULL, NULL, NULL, NULL, NULL, NULL, NULL), CSA2_ERR_INVALID_ARG, "encode n < 0");
  expect(csa2_encode_fp4(4, 48, FAKE(0x1000), NULL, FAKE(0x2000), FAKE(0x3000), NULL), CSA2_ERR_INVALID_ARG,
         "encode_fp4 width");
  expect(csa2_decode_step(&d, &q, 7, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1.0f, NULL,
                          NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), CSA2_ERR_INVALID_ARG, "step mode");

  /* page descriptors */
  const csa2_pages badp[] = {{NULL, 64, 0, 1024}, {(const int32_t*)FAKE(0x1000), 48, 0, 1024},
                             {(const int32_t*)FAKE(0x1000), 8, 0, 1024},
                             {(const int32_t*)FAKE(0x1000), 1 << 17, 0, 1 << 17},
                             {(const int32_t*)FAKE(0x1000), 64, 1, 1024}, {(const int32_t*)FAKE(0x1000), 64, 0, 1000},
                             {(const int32_t*)FAKE(0x1000), 64, 0, 0}, {(const int32_t*)FAKE(0x1000), 64, 0, 1 << 24}};
  for (size_t i = 0; i < sizeof badp / sizeof badp[0]; ++i) {
    expect(csa2_attend_paged(&d, &q, &badp[i], FAKE(0x1000), FAKE(0x2000), 1.0f, FAKE(0x3000), FAKE(0x4000),
                             FAKE(0x5000), FAKE(0x6000), FAKE(0x7000), FAKE(0x8000), FAKE(0x9000), FAKE(0xA000),
                             NULL, FAKE(0xB000), (size_t)1 << 30, NULL), CSA2_ERR_INVALID_ARG, "attend pages");
    if (i + 1 < sizeof badp / sizeof badp[0])   /* (2^24 rows are too many only for 256-byte rows) */
      expect(csa2_page_rows(&badp[i], 4, FAKE(0x1000), FAKE(0x2000), FAKE(0x3000), NULL), CSA2_ERR_INVALID_ARG,
             "page rows pages");
  }
  const csa2_pages okp = {(const int32_t*)FAKE(0x1000), 64, 0, 1024};
  expect(csa2_page_rows(&okp, -1, NULL, NULL, NULL, NULL), CSA2_ERR_INVALID_ARG, "page rows n");
  expect(csa2_index_full_paged(&d, &q, NULL, FAKE(0x1000), NULL, FAKE(0x2000), FAKE(0x3000), NULL, FAKE(0x4000),
                               FAKE(0x5000), NULL, 0, FAKE(0x6000), (size_t)1 << 30, NULL), CSA2_ERR_INVALID_ARG,
         "full paged NULL pages");
  expect(csa2_index_reindex_paged(&d, &q, &okp, FAKE(0x1000), FAKE(0x2000), FAKE(0x3000), FAKE(0x4000), NULL,
                                  FAKE(0x5000), FAKE(0x6000), FAKE(0x7000), FAKE(0x8000), NULL, FAKE(0x9000),
                                  (size_t)1 << 30, NULL), CSA2_ERR_INVALID_ARG, "reindex paged half FP4");

  if (failures) {
    fprintf(stderr, "%d host checks failed\n", failures);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
