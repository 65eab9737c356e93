/* Host-side memory and undefined-behaviour check of libqsa's C ABI: the
 * geometry validation, token widths, workspace sizes (including the
 * decode split layout) and every entry
 * point's argument checks, run in a build whose host code carries
 * AddressSanitizer and UndefinedBehaviorSanitizer.  Every call here is
 * decided on the host before any HIP call, so no GPU is needed; any report
 * aborts with a nonzero status.  Compiled and run by
 * tests/test_lib_host_sanitized.py. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "qsa.h"

static int failures = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      printf("FAILED line %d: %s\n", __LINE__, #cond);                \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static qsa_geometry geom(int hq, int hkv, int k, int kv, int indexer_mqa) {
  qsa_geometry g;
  g.num_q_heads = hq;
  g.num_kv_heads = hkv;
  g.head_dim = 256;
  g.page_size = 64;
  g.compress_ratio = 4;
  g.idx_heads = indexer_mqa ? 4 : 8;
  g.idx_dim = indexer_mqa ? 128 : 64;
  g.topk_groups = k;
  g.kv_dtype = kv;
  g.sm_scale = 0.0f;
  g.k_scale = 1.0f;
  g.v_scale = 1.0f;
  g.idx_key_heads = indexer_mqa ? 1 : 8;
  return g;
}

int main(void) {
  /* validation over a sweep of fields, valid and not */
  const int hqs[] = {1, 3, 6, 12, 16, 24, 32, 48, 0, -4};
  const int hkvs[] = {1, 2, 3, 4, 0, -1};
  const int ks[] = {-1, 0, 1, 7, 512, 1024, 2048, 2049, 1 << 30};
  int n_ok = 0;
  for (unsigned a = 0; a < sizeof hqs / sizeof *hqs; ++a)
    for (unsigned b = 0; b < sizeof hkvs / sizeof *hkvs; ++b)
      for (unsigned c = 0; c < sizeof ks / sizeof *ks; ++c)
        for (int kv = -1; kv <= 2; ++kv)
          for (int mqa = 0; mqa <= 1; ++mqa) {
            qsa_geometry g = geom(hqs[a], hkvs[b], ks[c], kv, mqa);
            const qsa_status st = qsa_validate(&g);
            EXPECT(st == QSA_OK || st == QSA_ERR_UNSUPPORTED);
            if (st != QSA_OK) {
              EXPECT(qsa_token_width(&g, 1) == 0);
              EXPECT(qsa_decode_workspace_size(&g, 8, 1, 262144) == 0);
              continue;
            }
            ++n_ok;
            for (int q = 0; q <= 5; ++q) (void)qsa_token_width(&g, q);
            /* sizes at the edges: empty, tiny, full capacity, past it */
            const int ctxs[] = {-7, 0, 1, 3, 4, 63, 64, 65, 8193, 65536, 65540, 262144, 262145};
            for (unsigned i = 0; i < sizeof ctxs / sizeof *ctxs; ++i) {
              const int ctx = ctxs[i];
              const size_t a1 = qsa_index_topk_workspace_size(&g, 3, ctx);
              const size_t a2 = qsa_prefill_workspace_size(&g, 4096, ctx);
              const size_t a3 = qsa_prefill_workspace_size(&g, 0, ctx);
              const size_t a4 = qsa_decode_workspace_size(&g, 8, 1, ctx);
              const size_t a5 = qsa_decode_workspace_size(&g, 4, 3, ctx);
              const int bad = ctx < 1 || ctx > 262144;
              EXPECT(!bad || (a1 == 0 && a2 == 0 && a3 == 0 && a4 == 0 && a5 == 0));
              EXPECT(bad || (a1 % 256 == 0 && a2 % 256 == 0 && a4 % 256 == 0));
            }
            EXPECT(qsa_prefill_workspace_size(&g, -1, 1000) == 0);
            EXPECT(qsa_decode_workspace_size(&g, -1, 1, 1000) == 0);
          }
  EXPECT(n_ok > 0);
  EXPECT(qsa_validate(NULL) == QSA_ERR_INVALID_ARG);
  for (int s = -6; s <= 1; ++s) EXPECT(qsa_status_string((qsa_status)s) != NULL);
  for (int n = -3; n <= 4100; n += 7) EXPECT(qsa_append_khat_slots(n) == (n > 0 ? (n + 3) / 4 : 0));

  /* entry points: refusals decided on the host before any HIP call */
  qsa_geometry g = geom(16, 2, 512, QSA_KV_FP8_E4M3, 0);
  g.k_scale = g.v_scale = 0.5f;
  int32_t* fake = (int32_t*)(uintptr_t)0x1000; /* never dereferenced */
  qsa_paged_cache c = {fake, fake, (const float*)fake, fake, 64, 64};
  qsa_paged_cache nulls = {NULL, NULL, NULL, NULL, 0, 0};
  EXPECT(qsa_decode(&g, &nulls, 1, 1, 100, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                    0, NULL) == QSA_ERR_INVALID_ARG);
  EXPECT(qsa_decode(&g, &c, 0, 1, 256, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                    NULL) == QSA_OK);
  EXPECT(qsa_decode(&g, &c, 1, 5, 256, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                    NULL) == QSA_ERR_INVALID_ARG);
  EXPECT(qsa_decode(&g, &c, 1, 1, 64 * 64 + 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                    NULL, 0, NULL) == QSA_ERR_INVALID_ARG);
  EXPECT(qsa_decode(&g, &c, 2, 1, 256, fake, (const float*)fake, (const float*)fake,
                    (const uint16_t*)fake, (float*)fake, NULL, NULL, NULL, NULL, 0,
                    NULL) == QSA_ERR_WORKSPACE);
  EXPECT(qsa_decode(&g, &c, 2, 1, 256, fake, (const float*)fake, (const float*)fake,
                    (const uint16_t*)fake, (float*)fake, NULL, NULL, NULL, (void*)0x1001,
                    1u << 30, NULL) == QSA_ERR_WORKSPACE); /* misaligned */
  EXPECT(qsa_prefill(&g, &c, 0, 100, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                     NULL) == QSA_OK);
  EXPECT(qsa_prefill(&g, &c, 0, 4000, 200, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                     NULL) == QSA_ERR_INVALID_ARG); /* past the page table */
  EXPECT(qsa_prefill(&g, &c, -1, 0, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                     NULL) == QSA_ERR_INVALID_ARG);
  EXPECT(qsa_prefill(&g, &c, 0, 10, 20, (const float*)fake, (const float*)fake,
                     (const uint16_t*)fake, (float*)fake, NULL, NULL, NULL, NULL, 0,
                     NULL) == QSA_ERR_WORKSPACE);
  EXPECT(qsa_index_topk(&g, &c, 0, 256, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
         QSA_OK);
  EXPECT(qsa_index_topk(&g, &c, 1, 256, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
         QSA_ERR_INVALID_ARG);
  EXPECT(qsa_index_score(&g, &c, 0, 256, NULL, NULL, NULL, NULL, NULL, NULL) == QSA_OK);
  EXPECT(qsa_index_score(&g, &c, 2, 0, NULL, NULL, NULL, NULL, NULL, NULL) ==
         QSA_ERR_INVALID_ARG);
  EXPECT(qsa_index_score_prefill(&g, &c, 0, 100, 0, NULL, NULL, NULL, NULL) == QSA_OK);
  EXPECT(qsa_index_score_prefill(&g, &c, 0, 262144, 1, NULL, NULL, NULL, NULL) ==
         QSA_ERR_INVALID_ARG);
  EXPECT(qsa_append_kv(&g, NULL, NULL, NULL, NULL, 4, 4, 1, NULL, NULL, 3, NULL, NULL, NULL,
                       NULL) == QSA_ERR_INVALID_ARG);
  EXPECT(qsa_append_kv(&g, NULL, NULL, NULL, NULL, 4, 4, 0, NULL, NULL, 3, NULL, NULL, NULL,
                       NULL) == QSA_OK);
  /* the allocation-free decode: argument checks, the size limit, batch 0 */
  EXPECT(qsa_decode_noalloc(&g, &nulls, 1, 1, 100, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                            NULL, NULL) == QSA_ERR_INVALID_ARG);
  qsa_paged_cache big = {fake, fake, (const float*)fake, fake, 4096, 4096};
  qsa_geometry g2 = geom(16, 2, 2048, QSA_KV_FP8_E4M3, 0);
  EXPECT(qsa_decode_noalloc(&g2, &big, 256, 1, 262144, fake, (const float*)fake,
                            (const float*)fake, (const uint16_t*)fake, (float*)fake, NULL, NULL,
                            NULL, NULL) == QSA_ERR_TOO_LARGE);
  EXPECT(qsa_decode_noalloc(&g2, &big, 0, 1, 262144, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                            NULL, NULL) == QSA_OK);
  EXPECT(qsa_noalloc_scratch_bytes() == QSA_NOALLOC_SCRATCH_BYTES);
  qsa_geometry bad = geom(16, 2, 512, 7, 0);
  EXPECT(qsa_prefill(&bad, &c, 0, 0, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                     NULL) == QSA_ERR_UNSUPPORTED);
  if (failures) {
    printf("%d failures\n", failures);
    return 1;
  }
  printf("library host code sanitized run: ok (%d supported geometries)\n", n_ok);
  return 0;
}
