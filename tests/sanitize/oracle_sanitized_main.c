/* Host-side memory and undefined-behaviour check of the oracle: every entry
 * point of oracle/qsa_oracle.c runs on small synthetic inputs (ragged
 * lengths, out-of-range page ids, ties, empty selections, appends at
 * negative and past-the-table positions) in a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer; any report aborts with a nonzero status.
 * Compiled and run by tests/test_oracle_sanitized.py. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/qsa_oracle.c"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
  state ^= state << 13; state ^= state >> 7; state ^= state << 17;
  return (uint32_t)(state >> 11);
}
static float uniform(void) { return (float)(next_u32() & 0xFFFFFF) / 16777216.0f * 2.0f - 1.0f; }

int main(void) {
  enum { P = 24, PAGE = 64, RATIO = 4, GPP = 16, HI = 8, DI = 64, HKV = 2, D = 256, HQ = 16 };
  enum { max_pages = 12, n_rows = 3 };
  int32_t pt[n_rows * max_pages];
  for (int i = 0; i < n_rows * max_pages; ++i) pt[i] = (int32_t)(i % P);
  pt[5] = P + 3;  /* out of range */
  pt[13] = -1;
  float* khat = malloc(sizeof(float) * P * GPP * HI * DI);
  for (int i = 0; i < P * GPP * HI * DI; ++i) khat[i] = uniform();
  float q_idx[n_rows * HI * DI], w_idx[n_rows * HI];
  for (int i = 0; i < n_rows * HI * DI; ++i) q_idx[i] = uniform();
  for (int i = 0; i < n_rows * HI; ++i) w_idx[i] = 0.5f + 0.5f * uniform();
  const int32_t row_req[n_rows] = {0, 1, 2};
  const int32_t row_len[n_rows] = {4 * 150 + 3, 17, -5};
  const int gstride = max_pages * GPP;
  float* scores = malloc(sizeof(float) * n_rows * gstride);
  qo_scores(n_rows, row_req, row_len, HI, HI, DI, PAGE, RATIO, q_idx, w_idx, khat, pt, max_pages, P,
            0, gstride, scores);
  qo_scores(n_rows, row_req, row_len, HI, HI, DI, PAGE, RATIO, q_idx, w_idx, khat, pt, max_pages, P,
            1, gstride, scores);
  /* multi-query form: 4 heads x 128 over one key head */
  qo_scores(n_rows, row_req, row_len, 4, 1, 128, PAGE, RATIO, q_idx, w_idx, khat, pt, max_pages,
            P, 0, gstride, scores);
  int32_t row_G[n_rows] = {150, 4, 0};
  enum { K = 64 };
  int32_t sel[n_rows * K];
  for (int i = 0; i < gstride; i += 7) scores[i] = 1.0f;  /* ties */
  if (qo_topk(n_rows, row_G, K, scores, gstride, sel) < 0) return 2;
  const int width = 4 * K + 3;
  int32_t* tokens = malloc(sizeof(int32_t) * n_rows * width);
  for (int r = 0; r < n_rows; ++r)
    if (qo_expand(K, sel + r * K, RATIO, 4 * row_G[r], 4 * row_G[r] + r, width,
                  tokens + r * width) < 0)
      return 3;
  uint8_t* kc = malloc((size_t)P * PAGE * HKV * D);
  uint8_t* vc = malloc((size_t)P * PAGE * HKV * D);
  for (size_t i = 0; i < (size_t)P * PAGE * HKV * D; ++i) {
    kc[i] = (uint8_t)(next_u32() & 0x7E);
    vc[i] = (uint8_t)(next_u32() & 0xFE);
  }
  uint16_t qv[n_rows * HQ * D];
  for (int i = 0; i < n_rows * HQ * D; ++i) qv[i] = (uint16_t)(0x3F00 + (next_u32() & 0xFF));
  double* out = malloc(sizeof(double) * n_rows * HQ * D);
  qo_attend(n_rows, row_req, tokens, width, HQ, HKV, D, PAGE, 1, kc, vc, 0.5, 0.25, 0.0625, pt,
            max_pages, P, qv, out);
  /* appends: in range, at a negative start, past the page table */
  const int32_t rows[3] = {0, 1, 2}, starts[3] = {61, -3, max_pages * PAGE - 2};
  const int n_tok = 9, slots = (n_tok + 3) / 4;
  uint16_t* kn = malloc(sizeof(uint16_t) * 3 * n_tok * HKV * D);
  uint16_t* vn = malloc(sizeof(uint16_t) * 3 * n_tok * HKV * D);
  for (int i = 0; i < 3 * n_tok * HKV * D; ++i) {
    kn[i] = (uint16_t)next_u32();
    vn[i] = (uint16_t)next_u32();
  }
  float* khn = malloc(sizeof(float) * 3 * slots * HI * DI);
  for (int i = 0; i < 3 * slots * HI * DI; ++i) khn[i] = uniform();
  qo_append(3, rows, starts, n_tok, HKV, D, 1, 0.37, 0.05, kn, vn, khn, slots, HI, DI, kc, vc,
            khat, pt, max_pages, P, PAGE, RATIO);
  uint16_t* kb = calloc((size_t)P * PAGE * HKV * D, sizeof(uint16_t));  /* BF16 caches */
  uint16_t* vb = calloc((size_t)P * PAGE * HKV * D, sizeof(uint16_t));
  qo_append(3, rows, starts, n_tok, HKV, D, 0, 1.0, 3.0, kn, vn, NULL, slots, HI, DI, kb, vb,
            khat, pt, max_pages, P, PAGE, RATIO);
  qo_attend(n_rows, row_req, tokens, width, HQ, HKV, D, PAGE, 0, kb, vb, 1.0, 1.0, 0.0625, pt,
            max_pages, P, qv, out);
  free(kb); free(vb);
  for (int c = 0; c < 256; ++c) (void)qo_fp8_e4m3_encode(qo_fp8_e4m3((uint8_t)c));
  free(khat); free(scores); free(tokens); free(kc); free(vc); free(out); free(kn); free(vn);
  free(khn);
  printf("oracle sanitized run: ok\n");
  return 0;
}
