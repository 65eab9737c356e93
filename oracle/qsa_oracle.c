/*
 * qsa_oracle.c — plain CPU oracle of one Qwen Sparse Attention layer step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this code.  It shares nothing
 * with the HIP library (no header, helper, table or constant) and the
 * library never calls it.
 *
 * Everything is computed with straightforward loops in fp64 from the exact
 * values of the stored inputs, in the order the method is described:
 *   indexer score -> exact top-K -> expansion to tokens -> attention.
 * Sources (page title, section):
 *   - "Qwen3.8-27B QSA - BF16 source weights", "QSA in brief": selection in
 *     4-token blocks by a learned compressed indexer, fixed K plus the
 *     current block, all KV retained.
 *   - TensorRT-LLM "QSASparseAttentionConfig": exact radix top-K over the
 *     compressed groups (enable_heuristic_topk), token-granular expanded
 *     selections (get_indices_block_size), selection sharing in the MTP
 *     draft loop with appended completed groups
 *     (index_share_for_mtp_iteration).
 *   - OrcaRouter article on SGLang PR #41855, "Neun bestandene Tests ...":
 *     -1 padded selections, zero output for rows that select nothing,
 *     causal tail of 0..3 tokens at ratio 4.
 * Readings where the pages are silent (the indexer formula, the tie order,
 * the FP8 flavour) are listed in the design notes and restated at each
 * function below.
 *
 * Pins: every function here is checked by tests against facts that do not
 * come from this file (format definitions, closed forms, brute force,
 * torch's CPU attention, invariants).  The indexer formula itself is an
 * assumed form: its pins check the code against that form, not against the
 * pages, which do not print it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* Exact values of stored elements                                        */
/* ---------------------------------------------------------------------- */

/* OCP 8-bit E4M3FN (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent field 0 is subnormal with weight 2^-6; field 15 with mantissa 7
 * is NaN; there is no infinity; largest finite 448). */
double qo_fp8_e4m3(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* bfloat16: the upper half of an IEEE binary32. */
double qo_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a binary32 to the nearest bfloat16 value, ties to even (used for
 * the prefill indexer, which multiplies bf16 operands). */
float qo_round_bf16(float x) {
  if (x != x) return x;
  uint32_t u;
  memcpy(&u, &x, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u = (u + 0x7FFFu + lsb) & 0xFFFF0000u;
  float r;
  memcpy(&r, &u, 4);
  return r;
}

static int page_ok(int32_t p, int num_pages) { return p >= 0 && p < num_pages; }

/* Nearest OCP E4M3FN code to x (the format above): the finite code whose
 * value is closest to x; on a tie, the code with an even mantissa field;
 * magnitudes beyond the largest finite value saturate to +-448 (the
 * library's reading: the pages name FP8 E4M3 KV but not an overflow rule);
 * NaN gives 0x7F.  Found by scanning all non-negative finite codes. */
uint8_t qo_fp8_e4m3_encode(double x) {
  if (x != x) return 0x7F;
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  const double a = fabs(x);
  if (a > 448.0) return (uint8_t)(sign | 0x7E); /* saturation, infinities included */
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    const double err = fabs(qo_fp8_e4m3((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(sign | best);
}

/* Nearest bfloat16 to a binary32 value, ties to even (bits). */
static uint16_t bf16_bits_rne(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if (x != x) return (uint16_t)((u >> 16) | 0x40u);
  u = u + 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* One stored K or V element for the new value x (a bfloat16) and the
 * per-tensor scale s of the cache: the binary32 quotient x / s (correctly
 * rounded), then its nearest FP8 E4M3 code, or its nearest bfloat16 for a
 * BF16 cache (x itself when s == 1).  Reading: the pages name FP8 E4M3 KV
 * with "prefill writes" (qsa-hisparse README, offload contract and entry
 * points) but print no quantiser; the per-tensor scale is the one the
 * attention decodes with.  The quotient of two binary32 values taken in
 * binary64 and then rounded to binary32 is the correctly rounded binary32
 * quotient (53 >= 2 * 24 + 2 bits, so the double rounding is innocuous). */
static void store_kv(void* cache, int kv_dtype, int64_t index, uint16_t x_bits, double scale) {
  const float q = (float)(qo_bf16(x_bits) / scale);
  if (kv_dtype == 0)
    ((uint16_t*)cache)[index] = scale == 1.0 ? x_bits : bf16_bits_rne(q);
  else
    ((uint8_t*)cache)[index] = qo_fp8_e4m3_encode((double)q);
}

/* Append n_tokens new tokens to each of n_req requests.  Request r uses
 * page-table row req_rows[r]; its new tokens take positions
 * start_pos[r] .. start_pos[r] + n_tokens - 1, token t landing in page
 * page_table[row][t / page_size], slot t % page_size.  k_new / v_new are
 * [n_req, n_tokens, Hkv, D] bfloat16.  khat_new (may be NULL) is
 * [n_req, khat_slots, Hi, Di] fp32: slot j holds group
 * floor(start_pos[r] / ratio) + j, and is written when that group's last
 * token (ratio * g + ratio - 1) is among the appended ones.  Positions
 * whose page-table entry lies outside the row or names a page outside
 * [0, num_pages) are not written. */
void qo_append(int n_req, const int32_t* req_rows, const int32_t* start_pos, int n_tokens, int Hkv,
               int D, int kv_dtype, double k_scale, double v_scale, const uint16_t* k_new,
               const uint16_t* v_new, const float* khat_new, int khat_slots, int Hi, int Di,
               void* k_cache, void* v_cache, float* khat_cache, const int32_t* page_table,
               int max_pages, int num_pages, int page_size, int ratio) {
  const int gpp = page_size / ratio;
  for (int r = 0; r < n_req; ++r) {
    const int32_t* pt = page_table + (int64_t)req_rows[r] * max_pages;
    for (int i = 0; i < n_tokens; ++i) {
      const int64_t t = (int64_t)start_pos[r] + i;
      if (t < 0 || t / page_size >= max_pages) continue;
      const int32_t p = pt[t / page_size];
      if (!page_ok(p, num_pages)) continue;
      const int64_t row = ((int64_t)p * page_size + t % page_size) * Hkv * D;
      const int64_t src = ((int64_t)r * n_tokens + i) * Hkv * D;
      for (int e = 0; e < Hkv * D; ++e) {
        store_kv(k_cache, kv_dtype, row + e, k_new[src + e], k_scale);
        store_kv(v_cache, kv_dtype, row + e, v_new[src + e], v_scale);
      }
    }
    if (khat_new == NULL) continue;
    const int64_t g0 = (int64_t)floor((double)start_pos[r] / ratio);
    for (int j = 0; j < khat_slots; ++j) {
      const int64_t g = g0 + j, last = g * ratio + ratio - 1;
      if (g < 0 || last < start_pos[r] || last >= (int64_t)start_pos[r] + n_tokens) continue;
      if (g / gpp >= max_pages) continue;
      const int32_t p = pt[g / gpp];
      if (!page_ok(p, num_pages)) continue;
      memcpy(khat_cache + ((int64_t)p * gpp + g % gpp) * Hi * Di,
             khat_new + ((int64_t)r * khat_slots + j) * Hi * Di, sizeof(float) * Hi * Di);
    }
  }
}

static double kv_value(const void* cache, int kv_dtype, int64_t index) {
  if (kv_dtype == 0) return qo_bf16(((const uint16_t*)cache)[index]);
  return qo_fp8_e4m3(((const uint8_t*)cache)[index]);
}


/* ---------------------------------------------------------------------- */
/* Step 1: indexer scores                                                 */
/* ---------------------------------------------------------------------- */

/* score[g] = sum_h w[h] * max(0, sum_d q[h][d] * khat[g][kh(h)][d]) for
 * every complete group g < floor(L/ratio) of the row; -inf for
 * g >= floor(L/ratio) and for groups whose page id is out of range.  The
 * form is the assumed ReLU-weighted indexer (the pages do not print one).
 * The k̂ of a group has Hk key heads; query head h reads key head
 * kh(h) = h * Hk / Hi.  Hk = Hi is the per-head form (8 x 64); Hk = 1 is the
 * multi-query form of the OrcaRouter article on PR #41855, "Warum QSA der
 * heikle Teil ist - in Zahlen" (4 query heads sharing 1 key head of
 * dimension 128).
 * Products of two binary32 values are exact in binary64 and the sums run in
 * binary64, so the single final rounding to binary32 gives (up to a
 * double-rounding tie) the correctly rounded score.  With round_bf16 != 0
 * q and khat are first rounded to bf16 (prefill precision).
 * gstride is the row stride of `out`; columns >= floor(L/ratio) up to
 * gstride are set to -inf.  Rows with L < 0 or floor(L/ratio) > gstride
 * (more complete groups than the row holds) get all -inf. */
void qo_scores(int n_rows, const int32_t* row_req, const int32_t* row_len, int Hi, int Hk, int Di,
               int page, int ratio, const float* q_idx, const float* w_idx, const float* khat,
               const int32_t* page_table, int max_pages, int num_pages, int round_bf16,
               int gstride, float* out) {
  int gpp = page / ratio; /* groups per page */
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < n_rows; ++r) {
    int L = row_len[r];
    int G = (L >= 0 && L / ratio <= gstride) ? L / ratio : 0;
    const float* q = q_idx + (int64_t)r * Hi * Di;
    const float* w = w_idx + (int64_t)r * Hi;
    float* o = out + (int64_t)r * gstride;
    for (int g = 0; g < gstride; ++g) o[g] = -INFINITY;
    for (int g = 0; g < G; ++g) {
      int32_t phys = page_table[(int64_t)row_req[r] * max_pages + g / gpp];
      if (!page_ok(phys, num_pages)) continue;
      const float* kg = khat + ((int64_t)phys * gpp + g % gpp) * Hk * Di;
      double s = 0.0;
      for (int h = 0; h < Hi; ++h) {
        double a = 0.0;
        for (int d = 0; d < Di; ++d) {
          float qv = q[h * Di + d], kv = kg[(h * Hk / Hi) * Di + d];
          if (round_bf16) { qv = qo_round_bf16(qv); kv = qo_round_bf16(kv); }
          a += (double)qv * (double)kv;
        }
        s += (double)w[h] * (a > 0.0 ? a : 0.0);
      }
      float s32 = (float)s;
      if (s32 == 0.0f) s32 = 0.0f; /* -0 -> +0 */
      o[g] = s32;
    }
  }
}

/* ---------------------------------------------------------------------- */
/* Step 2: exact top-K                                                    */
/* ---------------------------------------------------------------------- */

typedef struct { float s; int32_t g; } scored;

/* Total order of the selection: higher score first; equal scores (+0 and
 * -0 compare equal) go to the lower group index.  The pages do not state a
 * tie rule; lowest index first is the reading taken. */
static int by_rank(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->g > y->g) - (x->g < y->g);
}

static int ascending(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* For each row keep min(K, G) groups among g < G (G = row_G[r]): all of
 * them if G <= K, else the first K in the total order above.  Output is
 * ascending group ids padded with -1 to K entries.  Returns the number of
 * NaN scores met among candidates (NaN has no place in the order; callers
 * treat a nonzero return as an error). */
int qo_topk(int n_rows, const int32_t* row_G, int K, const float* scores, int gstride,
            int32_t* out) {
  int nan_count = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : nan_count)
  for (int r = 0; r < n_rows; ++r) {
    int G = row_G[r] < 0 ? 0 : (row_G[r] > gstride ? gstride : row_G[r]);
    const float* s = scores + (int64_t)r * gstride;
    int32_t* o = out + (int64_t)r * K;
    for (int i = 0; i < K; ++i) o[i] = -1;
    for (int g = 0; g < G; ++g) nan_count += (s[g] != s[g]);
    if (G <= K) {
      for (int g = 0; g < G; ++g) o[g] = g;
      continue;
    }
    scored* all = (scored*)malloc(sizeof(scored) * (size_t)G);
    for (int g = 0; g < G; ++g) { all[g].s = s[g]; all[g].g = g; }
    qsort(all, (size_t)G, sizeof(scored), by_rank);
    for (int i = 0; i < K; ++i) o[i] = all[i].g;
    qsort(o, (size_t)K, sizeof(int32_t), ascending);
    free(all);
  }
  return nan_count;
}

/* ---------------------------------------------------------------------- */
/* Step 3: expansion                                                      */
/* ---------------------------------------------------------------------- */

/* Token list of one query row: tokens ratio*g .. ratio*g+ratio-1 of every
 * selected group (ascending input, -1 entries ignored), followed by the
 * contiguous range [tail_begin, tail_end) (the current partial block, plus
 * any groups completed by draft positions).  Written ascending into
 * out[0..width), padded with -1.  Returns the count, or -1 if it exceeds
 * width. */
int qo_expand(int K, const int32_t* groups, int ratio, int tail_begin, int tail_end, int width,
              int32_t* out) {
  int n = 0;
  for (int i = 0; i < width; ++i) out[i] = -1;
  for (int i = 0; i < K; ++i) {
    if (groups[i] < 0) continue;
    for (int j = 0; j < ratio; ++j) {
      if (n >= width) return -1;
      out[n++] = groups[i] * ratio + j;
    }
  }
  for (int t = tail_begin; t < tail_end; ++t) {
    if (n >= width) return -1;
    out[n++] = t;
  }
  qsort(out, (size_t)n, sizeof(int32_t), ascending);
  return n;
}

/* ---------------------------------------------------------------------- */
/* Step 4: attention over a token list                                    */
/* ---------------------------------------------------------------------- */

/* For each query row r (page-table row row_req[r], token list
 * tokens[r*width .. ], -1 entries ignored) and query head h, with KV head
 * kh = h / (Hq / Hkv):
 *   z_t = sm_scale * sum_d q[r,h,d] * K[t,kh,d] * k_scale
 *   out[r,h,:] = sum_t exp(z_t - max z) * V[t,kh,:] * v_scale / sum_t exp(z_t - max z)
 * in binary64.  Tokens on out-of-range pages are skipped; a row with no
 * token gives exact zeros. */
void qo_attend(int n_rows, const int32_t* row_req, const int32_t* tokens, int width, int Hq,
               int Hkv, int D, int page, int kv_dtype, const void* k_cache, const void* v_cache,
               double k_scale, double v_scale, double sm_scale, const int32_t* page_table,
               int max_pages, int num_pages, const uint16_t* q, double* out) {
  int group = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int r = 0; r < n_rows; ++r) {
    for (int h = 0; h < Hq; ++h) {
      int kh = h / group;
      const int32_t* tl = tokens + (int64_t)r * width;
      const uint16_t* qh = q + ((int64_t)r * Hq + h) * D;
      double* o = out + ((int64_t)r * Hq + h) * D;
      double* z = (double*)malloc(sizeof(double) * (size_t)(width > 0 ? width : 1));
      int64_t* base = (int64_t*)malloc(sizeof(int64_t) * (size_t)(width > 0 ? width : 1));
      int n = 0;
      double zmax = -INFINITY;
      for (int i = 0; i < width; ++i) {
        int32_t t = tl[i];
        if (t < 0) continue;
        int32_t phys = page_table[(int64_t)row_req[r] * max_pages + t / page];
        if (!page_ok(phys, num_pages)) continue;
        int64_t b0 = (((int64_t)phys * page + t % page) * Hkv + kh) * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qo_bf16(qh[d]) * (kv_value(k_cache, kv_dtype, b0 + d) * k_scale);
        z[n] = sm_scale * dot;
        base[n] = b0;
        if (z[n] > zmax) zmax = z[n];
        ++n;
      }
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      if (n > 0) {
        double denom = 0.0;
        for (int i = 0; i < n; ++i) {
          double p = exp(z[i] - zmax);
          denom += p;
          for (int d = 0; d < D; ++d) o[d] += p * (kv_value(v_cache, kv_dtype, base[i] + d) * v_scale);
        }
        for (int d = 0; d < D; ++d) o[d] /= denom;
      }
      free(z);
      free(base);
    }
  }
}

int qo_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
