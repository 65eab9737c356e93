/*
 * qsa.h — C ABI of libqsa: one Qwen Sparse Attention (QSA) layer step on
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources: the "Qwen3.8-27B QSA - BF16 source
 * weights" model card, section "QSA in brief"; the TensorRT-LLM
 * "QSASparseAttentionConfig" reference; the OrcaRouter article on SGLang
 * PR #41855, sections "Was der Pull Request tatsächlich hinzufügt",
 * "Neun bestandene Tests ..." and "Warum QSA der heikle Teil ist – in Zahlen"):
 *
 *   1. Indexer score.  A learned, compressed indexer holds one key k̂ per
 *      group of 4 consecutive tokens (compress ratio 4, "C4").  The pages do
 *      not print the indexer formula; this library uses, per query row and
 *      complete group g,
 *          score[g] = sum_h  w[h] * max(0, sum_d q_idx[h,d] * khat[g,kh(h),d])
 *      with H_i = 8 indexer heads of dimension 64 and a key per head
 *      (kh(h) = h), or the multi-query form of 4 heads of dimension 128
 *      sharing one key (kh(h) = 0); all inputs fp32.
 *   2. Exact top-K.  Among the complete groups g < floor(L/4) (L = tokens
 *      including the current one) keep the K = topk_groups highest scores,
 *      ranking by (score descending, group index ascending); K is the group
 *      budget topk_groups, any value in 1..2048.  The pages' budgets are
 *      512, 1024 and 2048 groups at ratio 4; the TRT-LLM config
 *      (enable_heuristic_topk) names that set only as a prerequisite of
 *      its heuristic Guess-Verify-Refine selector, and otherwise falls back
 *      to the exact radix top-K, which this library always computes and
 *      which has no such limit.  If floor(L/4) <= K every complete group
 *      is kept, so the step equals dense causal attention.
 *   3. Expansion.  Each kept group g becomes tokens 4g..4g+3; the current
 *      partial block [4*floor(L/4), L) of 0..3 tokens is always added.  All
 *      KV stays in the cache; nothing is compressed or evicted (model card,
 *      "QSA in brief").  Selections address single tokens (TRT-LLM config,
 *      get_indices_block_size).
 *   4. Sparse GQA attention over exactly those tokens, read from a paged
 *      KV cache (page size 64, BF16 or FP8 E4M3 KV: qsa-hisparse offload
 *      contract), query head h using KV head floor(h * Hkv / Hq).  A row
 *      with no selected token outputs exact zeros (PR #41855 article,
 *      zero-output convention for fully masked rows).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers unless a comment says "host".
 *     The caller owns every buffer and the stream; the library allocates
 *     nothing and keeps no pointer after return.  Its only global state is
 *     the static scratch area of qsa_decode_noalloc (below).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *     the null stream).  No call synchronises the host or copies device
 *     data to the host, so the calls can be captured into a HIP graph.
 *   - Tensors are dense, row-major (C order), with the layouts below.
 *   - Argument and geometry errors are detected on the host and returned
 *     before anything is enqueued.  A failed kernel launch returns
 *     QSA_ERR_HIP.  Device-side contents (lengths, page ids) cannot be
 *     reported; their valid ranges are stated per argument and values
 *     outside them are handled as documented, never by faulting.
 *   - The workspace `ws` is a caller-allocated device buffer of at least
 *     the size reported by the matching *_workspace_size function, aligned
 *     to 256 bytes.  Its contents need not be initialised and are
 *     clobbered.  Two calls that share one workspace must be ordered.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qsa_status {
  QSA_OK = 0,
  QSA_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent lengths */
  QSA_ERR_UNSUPPORTED = -2, /* geometry outside what the kernels implement */
  QSA_ERR_WORKSPACE = -3,   /* workspace missing, too small or misaligned */
  QSA_ERR_HIP = -4,         /* a HIP launch or API call failed */
  QSA_ERR_TOO_LARGE = -5    /* the call needs more than the static scratch
                               of qsa_decode_noalloc holds */
} qsa_status;

/* KV element formats of the paged cache (qsa-hisparse offload contract:
 * FP8 E4M3 KV; PR #41855 article: BF16 KV with head dim 256). */
enum qsa_kv_dtype {
  QSA_KV_BF16 = 0,     /* 16-bit bfloat16 bit patterns */
  QSA_KV_FP8_E4M3 = 1  /* OCP E4M3FN bytes (max 448, no inf, 0x7F/0xFF NaN) */
};

/* Layer geometry.  The supported values follow the pages' configurations:
 * head_dim 256, page_size 64, compress_ratio 4 (C4), a group budget
 * topk_groups in [1, 2048] (the pages use 512, 1024 and 2048; the TRT-LLM
 * QSASparseAttentionConfig reference, enable_heuristic_topk, requires that
 * set only for its heuristic GVR selector, not for the exact top-K; values
 * outside [1, 2048] are refused as QSA_ERR_UNSUPPORTED), any GQA
 * ratio num_q_heads / num_kv_heads with (num_q_heads / num_kv_heads) *
 * q_per_req <= 64 query rows per KV head, and one of two indexer forms:
 *   - per head: idx_heads 8, idx_dim 64, idx_key_heads 8 (or 0), a key of
 *     8 x 64 fp32 per group (2 KiB);
 *   - multi-query (OrcaRouter article on PR #41855, "Warum QSA der heikle
 *     Teil ist - in Zahlen": 4 query heads share 1 key head of dimension
 *     128): idx_heads 4, idx_dim 128, idx_key_heads 1, a key of 128 fp32
 *     per group (512 B).  Query head h reads key head
 *     h * idx_key_heads / idx_heads. */
typedef struct qsa_geometry {
  int32_t num_q_heads;    /* Hq, e.g. 16 or 24 */
  int32_t num_kv_heads;   /* Hkv, e.g. 2; must divide num_q_heads */
  int32_t head_dim;       /* D = 256 */
  int32_t page_size;      /* tokens per KV page = 64 */
  int32_t compress_ratio; /* tokens per indexer group = 4 */
  int32_t idx_heads;      /* H_i = 8 (per-head form) or 4 (multi-query form) */
  int32_t idx_dim;        /* D_i = 64 or 128 */
  int32_t topk_groups;    /* K, group budget, 1..2048 */
  int32_t kv_dtype;       /* enum qsa_kv_dtype */
  float sm_scale;         /* softmax scale; <= 0 selects 1/sqrt(head_dim) */
  float k_scale;          /* K element = decoded code * k_scale (FP8 per-tensor
                             dequant factor; 1 for unscaled BF16) */
  float v_scale;          /* V element = decoded code * v_scale */
  int32_t idx_key_heads;  /* H_k: indexer key heads per group, 8 or 1 (0 = H_i) */
} qsa_geometry;

/* The paged caches of one attention layer.  Logical token t of the request
 * whose page-table row is r lives in physical page P = page_table[r *
 * max_pages + t / page_size], slot t % page_size.  The compressed indexer
 * keys are paged with the same table: group g of that request lives in page
 * page_table[r * max_pages + g / (page_size / compress_ratio)], slot
 * g % (page_size / compress_ratio).  A group never straddles a page.
 *
 * Page ids must lie in [0, num_pages).  An id outside that range is never
 * dereferenced: its groups score -inf (never selected) and its tokens are
 * skipped by attention. */
typedef struct qsa_paged_cache {
  const void* k;              /* [num_pages, page_size, Hkv, D] bf16 or fp8 */
  const void* v;              /* [num_pages, page_size, Hkv, D] bf16 or fp8 */
  const float* khat;          /* [num_pages, page_size/ratio, H_k, D_i] f32 */
  const int32_t* page_table;  /* [rows, max_pages] int32 */
  int32_t max_pages;          /* row stride of page_table (host) */
  int32_t num_pages;          /* physical pages in k, v and khat (host) */
} qsa_paged_cache;

/* Human-readable name of a status code (static string, host). */
const char* qsa_status_string(qsa_status s);

/* Host-only check that `g` describes a supported geometry.  Makes no HIP
 * call.  Returns QSA_OK, QSA_ERR_INVALID_ARG (null) or QSA_ERR_UNSUPPORTED.
 * Unsupported configurations are refused up front rather than silently
 * routed to another path (qsa-hisparse: unsupported configurations fail at
 * startup). */
qsa_status qsa_validate(const qsa_geometry* g);

/* Width of a per-query-row token list for `q_per_req` query positions:
 * 4*K selected-group tokens plus at most 3 + (q_per_req - 1) tokens of the
 * current block and of groups completed by draft positions.  For one
 * position this is 4K + 3, e.g. 2,051 at K = 512 (PR #41855 article: 2,051
 * selected slots per query).  Returns 0 for an invalid geometry. */
int32_t qsa_token_width(const qsa_geometry* g, int32_t q_per_req);

/* Workspace sizes in bytes (host).  max_ctx bounds every length the call
 * will see; 0 is returned for invalid arguments. */
size_t qsa_index_topk_workspace_size(const qsa_geometry* g, int32_t n_rows,
                                     int32_t max_ctx);
size_t qsa_decode_workspace_size(const qsa_geometry* g, int32_t batch,
                                 int32_t q_per_req, int32_t max_ctx);
size_t qsa_prefill_workspace_size(const qsa_geometry* g, int32_t n_q,
                                  int32_t max_ctx);

/* Indexer scores only (step 1 above), fp32, for independent query rows:
 * the decode-time GEMV over the paged k̂.  No workspace.
 *
 *   row_req   nullable [n_rows] int32: page-table row of each query row;
 *             NULL means row r uses page-table row r.
 *   row_len, q_idx, w_idx, max_ctx: as for qsa_index_topk.
 *   out_scores [n_rows, max_ctx / ratio] f32; entries g >= floor(L/4) are
 *             -inf, and so are groups on out-of-range pages.
 */
qsa_status qsa_index_score(const qsa_geometry* g, const qsa_paged_cache* cache,
                           int32_t n_rows, int32_t max_ctx, const int32_t* row_req,
                           const int32_t* row_len, const float* q_idx,
                           const float* w_idx, float* out_scores, void* stream);

/* Indexer scores of a prefill chunk (step 1 for every query of the chunk),
 * exactly as qsa_prefill computes them: a dense GEMM on the matrix cores
 * with q_idx and k̂ rounded to bf16 (round-to-nearest-even), exact
 * products, fp32 sums; w_idx, the ReLU and the head sum stay fp32.  No
 * workspace.
 *
 *   req, first_pos, n_q, q_idx, w_idx: as for qsa_prefill (query i has
 *             L = first_pos + i + 1).
 *   out_scores [n_q, (first_pos + n_q) / ratio] f32; entries
 *             g >= floor(L_i / 4) are -inf, and so are groups on
 *             out-of-range pages.
 */
qsa_status qsa_index_score_prefill(const qsa_geometry* g, const qsa_paged_cache* cache,
                                   int32_t req, int32_t first_pos, int32_t n_q,
                                   const float* q_idx, const float* w_idx,
                                   float* out_scores, void* stream);

/* Indexer score + exact top-K for independent query rows (steps 1-2 above),
 * fp32 arithmetic (a GEMV per row over the paged k̂).
 *
 *   n_rows, max_ctx  host; 1 <= max_ctx <= max_pages * page_size and
 *                    max_ctx <= 262,144 (the per-request capacity of the
 *                    qsa-hisparse contract).
 *   row_req   [n_rows] int32: page-table row of each query row.
 *   row_len   [n_rows] int32: L of each row (tokens including the current
 *             one).  Candidates are the groups g < floor(L/4).  A value
 *             outside [0, max_ctx] selects nothing.
 *   q_idx     [n_rows, H_i, D_i] f32;  w_idx [n_rows, H_i] f32.
 *   out_groups [n_rows, K] int32: selected group ids in ascending order,
 *             padded with -1 after the min(K, floor(L/4)) valid entries.
 *   out_scores nullable [n_rows, max_ctx / ratio] f32: the indexer scores;
 *             entries g >= floor(L/4) are -inf.
 */
qsa_status qsa_index_topk(const qsa_geometry* g, const qsa_paged_cache* cache,
                          int32_t n_rows, int32_t max_ctx,
                          const int32_t* row_req, const int32_t* row_len,
                          const float* q_idx, const float* w_idx,
                          int32_t* out_groups, float* out_scores, void* ws,
                          size_t ws_bytes, void* stream);

/* One decode step for `batch` requests (steps 1-4), each with q_per_req
 * query positions that share one selection (TRT-LLM config,
 * index_share_for_mtp_iteration: the draft loop reuses the indexer
 * selection of its base position and appends the groups that complete
 * during the loop).
 *
 *   batch, q_per_req, max_ctx  host; q_per_req in [1, 4]; request b uses
 *             page-table row b.
 *   ctx_lens  [batch] int32: L0 = tokens up to and including the base
 *             position.  Position j (0 <= j < q_per_req) has L_j = L0 + j
 *             and attends to expand(S0) plus every token in
 *             [4*floor(L0/4), L_j), where S0 is the top-K of the base
 *             position.  L0 + q_per_req - 1 must not exceed max_ctx; a
 *             request with L0 outside [0, max_ctx - q_per_req + 1] gets an
 *             empty selection and zero output.
 *   q_idx [batch, H_i, D_i] f32 and w_idx [batch, H_i] f32: indexer query
 *             of the base position.
 *   q         [batch, q_per_req, Hq, D] bf16 bit patterns (already rotated).
 *   out       [batch, q_per_req, Hq, D] f32.
 *   out_groups nullable [batch, K] int32: S0, ascending, -1 padded.
 *   out_tokens nullable [batch, q_per_req, W] int32 with
 *             W = qsa_token_width(g, q_per_req): the token list of each
 *             position, ascending, -1 padded.
 *   out_scores nullable [batch, max_ctx / ratio] f32 (as qsa_index_topk).
 */
qsa_status qsa_decode(const qsa_geometry* g, const qsa_paged_cache* cache,
                      int32_t batch, int32_t q_per_req, int32_t max_ctx,
                      const int32_t* ctx_lens, const float* q_idx,
                      const float* w_idx, const uint16_t* q, float* out,
                      int32_t* out_groups, int32_t* out_tokens,
                      float* out_scores, void* ws, size_t ws_bytes,
                      void* stream);

/* Chunked prefill of one request (steps 1-4 for every query of the chunk,
 * each query with its own causal selection; PR #41855 article: prefill
 * over selected token slots, long-prefill case).
 *
 *   req        host: page-table row of the request.
 *   first_pos  host: 0-based position of the first query; query i has
 *              L = first_pos + i + 1.  The chunk's own K/V and k̂ must
 *              already be in the cache.  first_pos + n_q <= 262,144 and
 *              <= max_pages * page_size.
 *   q_idx [n_q, H_i, D_i] f32, w_idx [n_q, H_i] f32: indexer queries.  The
 *              prefill indexer is a dense GEMM on the matrix cores in BF16
 *              with fp32 accumulation: q_idx and k̂ are rounded to bf16
 *              (round-to-nearest-even) before the products; w_idx, the
 *              ReLU and the head sum stay fp32.  Inputs that are already
 *              bf16-exact are used unchanged.
 *   q          [n_q, Hq, D] bf16 bit patterns.
 *   out        [n_q, Hq, D] f32.
 *   out_groups nullable [n_q, K]; out_tokens nullable [n_q, 4K + 3];
 *   out_scores nullable [n_q, (first_pos + n_q) / ratio] f32.
 */
qsa_status qsa_prefill(const qsa_geometry* g, const qsa_paged_cache* cache,
                       int32_t req, int32_t first_pos, int32_t n_q,
                       const float* q_idx, const float* w_idx,
                       const uint16_t* q, float* out, int32_t* out_groups,
                       int32_t* out_tokens, float* out_scores, void* ws,
                       size_t ws_bytes, void* stream);

/* Size in bytes of the static device scratch that qsa_decode_noalloc uses
 * in place of a workspace (one copy per GPU, held until the process ends). */
#define QSA_NOALLOC_SCRATCH_BYTES (32u << 20)
size_t qsa_noalloc_scratch_bytes(void);

/* qsa_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, semantics and
 * results as qsa_decode; the workspace is instead a file-scope device
 * array of QSA_NOALLOC_SCRATCH_BYTES (32 MiB) inside the library, one
 * copy per GPU.  The call never allocates or frees device memory: the
 * first call on a device only looks up that device's copy, with the
 * device current.  It holds, e.g., 32 requests at 262,144 tokens with
 * K = 2,048 groups (15.4 MiB; 8 such requests take 6.9 MiB).  A call whose
 * workspace would exceed it (qsa_decode_workspace_size(...) >
 * QSA_NOALLOC_SCRATCH_BYTES) returns QSA_ERR_TOO_LARGE after the argument
 * checks of qsa_decode and before any HIP call.
 *
 * Every call on one GPU uses that GPU's single scratch area, which keeps
 * whatever the last call left there (no call depends on it).  Calls that
 * overlap on one GPU (on different streams, or from several threads
 * without ordering) race on it and give undefined results: order them on
 * one stream.  QSA_ERR_HIP is returned if the device's copy cannot be
 * found. */
qsa_status qsa_decode_noalloc(const qsa_geometry* g, const qsa_paged_cache* cache,
                              int32_t batch, int32_t q_per_req, int32_t max_ctx,
                              const int32_t* ctx_lens, const float* q_idx,
                              const float* w_idx, const uint16_t* q, float* out,
                              int32_t* out_groups, int32_t* out_tokens,
                              float* out_scores, void* stream);

/* Number of k̂ slots per request that qsa_append_kv reads from khat_new for
 * n_tokens new tokens: floor((n_tokens + 3) / 4), the most groups that
 * many tokens can complete.  Returns 0 for n_tokens <= 0. */
int32_t qsa_append_khat_slots(int32_t n_tokens);

/* Cache append: the "prefill writes" of the attention backend (qsa-hisparse
 * README, entry points), in the cache format of the offload contract (FP8
 * E4M3 KV, page size 64).  Writes the keys and values of n_tokens new
 * tokens of each of n_req requests into the paged KV cache, and the
 * compressed indexer keys of the groups those tokens complete into the
 * paged k̂ cache.  The compressor that produces k̂ is learned and not part
 * of the library, so the caller supplies k̂.
 *
 *   n_req, n_tokens  host; >= 0.
 *   k_cache, v_cache, khat_cache  the caches of qsa_paged_cache (written;
 *             layouts as there); page_table [rows, max_pages] int32 with
 *             max_pages, num_pages host, as in qsa_paged_cache.
 *   req_rows  [n_req] int32: page-table row of each request.
 *   start_pos [n_req] int32: position of each request's first new token.
 *             New token i of request r is t = start_pos[r] + i and lands
 *             in page page_table[row][t / page_size], slot t % page_size.
 *   k_new, v_new [n_req, n_tokens, Hkv, D] bf16 bit patterns.  A stored
 *             element is the binary32 quotient x / k_scale (v_scale for V),
 *             correctly rounded, then rounded to the nearest FP8 E4M3FN
 *             code (ties to an even mantissa; magnitudes above 448
 *             saturate to +-448; NaN stays NaN) for an FP8 cache, or to the
 *             nearest bfloat16 (ties to even) for a BF16 cache, which is x
 *             itself when the scale is 1.  The pages print no quantiser;
 *             this is the library's reading.
 *   khat_new  nullable [n_req, qsa_append_khat_slots(n_tokens), H_k, D_i]
 *             f32.  Slot j of request r holds group
 *             g = floor(start_pos[r] / 4) + j.  It is written (copied) when
 *             that group's last token 4g + 3 is among the new tokens.
 * Tokens and groups at negative positions, at page-table indices
 * >= max_pages, or on page ids outside [0, num_pages) are skipped.  New
 * tokens of different requests that map to the same page slot race (a
 * valid page table gives requests distinct pages).  Ordering against other
 * calls that read the caches is the caller's, through `stream`.
 */
qsa_status qsa_append_kv(const qsa_geometry* g, void* k_cache, void* v_cache,
                         float* khat_cache, const int32_t* page_table,
                         int32_t max_pages, int32_t num_pages, int32_t n_req,
                         const int32_t* req_rows, const int32_t* start_pos,
                         int32_t n_tokens, const uint16_t* k_new,
                         const uint16_t* v_new, const float* khat_new,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
