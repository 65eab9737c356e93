// qsa_launch.h — internal host-side launchers of the QSA kernels.
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// Indexer scores of `n_rows` query rows over their request's paged k̂
// (fp32 GEMV); shared_key selects the multi-query form (4 heads x 128
// sharing one key head, 512 B of k̂ per group) over the per-head form.  scores is [n_rows, gstride]; columns g >= floor(L/4) get
// -inf.  Rows take (request, L) from row_req/row_len; with row_req null,
// row r uses page-table row r; with both null, rows are queries
// first_pos + row of request req0.  If samples is non-null and a row has
// G >= kTopkSamples groups, the kernel also writes that row's scores of
// groups floor(i * G / kTopkSamples), i < kTopkSamples, to
// samples[row * kTopkSamples + i] (the top-K's pruning sample).
constexpr int kTopkSamples = 512;
hipError_t launch_index_score_gemv(const float* khat, const int32_t* page_table, int max_pages,
                                   int num_pages, int n_rows, const int32_t* row_req,
                                   const int32_t* row_len, int req0, int first_pos, int max_ctx,
                                   const float* q_idx, const float* w_idx, float* scores,
                                   int gstride, hipStream_t stream, float* samples = nullptr,
                                   bool shared_key = false);

// Indexer scores of a prefill chunk on the matrix cores (bf16 operands,
// fp32 accumulation): query i of the chunk has L = first_pos + i + 1.
// shared_key: the multi-query indexer (4 heads x 128 sharing one key head)
// instead of the per-head form (8 heads x 64).
hipError_t launch_index_score_prefill(const float* khat, const int32_t* page_table,
                                      int max_pages, int num_pages, int req, int first_pos,
                                      int n_q, const float* q_idx, const float* w_idx,
                                      float* scores, int gstride, hipStream_t stream,
                                      bool shared_key = false);

// Exact top-K of each row: candidates g < G(row) where G = floor(L/4) for
// L = row_len[row] in [0, max_ctx] (else G = 0); when row_len is null,
// L = first_pos + row + 1.  out is [n_rows, K] ascending, -1 padded.  ws
// (256-byte aligned, topk_workspace_bytes) holds candidates of long rows.
size_t topk_workspace_bytes(int n_rows, int gstride);
// samples (nullable): the scoring kernel's per-row pruning sample.
hipError_t launch_topk(const float* scores, int gstride, int n_rows, const int32_t* row_len,
                       int first_pos, int max_ctx, int K, int32_t* out, void* ws,
                       hipStream_t stream, const float* samples = nullptr);

struct AttnArgs {
  const void* k;
  const void* v;
  int kv_dtype;  // 0 bf16, 1 fp8 e4m3
  const int32_t* page_table;
  int max_pages;
  int num_pages;
  const int32_t* sel;  // [items, K] ascending group ids, -1 padded
  int K;
  const int32_t* ctx_lens;  // decode: [B] L0; prefill: null
  int first_pos;            // prefill: position of query 0
  int req;                  // prefill: page-table row
  int max_ctx;
  int q_per_req;
  const uint16_t* q;  // decode [B, Q, Hq, D]; prefill [n_q, Hq, D]
  int Hq, Hkv;
  float sm_scale, k_scale, v_scale;
  int batch;            // decode: requests; prefill: queries
  int groups_per_split; // decode split size (groups)
  int n_splits;
  float* partial;  // decode: [B, Hkv, n_splits, Q*Hq/Hkv, 2 + D] (workspace)
  float* out;      // prefill: [n_q, Hq, D]; decode: [B, Q, Hq, D] (combine)
};

hipError_t launch_sparse_attn_decode(const AttnArgs& a, hipStream_t stream);
// Prefill attention needs no workspace: it writes the output rows directly.
hipError_t launch_sparse_attn_prefill(const AttnArgs& a, hipStream_t stream);

// Cache append: K/V of n_tokens new tokens per request (bf16 in, stored in
// the cache format with the per-tensor scales) and the k̂ of the groups they
// complete (khat_new nullable, (n_tokens + 3) / 4 slots per request).
hipError_t launch_append(void* k_cache, void* v_cache, float* khat_cache,
                         const int32_t* page_table, int max_pages, int num_pages, int n_req,
                         const int32_t* req_rows, const int32_t* start_pos, int n_tokens,
                         const uint16_t* k_new, const uint16_t* v_new, const float* khat_new,
                         int khat_group_floats, int row_elems, int kv_dtype, float k_scale,
                         float v_scale, hipStream_t stream);

// Expanded token lists: [rows, q_per_req, width], ascending, -1 padded.
hipError_t launch_expand_tokens(const int32_t* sel, int K, int n_rows, int q_per_req,
                                const int32_t* ctx_lens, int first_pos, int max_ctx, int width,
                                int32_t* out, hipStream_t stream);

}  // namespace qsa
