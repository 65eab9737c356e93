// qsa_api.hip — the C ABI of libqsa (declared in include/qsa.h): argument
// and geometry checks on the host, workspace carving, and the launch
// sequence of each entry point on the caller's stream.  No call allocates,
// synchronises or copies device data to the host.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "qsa.h"
#include "qsa_device.h"
#include "qsa_launch.h"

namespace {

using namespace qsa;

constexpr int kCapacity = 262144;  // tokens per request (qsa-hisparse offload contract)
constexpr int kMaxRows = 64;       // query rows per KV head and request
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int gstride_of(int max_ctx) { return max_ctx / kRatio; }

// multi-query indexer form (4 heads x 128, one shared key head per group)
bool shared_key(const qsa_geometry* g) { return g->idx_key_heads == 1; }

// Decode attention: selection entries per split-K workgroup.  The
// selection of each (request, KV head, 16-row block) item is cut into the
// largest power-of-two number of splits that keeps the whole batch at or
// under 384 workgroups and every split at 16 groups or more (64 tokens, one
// sub-tile per wavefront); equal splits, rounded up to 16 groups.  Measured
// per decode step (the wavefronts run a rolling pipeline, so longer splits
// amortise its start): 8 x 262,144 tokens, K = 2,048: 16 splits 196.3 us
// against 198.6 us for the former ~512-workgroup rule; 8 x 32-64K tokens,
// K = 512: 58.9 against 60.1 us; 4 x 3 MTP positions at 131K with 24 query
// heads, K = 1,024: 78.5 against 81.9 us.
int groups_per_split(const qsa_geometry* g, int batch, int q_per_req) {
  constexpr long long kMaxWorkgroups = 384;
  const int gq = g->num_q_heads / g->num_kv_heads;
  const int nblk = (q_per_req * gq + 15) / 16;
  const long long items = (long long)batch * g->num_kv_heads * nblk;
  const int K = g->topk_groups;
  long long n = 1;
  while (items * n * 2 <= kMaxWorkgroups && (K + 2 * n - 1) / (2 * n) >= 16) n *= 2;
  long long gps = (K + n - 1) / n;
  gps = (gps + 15) / 16 * 16;
  if (gps < 16) gps = 16;
  if (gps > K) gps = (K + 15) / 16 * 16;
  return (int)gps;
}

struct DecodeLayout {
  int gps, n_splits, gstride;
  size_t off_scores, off_samples, off_sel, off_partial, off_topk, total;
};

DecodeLayout decode_layout(const qsa_geometry* g, int batch, int q_per_req, int max_ctx) {
  DecodeLayout d;
  d.gps = groups_per_split(g, batch, q_per_req);
  d.n_splits = (g->topk_groups + d.gps - 1) / d.gps;
  d.gstride = gstride_of(max_ctx);
  const int rows = q_per_req * (g->num_q_heads / g->num_kv_heads);
  size_t off = 0;
  d.off_scores = off;
  off += align_up(sizeof(float) * (size_t)batch * d.gstride);
  d.off_samples = off;
  off += align_up(sizeof(float) * (size_t)batch * kTopkSamples);
  d.off_sel = off;
  off += align_up(sizeof(int32_t) * (size_t)batch * g->topk_groups);
  d.off_partial = off;
  off += align_up(sizeof(float) * (size_t)batch * g->num_kv_heads * d.n_splits * rows *
                  (2 + kHeadDim));
  d.off_topk = off;
  off += align_up(topk_workspace_bytes(batch, d.gstride));
  d.total = off;
  return d;
}

struct RowsLayout {
  int gstride;
  size_t off_scores, off_samples, off_sel, off_topk, total;
};

RowsLayout rows_layout(const qsa_geometry* g, int n_rows, int max_ctx) {
  RowsLayout r;
  r.gstride = gstride_of(max_ctx);
  size_t off = 0;
  r.off_scores = off;
  off += align_up(sizeof(float) * (size_t)n_rows * r.gstride);
  r.off_samples = off;
  off += align_up(sizeof(float) * (size_t)n_rows * kTopkSamples);
  r.off_sel = off;
  off += align_up(sizeof(int32_t) * (size_t)n_rows * g->topk_groups);
  r.off_topk = off;
  off += align_up(topk_workspace_bytes(n_rows, r.gstride));
  r.total = off;
  return r;
}


bool cache_ok(const qsa_paged_cache* c, bool need_kv) {
  if (!c || !c->khat || !c->page_table || c->max_pages <= 0 || c->num_pages <= 0) return false;
  if (need_kv && (!c->k || !c->v)) return false;
  return true;
}

qsa_status ws_ok(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return QSA_OK;
  if (!ws || ws_bytes < need || ((uintptr_t)ws % kAlign) != 0) return QSA_ERR_WORKSPACE;
  return QSA_OK;
}

float scale_of(const qsa_geometry* g) {
  return g->sm_scale > 0.0f ? g->sm_scale : 1.0f / sqrtf((float)g->head_dim);
}

AttnArgs attn_args(const qsa_geometry* g, const qsa_paged_cache* c) {
  AttnArgs a = {};
  a.k = c->k;
  a.v = c->v;
  a.kv_dtype = g->kv_dtype;
  a.page_table = c->page_table;
  a.max_pages = c->max_pages;
  a.num_pages = c->num_pages;
  a.K = g->topk_groups;
  a.Hq = g->num_q_heads;
  a.Hkv = g->num_kv_heads;
  a.sm_scale = scale_of(g);
  a.k_scale = g->k_scale;
  a.v_scale = g->v_scale;
  return a;
}

#define QSA_HIP(call)                                \
  do {                                               \
    if ((call) != hipSuccess) return QSA_ERR_HIP;    \
  } while (0)

// Scratch of qsa_decode_noalloc: a file-scope device array, one copy per
// GPU, alive until the process ends.  Host code never passes the array's
// name to a kernel or a copy (on the host it is only a stand-in for the
// symbol): it uses the device address hipGetSymbolAddress returns for the
// current device, looked up once per device.
constexpr size_t kScratchBytes = (size_t)QSA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`, or null on failure.
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* qsa_status_string(qsa_status s) {
  switch (s) {
    case QSA_OK: return "ok";
    case QSA_ERR_INVALID_ARG: return "invalid argument";
    case QSA_ERR_UNSUPPORTED: return "unsupported geometry";
    case QSA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case QSA_ERR_HIP: return "HIP error";
    case QSA_ERR_TOO_LARGE:
      return "call needs more scratch than the library's static scratch area holds";
  }
  return "unknown status";
}

qsa_status qsa_validate(const qsa_geometry* g) {
  if (!g) return QSA_ERR_INVALID_ARG;
  if (g->head_dim != kHeadDim || g->page_size != kPage || g->compress_ratio != kRatio)
    return QSA_ERR_UNSUPPORTED;
  // the two indexer forms: 8 heads x 64 with a key per head (idx_key_heads
  // 8, or 0), or 4 heads x 128 sharing one key head
  const bool per_head = g->idx_heads == kIdxHeads && g->idx_dim == kIdxDim &&
                        (g->idx_key_heads == kIdxHeads || g->idx_key_heads == 0);
  const bool shared = g->idx_heads == 4 && g->idx_dim == 128 && g->idx_key_heads == 1;
  if (!per_head && !shared) return QSA_ERR_UNSUPPORTED;
  if (g->topk_groups < 1 || g->topk_groups > 2048) return QSA_ERR_UNSUPPORTED;
  if (g->num_kv_heads < 1 || g->num_q_heads < g->num_kv_heads ||
      g->num_q_heads % g->num_kv_heads != 0 || g->num_q_heads / g->num_kv_heads > 16)
    return QSA_ERR_UNSUPPORTED;
  if (g->kv_dtype != QSA_KV_BF16 && g->kv_dtype != QSA_KV_FP8_E4M3) return QSA_ERR_UNSUPPORTED;
  if (!(g->k_scale > 0.0f) || !(g->v_scale > 0.0f) || !isfinite(g->k_scale) ||
      !isfinite(g->v_scale) || !isfinite(g->sm_scale))
    return QSA_ERR_INVALID_ARG;
  return QSA_OK;
}

int32_t qsa_token_width(const qsa_geometry* g, int32_t q_per_req) {
  if (qsa_validate(g) != QSA_OK || q_per_req < 1 || q_per_req > 4) return 0;
  return kRatio * g->topk_groups + (kRatio - 1) + (q_per_req - 1);
}

size_t qsa_index_topk_workspace_size(const qsa_geometry* g, int32_t n_rows, int32_t max_ctx) {
  if (qsa_validate(g) != QSA_OK || n_rows < 0 || max_ctx < 1 || max_ctx > kCapacity) return 0;
  return rows_layout(g, n_rows, max_ctx).total;
}

size_t qsa_decode_workspace_size(const qsa_geometry* g, int32_t batch, int32_t q_per_req,
                                 int32_t max_ctx) {
  if (qsa_validate(g) != QSA_OK || batch < 0 || q_per_req < 1 || q_per_req > 4 || max_ctx < 1 ||
      max_ctx > kCapacity || q_per_req * (g->num_q_heads / g->num_kv_heads) > kMaxRows)
    return 0;
  return decode_layout(g, batch, q_per_req, max_ctx).total;
}

size_t qsa_prefill_workspace_size(const qsa_geometry* g, int32_t n_q, int32_t max_ctx) {
  if (qsa_validate(g) != QSA_OK || n_q < 0 || max_ctx < 1 || max_ctx > kCapacity) return 0;
  return rows_layout(g, n_q, max_ctx).total;
}

qsa_status qsa_index_score(const qsa_geometry* g, const qsa_paged_cache* cache, int32_t n_rows,
                           int32_t max_ctx, const int32_t* row_req, const int32_t* row_len,
                           const float* q_idx, const float* w_idx, float* out_scores,
                           void* stream) {
  qsa_status st = qsa_validate(g);
  if (st != QSA_OK) return st;
  if (n_rows < 0 || max_ctx < 1 || max_ctx > kCapacity || !cache_ok(cache, false))
    return QSA_ERR_INVALID_ARG;
  if (max_ctx > cache->max_pages * kPage) return QSA_ERR_INVALID_ARG;
  if (n_rows == 0) return QSA_OK;
  if (!row_len || !q_idx || !w_idx || !out_scores) return QSA_ERR_INVALID_ARG;
  QSA_HIP(launch_index_score_gemv(cache->khat, cache->page_table, cache->max_pages,
                                  cache->num_pages, n_rows, row_req, row_len, 0, 0, max_ctx,
                                  q_idx, w_idx, out_scores, gstride_of(max_ctx),
                                  (hipStream_t)stream, nullptr, shared_key(g)));
  return QSA_OK;
}

qsa_status qsa_index_score_prefill(const qsa_geometry* g, const qsa_paged_cache* cache,
                                   int32_t req, int32_t first_pos, int32_t n_q, const float* q_idx,
                                   const float* w_idx, float* out_scores, void* stream) {
  qsa_status st = qsa_validate(g);
  if (st != QSA_OK) return st;
  if (req < 0 || first_pos < 0 || n_q < 0 || !cache_ok(cache, false)) return QSA_ERR_INVALID_ARG;
  const long long total = (long long)first_pos + n_q;
  if (total > kCapacity || total > (long long)cache->max_pages * kPage) return QSA_ERR_INVALID_ARG;
  if (n_q == 0) return QSA_OK;
  if (!q_idx || !w_idx || !out_scores) return QSA_ERR_INVALID_ARG;
  QSA_HIP(launch_index_score_prefill(cache->khat, cache->page_table, cache->max_pages,
                                     cache->num_pages, req, first_pos, n_q, q_idx, w_idx,
                                     out_scores, gstride_of((int)total), (hipStream_t)stream,
                                     shared_key(g)));
  return QSA_OK;
}

qsa_status qsa_index_topk(const qsa_geometry* g, const qsa_paged_cache* cache, int32_t n_rows,
                          int32_t max_ctx, const int32_t* row_req, const int32_t* row_len,
                          const float* q_idx, const float* w_idx, int32_t* out_groups,
                          float* out_scores, void* ws, size_t ws_bytes, void* stream) {
  qsa_status st = qsa_validate(g);
  if (st != QSA_OK) return st;
  if (n_rows < 0 || max_ctx < 1 || max_ctx > kCapacity || !cache_ok(cache, false))
    return QSA_ERR_INVALID_ARG;
  if (max_ctx > cache->max_pages * kPage) return QSA_ERR_INVALID_ARG;
  if (n_rows == 0) return QSA_OK;
  if (!row_req || !row_len || !q_idx || !w_idx || !out_groups) return QSA_ERR_INVALID_ARG;
  const RowsLayout lay = rows_layout(g, n_rows, max_ctx);
  if ((st = ws_ok(ws, ws_bytes, lay.total)) != QSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  float* scores = out_scores ? out_scores : (float*)((char*)ws + lay.off_scores);
  float* samples = (float*)((char*)ws + lay.off_samples);
  QSA_HIP(launch_index_score_gemv(cache->khat, cache->page_table, cache->max_pages,
                                  cache->num_pages, n_rows, row_req, row_len, 0, 0, max_ctx,
                                  q_idx, w_idx, scores, lay.gstride, s, samples, shared_key(g)));
  QSA_HIP(launch_topk(scores, lay.gstride, n_rows, row_len, 0, max_ctx, g->topk_groups,
                      out_groups, (char*)ws + lay.off_topk, s, samples));
  return QSA_OK;
}

qsa_status qsa_decode(const qsa_geometry* g, const qsa_paged_cache* cache, int32_t batch,
                      int32_t q_per_req, int32_t max_ctx, const int32_t* ctx_lens,
                      const float* q_idx, const float* w_idx, const uint16_t* q, float* out,
                      int32_t* out_groups, int32_t* out_tokens, float* out_scores, void* ws,
                      size_t ws_bytes, void* stream) {
  qsa_status st = qsa_validate(g);
  if (st != QSA_OK) return st;
  if (batch < 0 || q_per_req < 1 || q_per_req > 4 || max_ctx < 1 || max_ctx > kCapacity ||
      !cache_ok(cache, true))
    return QSA_ERR_INVALID_ARG;
  if (q_per_req * (g->num_q_heads / g->num_kv_heads) > kMaxRows) return QSA_ERR_UNSUPPORTED;
  if (max_ctx > cache->max_pages * kPage) return QSA_ERR_INVALID_ARG;
  if (batch == 0) return QSA_OK;
  if (!ctx_lens || !q_idx || !w_idx || !q || !out) return QSA_ERR_INVALID_ARG;
  const DecodeLayout lay = decode_layout(g, batch, q_per_req, max_ctx);
  if ((st = ws_ok(ws, ws_bytes, lay.total)) != QSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  float* scores = out_scores ? out_scores : (float*)(w + lay.off_scores);
  int32_t* sel = out_groups ? out_groups : (int32_t*)(w + lay.off_sel);
  float* samples = (float*)(w + lay.off_samples);
  // the indexer runs on the base position; draft positions reuse its selection
  QSA_HIP(launch_index_score_gemv(cache->khat, cache->page_table, cache->max_pages,
                                  cache->num_pages, batch, nullptr, ctx_lens, 0, 0,
                                  max_ctx - (q_per_req - 1), q_idx, w_idx, scores, lay.gstride, s,
                                  samples, shared_key(g)));
  QSA_HIP(launch_topk(scores, lay.gstride, batch, ctx_lens, 0, max_ctx - (q_per_req - 1),
                      g->topk_groups, sel, w + lay.off_topk, s, samples));
  AttnArgs a = attn_args(g, cache);
  a.sel = sel;
  a.ctx_lens = ctx_lens;
  a.max_ctx = max_ctx;
  a.q_per_req = q_per_req;
  a.q = q;
  a.batch = batch;
  a.groups_per_split = lay.gps;
  a.n_splits = lay.n_splits;
  a.partial = (float*)(w + lay.off_partial);
  a.out = out;
  QSA_HIP(launch_sparse_attn_decode(a, s));
  if (out_tokens)
    QSA_HIP(launch_expand_tokens(sel, g->topk_groups, batch, q_per_req, ctx_lens, 0, max_ctx,
                                 qsa_token_width(g, q_per_req), out_tokens, s));
  return QSA_OK;
}

qsa_status qsa_prefill(const qsa_geometry* g, const qsa_paged_cache* cache, int32_t req,
                       int32_t first_pos, int32_t n_q, const float* q_idx, const float* w_idx,
                       const uint16_t* q, float* out, int32_t* out_groups, int32_t* out_tokens,
                       float* out_scores, void* ws, size_t ws_bytes, void* stream) {
  qsa_status st = qsa_validate(g);
  if (st != QSA_OK) return st;
  if (req < 0 || first_pos < 0 || n_q < 0 || !cache_ok(cache, true)) return QSA_ERR_INVALID_ARG;
  const long long total = (long long)first_pos + n_q;
  if (total > kCapacity || total > (long long)cache->max_pages * kPage) return QSA_ERR_INVALID_ARG;
  if (n_q == 0) return QSA_OK;
  if (!q_idx || !w_idx || !q || !out) return QSA_ERR_INVALID_ARG;
  const int max_ctx = (int)total;
  const RowsLayout lay = rows_layout(g, n_q, max_ctx);
  if ((st = ws_ok(ws, ws_bytes, lay.total)) != QSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  float* scores = out_scores ? out_scores : (float*)(w + lay.off_scores);
  int32_t* sel = out_groups ? out_groups : (int32_t*)(w + lay.off_sel);
  QSA_HIP(launch_index_score_prefill(cache->khat, cache->page_table, cache->max_pages,
                                     cache->num_pages, req, first_pos, n_q, q_idx, w_idx, scores,
                                     lay.gstride, s, shared_key(g)));
  QSA_HIP(launch_topk(scores, lay.gstride, n_q, nullptr, first_pos, max_ctx, g->topk_groups, sel,
                      w + lay.off_topk, s));
  AttnArgs a = attn_args(g, cache);
  a.sel = sel;
  a.first_pos = first_pos;
  a.req = req;
  a.max_ctx = max_ctx;
  a.q_per_req = 1;
  a.q = q;
  a.batch = n_q;
  a.out = out;
  QSA_HIP(launch_sparse_attn_prefill(a, s));
  if (out_tokens)
    QSA_HIP(launch_expand_tokens(sel, g->topk_groups, n_q, 1, nullptr, first_pos, max_ctx,
                                 qsa_token_width(g, 1), out_tokens, s));
  return QSA_OK;
}

size_t qsa_noalloc_scratch_bytes(void) { return kScratchBytes; }

qsa_status qsa_decode_noalloc(const qsa_geometry* g, const qsa_paged_cache* cache, int32_t batch,
                              int32_t q_per_req, int32_t max_ctx, const int32_t* ctx_lens,
                              const float* q_idx, const float* w_idx, const uint16_t* q,
                              float* out, int32_t* out_groups, int32_t* out_tokens,
                              float* out_scores, void* stream) {
  // the argument checks of qsa_decode, then the size check, all before
  // any HIP call
  qsa_status st = qsa_validate(g);
  if (st != QSA_OK) return st;
  if (batch < 0 || q_per_req < 1 || q_per_req > 4 || max_ctx < 1 || max_ctx > kCapacity ||
      !cache_ok(cache, true))
    return QSA_ERR_INVALID_ARG;
  if (q_per_req * (g->num_q_heads / g->num_kv_heads) > kMaxRows) return QSA_ERR_UNSUPPORTED;
  if (max_ctx > cache->max_pages * kPage) return QSA_ERR_INVALID_ARG;
  if (batch == 0) return QSA_OK;
  if (!ctx_lens || !q_idx || !w_idx || !q || !out) return QSA_ERR_INVALID_ARG;
  const size_t need = decode_layout(g, batch, q_per_req, max_ctx).total;
  if (need > kScratchBytes) return QSA_ERR_TOO_LARGE;
  void* ws = scratch_of_current_device();
  if (!ws) return QSA_ERR_HIP;
  // the decode kernels keep nothing in their workspace between calls, so
  // the scratch needs no clearing
  return qsa_decode(g, cache, batch, q_per_req, max_ctx, ctx_lens, q_idx, w_idx, q, out,
                    out_groups, out_tokens, out_scores, ws, kScratchBytes, stream);
}

int32_t qsa_append_khat_slots(int32_t n_tokens) {
  return n_tokens > 0 ? (n_tokens + kRatio - 1) / kRatio : 0;
}

qsa_status qsa_append_kv(const qsa_geometry* g, void* k_cache, void* v_cache, float* khat_cache,
                         const int32_t* page_table, int32_t max_pages, int32_t num_pages,
                         int32_t n_req, const int32_t* req_rows, const int32_t* start_pos,
                         int32_t n_tokens, const uint16_t* k_new, const uint16_t* v_new,
                         const float* khat_new, void* stream) {
  qsa_status st = qsa_validate(g);
  if (st != QSA_OK) return st;
  if (n_req < 0 || n_tokens < 0 || max_pages < 1 || num_pages < 0) return QSA_ERR_INVALID_ARG;
  if (n_req == 0 || n_tokens == 0) return QSA_OK;
  if (!k_cache || !v_cache || !page_table || !req_rows || !start_pos || !k_new || !v_new)
    return QSA_ERR_INVALID_ARG;
  if (khat_new && !khat_cache) return QSA_ERR_INVALID_ARG;
  if (!(g->k_scale > 0.0f) || !(g->v_scale > 0.0f)) return QSA_ERR_INVALID_ARG;
  QSA_HIP(launch_append(k_cache, v_cache, khat_cache, page_table, max_pages, num_pages, n_req,
                        req_rows, start_pos, n_tokens, k_new, v_new, khat_new,
                        (shared_key(g) ? 1 : g->idx_heads) * g->idx_dim,
                        g->num_kv_heads * g->head_dim, g->kv_dtype, g->k_scale, g->v_scale,
                        (hipStream_t)stream));
  return QSA_OK;
}

}  // extern "C"
