// sparse_attn.hip — grouped-query attention over the expanded QSA token
// selection, read straight from the paged KV cache.
//
// Each selected group g stands for tokens 4g..4g+3 (selections address
// single tokens: TensorRT-LLM QSASparseAttentionConfig,
// get_indices_block_size); the current partial block and, for draft
// positions, the groups completed since the base position follow as one
// contiguous token range (index_share_for_mtp_iteration).  Query head h
// reads KV head h / (Hq / Hkv); a row with no visible token yields zeros
// (OrcaRouter article on SGLang PR #41855, zero-output convention).
//
// One workgroup (4 wavefronts) owns one work item: a KV head, a slice of the
// selection list and the query rows that share it (the GQA heads of one
// query, or of every draft position of a request).  The item's token
// stream is translated once into physical row offsets in LDS; then each
// wavefront walks 16-token sub-tiles of it:
//   S^T[16 tok x 16 rows] = K[16 tok x 256] . Q^T     (8 x mfma 16x16x32 bf16)
//   online softmax per query row (exp2 domain, fp32)
//   O^T[256 x 16 rows]   += V^T[256 x 16 tok] . P^T   (2 x 16 x mfma 16x16x16 bf16,
//                                                      P as a bf16 hi + lo pair)
// K and V go from HBM to registers already in MFMA operand order: lane l
// reads 64 contiguous bytes of token l%16's K row and 16 contiguous bytes
// of four V rows, so no LDS staging or transposition is needed; FP8 E4M3
// elements are widened to bf16 exactly by the hardware converter and the
// per-tensor scales are folded into the logit scale and the final output.
// The contraction dimension is permuted consistently between the two MFMA
// operands (dot products do not depend on the order of d), which is what
// makes those contiguous loads possible.  Waves merge their (max, sum,
// accumulator) through LDS at the end.  Decode splits the selection over
// several workgroups and writes (max, sum, accumulator) partials that
// combine_kernel merges; prefill writes normalised rows directly.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kAccPitch = kHeadDim + 1;  // LDS row pitch of the merged accumulator
constexpr float kLog2e = 1.4426950408889634f;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct ItemDesc {
  int req;           // page-table row
  const int32_t* sel;
  int g_begin, g_end;  // selection-list entries of this item
  int x_begin, x_end;  // contiguous extra tokens of this item
  int base_len;        // query row r sees extra tokens t < base_len + r / gq
};

// Widen 8 FP8 bytes (two dwords) to 8 bf16 (an MFMA operand).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r.x = fp8x2_to_bf16x2<false>(lo);
  r.y = fp8x2_to_bf16x2<true>(lo);
  r.z = fp8x2_to_bf16x2<false>(hi);
  r.w = fp8x2_to_bf16x2<true>(hi);
  return __builtin_bit_cast(bf16x8, r);
}

// Registers of one 16-token sub-tile in flight: lane l holds 64 contiguous
// K bytes (fp8) / 128 bytes (bf16) of token lq = l % 16, and 16 / 32 bytes
// of the V rows of tokens 4*lg + j (lg = l / 16).
template <bool kFp8>
struct SubTile {
  u32x4 k[kFp8 ? 4 : 8];
  u32x4 v[4][kFp8 ? 1 : 2];
  int rv[4];  // physical rows of the four V tokens (-1: absent)
};

// One work item: the 16 query rows row_base .. row_base + 15 (row r =
// position r / gq, head r % gq of the KV head's group; rows >= n_rows are
// padding) over the item's token stream.
template <bool kFp8>
__device__ __forceinline__ void attend_item(const AttnArgs& a, const ItemDesc& it, int kvh,
                                            const uint16_t* q_rows, int q_row_stride,
                                            int row_base, int n_rows, int gq, float* acc_lds,
                                            float* ml_lds, uint16_t* q_lds, int32_t* tok_row,
                                            float* out_final, float* out_partial) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int lq = lane & 15, lg = lane >> 4;
  constexpr int kEsize = kFp8 ? 1 : 2;
  constexpr int kRowBytes = kHeadDim * kEsize;
  constexpr int kQPitch = kHeadDim + 8;  // bf16 elements; spreads the 16 rows over LDS banks

  // ---- token stream -> physical row offsets (page * 64 + slot), -1 if absent
  const int n_groups = max(0, it.g_end - it.g_begin);
  const int n_extra = max(0, it.x_end - it.x_begin);
  const int n_stream = 4 * n_groups + n_extra;
  const int n_sub = (n_stream + 15) / 16;
  const int32_t* pt = a.page_table + (size_t)it.req * a.max_pages;
  // Selected groups: a group's 4 tokens share one page (4 divides the page
  // size), so each thread takes whole groups, kGroupBatch at a time, with
  // all their selection loads issued before any page-table load: a long
  // (prefill) selection then costs two memory round trips per batch, not
  // two per token.
  constexpr int kGroupBatch = 4;
  for (int j0 = 0; j0 < n_groups; j0 += kGroupBatch * kAttnThreads) {
    int gs[kGroupBatch], ph[kGroupBatch];
#pragma unroll
    for (int u = 0; u < kGroupBatch; ++u) {
      const int j = j0 + u * kAttnThreads + tid;
      gs[u] = j < n_groups ? it.sel[it.g_begin + j] : -1;
    }
#pragma unroll
    for (int u = 0; u < kGroupBatch; ++u) ph[u] = gs[u] >= 0 ? pt[(kRatio * gs[u]) / kPage] : -1;
#pragma unroll
    for (int u = 0; u < kGroupBatch; ++u) {
      const int j = j0 + u * kAttnThreads + tid;
      if (j < n_groups) {
        int4 r = make_int4(-1, -1, -1, -1);
        if (gs[u] >= 0 && ph[u] >= 0 && ph[u] < a.num_pages) {
          const int base = ph[u] * kPage + (kRatio * gs[u]) % kPage;
          r = make_int4(base, base + 1, base + 2, base + 3);
        }
        *reinterpret_cast<int4*>(tok_row + kRatio * j) = r;
      }
    }
  }
  // the contiguous extra tokens, then padding to whole sub-tiles
  for (int i = kRatio * n_groups + tid; i < n_sub * 16; i += kAttnThreads) {
    int r = -1;
    if (i < n_stream) {
      const int t = it.x_begin + (i - kRatio * n_groups);
      const int phys = pt[t / kPage];
      if (phys >= 0 && phys < a.num_pages) r = phys * kPage + (t % kPage);
    }
    tok_row[i] = r;
  }
  // ---- the 16 query rows into LDS (zeros for padding rows)
  for (int i = tid; i < 16 * (kHeadDim / 8); i += kAttnThreads) {
    const int rl = i / (kHeadDim / 8), c = i % (kHeadDim / 8);
    const int r = row_base + rl;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < n_rows)
      v = *reinterpret_cast<const u32x4*>(q_rows + (size_t)(r / gq) * q_row_stride +
                                          (size_t)(r % gq) * kHeadDim + 8 * c);
    *reinterpret_cast<u32x4*>(q_lds + rl * kQPitch + 8 * c) = v;
  }
  __syncthreads();

  // causal limit of this lane's query row (only extra tokens can exceed it)
  const int limit = it.base_len + (row_base + lq) / gq;
  const float qk_scale = a.sm_scale * a.k_scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.0f;
  float4_t acc[16];
#pragma unroll
  for (int mb = 0; mb < 16; ++mb) acc[mb] = (float4_t){0.f, 0.f, 0.f, 0.f};

  const uint8_t* kc = reinterpret_cast<const uint8_t*>(a.k);
  const uint8_t* vc = reinterpret_cast<const uint8_t*>(a.v);
  const int Hkv = a.Hkv;

  // K rows are fetched in four 16-byte pieces by separate instructions, so
  // they are cached normally (the pieces meet in L2); each lane's V piece is
  // read once, whole, and streamed past the caches.
  auto load = [&](SubTile<kFp8>& b, int s) {
    const int rk = tok_row[16 * s + lq];
    const uint8_t* kp = kc + ((size_t)max(rk, 0) * Hkv + kvh) * kRowBytes + 64 * lg * kEsize;
#pragma unroll
    for (int i = 0; i < (kFp8 ? 4 : 8); ++i) b.k[i] = *reinterpret_cast<const u32x4*>(kp + 16 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b.rv[j] = tok_row[16 * s + 4 * lg + j];
      const uint8_t* vp = vc + ((size_t)max(b.rv[j], 0) * Hkv + kvh) * kRowBytes + 16 * lq * kEsize;
#pragma unroll
      for (int i = 0; i < (kFp8 ? 1 : 2); ++i) b.v[j][i] = stream_load_u4(vp + 16 * i);
    }
  };

  auto compute = [&](const SubTile<kFp8>& b, int s) {
    // S^T = K . Q^T (Q operand from LDS: row lq, d = 64*lg + 8*ks + 0..7)
    float4_t sc = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bf16x8 kop;
      if (kFp8) {
        const u32x4 w = b.k[ks / 2];
        kop = (ks & 1) ? fp8x8_to_bf16x8(w.z, w.w) : fp8x8_to_bf16x8(w.x, w.y);
      } else {
        kop = __builtin_bit_cast(bf16x8, b.k[ks]);
      }
      const bf16x8 qop = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(q_lds + lq * kQPitch + 64 * lg + 8 * ks));
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop, sc, 0, 0, 0);
    }
    // token of D row 4*lg + i is stream entry 16s + 4*lg + i (= V token i)
    float sv[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int si = 16 * s + 4 * lg + i;
      const int tok = si < 4 * n_groups ? -1 : it.x_begin + (si - 4 * n_groups);  // -1: visible
      const bool vis = b.rv[i] >= 0 && tok < limit;
      sv[i] = vis ? sc[i] * qk_scale : -INFINITY;
      tmax = fmaxf(tmax, sv[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    // Lazy running max: the accumulators (held in AGPRs) are rescaled only
    // when a row's max grows by more than 2^8, so weights stay <= 256.
    const bool grow = tmax > m_run + 8.0f;
    if (__any(grow)) {
      const float m_new = grow ? tmax : m_run;
      const float alpha = (m_run == -INFINITY || m_new == -INFINITY) ? 1.0f : exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < 16; ++mb) acc[mb] *= alpha;
      m_run = m_new;
    }
    // weights as a bf16 hi + lo pair (~16 significant bits) for the PV MFMA
    float psum = 0.0f;
    uint32_t hb[4], lb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = (m_run == -INFINITY) ? 0.0f : exp2f(sv[i] - m_run);
      hb[i] = bf16_rne_bits(p);
      lb[i] = bf16_rne_bits(p - __uint_as_float(hb[i] << 16));
      psum += p;
    }
    l_run += psum;
    const short4_t p_hi = (short4_t){(short)hb[0], (short)hb[1], (short)hb[2], (short)hb[3]};
    const short4_t p_lo = (short4_t){(short)lb[0], (short)lb[1], (short)lb[2], (short)lb[3]};
    // O^T += V^T . P^T; m-block mb holds d = 64*lg' + 16*i + mb for D row 4*lg' + i
#pragma unroll
    for (int qd = 0; qd < 8; ++qd) {
      uint32_t cv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (kFp8) {
          const u32x4 w = b.rv[j] >= 0 ? b.v[j][0] : (u32x4){0u, 0u, 0u, 0u};
          const uint32_t word = qd < 2 ? w.x : qd < 4 ? w.y : qd < 6 ? w.z : w.w;
          cv[j] = (qd & 1) ? fp8x2_to_bf16x2<true>(word) : fp8x2_to_bf16x2<false>(word);
        } else {
          const u32x4 w = b.rv[j] >= 0 ? b.v[j][qd / 4] : (u32x4){0u, 0u, 0u, 0u};
          const int e = qd % 4;
          cv[j] = e == 0 ? w.x : e == 1 ? w.y : e == 2 ? w.z : w.w;
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int mb = 2 * qd + h;
        const uint32_t sel = h ? 0x07060302u : 0x05040100u;
        const uint32_t lo = __builtin_amdgcn_perm(cv[1], cv[0], sel);
        const uint32_t hi = __builtin_amdgcn_perm(cv[3], cv[2], sel);
        const short4_t vop = __builtin_bit_cast(short4_t, (u32x2){lo, hi});
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, p_hi, acc[mb], 0, 0, 0);
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, p_lo, acc[mb], 0, 0, 0);
      }
    }
  };

  // ---- main loop: rounds of kNS sub-tiles per wave (sub-tiles
  // wave + 4*i); a round issues all of its loads before computing any of
  // them, so one memory latency covers kNS sub-tiles
  constexpr int kNS = kFp8 ? 2 : 1;
  for (int s0 = wave; s0 < n_sub; s0 += kNS * kAttnWaves) {
    SubTile<kFp8> bt[kNS];
#pragma unroll
    for (int i = 0; i < kNS; ++i)
      if (s0 + i * kAttnWaves < n_sub) load(bt[i], s0 + i * kAttnWaves);
#pragma unroll
    for (int i = 0; i < kNS; ++i)
      if (s0 + i * kAttnWaves < n_sub) compute(bt[i], s0 + i * kAttnWaves);
  }

  // ---- merge the 4 waves.  Each wave publishes its row maxima and sums,
  // then writes its accumulators, rescaled to the row's common max, into
  // its own LDS slice; the block sums the slices while writing out.
  {
    float l = l_run;
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    if (lg == 0) {
      ml_lds[wave * 32 + lq] = m_run;
      ml_lds[wave * 32 + 16 + lq] = l;
    }
  }
  __syncthreads();
  const int rows_here = min(16, n_rows - row_base);
  {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, ml_lds[w * 32 + lq]);
    const float fac = (M == -INFINITY || m_run == -INFINITY) ? 0.0f : exp2f(m_run - M);
    if (lq < rows_here) {
      float* rowp = acc_lds + ((size_t)wave * 16 + lq) * kAccPitch;
#pragma unroll
      for (int mb = 0; mb < 16; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) rowp[64 * lg + 16 * i + mb] = acc[mb][i] * fac;
    }
  }
  // row statistics: common max and the sum of the rescaled row sums
  if (tid < 16) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, ml_lds[w * 32 + tid]);
    float Lsum = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float mw = ml_lds[w * 32 + tid];
        if (mw != -INFINITY) Lsum += exp2f(mw - M) * ml_lds[w * 32 + 16 + tid];
      }
    }
    ml_lds[kAttnWaves * 32 + tid] = M;
    ml_lds[kAttnWaves * 32 + 16 + tid] = Lsum;
  }
  __syncthreads();

  // ---- write: normalised rows, or (max, sum, accumulator) partials
  for (int e = tid; e < rows_here * kHeadDim; e += kAttnThreads) {
    const int r = e / kHeadDim, d = e % kHeadDim;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) v += acc_lds[((size_t)w * 16 + r) * kAccPitch + d];
    const int rg = row_base + r;
    if (out_final) {
      const float Lsum = ml_lds[kAttnWaves * 32 + 16 + r];
      out_final[(size_t)(rg / gq) * ((size_t)a.Hq * kHeadDim) + (size_t)(rg % gq) * kHeadDim + d] =
          Lsum > 0.0f ? v * (a.v_scale / Lsum) : 0.0f;
    } else {
      out_partial[(size_t)rg * (2 + kHeadDim) + 2 + d] = v;
    }
  }
  if (!out_final && tid < rows_here) {
    out_partial[(size_t)(row_base + tid) * (2 + kHeadDim)] = ml_lds[kAttnWaves * 32 + tid];
    out_partial[(size_t)(row_base + tid) * (2 + kHeadDim) + 1] = ml_lds[kAttnWaves * 32 + 16 + tid];
  }
}

// Dynamic LDS: the row statistics, then one region that holds the query
// tile and the token rows during the main loop and the per-wave
// accumulators during the merge (the barrier before the merge writes
// separates the two uses).
constexpr int kQLdsElems = 16 * (kHeadDim + 8);
constexpr int kMlFloats = (kAttnWaves + 1) * 32;

template <bool kFp8>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_decode_kernel(AttnArgs a) {
  extern __shared__ float smem[];
  const int gq = a.Hq / a.Hkv;
  const int Q = a.q_per_req;
  const int n_rows = Q * gq;
  const int nblk = (n_rows + 15) / 16;
  const int split = blockIdx.x / nblk, rb = blockIdx.x % nblk;
  const int kvh = blockIdx.y, b = blockIdx.z;
  float* ml_lds = smem;
  float* acc_lds = smem + kMlFloats;
  uint16_t* q_lds = reinterpret_cast<uint16_t*>(acc_lds);
  int32_t* tok_row = reinterpret_cast<int32_t*>(q_lds + kQLdsElems);

  const int L0 = a.ctx_lens[b];
  const bool valid = L0 >= 0 && L0 <= a.max_ctx - (Q - 1);
  const int G = valid ? L0 / kRatio : 0;
  const int n_valid = min(a.K, G);
  ItemDesc it;
  it.req = b;
  it.sel = a.sel + (size_t)b * a.K;
  it.g_begin = split * a.groups_per_split;
  it.g_end = min(n_valid, it.g_begin + a.groups_per_split);
  const bool last = split == a.n_splits - 1;
  it.x_begin = kRatio * G;
  it.x_end = (valid && last) ? L0 + Q - 1 : kRatio * G;
  it.base_len = L0;

  const uint16_t* q_rows = a.q + ((size_t)b * Q * a.Hq + (size_t)kvh * gq) * kHeadDim;
  float* part = a.partial + (((size_t)b * a.Hkv + kvh) * a.n_splits + split) * n_rows * (2 + kHeadDim);
  attend_item<kFp8>(a, it, kvh, q_rows, a.Hq * kHeadDim, rb * 16, n_rows, gq, acc_lds, ml_lds,
                    q_lds, tok_row, nullptr, part);
}

template <bool kFp8>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_prefill_kernel(AttnArgs a) {
  extern __shared__ float smem[];
  const int qi = blockIdx.x, kvh = blockIdx.y;
  const int gq = a.Hq / a.Hkv;
  float* ml_lds = smem;
  float* acc_lds = smem + kMlFloats;
  uint16_t* q_lds = reinterpret_cast<uint16_t*>(acc_lds);
  int32_t* tok_row = reinterpret_cast<int32_t*>(q_lds + kQLdsElems);

  const int L = a.first_pos + qi + 1;
  const int G = L / kRatio;
  ItemDesc it;
  it.req = a.req;
  it.sel = a.sel + (size_t)qi * a.K;
  it.g_begin = 0;
  it.g_end = min(a.K, G);
  it.x_begin = kRatio * G;
  it.x_end = L;
  it.base_len = L;
  const uint16_t* q_rows = a.q + ((size_t)qi * a.Hq + (size_t)kvh * gq) * kHeadDim;
  float* outp = a.out + ((size_t)qi * a.Hq + (size_t)kvh * gq) * kHeadDim;
  attend_item<kFp8>(a, it, kvh, q_rows, 0, 0, gq, gq, acc_lds, ml_lds, q_lds, tok_row, outp,
                    nullptr);
}

// Merge split partials: out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
// Thread s first fetches split s's (m, l) so all splits are read at once;
// then thread d sums the accumulators with independent loads.
constexpr int kMaxSplits = kHeadDim;
__global__ __launch_bounds__(kHeadDim) void combine_kernel(const float* __restrict__ partial,
                                                           int n_splits, int Hq, int Hkv, int Q,
                                                           float v_scale, float* __restrict__ out) {
  __shared__ float fac[kMaxSplits];
  __shared__ float red[kHeadDim / kWave];
  const int h = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int gq = Hq / Hkv, kvh = h / gq, r = j * gq + (h % gq);
  const int R = Q * gq;
  const size_t split_stride = (size_t)R * (2 + kHeadDim);
  const float* p = partial + ((size_t)(b * Hkv + kvh) * n_splits) * split_stride +
                   (size_t)r * (2 + kHeadDim);
  const int t = threadIdx.x, lane = t & (kWave - 1), wid = t / kWave;
  // the first kEarly splits' accumulators are fetched together with the
  // (max, sum) pairs, so both come back in one memory round trip
  constexpr int kEarly = 32;
  float early[kEarly];
#pragma unroll
  for (int s = 0; s < kEarly; ++s) early[s] = s < n_splits ? p[s * split_stride + 2 + t] : 0.0f;
  const float m = t < n_splits ? p[t * split_stride] : -INFINITY;
  const float l = t < n_splits ? p[t * split_stride + 1] : 0.0f;
  float M = wave_max(m);
  if (lane == 0) red[wid] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float f = (m == -INFINITY) ? 0.0f : exp2f(m - M);
  fac[t] = f;  // 0 for t >= n_splits (m = -inf there)
  __syncthreads();
  float den = wave_sum(f * l);
  if (lane == 0) red[wid] = den;  // (every thread has read red[] above)
  __syncthreads();
  den = (red[0] + red[1]) + (red[2] + red[3]);
  float num = 0.0f;
#pragma unroll
  for (int s = 0; s < kEarly; ++s) num += fac[s] * early[s];  // fac[s] = 0 past n_splits
#pragma unroll 8
  for (int s = kEarly; s < n_splits; ++s) num += fac[s] * p[s * split_stride + 2 + t];
  out[(((size_t)b * Q + j) * Hq + h) * kHeadDim + t] = den > 0.0f ? num * (v_scale / den) : 0.0f;
}

// Token lists: slot i < 4*n_valid -> 4*sel[i/4] + i%4; then the extra range.
__global__ void expand_tokens_kernel(const int32_t* __restrict__ sel, int K,
                                     const int32_t* __restrict__ ctx_lens, int first_pos,
                                     int max_ctx, int Q, int width, int32_t* __restrict__ out) {
  const int row = blockIdx.x, j = blockIdx.y;
  const int L0 = ctx_lens ? ctx_lens[row] : first_pos + row + 1;
  const bool valid = L0 >= 0 && L0 <= max_ctx - (Q - 1);
  const int G = valid ? L0 / kRatio : 0;
  const int n_valid = min(K, G);
  const int n_extra = valid ? L0 + j - kRatio * G : 0;
  int32_t* o = out + ((size_t)row * Q + j) * width;
  const int32_t* s = sel + (size_t)row * K;
  for (int i = threadIdx.x; i < width; i += blockDim.x) {
    int t = -1;
    if (i < kRatio * n_valid) t = kRatio * s[i / kRatio] + (i % kRatio);
    else if (i - kRatio * n_valid < n_extra) t = kRatio * G + (i - kRatio * n_valid);
    o[i] = t;
  }
}

size_t attn_smem_bytes(int stream_cap) {
  const size_t acc = sizeof(float) * (size_t)kAttnWaves * 16 * kAccPitch;
  const size_t loop = sizeof(uint16_t) * (size_t)kQLdsElems +
                      sizeof(int32_t) * (size_t)((stream_cap + 15) / 16 * 16);
  return sizeof(float) * (size_t)kMlFloats + (acc > loop ? acc : loop);
}

template <bool kFp8>
hipError_t launch_decode_t(const AttnArgs& a, hipStream_t stream) {
  if (a.n_splits > kMaxSplits) return hipErrorInvalidValue;
  const int cap = 4 * a.groups_per_split + 3 + (a.q_per_req - 1);
  const size_t smem = attn_smem_bytes(cap);
  const int rows = a.q_per_req * (a.Hq / a.Hkv);
  const int nblk = (rows + 15) / 16;
  dim3 grid(a.n_splits * nblk, a.Hkv, a.batch);
  hipLaunchKernelGGL((attn_decode_kernel<kFp8>), grid, dim3(kAttnThreads), smem, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 cgrid(a.Hq, a.q_per_req, a.batch);
  hipLaunchKernelGGL(combine_kernel, cgrid, dim3(kHeadDim), 0, stream, a.partial, a.n_splits, a.Hq,
                     a.Hkv, a.q_per_req, a.v_scale, a.out);
  return hipGetLastError();
}

template <bool kFp8>
hipError_t launch_prefill_t(const AttnArgs& a, hipStream_t stream) {
  if (a.Hq / a.Hkv > 16) return hipErrorInvalidValue;
  const size_t smem = attn_smem_bytes(4 * a.K + 3);
  dim3 grid(a.batch, a.Hkv);
  hipLaunchKernelGGL((attn_prefill_kernel<kFp8>), grid, dim3(kAttnThreads), smem, stream, a);
  return hipGetLastError();
}

// One 16-row block per workgroup: query rows beyond 16 (e.g. 12 heads x 3
// draft positions) take further workgroups over the same tokens, which
// then mostly come from the caches.
hipError_t dispatch(const AttnArgs& a, hipStream_t stream, bool prefill) {
  if (a.kv_dtype == 1)
    return prefill ? launch_prefill_t<true>(a, stream) : launch_decode_t<true>(a, stream);
  return prefill ? launch_prefill_t<false>(a, stream) : launch_decode_t<false>(a, stream);
}

}  // namespace

hipError_t launch_sparse_attn_decode(const AttnArgs& a, hipStream_t stream) {
  if (a.batch <= 0) return hipSuccess;
  return dispatch(a, stream, false);
}

hipError_t launch_sparse_attn_prefill(const AttnArgs& a, hipStream_t stream) {
  if (a.batch <= 0) return hipSuccess;
  return dispatch(a, stream, true);
}

hipError_t launch_expand_tokens(const int32_t* sel, int K, int n_rows, int q_per_req,
                                const int32_t* ctx_lens, int first_pos, int max_ctx, int width,
                                int32_t* out, hipStream_t stream) {
  if (n_rows <= 0) return hipSuccess;
  dim3 grid(n_rows, q_per_req);
  hipLaunchKernelGGL(expand_tokens_kernel, grid, dim3(256), 0, stream, sel, K, ctx_lens, first_pos,
                     max_ctx, q_per_req, width, out);
  return hipGetLastError();
}

}  // namespace qsa
