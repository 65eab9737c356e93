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
// Decode: one workgroup (4 wavefronts) owns one work item: a KV head, a
// slice of the selection list and the query rows that share it (the GQA
// heads of one query, or of every draft position of a request).  The
// item's token stream is translated once into physical row offsets in LDS;
// then each wavefront walks 16-token sub-tiles of it:
//   S^T[16 tok x 16 rows] = K[16 tok x 256] . Q^T     (8 x mfma 16x16x32 bf16)
//   online softmax per query row (exp2 domain, fp32)
//   O^T[256 x 16 rows]   += V^T[256 x 16 tok] . P^T   (2 x 16 x mfma 16x16x16 bf16,
//                                                      P as a bf16 hi + lo pair)
// Waves merge their (max, sum, accumulator) through LDS, and combine_kernel
// merges the partials of the workgroups the selection is split over.
// Prefill: one wavefront per (query, KV head) walks the query's whole
// selection with the same sub-tile step and writes normalised rows.  The
// wavefronts of an XCD share its L2 only while they sweep nearby tokens;
// random selections let them drift apart, so where the expected drift is
// large (BF16 rows, sparse selections) a wavefront that runs ahead in the
// token space waits (pacing; timing only, the order of work is unchanged).
//
// V goes from HBM to registers already in MFMA operand order (16 lanes
// read 256 contiguous bytes of one token's row).  K is loaded with
// contiguous lane quads into a per-wavefront LDS tile and read back as
// operands (see the K-through-LDS helpers).  FP8 E4M3 elements are widened
// to bf16 exactly by the hardware converter and the per-tensor scales are
// folded into the logit scale and the final output.  The contraction
// dimension is permuted consistently between the two MFMA operands (dot
// products do not depend on the order of d), which is what makes those
// contiguous loads possible.
#include <algorithm>
#include <cmath>

#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;
// LDS rows of the merged accumulator: dimension d of a row sits at float
// acc_col(d) = d + d / 64 of a 260-float row.  A wavefront stores the
// accumulators of one (i, mb) pair at once, lane (lq, lg) writing
// dimension out_dim(lg, i, mb) of row lq; with the pitch = 4 (mod 64) and
// the skew, the 64 lanes of an FP8 store land on 64 different banks (a
// 257-float pitch put the four lane groups on one bank).
constexpr int kAccPitch = kHeadDim + 4;
__device__ __forceinline__ int acc_col(int d) { return d + (d >> 6); }
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

// Dimension order.  A dot product does not depend on the order of its terms,
// so the contraction index of S^T = K . Q^T is permuted identically in both
// operands; in k-step ks, lane group lg supplies
//   bf16 K: d = 32*ks + 8*lg + 0..7,
//   fp8 K:  d = 64*(ks/2) + 16*lg + 8*(ks%2) + 0..7 (one 16-byte chunk of
//           the row serves two k-steps),
// so each K operand is one 16-byte chunk of the token's row in LDS.
// The output dimension of O^T = V^T . P^T is permuted through the V^T
// operand: lane lq of m-block mb supplies d = dv(lq, mb) with
//   bf16 V: dv = 8*lq + (mb % 8) + 128*(mb / 8) (two loads of 256
//           contiguous bytes per token across the 16 lanes),
//   fp8 V:  dv = 16*lq + mb (one load of the whole 256-byte row);
// so accumulator acc[mb][i] of lane (lq, lg) holds output dimension
// dv(4*lg + i, mb) of query row lq (out_dim below).

// First of the 8 dimensions that k-step ks of lane group lg covers.
template <bool kFp8>
__device__ __forceinline__ int qk_dim(int ks, int lg) {
  return kFp8 ? 64 * (ks >> 1) + 16 * lg + 8 * (ks & 1) : 32 * ks + 8 * lg;
}

// Output dimension held in accumulator acc[mb][i] of lane group lg.
template <bool kFp8>
__device__ __forceinline__ int out_dim(int lg, int i, int mb) {
  const int r = 4 * lg + i;
  return kFp8 ? 16 * r + mb : 8 * r + (mb & 7) + 128 * (mb >> 3);
}

// Loads the V part of one sub-tile in MFMA operand order: rv[j] = row of
// token 4*lg + j; fp8: bytes 16*lq .. +15 of its V row, bf16: elements
// 8*lq + 128*i .. +7 (i = 0, 1).  kStreamV reads past the caches (decode
// reads each selected row once).
template <bool kFp8, bool kStreamV>
__device__ __forceinline__ void load_v_rows(u32x4 (&v)[4][kFp8 ? 1 : 2], int (&rv)[4],
                                            const int32_t* tok, const uint8_t* vc, int Hkv,
                                            int kvh) {
  const int lane = threadIdx.x & (kWave - 1), lq = lane & 15, lg = lane >> 4;
  constexpr int kRowBytes = kHeadDim * (kFp8 ? 1 : 2);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    rv[j] = tok[4 * lg + j];
    const uint8_t* vp = vc + ((size_t)max(rv[j], 0) * Hkv + kvh) * kRowBytes + 16 * lq;
#pragma unroll
    for (int i = 0; i < (kFp8 ? 1 : 2); ++i)
      v[j][i] = kStreamV ? stream_load_u4(vp + 256 * i)
                         : *reinterpret_cast<const u32x4*>(vp + 256 * i);
  }
}

// K rows through LDS.  Read straight into MFMA operand order, the 64
// lanes of one load instruction would touch 16
// different rows with adjacent lanes in different rows, so no four lanes
// would share a 64-byte segment and the vector L1 would serve 64 separate
// accesses per instruction, four times the 16 of a load whose lane quads
// read contiguous 64 bytes; where the gathers run at L1 rate, that access
// count bounds them.  Instead lane 4t + c reads bytes 64j + 16c of token t's row in load
// j (contiguous quads), stores them to a per-wavefront LDS tile, and the
// operands are read back per k-step.  The 16-byte chunk k of token t's row
// sits at chunk position k ^ k_swizzle(t) of LDS row t.  This XOR pattern
// was picked by measurement (rocprofv3 SQ_LDS_BANK_CONFLICT over probes of
// all candidate patterns): it leaves both the 16-byte stores (lane 4t + c,
// chunk 4j + c) and the operand reads (lane lq + 16 lg, chunk 4 ks + lg)
// without bank conflicts for every j and ks; other patterns that a plain
// bank model calls conflict-free cost the reads 4 cycles per instruction.
__device__ __forceinline__ int k_swizzle(int t) {
  return ((t & 1) ? 4 : 0) ^ ((t & 2) ? 1 : 0) ^ ((t & 4) ? 2 : 0) ^ ((t & 8) ? 8 : 0);
}

// Bytes of one sub-tile's K rows in LDS (16 tokens).
template <bool kFp8>
__host__ __device__ constexpr int k_tile_bytes() {
  return 16 * kHeadDim * (kFp8 ? 1 : 2);
}

// Loads one sub-tile's K rows with contiguous lane quads: load j of lane
// 4t + c holds bytes 64j + 16c of the row of token tok[t] (-1: row 0).
template <bool kFp8>
__device__ __forceinline__ void load_k_quads(u32x4 (&k)[kFp8 ? 4 : 8], const int32_t* tok,
                                             const uint8_t* kc, int Hkv, int kvh) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int kRowBytes = kHeadDim * (kFp8 ? 1 : 2);
  const uint8_t* kp =
      kc + ((size_t)max(tok[lane >> 2], 0) * Hkv + kvh) * kRowBytes + 16 * (lane & 3);
#pragma unroll
  for (int j = 0; j < (kFp8 ? 4 : 8); ++j) k[j] = *reinterpret_cast<const u32x4*>(kp + 64 * j);
}

// Stores load_k_quads' registers into the wavefront's LDS tile.
template <bool kFp8>
__device__ __forceinline__ void store_k_tile(const u32x4 (&k)[kFp8 ? 4 : 8], uint8_t* tile) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int kRowBytes = kHeadDim * (kFp8 ? 1 : 2);
  const int t = lane >> 2, c = lane & 3, sw = k_swizzle(t);
#pragma unroll
  for (int j = 0; j < (kFp8 ? 4 : 8); ++j)
    *reinterpret_cast<u32x4*>(tile + t * kRowBytes + 16 * ((4 * j + c) ^ sw)) = k[j];
}

// The BF16 K operand of k-step ks (token lq, dims qk_dim(ks, lg) + 0..7)
// from the LDS tile; sw = k_swizzle(lq).
__device__ __forceinline__ bf16x8 k_operand_lds_bf16(const uint8_t* tile, int ks, int lq, int lg,
                                                     int sw) {
  return *reinterpret_cast<const bf16x8*>(tile + lq * (2 * kHeadDim) + 16 * ((4 * ks + lg) ^ sw));
}

// LDS of one wavefront's K tile (room for either element type)
constexpr int kItemKBytesPerWave = k_tile_bytes<false>();

// S^T = K . Q^T of one sub-tile (16 tokens x 16 query rows): k-step ks
// takes the K operand kop(ks) (token lq, dims qk_dim(ks, lg) + 0..7, as
// bf16) and the Q^T operand qop(ks) (row lq, the same dims).
template <typename KOp, typename QOp>
__device__ __forceinline__ float4_t subtile_logits(KOp kop, QOp qop) {
  float4_t sc = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop(ks), __builtin_bit_cast(bf16x8, qop(ks)), sc,
                                                0, 0, 0);
  return sc;
}

// S^T = K . Q^T of one sub-tile with K from the LDS tile (sw =
// k_swizzle(lq)) and the Q^T operand qop(ks).  For FP8 the four 16-byte
// chunks of the lane's row are read whole before the products: each serves
// two k-steps, and reading each k-step's half on its own (two dwords, which
// the compiler does when one half is used at a time) costs those reads
// two-way bank conflicts.
template <bool kFp8, typename QOp>
__device__ __forceinline__ float4_t subtile_logits_lds(const uint8_t* tile, int lq, int lg, int sw,
                                                       QOp qop) {
  if constexpr (kFp8) {
    u32x4 c[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      c[m] = *reinterpret_cast<const u32x4*>(tile + lq * kHeadDim + 16 * ((4 * m + lg) ^ sw));
    return subtile_logits(
        [&](int ks) {
          const u32x4 w = c[ks >> 1];
          return (ks & 1) ? fp8x8_to_bf16x8(w.z, w.w) : fp8x8_to_bf16x8(w.x, w.y);
        },
        qop);
  } else {
    return subtile_logits([&](int ks) { return k_operand_lds_bf16(tile, ks, lq, lg, sw); }, qop);
  }
}

// The online-softmax update of one sub-tile from its logits sc: the
// weights of the visible tokens (vis[i] for D row 4*lg + i) update the
// running max m_run, sum l_run and the O^T accumulators acc with V^T . P^T.
template <bool kFp8>
__device__ __forceinline__ void subtile_accumulate(float4_t sc, u32x4 (&v)[4][kFp8 ? 1 : 2],
                                                   const int (&rv)[4], const bool (&vis)[4],
                                                   float qk_scale, float& m_run, float& l_run,
                                                   float4_t (&acc)[16]) {
  // Absent tokens (padding, out-of-range pages) were loaded from row 0 of
  // the cache, which may hold anything: their V operands are cleared so a
  // zero weight cannot meet a NaN.  Nearly every sub-tile is full, so the
  // clearing runs only when the wavefront holds an absent token.
  if (!__all(rv[0] >= 0 && rv[1] >= 0 && rv[2] >= 0 && rv[3] >= 0)) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < (kFp8 ? 1 : 2); ++i)
        if (rv[j] < 0) v[j][i] = (u32x4){0u, 0u, 0u, 0u};
  }
  float sv[4];
  float tmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sv[i] = vis[i] ? sc[i] * qk_scale : -INFINITY;
    tmax = fmaxf(tmax, sv[i]);
  }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
  // Lazy running max: the accumulators are rescaled only when a row's max
  // grows by more than 2^8, so weights stay <= 256.
  const bool grow = tmax > m_run + 8.0f;
  if (__any(grow)) {
    const float m_new = grow ? tmax : m_run;
    const float alpha = (m_run == -INFINITY || m_new == -INFINITY) ? 1.0f : exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int mb = 0; mb < 16; ++mb) acc[mb] *= alpha;
    m_run = m_new;
  }
  // The weights for the P.V MFMA.  BF16 K/V: a bf16 hi + lo pair (~16
  // significant bits), which keeps the output within ~1e-6 of exact.  FP8
  // K/V: one bf16 value per weight (V itself carries 3 mantissa bits), and
  // the sum l takes the rounded weights, so the output is exactly the
  // average of V under those weights: max-abs error ~4e-4 against 2e-2
  // allowed, 16 fewer MFMAs per sub-tile (measured: FP8 prefill attention
  // 796-814 -> 692-701 us, decode 195.85 -> 195.05 us per step; with BF16
  // K/V the single form measured slower, 951 -> 1,108-1,139 us).
  float psum = 0.0f;
  uint32_t hb[4], lb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float pw = (m_run == -INFINITY) ? 0.0f : exp2f(sv[i] - m_run);
    hb[i] = bf16_rne_bits(pw);
    if (kFp8) {
      psum += __uint_as_float(hb[i] << 16);
    } else {
      lb[i] = bf16_rne_bits(pw - __uint_as_float(hb[i] << 16));
      psum += pw;
    }
  }
  l_run += psum;
  const short4_t p_hi = (short4_t){(short)hb[0], (short)hb[1], (short)hb[2], (short)hb[3]};
  short4_t p_lo = {};
  if (!kFp8) p_lo = (short4_t){(short)lb[0], (short)lb[1], (short)lb[2], (short)lb[3]};
  // O^T += V^T . P^T; m-block mb holds d = out_dim(lg', i, mb) for D row 4*lg' + i
#pragma unroll
  for (int qd = 0; qd < 8; ++qd) {
    uint32_t cv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (kFp8) {
        const u32x4 w = v[j][0];
        const uint32_t word = qd < 2 ? w.x : qd < 4 ? w.y : qd < 6 ? w.z : w.w;
        cv[j] = (qd & 1) ? fp8x2_to_bf16x2<true>(word) : fp8x2_to_bf16x2<false>(word);
      } else {
        const u32x4 w = v[j][qd / 4];
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
      if (!kFp8) acc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, p_lo, acc[mb], 0, 0, 0);
    }
  }
}


// One decode work item: the 16 query rows row_base .. row_base + 15 (row
// r = position r / gq, head r % gq of the KV head's group; rows >= n_rows
// are padding) over the item's token stream, written as (max, sum,
// accumulator) partial rows.  V rows are read past the caches (decode
// reads each selected row once); K rows go through the wavefronts' LDS
// tiles at k_lds (kAttnWaves x kItemKBytesPerWave bytes).
template <bool kFp8>
__device__ __forceinline__ void attend_item(const AttnArgs& a, const ItemDesc& it, int kvh,
                                            const uint16_t* q_rows, int q_row_stride,
                                            int row_base, int n_rows, int gq, float* acc_lds,
                                            float* ml_lds, uint16_t* q_lds, uint8_t* k_lds,
                                            int32_t* tok_row, float* out_partial) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int lq = lane & 15, lg = lane >> 4;
  // bf16 elements (544 bytes): the operand reads of the 16 rows hit every
  // LDS bank once (measured: a 528-byte pitch costs each read 4 conflict
  // cycles)
  constexpr int kQPitch = kHeadDim + 16;

  // ---- token stream -> physical row offsets (page * 64 + slot), -1 if absent
  const int n_groups = max(0, it.g_end - it.g_begin);
  const int n_extra = max(0, it.x_end - it.x_begin);
  const int n_stream = 4 * n_groups + n_extra;
  const int n_sub = (n_stream + 15) / 16;
  const int32_t* pt = a.page_table + (size_t)it.req * a.max_pages;
  // Selected groups: a group's 4 tokens share one page (4 divides the page
  // size), so each thread takes whole groups, kGroupBatch at a time, with
  // all their selection loads issued before any page-table load: a long
  // selection then costs two memory round trips per batch, not two per
  // token.
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
  // (one sub-tile per wavefront more: the main loop's prefetch past the
  // last sub-tile reads those absent entries, i.e. row 0)
  for (int i = kRatio * n_groups + tid; i < (n_sub + kAttnWaves) * 16; i += kAttnThreads) {
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

  // ---- main loop, rolling: the wave's sub-tiles wave + 4*i in turn;
  // the next sub-tile's K rows (contiguous lane quads, staged through this
  // wave's LDS tile) and V rows are requested before the current one
  // computes, so each memory latency overlaps a sub-tile of work
  // (measured: 199.0 -> 197.9 us per decode step of 8 x 262,144 tokens).
  const int kr_swz = k_swizzle(lq);
  uint8_t* tile = k_lds + (size_t)wave * kItemKBytesPerWave;
  u32x4 kst[kFp8 ? 4 : 8];
  u32x4 vb[2][4][kFp8 ? 1 : 2];
  int rb[2][4];
  if (wave < n_sub) {
    load_k_quads<kFp8>(kst, tok_row + 16 * wave, kc, Hkv, kvh);
    load_v_rows<kFp8, true>(vb[0], rb[0], tok_row + 16 * wave, vc, Hkv, kvh);
  }
  auto step = [&](int s, u32x4 (&vcur)[4][kFp8 ? 1 : 2], int (&rcur)[4],
                  u32x4 (&vnext)[4][kFp8 ? 1 : 2], int (&rnext)[4]) {
    store_k_tile<kFp8>(kst, tile);
    // unconditional (past the last sub-tile it reads absent entries): under
    // a branch, the compiler's wait before the P.V products covered this
    // prefetch too (vmcnt(0) instead of a count that leaves it in flight)
    const int sn = s + kAttnWaves;
    load_k_quads<kFp8>(kst, tok_row + 16 * sn, kc, Hkv, kvh);
    load_v_rows<kFp8, true>(vnext, rnext, tok_row + 16 * sn, vc, Hkv, kvh);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    u32x4 qop[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qop[ks] = *reinterpret_cast<const u32x4*>(q_lds + lq * kQPitch + qk_dim<kFp8>(ks, lg));
    bool vis[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int si = 16 * s + 4 * lg + i;
      const int tok = si < 4 * n_groups ? -1 : it.x_begin + (si - 4 * n_groups);  // -1: visible
      vis[i] = rcur[i] >= 0 && tok < limit;
    }
    const float4_t sc =
        subtile_logits_lds<kFp8>(tile, lq, lg, kr_swz, [&](int ks) { return qop[ks]; });
    subtile_accumulate<kFp8>(sc, vcur, rcur, vis, qk_scale, m_run, l_run, acc);
    // the next store to the tile comes after these operand reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  for (int s = wave; s < n_sub; s += 2 * kAttnWaves) {
    step(s, vb[0], rb[0], vb[1], rb[1]);
    if (s + kAttnWaves < n_sub) step(s + kAttnWaves, vb[1], rb[1], vb[0], rb[0]);
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
        for (int i = 0; i < 4; ++i) rowp[acc_col(out_dim<kFp8>(lg, i, mb))] = acc[mb][i] * fac;
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

  // ---- write the (max, sum, accumulator) partial rows
  for (int e = tid; e < rows_here * kHeadDim; e += kAttnThreads) {
    const int r = e / kHeadDim, d = e % kHeadDim;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) v += acc_lds[((size_t)w * 16 + r) * kAccPitch + acc_col(d)];
    out_partial[(size_t)(row_base + r) * (2 + kHeadDim) + 2 + d] = v;
  }
  if (tid < rows_here) {
    out_partial[(size_t)(row_base + tid) * (2 + kHeadDim)] = ml_lds[kAttnWaves * 32 + tid];
    out_partial[(size_t)(row_base + tid) * (2 + kHeadDim) + 1] = ml_lds[kAttnWaves * 32 + 16 + tid];
  }
}

// Dynamic LDS of a decode workgroup: the row statistics, then one region
// that holds the query tile, the wavefronts' K tiles and the token rows
// during the main loop and the per-wave accumulators during the merge (the
// barrier before the merge writes separates the two uses).
constexpr int kQLdsElems = 16 * (kHeadDim + 16);
constexpr int kMlFloats = (kAttnWaves + 1) * 32;

template <bool kFp8>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_decode_kernel(AttnArgs a) {
  extern __shared__ float smem[];
  const int gq = a.Hq / a.Hkv;
  const int Q = a.q_per_req;
  const int n_rows = Q * gq;
  const int nblk = (n_rows + 15) / 16;
  // workgroup id -> request b = id % batch first: workgroups are dealt to
  // the XCDs round-robin, so with 8 | batch request b's workgroups run on
  // the XCD where the top-K wrote its selection (measured: 4 x 3 MTP
  // positions 78.2 -> 76.7 us per step; 8 x 262,144 tokens unchanged)
  const int b = blockIdx.x % a.batch, rest = blockIdx.x / a.batch;
  const int per_kvh = a.n_splits * nblk;
  const int kvh = rest / per_kvh, sr = rest - kvh * per_kvh;
  const int split = sr / nblk, rb = sr % nblk;
  float* ml_lds = smem;
  float* acc_lds = smem + kMlFloats;
  uint16_t* q_lds = reinterpret_cast<uint16_t*>(acc_lds);
  uint8_t* k_lds = reinterpret_cast<uint8_t*>(q_lds + kQLdsElems);
  int32_t* tok_row = reinterpret_cast<int32_t*>(k_lds + kAttnWaves * kItemKBytesPerWave);

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
                    q_lds, k_lds, tok_row, part);
}

// ---------------------------------------------------------------------------
// Prefill attention: one wavefront per (query, KV head).
//
// The queries of a chunk gather their selected rows from the whole request
// cache (64 MiB for 32,768 BF16 tokens and two KV heads), far more than one
// XCD's 4 MiB L2.  A wavefront walks its query's selection in ascending
// token order (the selection is sorted, the current-block tokens come
// last), so the wavefronts resident on an XCD move through the cache
// together and the rows they read fall in a sliding window.  Workgroups are
// numbered so that each XCD serves one KV head (when the number of KV heads
// divides the 8 XCDs), so that window holds one head's rows (worth about
// 1 % against the plain order).  A workgroup takes four consecutive queries,
// one per wavefront, and each wavefront writes its query's normalised rows
// for the heads of its KV head.  Measured on the 4,096-query chunk over
// 32,768 tokens (K = 512), against cutting the token axis into four ranges,
// one XCD's partition each, with per-range partials merged by a second
// kernel: BF16 1,204-1,241 -> 1,085-1,108 us per prefill step and 4.8 ->
// 3.7-4.4 GB past L2; FP8, against one workgroup per query, 963-973 ->
// 883-889 us and 3.7 -> 1.1 GB.
//
// Random selections make that window wider than it looks: a wavefront's
// position in the token space after a given share of its work varies with
// how its selected groups fall, so the wavefronts of an XCD drift apart
// (a bare gather of random sorted selections took 1.04 ms against 0.69 ms
// for evenly spread ones).  Where the expected drift is large (BF16 rows,
// sparse selections; prefill_paced below) the sweep is paced: a wavefront
// whose position runs ahead of its share of the work, by more than
// kPaceSlack bytes of rows, sleeps until its own average rate catches up,
// its waits kept under kPaceMaxShare of its working time.  Only timing
// changes.  Measured on the BF16 chunk: 1.243 -> 1.065 ms per prefill step,
// L2 hits 75 -> 78 %, 4.33 -> 3.69 GB past L2.

constexpr int kXcds = 8;
constexpr int kPrefillTok = 1024;  // stream entries translated at a time per wavefront
constexpr int kPrefillGpl = kPrefillTok / (kRatio * kWave);  // groups per lane per step
// LDS row of one head's output in the write-out: the accumulator at +4 of a
// 260-float row (the transposed 16-byte stores below then spread over the
// banks)
constexpr int kOutPitch = kHeadDim + 4;
// LDS per wavefront, in floats: the token rows of one translation step,
// then one sub-tile's K tile, then (paced sweeps) the group id that each
// sub-tile of the step starts at; at the end (reused) the transposed output
// rows of the query's heads.
constexpr int kPrefillKFloats = k_tile_bytes<false>() / 4;  // room for either element type
constexpr int kPrefillSubs = kPrefillTok / 16;  // sub-tiles per translation step
// Pacing of the prefill sweep (see attn_prefill_kernel):
//   kPaceSlack     bytes of one KV head's K and V rows a wavefront may run
//                  ahead of its own rate before it waits;
//   kPaceGate      paced only if the expected spread of the wavefronts'
//                  positions exceeds this many bytes;
//   kPaceMaxShare  the waits of a wavefront stay under this share of its
//                  working time.
constexpr int kPaceSlack = 1 << 18;
constexpr int kPaceGate = 1 << 20;
constexpr float kPaceMaxShare = 0.05f;
// K and V bytes of one group (4 tokens) of one KV head
template <bool kFp8>
constexpr int kPaceGroupBytes() { return 2 * kRatio * kHeadDim * (kFp8 ? 1 : 2); }
constexpr int kPrefillWaveFloats = kPrefillTok + 16 + kPrefillKFloats + kPrefillSubs;
constexpr int kOutRowsLds = kPrefillWaveFloats / kOutPitch;  // output rows per LDS pass
static_assert(kOutRowsLds >= 8, "a pass holds at least 8 output rows");

// kWaves queries (one per wavefront) per workgroup; two wavefronts per SIMD
template <bool kFp8, bool kPace, int kWaves>
__global__ __launch_bounds__(kWave * kWaves, 2) void attn_prefill_kernel(AttnArgs a, int n_qb) {
  extern __shared__ float smem[];
  const int gq = a.Hq / a.Hkv;
  // workgroup -> (KV head, query block qb).  With nx = 8 / Hkv, XCD x (=
  // blockIdx % 8, the order in which workgroups are dealt to the XCDs)
  // serves KV head x / nx; other head counts take the linear order.
  const int b = blockIdx.x;
  int kvh, qb;
  if (kXcds % a.Hkv == 0) {
    const int nx = kXcds / a.Hkv, xcd = b % kXcds;
    kvh = xcd / nx;
    qb = (b / kXcds) * nx + xcd % nx;
  } else {
    kvh = b % a.Hkv;
    qb = b / a.Hkv;
  }
  if (qb >= n_qb) return;  // padding: the whole workgroup leaves
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int lq = lane & 15, lg = lane >> 4;
  const int q = qb * kWaves + wave;
  if (q >= a.batch) return;  // whole wavefronts; nothing below synchronises the block
  float* wl = smem + (size_t)wave * kPrefillWaveFloats;
  int32_t* tok = reinterpret_cast<int32_t*>(wl);
  uint8_t* k_lds = reinterpret_cast<uint8_t*>(wl + kPrefillTok + 16);
  // group id of each sub-tile's first selected group in the current step
  int32_t* sgid = reinterpret_cast<int32_t*>(wl + kPrefillTok + 16 + kPrefillKFloats);
  // the 16 entries past a translation step: absent, so the K prefetch past
  // a step's last sub-tile reads row 0 (the translation writes the rest)
  if (lane < 16) tok[kPrefillTok + lane] = -1;

  // the query's selected groups (all complete, all visible), then its
  // current-block tokens 4G .. L - 1
  const int L = a.first_pos + q + 1;
  const int G = L / kRatio;
  const int n_groups = min(a.K, G);
  const int x0 = kRatio * G, n_extra = L - x0;
  const int n_stream = kRatio * n_groups + n_extra;

  // the query rows as the Q^T operand, held in registers: row lq (head
  // kvh * gq + lq, zero past gq), dims qk_dim(ks, lg) + 0..7
  u32x4 qop[8];
  {
    const uint16_t* qr = a.q + ((size_t)q * a.Hq + (size_t)kvh * gq + min(lq, gq - 1)) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qr + qk_dim<kFp8>(ks, lg));
      qop[ks] = lq < gq ? v : (u32x4){0u, 0u, 0u, 0u};
    }
  }
  const int kr_swz = k_swizzle(lq);  // this lane's operand reads: LDS row lq
  const float qk_scale = a.sm_scale * a.k_scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.0f;
  float4_t acc[16];
#pragma unroll
  for (int mb = 0; mb < 16; ++mb) acc[mb] = (float4_t){0.f, 0.f, 0.f, 0.f};
  const uint8_t* kc = reinterpret_cast<const uint8_t*>(a.k);
  const uint8_t* vc = reinterpret_cast<const uint8_t*>(a.v);
  const int32_t* pt = a.page_table + (size_t)a.req * a.max_pages;
  const int32_t* srow = a.sel + (size_t)q * a.K;
  const uint64_t t0 = kPace ? __builtin_amdgcn_s_memrealtime() : 0;
  uint64_t waited = 0;  // pacing waits so far
  const float slack_groups = (float)kPaceSlack / (float)kPaceGroupBytes<kFp8>();

  // the group ids and page ids of a translation step's selected entries:
  // those of the first step are loaded here, those of each next step while
  // the current step's sub-tiles compute (group ids at its start, page ids
  // from its kPhAt-th sub-tile on), so only the first step waits for them
  int gs[kPrefillGpl], ph[kPrefillGpl];
  auto load_gs = [&](int c) {
#pragma unroll
    for (int u = 0; u < kPrefillGpl; ++u) {
      const int e = c + kRatio * (u * kWave + lane);
      gs[u] = e < kRatio * n_groups ? srow[e / kRatio] : -1;
    }
  };
  auto load_ph = [&]() {
#pragma unroll
    for (int u = 0; u < kPrefillGpl; ++u) ph[u] = gs[u] >= 0 ? pt[(kRatio * gs[u]) / kPage] : -1;
  };
  constexpr int kPhAt = 8;
  load_gs(0);
  load_ph();
  for (int c0 = 0; c0 < n_stream; c0 += kPrefillTok) {
    // stream entries c0 + 4*(u*64 + lane) .. + 3 -> physical rows: a selected
    // group's four tokens (one page), or up to four current-block tokens.
    {
      if (kPace) {
#pragma unroll
        for (int u = 0; u < kPrefillGpl; ++u)
          if ((lane & 3) == 0) sgid[u * (kWave / 4) + lane / 4] = gs[u];
      }
#pragma unroll
      for (int u = 0; u < kPrefillGpl; ++u) {
        const int e = c0 + kRatio * (u * kWave + lane);
        int4 rr = make_int4(-1, -1, -1, -1);
        if (e < kRatio * n_groups) {
          if (gs[u] >= 0 && ph[u] >= 0 && ph[u] < a.num_pages) {
            const int base = ph[u] * kPage + (kRatio * gs[u]) % kPage;
            rr = make_int4(base, base + 1, base + 2, base + 3);
          }
        } else if (e < n_stream) {
          int t4[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int sx = e + k - kRatio * n_groups;
            t4[k] = -1;
            if (sx >= 0 && sx < n_extra) {
              const int t = x0 + sx;
              const int pg = pt[t / kPage];
              if (pg >= 0 && pg < a.num_pages) t4[k] = pg * kPage + t % kPage;
            }
          }
          rr = make_int4(t4[0], t4[1], t4[2], t4[3]);
        }
        *reinterpret_cast<int4*>(tok + kRatio * (u * kWave + lane)) = rr;
      }
    }
    const bool has_next = c0 + kPrefillTok < n_stream;
    if (has_next) load_gs(c0 + kPrefillTok);
    // LDS operations of one wavefront execute in order; the fences keep the
    // compiler from moving the reads below above the writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int n_sub = min(kPrefillTok / 16, (n_stream - c0 + 15) / 16);
    // K rows one sub-tile ahead: sub-tile s + 1's loads are issued into the
    // registers s's rows leave once they are in LDS, so they arrive while s
    // computes.  The prefetch is unconditional (past the step's last
    // sub-tile it reads absent entries, i.e. row 0): with it under a branch,
    // the compiler's wait before the P.V products covered the prefetch too
    // (vmcnt(0) instead of a count that leaves it in flight).
    u32x4 kst[kFp8 ? 4 : 8];
    if (n_sub > 0) load_k_quads<kFp8>(kst, tok, kc, a.Hkv, kvh);
    for (int s = 0; s < n_sub; ++s) {
      const int32_t* ts = tok + 16 * s;
      if (s == kPhAt && has_next) load_ph();  // a step with a next one is full
      // pacing: a wavefront whose position in the token space (group id over
      // G) runs ahead of its share of the work (selection index over
      // n_groups) waits until its own average rate catches up, so that the
      // wavefronts of an XCD sweep the cache together
      if (kPace && (s & 3) == 0) {
        const int j = (c0 + 16 * s) / kRatio;
        if (j >= 64 && j < n_groups) {
          const int gid = __builtin_amdgcn_readfirstlane(sgid[s]);
          // position fraction less the slack a wavefront may run ahead
          // (kPaceSlack bytes of one KV head's K and V rows)
          const float x = ((float)gid - slack_groups) * __builtin_amdgcn_rcpf((float)G);
          const float lead = x * (float)n_groups * __builtin_amdgcn_rcpf((float)j) - 1.0f;
          if (lead > 0.0f) {
            // work time so far (elapsed minus earlier waits) sets the
            // wavefront's own rate; the wait brings its position and its
            // elapsed time back into that ratio, less what it already waited
            const uint64_t now = __builtin_amdgcn_s_memrealtime();
            const float work = (float)(now - t0 - waited);
            const float w = fminf(lead, kPaceMaxShare) * work - (float)waited;
            if (w > 0.0f) {
              // the real-time counter runs at 100 MHz; the spin is also
              // bounded by a count of sleeps (each >= 128 clocks), so it
              // ends even if the counter stood still
              const uint64_t until = now + (uint64_t)w;
              uint64_t t = now;
              for (int spins = 0; t < until && spins < (1 << 16); ++spins) {
                __builtin_amdgcn_s_sleep(2);
                t = __builtin_amdgcn_s_memrealtime();
              }
              waited += t - now;
            }
          }
        }
      }
      // V rows in operand order
      u32x4 vr[4][kFp8 ? 1 : 2];
      int rv[4];
      load_v_rows<kFp8, false>(vr, rv, ts, vc, a.Hkv, kvh);
      store_k_tile<kFp8>(kst, k_lds);
      load_k_quads<kFp8>(kst, ts + 16, kc, a.Hkv, kvh);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      bool vis[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) vis[k] = rv[k] >= 0;
      const float4_t sc =
          subtile_logits_lds<kFp8>(k_lds, lq, lg, kr_swz, [&](int ks) { return qop[ks]; });
      subtile_accumulate<kFp8>(sc, vr, rv, vis, qk_scale, m_run, l_run, acc);
      // the next sub-tile's stores come after these operand reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- the query's rows: row lq's sum over its four lanes, the normalised
  // accumulator transposed through LDS (acc[mb][i] of lane (lq, lg) is
  // dimension out_dim(lg, i, mb); runs of four consecutive mb are four
  // consecutive dimensions) and written with 16-byte stores, up to
  // kOutRowsLds rows at a time
  float l = l_run;
  l += __shfl_xor(l, 16, kWave);
  l += __shfl_xor(l, 32, kWave);
  const float f = l > 0.0f ? a.v_scale / l : 0.0f;  // no visible token: zeros
#pragma unroll
  for (int mb = 0; mb < 16; ++mb)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[mb][k] *= f;
  float4* dst = reinterpret_cast<float4*>(a.out + ((size_t)q * a.Hq + (size_t)kvh * gq) * kHeadDim);
  const float4* srcl = reinterpret_cast<const float4*>(wl);
  for (int h0 = 0; h0 < gq; h0 += kOutRowsLds) {
    if (lq >= h0 && lq < min(gq, h0 + kOutRowsLds)) {
      float* rowp = wl + (lq - h0) * kOutPitch;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          *reinterpret_cast<float4*>(rowp + 4 + out_dim<kFp8>(lg, i, 4 * c)) =
              make_float4(acc[4 * c][i], acc[4 * c + 1][i], acc[4 * c + 2][i], acc[4 * c + 3][i]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int nf4 = (min(gq, h0 + kOutRowsLds) - h0) * (kHeadDim / 4);
    for (int e = lane; e < nf4; e += kWave) {
      const int rw = e / (kHeadDim / 4), c = e % (kHeadDim / 4);
      dst[(h0 + rw) * (kHeadDim / 4) + c] = srcl[rw * (kOutPitch / 4) + 1 + c];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Merge split partials: out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
// Thread s first fetches split s's (m, l) so all splits are read at once;
// then thread d sums the accumulators with independent loads.
// A partial row is 2 + 256 floats: max, sum, then the accumulator.
constexpr int kMaxSplits = kHeadDim;
__global__ __launch_bounds__(kHeadDim) void combine_kernel(const float* __restrict__ partial,
                                                           int n_splits, int Hq, int Hkv, int Q,
                                                           float v_scale, float* __restrict__ out) {
  constexpr int pitch = 2 + kHeadDim, acc_off = 2;
  __shared__ float fac[kMaxSplits];
  __shared__ float red[kHeadDim / kWave];
  // request first, as the attention workgroups that wrote the partials
  const int B = gridDim.x / (Hq * Q);
  const int b = blockIdx.x % B, rest = blockIdx.x / B;
  const int h = rest % Hq, j = rest / Hq;
  const int gq = Hq / Hkv, kvh = h / gq, r = j * gq + (h % gq);
  const int R = Q * gq;
  const size_t split_stride = (size_t)R * pitch;
  const float* p = partial + ((size_t)(b * Hkv + kvh) * n_splits) * split_stride +
                   (size_t)r * pitch;
  const int t = threadIdx.x, lane = t & (kWave - 1), wid = t / kWave;
  // the first kEarly splits' accumulators are fetched together with the
  // (max, sum) pairs, so both come back in one memory round trip
  constexpr int kEarly = 32;
  float early[kEarly];
#pragma unroll
  for (int s = 0; s < kEarly; ++s) early[s] = s < n_splits ? p[s * split_stride + acc_off + t] : 0.0f;
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
  for (int s = kEarly; s < n_splits; ++s) num += fac[s] * p[s * split_stride + acc_off + t];
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
                      (size_t)kAttnWaves * kItemKBytesPerWave +
                      sizeof(int32_t) * (size_t)((stream_cap + 15) / 16 * 16 + 16 * kAttnWaves);
  return sizeof(float) * (size_t)kMlFloats + (acc > loop ? acc : loop);
}

template <bool kFp8>
hipError_t launch_decode_t(const AttnArgs& a, hipStream_t stream) {
  if (a.n_splits > kMaxSplits) return hipErrorInvalidValue;
  const int cap = 4 * a.groups_per_split + 3 + (a.q_per_req - 1);
  const size_t smem = attn_smem_bytes(cap);
  const int rows = a.q_per_req * (a.Hq / a.Hkv);
  const int nblk = (rows + 15) / 16;
  dim3 grid(a.n_splits * nblk * a.Hkv * a.batch);
  hipLaunchKernelGGL((attn_decode_kernel<kFp8>), grid, dim3(kAttnThreads), smem, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 cgrid(a.Hq * a.q_per_req * a.batch);
  hipLaunchKernelGGL(combine_kernel, cgrid, dim3(kHeadDim), 0, stream, a.partial, a.n_splits, a.Hq,
                     a.Hkv, a.q_per_req, a.v_scale, a.out);
  return hipGetLastError();
}

template <bool kFp8, bool kPace, int kWaves>
hipError_t launch_prefill_t(const AttnArgs& a, hipStream_t stream) {
  if (a.Hq / a.Hkv > 16) return hipErrorInvalidValue;
  const int n_qb = (a.batch + kWaves - 1) / kWaves;
  size_t n_wg = (size_t)n_qb * a.Hkv;
  if (kXcds % a.Hkv == 0) {
    const int nx = kXcds / a.Hkv;
    n_wg = (size_t)((n_qb + nx - 1) / nx) * kXcds;
  }
  const size_t smem = sizeof(float) * (size_t)kWaves * kPrefillWaveFloats;
  hipLaunchKernelGGL((attn_prefill_kernel<kFp8, kPace, kWaves>), dim3((unsigned)n_wg), dim3(kWave * kWaves), smem,
                     stream, a, n_qb);
  return hipGetLastError();
}

// Whether a prefill chunk's sweep is paced.  With n groups drawn evenly at
// random from G, the position of a wavefront's middle group varies by about
// G / (2 sqrt(n)) groups; the chunk is paced when twice that, in bytes of one
// KV head's K and V, exceeds kPaceGate (and each query keeps >= 128 groups).
bool prefill_paced(const AttnArgs& a) {
  const double G = (double)(a.first_pos + a.batch) / kRatio;
  const double n = std::min((double)a.K, G);
  if (n < 128) return false;
  const int gb = a.kv_dtype == 1 ? kPaceGroupBytes<true>() : kPaceGroupBytes<false>();
  return G / std::sqrt(n) * gb > (double)kPaceGate;
}

// One 16-row block per workgroup: query rows beyond 16 (e.g. 12 heads x 3
// draft positions) take further workgroups over the same tokens, which
// then mostly come from the caches.
hipError_t dispatch(const AttnArgs& a, hipStream_t stream, bool prefill) {
  if (!prefill)
    return a.kv_dtype == 1 ? launch_decode_t<true>(a, stream) : launch_decode_t<false>(a, stream);
  // Paced BF16 sweeps take eight queries per workgroup (one per CU), the
  // rest four (two per CU): eight made the BF16 chunk at K = 512 5 % faster
  // and FP8 and K = 2,048 2-5 % slower.
  const bool pace = prefill_paced(a);
  if (a.kv_dtype == 1)
    return pace ? launch_prefill_t<true, true, 4>(a, stream)
                : launch_prefill_t<true, false, 4>(a, stream);
  return pace ? launch_prefill_t<false, true, 8>(a, stream)
              : launch_prefill_t<false, false, 4>(a, stream);
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
