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
// V goes from HBM to registers already in MFMA operand order (16 lanes
// read 256 contiguous bytes of one token's row).  K is either loaded the
// same way (prefill over FP8 caches: lane l reads 64 bytes of token l%16's
// row per instruction) or, in decode and the BF16 range kernel, loaded
// with contiguous lane quads into a per-wavefront LDS tile and read back
// as operands (see the K-through-LDS helpers).  FP8 E4M3 elements are
// widened to bf16 exactly by the hardware converter and the per-tensor
// scales are folded into the logit scale and the final output.  The
// contraction dimension is permuted consistently between the two MFMA
// operands (dot products do not depend on the order of d), which is what
// makes those contiguous loads possible.  Waves merge their (max, sum,
// accumulator) through LDS at the end.  Decode splits the selection over
// several workgroups and writes (max, sum, accumulator) partials that
// combine_kernel merges.  Prefill over FP8 caches writes normalised rows
// directly; over BF16 caches it works in token-range partitions (below).
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

// Registers of one 16-token sub-tile in flight: lane l holds 64 (fp8) /
// 128 (bf16) K bytes of token lq = l % 16, and 16 / 32 bytes of the V rows
// of tokens 4*lg + j (lg = l / 16).
//
// Dimension order.  A dot product does not depend on the order of its terms,
// so the contraction index of S^T = K . Q^T is permuted identically in both
// operands, chosen so that the four lanes of one token read 64 contiguous
// bytes of its K row in each load instruction (16 cache lines per
// instruction rather than 64): in k-step ks, lane group lg supplies
//   bf16 K: d = 32*ks + 8*lg + 0..7,
//   fp8 K:  d = 64*(ks/2) + 16*lg + 8*(ks%2) + 0..7 (one 16-byte load
//           serves two k-steps).
// The output dimension of O^T = V^T . P^T is permuted through the V^T
// operand: lane lq of m-block mb supplies d = dv(lq, mb) with
//   bf16 V: dv = 8*lq + (mb % 8) + 128*(mb / 8) (two loads of 256
//           contiguous bytes per token across the 16 lanes),
//   fp8 V:  dv = 16*lq + mb (one load of the whole 256-byte row);
// so accumulator acc[mb][i] of lane (lq, lg) holds output dimension
// dv(4*lg + i, mb) of query row lq (out_dim below).
template <bool kFp8>
struct SubTile {
  u32x4 k[kFp8 ? 4 : 8];
  u32x4 v[4][kFp8 ? 1 : 2];
  int rv[4];  // physical rows of the four V tokens (-1: absent)
};

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

// Loads the K part of one 16-token sub-tile: the K rows of tokens
// tok[0..16) (physical row offsets, -1 if absent; absent rows read row 0).
// Load i holds bytes 64*i + 16*lg .. +15 of token lq's K row (k-step i for
// bf16, k-steps 2i and 2i + 1 for fp8).
template <bool kFp8>
__device__ __forceinline__ void load_k_rows(u32x4 (&k)[kFp8 ? 4 : 8], const int32_t* tok,
                                            const uint8_t* kc, int Hkv, int kvh) {
  const int lane = threadIdx.x & (kWave - 1), lq = lane & 15, lg = lane >> 4;
  constexpr int kRowBytes = kHeadDim * (kFp8 ? 1 : 2);
  const uint8_t* kp = kc + ((size_t)max(tok[lq], 0) * Hkv + kvh) * kRowBytes + 16 * lg;
#pragma unroll
  for (int i = 0; i < (kFp8 ? 4 : 8); ++i) k[i] = *reinterpret_cast<const u32x4*>(kp + 64 * i);
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

// Loads one whole sub-tile, K first.
template <bool kFp8, bool kStreamV>
__device__ __forceinline__ void load_subtile(SubTile<kFp8>& b, const int32_t* tok,
                                             const uint8_t* kc, const uint8_t* vc, int Hkv,
                                             int kvh) {
  load_k_rows<kFp8>(b.k, tok, kc, Hkv, kvh);
  load_v_rows<kFp8, kStreamV>(b.v, b.rv, tok, vc, Hkv, kvh);
}

// K rows through LDS (the BF16 prefill range kernel).  Read straight into
// MFMA operand order, the 64 lanes of one load instruction touch 16
// different rows with adjacent lanes in different rows, so no four lanes
// share a 64-byte segment and the vector L1 serves 64 separate accesses per
// instruction, four times the 16 of a load whose lane quads read contiguous
// 64 bytes; where the gathers run at L1 rate, that access count bounds
// them.  Instead lane 4t + c reads bytes 64j + 16c of token t's row in load
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

// The K operand of k-step ks (token lq, dims qk_dim(ks, lg) + 0..7, as
// bf16) from the LDS tile; sw = k_swizzle(lq).
template <bool kFp8>
__device__ __forceinline__ bf16x8 k_operand_lds(const uint8_t* tile, int ks, int lq, int lg,
                                                int sw) {
  constexpr int kRowBytes = kHeadDim * (kFp8 ? 1 : 2);
  if (kFp8) {
    // chunk 4 (ks / 2) + lg holds dims 64 (ks / 2) + 16 lg .. + 15
    const u32x4 w =
        *reinterpret_cast<const u32x4*>(tile + lq * kRowBytes + 16 * ((4 * (ks >> 1) + lg) ^ sw));
    return (ks & 1) ? fp8x8_to_bf16x8(w.z, w.w) : fp8x8_to_bf16x8(w.x, w.y);
  }
  return *reinterpret_cast<const bf16x8*>(tile + lq * kRowBytes + 16 * ((4 * ks + lg) ^ sw));
}

// LDS of one wavefront's K tile in a decode work item (room for either
// element type)
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

// The K operand of k-step ks from a sub-tile's K registers (fp8 widened).
template <bool kFp8>
__device__ __forceinline__ bf16x8 k_operand(const u32x4 (&k)[kFp8 ? 4 : 8], int ks) {
  if (kFp8) {
    const u32x4 w = k[ks / 2];
    return (ks & 1) ? fp8x8_to_bf16x8(w.z, w.w) : fp8x8_to_bf16x8(w.x, w.y);
  }
  return __builtin_bit_cast(bf16x8, k[ks]);
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
  // weights as a bf16 hi + lo pair (~16 significant bits) for the PV MFMA
  float psum = 0.0f;
  uint32_t hb[4], lb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float pw = (m_run == -INFINITY) ? 0.0f : exp2f(sv[i] - m_run);
    hb[i] = bf16_rne_bits(pw);
    lb[i] = bf16_rne_bits(pw - __uint_as_float(hb[i] << 16));
    psum += pw;
  }
  l_run += psum;
  const short4_t p_hi = (short4_t){(short)hb[0], (short)hb[1], (short)hb[2], (short)hb[3]};
  const short4_t p_lo = (short4_t){(short)lb[0], (short)lb[1], (short)lb[2], (short)lb[3]};
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
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, p_lo, acc[mb], 0, 0, 0);
    }
  }
}

// One sub-tile's contribution to the online softmax of the 16 query rows,
// with the Q^T operands qop[ks] in registers.
template <bool kFp8>
__device__ __forceinline__ void subtile_update(SubTile<kFp8>& b, const u32x4 (&qop)[8],
                                               const bool (&vis)[4], float qk_scale,
                                               float& m_run, float& l_run, float4_t (&acc)[16]) {
  const float4_t sc = subtile_logits([&](int ks) { return k_operand<kFp8>(b.k, ks); },
                                     [&](int ks) { return qop[ks]; });
  subtile_accumulate<kFp8>(sc, b.v, b.rv, vis, qk_scale, m_run, l_run, acc);
}

// One work item: the 16 query rows row_base .. row_base + 15 (row r =
// position r / gq, head r % gq of the KV head's group; rows >= n_rows are
// padding) over the item's token stream.  kStreamV (decode): V rows are
// read past the caches (decode reads each selected row once) and K rows go
// through the wavefronts' LDS tiles at k_lds (kAttnWaves x
// kItemKBytesPerWave bytes); prefill keeps V cacheable, since the queries
// of a chunk share the request's KV rows, loads K straight into operand
// order and takes no K tiles (k_lds unused).
template <bool kFp8, bool kStreamV>
__device__ __forceinline__ void attend_item(const AttnArgs& a, const ItemDesc& it, int kvh,
                                            const uint16_t* q_rows, int q_row_stride,
                                            int row_base, int n_rows, int gq, float* acc_lds,
                                            float* ml_lds, uint16_t* q_lds, uint8_t* k_lds,
                                            int32_t* tok_row, float* out_final,
                                            float* out_partial) {
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

  auto load = [&](SubTile<kFp8>& b, int s) {
    load_subtile<kFp8, kStreamV>(b, tok_row + 16 * s, kc, vc, Hkv, kvh);
  };

  auto compute = [&](SubTile<kFp8>& b, int s) {
    // Q operand from LDS: row lq, dims qk_dim(ks, lg) + 0..7
    u32x4 qop[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qop[ks] = *reinterpret_cast<const u32x4*>(q_lds + lq * kQPitch + qk_dim<kFp8>(ks, lg));
    // token of D row 4*lg + i is stream entry 16s + 4*lg + i (= V token i)
    bool vis[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int si = 16 * s + 4 * lg + i;
      const int tok = si < 4 * n_groups ? -1 : it.x_begin + (si - 4 * n_groups);  // -1: visible
      vis[i] = b.rv[i] >= 0 && tok < limit;
    }
    subtile_update<kFp8>(b, qop, vis, qk_scale, m_run, l_run, acc);
  };

  if constexpr (kStreamV) {
  // ---- decode main loop, rolling: the wave's sub-tiles wave + 4*i in turn;
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
    load_v_rows<kFp8, kStreamV>(vb[0], rb[0], tok_row + 16 * wave, vc, Hkv, kvh);
  }
  auto step = [&](int s, u32x4 (&vcur)[4][kFp8 ? 1 : 2], int (&rcur)[4],
                  u32x4 (&vnext)[4][kFp8 ? 1 : 2], int (&rnext)[4]) {
    store_k_tile<kFp8>(kst, tile);
    const int sn = s + kAttnWaves;
    if (sn < n_sub) {
      load_k_quads<kFp8>(kst, tok_row + 16 * sn, kc, Hkv, kvh);
      load_v_rows<kFp8, kStreamV>(vnext, rnext, tok_row + 16 * sn, vc, Hkv, kvh);
    }
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
        subtile_logits([&](int ks) { return k_operand_lds<kFp8>(tile, ks, lq, lg, kr_swz); },
                       [&](int ks) { return qop[ks]; });
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
  } else {
  // ---- prefill main loop: rounds of kNS sub-tiles per wave (sub-tiles
  // wave + 4*i), K loaded straight into operand order; a round issues all
  // of its loads before computing any of them, so one memory latency
  // covers kNS sub-tiles (the rolling loop above measured slower here:
  // 955 -> 1,023 us per FP8 prefill step of the 4,096-query chunk)
  constexpr int kNS = kFp8 ? 2 : 1;  // fp8: 3 measured 990 against 966 us, 4 spills
  for (int s0 = wave; s0 < n_sub; s0 += kNS * kAttnWaves) {
    SubTile<kFp8> bt[kNS];
#pragma unroll
    for (int i = 0; i < kNS; ++i)
      if (s0 + i * kAttnWaves < n_sub) load(bt[i], s0 + i * kAttnWaves);
#pragma unroll
    for (int i = 0; i < kNS; ++i)
      if (s0 + i * kAttnWaves < n_sub) compute(bt[i], s0 + i * kAttnWaves);
  }
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

  // ---- write: normalised rows, or (max, sum, accumulator) partials
  for (int e = tid; e < rows_here * kHeadDim; e += kAttnThreads) {
    const int r = e / kHeadDim, d = e % kHeadDim;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) v += acc_lds[((size_t)w * 16 + r) * kAccPitch + acc_col(d)];
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
  attend_item<kFp8, true>(a, it, kvh, q_rows, a.Hq * kHeadDim, rb * 16, n_rows, gq, acc_lds, ml_lds,
                          q_lds, k_lds, tok_row, nullptr, part);
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
  attend_item<kFp8, false>(a, it, kvh, q_rows, 0, 0, gq, gq, acc_lds, ml_lds, q_lds, nullptr,
                           tok_row, outp, nullptr);
}

// ---------------------------------------------------------------------------
// Prefill attention over token partitions.
//
// The queries of a chunk gather their selected rows from the whole request
// cache (64 MiB for 32,768 BF16 tokens and two KV heads), far more than one
// XCD's 4 MiB L2, so a kernel that gives each workgroup one query's whole
// selection reads most rows from beyond L2.  Here the token axis is cut into
// ranges of R tokens whose K and V rows for one KV head take about 2 MiB; a
// partition is (range, KV head).  Workgroups are numbered so that each XCD
// works through its partitions one after another, each for every query of
// the chunk, so the current partition's rows stay in that XCD's L2.  A
// workgroup takes one partition and four consecutive queries, one per
// wavefront; a wavefront attends over its query's selected tokens inside
// the range and writes (max, sum, accumulator) rows for the query's heads
// of that KV head, which combine_ranges_kernel merges over the ranges.

constexpr int kXcds = 8;
constexpr int kRangePitch = kHeadDim + 4;  // partial row: max, sum, 2 unused, accumulator
// Bytes of K and V rows of one KV head per range (an XCD's L2 holds 4 MiB;
// measured on the 4,096-query chunk over 32,768 BF16 tokens: 2 MiB ranges
// 1,824 us per prefill step, 4 MiB 1,648 us, 8 MiB 1,608 us, the per-query
// kernel 1,950 us).
#ifndef QSA_RANGE_KIB
#define QSA_RANGE_KIB 8192
#endif
constexpr int kRangeBytes = QSA_RANGE_KIB << 10;
constexpr int kRangeTok = 1024;            // stream entries translated at a time per wavefront
constexpr int kRangeGpl = kRangeTok / (kRatio * kWave);  // groups per lane per translation step

// LDS per wavefront, in floats: the token rows of one translation step,
// then one sub-tile's K tile; at the end (reused) the transposed partial
// rows of the query's heads.
constexpr int kRangeKFloats = k_tile_bytes<false>() / 4;  // room for either element type

constexpr int kRangeWaveFloats = kRangeTok + 16 + kRangeKFloats;
constexpr int kRangeRowsLds = kRangeWaveFloats / kRangePitch;  // partial rows per LDS pass
static_assert(kRangeRowsLds >= 8, "a pass holds at least 8 partial rows");

// off[q * (NR + 1) + r] = number of entries of query q's selection (ascending
// group ids, -1 padded) whose group lies below range r (group < r * R / 4),
// r = 0 .. NR.  One wavefront per query reads the row in coalesced chunks
// of 64 entries.  Since the entries ascend, off[r] is the index of the
// first entry at or past range r: entry e writes the boundaries between the
// range of entry e - 1 and its own, so every boundary is written once.
__global__ __launch_bounds__(kAttnThreads) void range_offsets_kernel(
    const int32_t* __restrict__ sel, int K, int n_q, int R, int NR, int32_t* __restrict__ off) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int q = blockIdx.x * kAttnWaves + w;
  if (q >= n_q) return;
  const int gpr = R / kRatio;  // groups per range
  const int32_t* row = sel + (size_t)q * K;
  int32_t* o = off + (size_t)q * (NR + 1);
  int prev_r = -1;   // range of the entry before this chunk (wave-uniform)
  int n_valid = 0;   // valid entries so far (a prefix of the row)
  for (int c0 = 0; c0 < K; c0 += kWave) {
    const int e = c0 + lane;
    const int v = e < K ? row[e] : -1;
    const int rr = v >= 0 ? min(v / gpr, NR) : -1;
    int before = __shfl_up(rr, 1, kWave);  // range of entry e - 1
    if (lane == 0) before = prev_r;
    if (v >= 0)
      for (int b = max(before, -1) + 1; b <= rr; ++b) o[b] = e;
    const uint64_t valid = __ballot(v >= 0);
    n_valid += __popcll(valid);
    const int last = valid ? 63 - __clzll(valid) : -1;  // last valid lane of the chunk
    if (last >= 0) prev_r = __shfl(rr, last, kWave);
    if (valid != ~0ull) break;  // the valid entries have ended
  }
  // boundaries past the last valid entry's range (all of them when the
  // selection is empty)
  for (int b = prev_r + 1 + lane; b <= NR; b += kWave) o[b] = n_valid;
}

// Merge of the prefill range partials, one workgroup per (query, KV head):
// out = sum_r 2^(m_r - M) acc_r / sum_r 2^(m_r - M) l_r over the ranges r.
// The first gq threads turn each head's (max, sum) pairs into one factor
// per partial row; then every thread owns four output dimensions of one
// head at a time, with all of that head's range loads in flight together.
constexpr int kMaxRanges = 32;
__global__ __launch_bounds__(kHeadDim) void combine_ranges_kernel(
    const float* __restrict__ part, int NR, int Hq, int Hkv, float v_scale,
    float* __restrict__ out) {
  __shared__ float fac[kMaxRanges * 16];
  const int b = blockIdx.x / Hkv, kvh = blockIdx.x - b * Hkv;
  const int gq = Hq / Hkv, t = threadIdx.x;
  const float* p = part + ((size_t)b * Hkv + kvh) * NR * gq * kRangePitch;
  if (t < gq) {
    float M = -INFINITY;
    for (int s = 0; s < NR; ++s) M = fmaxf(M, p[((size_t)s * gq + t) * kRangePitch]);
    float den = 0.0f;
    for (int s = 0; s < NR; ++s) {
      const float* row = p + ((size_t)s * gq + t) * kRangePitch;
      const float f = row[0] == -INFINITY ? 0.0f : exp2f(row[0] - M);
      fac[s * gq + t] = f;
      den += f * row[1];
    }
    // a head with no visible token (den = 0) outputs exact zeros
    const float sc = den > 0.0f ? v_scale / den : 0.0f;
    for (int s = 0; s < NR; ++s) fac[s * gq + t] *= sc;
  }
  __syncthreads();
  constexpr int kRowsPerPass = kHeadDim / (kHeadDim / 4);  // 4 heads per pass
  const int d4 = t % (kHeadDim / 4), r0 = t / (kHeadDim / 4);
  for (int r = r0; r < gq; r += kRowsPerPass) {
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int s = 0; s < NR; ++s) {
      const float4 v = *reinterpret_cast<const float4*>(p + ((size_t)s * gq + r) * kRangePitch +
                                                        4 + 4 * d4);
      const float f = fac[s * gq + r];
      num.x += f * v.x; num.y += f * v.y; num.z += f * v.z; num.w += f * v.w;
    }
    *reinterpret_cast<float4*>(out + ((size_t)b * Hq + (size_t)kvh * gq + r) * kHeadDim +
                               4 * d4) = num;
  }
}

template <bool kFp8>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_prefill_ranges_kernel(
    AttnArgs a, int R, int NR, int n_qb, const int32_t* __restrict__ off,
    float* __restrict__ part) {
  extern __shared__ float smem[];
  const int gq = a.Hq / a.Hkv;
  // workgroup -> (partition p, query block qb): XCD x (= blockIdx % 8, the
  // order in which workgroups are dealt to the XCDs) takes partitions
  // x, x + 8, ... in turn, every query block of one before the next
  const int b = blockIdx.x;
  const int xcd = b % kXcds, i = b / kXcds;
  const int j = i / n_qb, qb = i - j * n_qb;
  const int p = kXcds * j + xcd;
  if (p >= NR * a.Hkv) return;  // padding partition: the whole workgroup leaves
  const int r = p / a.Hkv, kvh = p - r * a.Hkv;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int lq = lane & 15, lg = lane >> 4;
  const int q = qb * kAttnWaves + wave;
  if (q >= a.batch) return;  // whole wavefronts; nothing below synchronises the block
  float* wl = smem + (size_t)wave * kRangeWaveFloats;
  int32_t* tok = reinterpret_cast<int32_t*>(wl);
  uint8_t* k_lds = reinterpret_cast<uint8_t*>(wl + kRangeTok + 16);

  // the query's selected groups and current-block tokens inside the range
  const int L = a.first_pos + q + 1;
  const int G = L / kRatio;
  const int n_valid = min(a.K, G);
  const int t0 = r * R, t1 = min(t0 + R, L);
  int lo = 0, hi = 0, x0 = 0, x1 = 0;
  if (t0 < L) {
    lo = min(off[(size_t)q * (NR + 1) + r], n_valid);
    hi = min(off[(size_t)q * (NR + 1) + r + 1], n_valid);
    x0 = max(kRatio * G, t0);
    x1 = max(x0, t1);
  }
  const int n_groups = max(0, hi - lo), n_extra = x1 - x0;
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
  const int32_t* srow = a.sel + (size_t)q * a.K + lo;

  for (int c0 = 0; c0 < n_stream; c0 += kRangeTok) {
    // stream entries c0 + 4*(u*64 + lane) .. + 3 -> physical rows: a selected
    // group's four tokens (one page), or up to four current-block tokens.
    // All of a lane's selection loads are issued before its page-table
    // loads, so a step costs two memory round trips.
    {
      int gs[kRangeGpl], ph[kRangeGpl];
#pragma unroll
      for (int u = 0; u < kRangeGpl; ++u) {
        const int e = c0 + kRatio * (u * kWave + lane);
        gs[u] = e < kRatio * n_groups ? srow[e / kRatio] : -1;
      }
#pragma unroll
      for (int u = 0; u < kRangeGpl; ++u) ph[u] = gs[u] >= 0 ? pt[(kRatio * gs[u]) / kPage] : -1;
#pragma unroll
      for (int u = 0; u < kRangeGpl; ++u) {
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
    // LDS operations of one wavefront execute in order; the fences keep the
    // compiler from moving the reads below above the writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int n_sub = min(kRangeTok / 16, (n_stream - c0 + 15) / 16);
    // K rows one sub-tile ahead: sub-tile s + 1's loads are issued into the
    // registers s's rows leave once they are in LDS, so they arrive while s
    // computes
    u32x4 kst[kFp8 ? 4 : 8];
    if (n_sub > 0) load_k_quads<kFp8>(kst, tok, kc, a.Hkv, kvh);
    for (int s = 0; s < n_sub; ++s) {
      const int32_t* ts = tok + 16 * s;
      // V rows in operand order
      u32x4 vr[4][kFp8 ? 1 : 2];
      int rv[4];
      load_v_rows<kFp8, false>(vr, rv, ts, vc, a.Hkv, kvh);
      store_k_tile<kFp8>(kst, k_lds);
      if (s + 1 < n_sub) load_k_quads<kFp8>(kst, ts + 16, kc, a.Hkv, kvh);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      bool vis[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) vis[k] = rv[k] >= 0;
      const float4_t sc =
          subtile_logits([&](int ks) { return k_operand_lds<kFp8>(k_lds, ks, lq, lg, kr_swz); },
                         [&](int ks) { return qop[ks]; });
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

  // ---- the partial rows: row lq's sum over its four lanes, then the
  // accumulator transposed through LDS (acc[mb][i] of lane (lq, lg) is
  // dimension out_dim(lg, i, mb); runs of four consecutive mb are four
  // consecutive dimensions) and written with 16-byte stores, up to
  // kRangeRowsLds rows at a time
  float l = l_run;
  l += __shfl_xor(l, 16, kWave);
  l += __shfl_xor(l, 32, kWave);
  float4* dst = reinterpret_cast<float4*>(part + (((size_t)q * a.Hkv + kvh) * NR + r) * gq *
                                                     kRangePitch);
  const float4* srcl = reinterpret_cast<const float4*>(wl);
  for (int h0 = 0; h0 < gq; h0 += kRangeRowsLds) {
    if (lq >= h0 && lq < min(gq, h0 + kRangeRowsLds)) {
      float* rowp = wl + (lq - h0) * kRangePitch;
      if (lg == 0) *reinterpret_cast<float4*>(rowp) = make_float4(m_run, l, 0.0f, 0.0f);
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
    const int nf4 = (min(gq, h0 + kRangeRowsLds) - h0) * (kRangePitch / 4);
    for (int e = lane; e < nf4; e += kWave) dst[h0 * (kRangePitch / 4) + e] = srcl[e];
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

size_t attn_smem_bytes(int stream_cap, bool k_tiles) {
  const size_t acc = sizeof(float) * (size_t)kAttnWaves * 16 * kAccPitch;
  const size_t loop = sizeof(uint16_t) * (size_t)kQLdsElems +
                      (k_tiles ? (size_t)kAttnWaves * kItemKBytesPerWave : 0) +
                      sizeof(int32_t) * (size_t)((stream_cap + 15) / 16 * 16);
  return sizeof(float) * (size_t)kMlFloats + (acc > loop ? acc : loop);
}

template <bool kFp8>
hipError_t launch_decode_t(const AttnArgs& a, hipStream_t stream) {
  if (a.n_splits > kMaxSplits) return hipErrorInvalidValue;
  const int cap = 4 * a.groups_per_split + 3 + (a.q_per_req - 1);
  const size_t smem = attn_smem_bytes(cap, true);
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

// FP8 K/V: one workgroup per (query, KV head) over the query's whole
// selection.  Its rows are half the size of BF16 rows, and the per-query
// kernel already finds over half of them in L2 (measured: 1,010 us per
// prefill step of the 4,096-query chunk against 1,143 us with ranges).
hipError_t launch_prefill_per_query(const AttnArgs& a, hipStream_t stream) {
  if (a.Hq / a.Hkv > 16) return hipErrorInvalidValue;
  const size_t smem = attn_smem_bytes(4 * a.K + 3, false);
  dim3 grid(a.batch, a.Hkv);
  hipLaunchKernelGGL((attn_prefill_kernel<true>), grid, dim3(kAttnThreads), smem, stream, a);
  return hipGetLastError();
}

// Range partitions (attn_prefill_ranges_kernel), then the merge; taken for
// BF16 K/V (FP8 measured slower here than the per-query kernel: 1,055 against
// 983 us per prefill step of the 4,096-query chunk).
template <bool kFp8>
hipError_t launch_prefill_ranges(const AttnArgs& a, hipStream_t stream) {
  if (a.Hq / a.Hkv > 16) return hipErrorInvalidValue;
  if (!a.range_offsets || !a.partial) return hipErrorInvalidValue;
  int R, NR;
  prefill_ranges(a.kv_dtype, a.Hkv, a.max_ctx, &R, &NR);
  const int n_qb = (a.batch + kAttnWaves - 1) / kAttnWaves;
  hipLaunchKernelGGL(range_offsets_kernel, dim3(n_qb), dim3(kAttnThreads), 0, stream, a.sel, a.K,
                     a.batch, R, NR, a.range_offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int np_pad = (NR * a.Hkv + kXcds - 1) / kXcds * kXcds;
  const size_t smem = sizeof(float) * (size_t)kAttnWaves * kRangeWaveFloats;
  hipLaunchKernelGGL((attn_prefill_ranges_kernel<kFp8>), dim3((unsigned)((size_t)n_qb * np_pad)),
                     dim3(kAttnThreads), smem, stream, a, R, NR, n_qb, a.range_offsets, a.partial);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(combine_ranges_kernel, dim3((unsigned)((size_t)a.batch * a.Hkv)),
                     dim3(kHeadDim), 0, stream, a.partial, NR, a.Hq, a.Hkv, a.v_scale, a.out);
  return hipGetLastError();
}

// One 16-row block per workgroup: query rows beyond 16 (e.g. 12 heads x 3
// draft positions) take further workgroups over the same tokens, which
// then mostly come from the caches.
hipError_t dispatch(const AttnArgs& a, hipStream_t stream, bool prefill) {
  if (a.kv_dtype == 1)
    return prefill ? launch_prefill_per_query(a, stream) : launch_decode_t<true>(a, stream);
  return prefill ? launch_prefill_ranges<false>(a, stream) : launch_decode_t<false>(a, stream);
}

}  // namespace

void prefill_ranges(int kv_dtype, int Hkv, int max_ctx, int* R, int* NR) {
  // K + V rows of one KV head for R tokens take kRangeBytes; at least 8
  // partitions so every XCD has one; at most 32 ranges
  const int esize = kv_dtype == 1 ? 1 : 2;
  const int r_l2 = kRangeBytes / (2 * kHeadDim * esize);
  const int ctx = max(max_ctx, 1);
  int nr = (ctx + r_l2 - 1) / r_l2;
  nr = max(nr, (kXcds + Hkv - 1) / Hkv);
  nr = min(nr, kMaxRanges);
  int r = (ctx + nr - 1) / nr;
  r = (r + kPage - 1) / kPage * kPage;
  *R = r;
  *NR = (ctx + r - 1) / r;
}

size_t prefill_attn_workspace_bytes(int kv_dtype, int Hq, int Hkv, int n_q, int max_ctx,
                                    size_t* off_bytes) {
  if (kv_dtype == 1) {  // the per-query kernel needs no workspace
    if (off_bytes) *off_bytes = 0;
    return 0;
  }
  int R, NR;
  prefill_ranges(kv_dtype, Hkv, max_ctx, &R, &NR);
  const size_t ob = ((size_t)n_q * (NR + 1) * sizeof(int32_t) + 255) / 256 * 256;
  if (off_bytes) *off_bytes = ob;
  return ob + sizeof(float) * (size_t)n_q * Hkv * NR * (Hq / Hkv) * kRangePitch;
}

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
