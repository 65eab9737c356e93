// index_score_prefill.hip — indexer scoring of a prefill chunk on the
// matrix cores.
//
// For every query i of the chunk (L_i = first_pos + i + 1 tokens) and every
// complete group g < floor(L_i / 4) of the request (the 4-token groups of
// the "QSA in brief" section of the Qwen3.8-27B QSA model card; the scoring
// form is the library's stated reading, since the pages give none):
//   score[i][g] = sum_h w[i][h] * max(0, sum_d q[i][h][d] * khat[g][h][d])
// with 8 heads of 64 dims; other entries are -inf.  With thousands of
// queries this is a dense contraction (4,096 queries x 8,192 groups x 512
// for the long-prefill chunk), so it runs on the bf16 MFMA units: q and k̂
// are rounded to bf16 (nearest-even), every product is exact and the sums
// are fp32.
//
// Work split.  A workgroup of 8 wavefronts owns 256 queries (32 per wave)
// and sweeps a range of 32-group blocks:
//   - each wave keeps its 32 queries' q, all 8 heads, as MFMA B operands
//     in registers for the whole sweep (128 VGPRs) and its weights w;
//   - per block, the workgroup converts the block's k̂ (32 groups x 2 KiB
//     fp32) to bf16 into one of two LDS buffers, in exactly the operand
//     order of v_mfma_f32_32x32x16_bf16, so every A-operand read is one
//     conflict-free 16-byte LDS load; the next block's k̂ is fetched from
//     memory while the current block is computed;
//   - per block and head a wave issues 4 MFMAs (the 64-dim contraction)
//     into a 32 x 32 tile (groups x queries), then folds
//     w * max(0, .) into the running score tile;
//   - the finished 32 x 32 tile is masked and stored, each lane writing 16
//     consecutive bytes of its query's score row per store.
// The contraction index inside a head is permuted identically in both
// operands (a dot product does not depend on the order of its terms): lane
// half hf, k-step s, element j covers dim 32*hf + 8*s + j, so each lane's
// q operands and each k̂ staging thread read 128 contiguous bytes.
// Workgroups are numbered so that those sharing a sweep of k̂ run on the
// same XCD and find it in that XCD's L2.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {
namespace {

constexpr int kPfWaves = 8;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfQueries = 32 * kPfWaves;  // queries per workgroup
constexpr int kPfGroups = 32;              // groups per block
// LDS slots are 16 bytes (8 bf16, one MFMA operand per lane).  A k̂ block
// is [key head][k-step][half] rows of 32 group slots; q staging is rows of
// 256 query slots.  Each row is padded by one slot, so that the 32 rows a
// wavefront writes at once (one group or query, all heads) start in
// different LDS banks.
constexpr int kKPitch = kPfGroups + 1;
constexpr int kQPitch = kPfQueries + 1;
constexpr int kXcds = 8;

// Indexer forms: kH query heads of kD dims per query row; each group's k̂
// holds kHk key heads, query head h reading key head h * kHk / kH.
//   - per-head form: 8 heads x 64 dims, one key per head (2 KiB per group);
//   - multi-query form (OrcaRouter article on PR #41855, "Warum QSA der
//     heikle Teil ist - in Zahlen"): 4 heads x 128 dims sharing one key
//     head (512 B per group).
template <int H, int Hk, int D>
struct Form {
  static constexpr int kH = H, kHk = Hk, kD = D;
  static constexpr int kS = D / 16;           // MFMA k-steps per head
  static constexpr int kGF = Hk * D;          // fp32 per group of k̂
  static constexpr int kQF = H * D;           // fp32 per query row
  static constexpr int kKBlockSlots = Hk * kS * 2 * kKPitch;
  static constexpr int kQRoundHeads = 16 / kS;  // 256 fp32 of a query row per staging round
  static constexpr int kQRounds = H / kQRoundHeads;
  static constexpr int kQSlots = kQRoundHeads * kS * 2 * kQPitch;  // 8,224 slots = 128.5 KiB
  static constexpr int kLdsSlots = kQSlots > 2 * kKBlockSlots ? kQSlots : 2 * kKBlockSlots;
  static constexpr int kPagesF4 = kGroupsPerPage * kGF / 4;  // float4 per k̂ page
  static constexpr int kFetch = 2 * kPagesF4 / kPfThreads;    // float4 per thread per block
  static_assert(kQRoundHeads * D == 256 && H % kQRoundHeads == 0 && H % Hk == 0, "form");
  static_assert(kFetch >= 1 && (kPagesF4 & (kPagesF4 - 1)) == 0, "form");
};
using PerHeadForm = Form<kIdxHeads, kIdxHeads, kIdxDim>;
using SharedKeyForm = Form<4, 1, 128>;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 4 fp32 -> 4 bf16 (round to nearest even): half an operand slot.
__device__ __forceinline__ u32x2 pack4_bf16(float4 a) {
  const bf16x2_t p0 = {(__bf16)a.x, (__bf16)a.y};
  const bf16x2_t p1 = {(__bf16)a.z, (__bf16)a.w};
  return (u32x2){__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
}

template <class F>
__global__ __launch_bounds__(kPfThreads, 1) void index_score_mfma_kernel(
    const float* __restrict__ khat, const int32_t* __restrict__ page_table, int max_pages,
    int num_pages, int req, int first_pos, int n_q, const float* __restrict__ q_idx,
    const float* __restrict__ w_idx, float* __restrict__ scores, int gstride, int n_qt,
    int blocks_per_sweep) {
  // two k̂ block buffers; at the start the same memory stages q
  constexpr int kH = F::kH, kS = F::kS, kD = F::kD, kQRoundHeads = F::kQRoundHeads;
  constexpr int kKBlockSlots = F::kKBlockSlots;
  __shared__ u32x4 lds[F::kLdsSlots];

  // workgroup -> (query tile, sweep).  Workgroups are dealt to the XCDs
  // round-robin, so linear id lin = (b % 8) * (nb / 8) + b / 8 gives each
  // XCD a contiguous range of lin; lin is laid out in groups of 4 query
  // tiles x all sweeps, so an XCD's range covers a few query tiles (whose q
  // it reads once into its L2) and a run of sweeps shared by those tiles.
  const int nb = gridDim.x, b = blockIdx.x;
  const int lin = (nb % kXcds == 0) ? (b % kXcds) * (nb / kXcds) + b / kXcds : b;
  const int n_sw = nb / n_qt;
  const int qgrp = (n_qt % 4 == 0) ? 4 : 1;
  const int qt = (lin / (qgrp * n_sw)) * qgrp + lin % qgrp;
  const int sw = (lin % (qgrp * n_sw)) / qgrp;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int ql = lane & 31, hf = lane >> 5;
  const int q_wave = qt * kPfQueries + wave * 32;
  const int qi = q_wave + ql;  // this lane's query (MFMA column)
  const bool q_ok = qi < n_q;
  const int n_gb = (gstride + kPfGroups - 1) / kPfGroups;
  const int gb_begin = sw * blocks_per_sweep;
  const int gb_end = min(n_gb, gb_begin + blocks_per_sweep);
  // groups visible to any query of the wave / the workgroup (G grows with i)
  const int G_wave = q_wave < n_q ? (first_pos + min(q_wave + 32, n_q)) / kRatio : 0;
  const int G_wg = (first_pos + min(qt * kPfQueries + kPfQueries, n_q)) / kRatio;
  const int G_q = q_ok ? (first_pos + qi + 1) / kRatio : 0;
  const int gb_live = min(gb_end, (G_wg + kPfGroups - 1) / kPfGroups);
  const int32_t* pt = page_table + (size_t)req * max_pages;

  // ---- this lane's query: q as B operands (all heads) and its weights.
  // The workgroup's 256 q rows are contiguous in memory; they are staged
  // through LDS in two rounds of four heads.  In each round a wavefront
  // load instruction reads 1 KiB of one row (coalesced), each lane
  // converts its 4 values to bf16 and writes them to their operand slot;
  // then every lane picks up its own query's 16 operands.  Rows past the
  // chunk repeat the last row: a query column only feeds its own scores,
  // which are not stored.
  u32x4 qb[kH][kS];
  float wv[kH];
  {
    const int qr = min(qi, n_q - 1);
#pragma unroll
    for (int h = 0; h < kH; ++h) wv[h] = w_idx[(size_t)qr * kH + h];
    u32x2* lds8 = reinterpret_cast<u32x2*>(lds);
#pragma unroll
    for (int rd = 0; rd < F::kQRounds; ++rd) {
      constexpr int kPer = kPfQueries * kQRoundHeads * (kD / 4) / kPfThreads;  // 32 float4
      float4 x[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int f = i * kPfThreads + tid;
        const int r = f >> 6, c = f & 63;  // row, float4 within the round's heads
        const int row = min(qt * kPfQueries + r, n_q - 1);
        x[i] = reinterpret_cast<const float4*>(q_idx + (size_t)row * F::kQF +
                                               rd * kQRoundHeads * kD)[c];
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int f = i * kPfThreads + tid;
        const int r = f >> 6, c = f & 63;
        // dims 4m.. of head hh = chunk cc (k-step cc % kS, lane half cc / kS)
        const int hh = c / (kD / 4), m = c % (kD / 4), cc = m >> 1;
        const int slot = ((hh * kS + cc % kS) * 2 + cc / kS) * kQPitch + r;
        lds8[2 * slot + (m & 1)] = pack4_bf16(x[i]);
      }
      __syncthreads();
#pragma unroll
      for (int hh = 0; hh < kQRoundHeads; ++hh)
#pragma unroll
        for (int s = 0; s < kS; ++s)
          qb[rd * kQRoundHeads + hh][s] =
              lds[((hh * kS + s) * 2 + hf) * kQPitch + wave * 32 + ql];
      __syncthreads();
    }
  }

  // ---- staging of a block (2 pages, 64 KiB of fp32): thread t loads
  // float4 number i * 512 + t of the block, so a wavefront instruction
  // reads 1 KiB of one page (coalesced).  The two page ids of a block are
  // workgroup-uniform and come through the scalar cache one block ahead.
  struct Pages { int p0, p1; };
  auto pages_of = [&](int gb) {
    Pages r = {-1, -1};
    if (gb < gb_live) {
      const int pg = gb * (kPfGroups / kGroupsPerPage);
      r.p0 = pt[pg];
      if (gb * kPfGroups + kGroupsPerPage < gstride) r.p1 = pt[pg + 1];
    }
    return r;
  };
  auto page_valid = [&](int p) { return p >= 0 && p < num_pages; };
  constexpr int kPagesF4 = F::kPagesF4;  // 2,048 (per-head form) or 512 float4 per page
  constexpr int kFetch = F::kFetch;      // 8 or 2 float4 per thread
  float4 pre[kFetch];
  // A page that is out of range (or past the row) is read as page 0
  // instead, always a valid address: its groups' k̂ feed only their own
  // score columns, which the store masks to -inf.  Loading unconditionally
  // also keeps the destination registers free of VALU writes, so no wait
  // for the previous block's score stores is needed here.
  auto fetch = [&](int gb, Pages pg) {
    const float* base0 = khat + (size_t)(page_valid(pg.p0) ? pg.p0 : 0) * kPagesF4 * 4;
    const float* base1 = khat + (size_t)(page_valid(pg.p1) ? pg.p1 : 0) * kPagesF4 * 4;
#pragma unroll
    for (int i = 0; i < kFetch; ++i) {
      const int f = i * kPfThreads + tid;
      const float* base = (f < kPagesF4) ? base0 : base1;
      pre[i] = reinterpret_cast<const float4*>(base)[f & (kPagesF4 - 1)];
    }
  };
  auto stash = [&](int buf) {
    u32x2* kl8 = reinterpret_cast<u32x2*>(lds + buf * kKBlockSlots);
#pragma unroll
    for (int i = 0; i < kFetch; ++i) {
      const int f = i * kPfThreads + tid;
      const int e = f & (kPagesF4 - 1);
      const int g = (f / kPagesF4) * kGroupsPerPage + e / (F::kGF / 4);  // group within the block
      const int col = e % (F::kGF / 4), kh = col / (kD / 4), m = col % (kD / 4), cc = m >> 1;
      const int slot = ((kh * kS + cc % kS) * 2 + cc / kS) * kKPitch + g;
      kl8[2 * slot + (m & 1)] = pack4_bf16(pre[i]);
    }
  };

  // ---- output of one 32 x 32 tile: lane (query ql) owns groups
  // g0 + 8*k + 4*hf + 0..3 in registers 4k .. 4k+3 (page g0/16 + k/2)
  const bool vec_ok = (gstride & 3) == 0;
  float* srow = scores + (size_t)(q_ok ? qi : 0) * gstride;
  auto store = [&](int gb, const f32x16& sc, bool live, Pages pg) {
    if (!q_ok) return;
    const int g0 = gb * kPfGroups;
    const bool ok0 = live && page_valid(pg.p0), ok1 = live && page_valid(pg.p1);
    // common case: the whole block is visible to every query of the wave
    if (vec_ok && ok0 && ok1 && g0 + kPfGroups <= gstride &&
        g0 + kPfGroups <= (first_pos + q_wave + 1) / kRatio) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *reinterpret_cast<float4*>(srow + g0 + 8 * k + 4 * hf) =
            make_float4(sc[4 * k], sc[4 * k + 1], sc[4 * k + 2], sc[4 * k + 3]);
      return;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int gq = g0 + 8 * k + 4 * hf;
      const bool page_ok = k < 2 ? ok0 : ok1;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = (page_ok && gq + i < G_q) ? sc[4 * k + i] : -INFINITY;
      if (vec_ok) {
        if (gq < gstride)
          *reinterpret_cast<float4*>(srow + gq) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (gq + i < gstride) srow[gq + i] = v[i];
      }
    }
  };

  // ---- blocks that some query of the workgroup can see
  Pages pg_cur = pages_of(gb_begin), pg_next = pages_of(gb_begin + 1);
  if (gb_begin < gb_live) {
    fetch(gb_begin, pg_cur);
    stash(0);
  }
  __syncthreads();
  for (int gb = gb_begin; gb < gb_live; ++gb) {
    const int buf = (gb - gb_begin) & 1;
    const bool more = gb + 1 < gb_live;
    if (more) fetch(gb + 1, pg_next);
    const Pages pg_after = pages_of(gb + 2);
    f32x16 sc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = 0.0f;
    const bool live = gb * kPfGroups < G_wave;
    if (live) {
      // Two heads in flight: the MFMAs of head h are issued before the VALU
      // fold of head h - 1, so the matrix pipe works while the fold runs;
      // the fences keep the compiler from hoisting further heads (16 more
      // VGPRs each).  ReLU is an integer max on the bit pattern (negative
      // floats are negative integers; -0 becomes +0).
      const u32x4* kb = lds + buf * kKBlockSlots + hf * kKPitch + ql;
      // with one key head (multi-query form) all heads share the A
      // operands: they are read from LDS once per block
      constexpr bool kShared = F::kHk == 1;
      u32x4 ash[kShared ? kS : 1];
      if (kShared) {
#pragma unroll
        for (int s = 0; s < kS; ++s) ash[s] = kb[s * 2 * kKPitch];
      }
      auto head = [&](int h) {
        f32x16 acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int s = 0; s < kS; ++s) {
          const u32x4 a = kShared ? ash[kShared ? s : 0]
                                  : kb[((h * F::kHk / kH) * kS + s) * 2 * kKPitch];
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, qb[h][s]), acc,
                                                        0, 0, 0);
        }
        return acc;
      };
      f32x16 prev = head(0);
#pragma unroll
      for (int h = 1; h <= kH; ++h) {
        f32x16 cur;
        if (h < kH) cur = head(h);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sc[i] += wv[h - 1] * __int_as_float(max(__float_as_int(prev[i]), 0));
        __builtin_amdgcn_sched_barrier(0);
        if (h < kH) prev = cur;
      }
    }
    if (more) stash(buf ^ 1);
    store(gb, sc, live, pg_cur);
    pg_cur = pg_next;
    pg_next = pg_after;
    __syncthreads();
  }
  // ---- blocks past every query's causal limit: -inf only, written by the
  // whole workgroup with row-contiguous stores
  const int c0 = max(gb_begin, gb_live) * kPfGroups, c1 = min(gb_end * kPfGroups, gstride);
  if (c0 < c1) {
    const int row0 = qt * kPfQueries;
    const int rows = min(kPfQueries, n_q - row0);
    if (vec_ok) {
      const int nf4 = (c1 - c0) / 4;
      const float4 ninf = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      for (int idx = tid; idx < rows * nf4; idx += kPfThreads) {
        const int r = idx / nf4, j = idx - r * nf4;
        *reinterpret_cast<float4*>(scores + (size_t)(row0 + r) * gstride + c0 + 4 * j) = ninf;
      }
    } else {
      const int n = c1 - c0;
      for (int idx = tid; idx < rows * n; idx += kPfThreads) {
        const int r = idx / n, j = idx - r * n;
        scores[(size_t)(row0 + r) * gstride + c0 + j] = -INFINITY;
      }
    }
  }
}

}  // namespace

hipError_t launch_index_score_prefill(const float* khat, const int32_t* page_table,
                                      int max_pages, int num_pages, int req, int first_pos,
                                      int n_q, const float* q_idx, const float* w_idx,
                                      float* scores, int gstride, hipStream_t stream,
                                      bool shared_key) {
  if (n_q <= 0 || gstride <= 0) return hipSuccess;
  const int n_qt = (n_q + kPfQueries - 1) / kPfQueries;
  const int n_gb = (gstride + kPfGroups - 1) / kPfGroups;
  // about one workgroup per compute unit: 256 / n_qt sweeps per query tile
  int sweeps = max(1, 256 / n_qt);
  sweeps = min(sweeps, n_gb);
  const int bps = (n_gb + sweeps - 1) / sweeps;
  sweeps = (n_gb + bps - 1) / bps;
  const int grid = n_qt * sweeps;
  auto kern = shared_key ? index_score_mfma_kernel<SharedKeyForm>
                        : index_score_mfma_kernel<PerHeadForm>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kPfThreads), 0, stream, khat,
                     page_table, max_pages, num_pages, req, first_pos, n_q, q_idx, w_idx, scores,
                     gstride, n_qt, bps);
  return hipGetLastError();
}

}  // namespace qsa
